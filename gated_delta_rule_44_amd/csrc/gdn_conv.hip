// Standalone causal conv1d + SiLU over [saved tail | chunk] with the tail update (gfx950).
//
// y[t][c] = silu(sum_{j<4} w[c][j] * xin[t+j][c]) with xin = [tail (3 rows) | mixed (Lb rows)]; the new
// tail is rows len .. len+2 of xin (the "qev_fast/statecache.py" page, CacheQwen35._gdn: conv on
// [saved conv inputs | chunk] with SiLU and no bias, then the copy of the last Kc real inputs).
//
// HBM-bound elementwise work: each thread owns 4 adjacent channels and walks 16 tokens with a sliding
// window, so every input row is read once per 16 outputs (plus the 3-row halo).  Only the workgroups
// of the first token block read the old tail, and each of them rewrites the tail of exactly its own
// channels after its reads, so no other workgroup can observe a half-updated tail.
#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

constexpr int kTok = 16;
constexpr int kThreads = 256;

template <typename ActT>
struct Vec4;
template <>
struct Vec4<float> {
  static __device__ __forceinline__ float4 load(const float* p) { return *(const float4*)p; }
  static __device__ __forceinline__ void store(float* p, float4 v) { *(float4*)p = v; }
};
template <>
struct Vec4<bf16_t> {
  static __device__ __forceinline__ float4 load(const bf16_t* p) {
    const uint2 u = *(const uint2*)p;
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
  }
  static __device__ __forceinline__ void store(bf16_t* p, float4 v) {
    uint2 u;
    u.x = (uint32_t)from_f32<bf16_t>(v.x).bits | ((uint32_t)from_f32<bf16_t>(v.y).bits << 16);
    u.y = (uint32_t)from_f32<bf16_t>(v.z).bits | ((uint32_t)from_f32<bf16_t>(v.w).bits << 16);
    *(uint2*)p = u;
  }
};

template <typename ActT>
__global__ __launch_bounds__(kThreads) void conv_kernel(ConvArgs p) {
  const int C = p.C, Lb = p.Lb;
  const int c0 = (blockIdx.x * kThreads + threadIdx.x) * 4;
  if (c0 >= C) return;
  const int b = blockIdx.z;
  const int t0 = blockIdx.y * kTok;
  const ActT* mixed = (const ActT*)p.mixed + (long)b * Lb * C;
  ActT* tail = (ActT*)p.tail + (long)b * 3 * C;
  ActT* y = (ActT*)p.y + (long)b * Lb * C;
  const ActT* cw = (const ActT*)p.conv_w;

  float w[4][4];  // [channel][tap]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 v = Vec4<ActT>::load(cw + (long)(c0 + i) * 4);
    w[i][0] = v.x; w[i][1] = v.y; w[i][2] = v.z; w[i][3] = v.w;
  }
  float4 x[kTok + 3];
#pragma unroll
  for (int i = 0; i < kTok + 3; ++i) {  // unconditional loads from clamped rows, masked after
    const int t = t0 - 3 + i;
    const ActT* src = t < 0 ? tail + (long)(t + 3) * C : mixed + (long)(t < Lb ? t : Lb - 1) * C;
    const float4 v = Vec4<ActT>::load(src + c0);
    x[i] = t < Lb ? v : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int tt = 0; tt < kTok; ++tt) {
    const int t = t0 + tt;
    if (t < Lb) {
      float4 o;
      o.x = silu(w[0][0] * x[tt].x + w[0][1] * x[tt + 1].x + w[0][2] * x[tt + 2].x + w[0][3] * x[tt + 3].x);
      o.y = silu(w[1][0] * x[tt].y + w[1][1] * x[tt + 1].y + w[1][2] * x[tt + 2].y + w[1][3] * x[tt + 3].y);
      o.z = silu(w[2][0] * x[tt].z + w[2][1] * x[tt + 1].z + w[2][2] * x[tt + 2].z + w[2][3] * x[tt + 3].z);
      o.w = silu(w[3][0] * x[tt].w + w[3][1] * x[tt + 1].w + w[3][2] * x[tt + 2].w + w[3][3] * x[tt + 3].w);
      Vec4<ActT>::store(y + (long)t * C + c0, o);
    }
  }
  if (blockIdx.y == 0) {
    // new tail = rows len .. len+2 of [tail | mixed]; x[0..2] still hold the old tail rows
    const int len = p.len[b];
    float4 nt[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int src = len + i;
      const float4 v = Vec4<ActT>::load(mixed + (long)(src >= 3 ? src - 3 : 0) * C + c0);
      nt[i] = src < 3 ? (src == 0 ? x[0] : src == 1 ? x[1] : x[2]) : v;
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) Vec4<ActT>::store(tail + (long)i * C + c0, nt[i]);
  }
}

}  // namespace

hipError_t launch_conv(const ConvArgs& p, int act_dtype, hipStream_t st) {
  dim3 grid((p.C / 4 + kThreads - 1) / kThreads, (p.Lb + kTok - 1) / kTok, p.B), block(kThreads);
  timing_before("conv", st);
  if (act_dtype == kActBf16) hipLaunchKernelGGL(conv_kernel<bf16_t>, grid, block, 0, st, p);
  else hipLaunchKernelGGL(conv_kernel<float>, grid, block, 0, st, p);
  timing_after(st);
  return hipGetLastError();
}

}  // namespace gdn
