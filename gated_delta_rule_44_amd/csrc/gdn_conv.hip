// Standalone causal conv1d + SiLU over [saved tail | chunk] with the tail update (gfx950).
//
// y[t][c] = silu(sum_{j<4} w[c][j] * xin[t+j][c]) with xin = [tail (3 rows) | mixed (Lb rows)]; the new
// tail is rows len .. len+2 of xin (the "qev_fast/statecache.py" page, CacheQwen35._gdn: conv on
// [saved conv inputs | chunk] with SiLU and no bias, then the copy of the last Kc real inputs).
//
// HBM-bound elementwise work.  Each thread owns 4 adjacent channels and a span of kSpan tokens, which it
// walks in groups of kG rows with a rolling 3-row window: the next group's rows are loaded before the
// current group is computed, so every input row is read once (plus a 3-row halo per span) and loads
// stay in flight under the arithmetic.  Workgroup w runs job J = (w % 8) * (N / 8) + w / 8 so that each
// XCD walks consecutive spans of one channel stripe and finds the halo rows in its own L2.  Only the
// workgroups of the first span read the old tail, and each rewrites the tail of exactly its own
// channels after its reads, so no other workgroup can observe a half-updated tail.
#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

constexpr int kG = 8;
constexpr int kGroups = 8;
constexpr int kSpan = kG * kGroups;
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
    u.x = pack_bf16x2(v.x, v.y);
    u.y = pack_bf16x2(v.z, v.w);
    *(uint2*)p = u;
  }
};

template <typename ActT>
__global__ __launch_bounds__(kThreads) void conv_kernel(ConvArgs p) {
  const int C = p.C, Lb = p.Lb;
  const int nx = (C / 4 + kThreads - 1) / kThreads, ny = (Lb + kSpan - 1) / kSpan;
  const long N = (long)nx * ny * p.B;
  const long wg = blockIdx.x;
  const long J = wg < (N / 8) * 8 ? (wg % 8) * (N / 8) + wg / 8 : wg;
  const int by = (int)(J % ny);
  const int bx = (int)((J / ny) % nx);
  const int b = (int)(J / ((long)ny * nx));
  const int c0 = (bx * kThreads + threadIdx.x) * 4;
  if (c0 >= C) return;
  const int t0 = by * kSpan;
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
  float4 h[3];  // the 3 rows before the current group
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int t = t0 - 3 + i;
    const ActT* src = t < 0 ? tail + (long)(t + 3) * C : mixed + (long)(t < Lb ? t : Lb - 1) * C;
    const float4 v = Vec4<ActT>::load(src + c0);
    h[i] = t < Lb ? v : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const float4 old0 = h[0], old1 = h[1], old2 = h[2];
  const int ng = min(kGroups, (Lb - t0 + kG - 1) / kG);
  float4 cur[kG], nxt[kG];
#pragma unroll
  for (int i = 0; i < kG; ++i) cur[i] = Vec4<ActT>::load(mixed + (long)min(t0 + i, Lb - 1) * C + c0);
#pragma unroll 1
  for (int g = 0; g < ng; ++g) {
    const int tg = t0 + g * kG;
    if (g + 1 < ng) {
#pragma unroll
      for (int i = 0; i < kG; ++i) nxt[i] = Vec4<ActT>::load(mixed + (long)min(tg + kG + i, Lb - 1) * C + c0);
    }
    const bool whole = tg + kG <= Lb;
    if (!whole) {
#pragma unroll
      for (int i = 0; i < kG; ++i)
        if (tg + i >= Lb) cur[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int tt = 0; tt < kG; ++tt) {
      const float4 x0 = tt >= 3 ? cur[tt - 3] : h[tt];
      const float4 x1 = tt >= 2 ? cur[tt - 2] : h[tt + 1];
      const float4 x2 = tt >= 1 ? cur[tt - 1] : h[2];
      const float4 x3 = cur[tt];
      float4 o;
      o.x = silu(w[0][0] * x0.x + w[0][1] * x1.x + w[0][2] * x2.x + w[0][3] * x3.x);
      o.y = silu(w[1][0] * x0.y + w[1][1] * x1.y + w[1][2] * x2.y + w[1][3] * x3.y);
      o.z = silu(w[2][0] * x0.z + w[2][1] * x1.z + w[2][2] * x2.z + w[2][3] * x3.z);
      o.w = silu(w[3][0] * x0.w + w[3][1] * x1.w + w[3][2] * x2.w + w[3][3] * x3.w);
      if (whole || tg + tt < Lb) Vec4<ActT>::store(y + (long)(tg + tt) * C + c0, o);
    }
    h[0] = cur[kG - 3]; h[1] = cur[kG - 2]; h[2] = cur[kG - 1];
#pragma unroll
    for (int i = 0; i < kG; ++i) cur[i] = nxt[i];
  }
  if (by == 0) {
    // new tail = rows len .. len+2 of [tail | mixed]; old0..2 hold the old tail rows
    const int len = p.len[b];
    float4 nt[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int src = len + i;
      const float4 v = Vec4<ActT>::load(mixed + (long)(src >= 3 ? src - 3 : 0) * C + c0);
      nt[i] = src < 3 ? (src == 0 ? old0 : src == 1 ? old1 : old2) : v;
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) Vec4<ActT>::store(tail + (long)i * C + c0, nt[i]);
  }
}

}  // namespace

hipError_t launch_conv(const ConvArgs& p, int act_dtype, hipStream_t st) {
  // one workgroup per (batch, 1024-channel stripe, kSpan-token span), flattened into grid.x
  const long n = (long)((p.C / 4 + kThreads - 1) / kThreads) * ((p.Lb + kSpan - 1) / kSpan) * p.B;
  if (n >= (1L << 31)) return hipErrorInvalidValue;
  dim3 grid((unsigned)n), block(kThreads);
  timing_before("conv", st);
  if (act_dtype == kActBf16) hipLaunchKernelGGL(conv_kernel<bf16_t>, grid, block, 0, st, p);
  else hipLaunchKernelGGL(conv_kernel<float>, grid, block, 0, st, p);
  timing_after(st);
  return hipGetLastError();
}

}  // namespace gdn
