// Standalone causal conv1d + SiLU over [saved tail | chunk] with the tail update (gfx950).
//
// y[t][c] = silu(sum_{j<4} w[c][j] * xin[t+j][c]) with xin = [tail (3 rows) | mixed (Lb rows)]; the new
// tail is rows len .. len+2 of xin (the "qev_fast/statecache.py" page, CacheQwen35._gdn: conv on
// [saved conv inputs | chunk] with SiLU and no bias, then the copy of the last Kc real inputs).
//
// HBM-bound elementwise work.  Each thread owns 8 adjacent bf16 channels (one 16-byte access per row;
// 4 fp32 channels) and a span of kSpan tokens, which it walks in groups of kG rows with a rolling 3-row
// window: the next group's rows are loaded before the current group is computed, so every input row is
// read once (plus a 3-row halo per span) and loads stay in flight under the arithmetic.  Rows are
// streamed, so they are loaded and stored non-temporally.  Workgroup w runs job
// J = (w % 8) * (N / 8) + w / 8 so that each XCD walks consecutive spans of one channel stripe and
// finds the halo rows in its own L2.  Only the workgroups of the first span read the old tail, and
// each rewrites the tail of exactly its own channels after its reads, so no other workgroup can
// observe a half-updated tail.
#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

constexpr int kG = 8;
constexpr int kGroups = 8;
constexpr int kSpan = kG * kGroups;
constexpr int kThreads = 256;

// the channels one thread owns in one row: 8 bf16 (one 16-byte access) or 4 fp32, widened to fp32
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <typename ActT>
struct Row;
template <>
struct Row<float> {
  static constexpr int kC = 4;
  typedef float4 raw;
  static __device__ __forceinline__ raw ld(const float* p) { const f32x4 v = __builtin_nontemporal_load((const f32x4*)p); return make_float4(v[0], v[1], v[2], v[3]); }
  static __device__ __forceinline__ void widen(raw v, float (&f)[kC]) { f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w; }
  static __device__ __forceinline__ void store(float* p, const float (&f)[kC]) { const f32x4 v = {f[0], f[1], f[2], f[3]}; __builtin_nontemporal_store(v, (f32x4*)p); }
};
template <>
struct Row<bf16_t> {
  static constexpr int kC = 8;
  typedef uint4 raw;
  static __device__ __forceinline__ raw ld(const bf16_t* p) { const u32x4 v = __builtin_nontemporal_load((const u32x4*)p); return make_uint4(v[0], v[1], v[2], v[3]); }
  static __device__ __forceinline__ void widen(raw u, float (&f)[kC]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float (&f)[kC]) {
    const u32x4 v = {pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
    __builtin_nontemporal_store(v, (u32x4*)p);
  }
};

template <typename ActT>
__global__ __launch_bounds__(kThreads) void conv_kernel(ConvArgs p) {
  typedef Row<ActT> V;
  constexpr int K = V::kC;
  const int C = p.C, Lb = p.Lb;
  const int nx = (C / K + kThreads - 1) / kThreads, ny = (Lb + kSpan - 1) / kSpan;
  const long N = (long)nx * ny * p.B;
  const long wg = blockIdx.x;
  const long J = wg < (N / 8) * 8 ? (wg % 8) * (N / 8) + wg / 8 : wg;
  const int by = (int)(J % ny);
  const int bx = (int)((J / ny) % nx);
  const int b = (int)(J / ((long)ny * nx));
  const int c0 = (bx * kThreads + threadIdx.x) * K;
  if (c0 >= C) return;
  const int t0 = by * kSpan;
  const ActT* mixed = (const ActT*)p.mixed + (long)b * Lb * C;
  ActT* tail = (ActT*)p.tail + (long)b * 3 * C;
  ActT* y = (ActT*)p.y + (long)b * Lb * C;
  const ActT* cw = (const ActT*)p.conv_w;

  float w[K][4];  // [channel][tap]
#pragma unroll
  for (int i = 0; i < K; ++i) {
    float f[4];
    f[0] = to_f32(cw[(long)(c0 + i) * 4 + 0]); f[1] = to_f32(cw[(long)(c0 + i) * 4 + 1]);
    f[2] = to_f32(cw[(long)(c0 + i) * 4 + 2]); f[3] = to_f32(cw[(long)(c0 + i) * 4 + 3]);
    w[i][0] = f[0]; w[i][1] = f[1]; w[i][2] = f[2]; w[i][3] = f[3];
  }
  float h[3][K];  // the 3 rows before the current group
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int t = t0 - 3 + i;
    const ActT* src = t < 0 ? tail + (long)(t + 3) * C : mixed + (long)(t < Lb ? t : Lb - 1) * C;
    V::widen(V::ld(src + c0), h[i]);
    if (t >= Lb) {
#pragma unroll
      for (int k = 0; k < K; ++k) h[i][k] = 0.f;
    }
  }
  float old[3][K];
#pragma unroll
  for (int i = 0; i < 3; ++i)
#pragma unroll
    for (int k = 0; k < K; ++k) old[i][k] = h[i][k];
  const int ng = min(kGroups, (Lb - t0 + kG - 1) / kG);
  typename V::raw cur[kG], nxt[kG];
#pragma unroll
  for (int i = 0; i < kG; ++i) cur[i] = V::ld(mixed + (long)min(t0 + i, Lb - 1) * C + c0);
#pragma unroll 1
  for (int g = 0; g < ng; ++g) {
    const int tg = t0 + g * kG;
    if (g + 1 < ng) {
#pragma unroll
      for (int i = 0; i < kG; ++i) nxt[i] = V::ld(mixed + (long)min(tg + kG + i, Lb - 1) * C + c0);
    }
    const bool whole = tg + kG <= Lb;
    float win[3][K];  // rows tg + tt - 3 .. tg + tt - 1
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
      for (int k = 0; k < K; ++k) win[i][k] = h[i][k];
#pragma unroll
    for (int tt = 0; tt < kG; ++tt) {
      float x3[K];
      V::widen(cur[tt], x3);
      if (!whole && tg + tt >= Lb) {
#pragma unroll
        for (int k = 0; k < K; ++k) x3[k] = 0.f;
      }
      float o[K];
#pragma unroll
      for (int k = 0; k < K; ++k)
        o[k] = silu(w[k][0] * win[0][k] + w[k][1] * win[1][k] + w[k][2] * win[2][k] + w[k][3] * x3[k]);
      if (whole || tg + tt < Lb) V::store(y + (long)(tg + tt) * C + c0, o);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        win[0][k] = win[1][k];
        win[1][k] = win[2][k];
        win[2][k] = x3[k];
      }
    }
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
      for (int k = 0; k < K; ++k) h[i][k] = win[i][k];
#pragma unroll
    for (int i = 0; i < kG; ++i) cur[i] = nxt[i];
  }
  if (by == 0) {
    // new tail = rows len .. len+2 of [tail | mixed]; old[] holds the old tail rows
    const int len = p.len[b];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int src = len + i;
      float v[K];
      V::widen(V::ld(mixed + (long)(src >= 3 ? src - 3 : 0) * C + c0), v);
      if (src < 3) {
#pragma unroll
        for (int k = 0; k < K; ++k) v[k] = src == 0 ? old[0][k] : src == 1 ? old[1][k] : old[2][k];
      }
      V::store(tail + (long)i * C + c0, v);
    }
  }
}

}  // namespace

hipError_t launch_conv(const ConvArgs& p, int act_dtype, hipStream_t st) {
  // one workgroup per (batch, 256-thread channel stripe, kSpan-token span), flattened into grid.x
  const int k = act_dtype == kActBf16 ? Row<bf16_t>::kC : Row<float>::kC;
  const long n = (long)((p.C / k + kThreads - 1) / kThreads) * ((p.Lb + kSpan - 1) / kSpan) * p.B;
  if (n >= (1L << 31)) return hipErrorInvalidValue;
  dim3 grid((unsigned)n), block(kThreads);
  timing_before("conv", st);
  if (act_dtype == kActBf16) hipLaunchKernelGGL(conv_kernel<bf16_t>, grid, block, 0, st, p);
  else hipLaunchKernelGGL(conv_kernel<float>, grid, block, 0, st, p);
  timing_after(st);
  return hipGetLastError();
}

}  // namespace gdn
