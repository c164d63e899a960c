// Zero-padded heads for prefill with d_k != d_v (gfx950).
//
// The layer allows different key and value head dims (both in {32, 64, 128}; the conv channels are
// [q heads of d_k | k heads of d_k | v heads of d_v], and the state of a value head is d_k x d_v).
// Prefill runs such a layer through the square kernels at D = max(d_k, d_v), on copies in the
// workspace whose extra channels, conv weights, tail entries and state rows/columns are zero:
//  - an extra q or k channel has zero inputs, zero conv weights and a zero tail, so its conv output
//    is silu(0) = 0; it adds nothing to the L2 norms, the Gram products or k^T H, and the state rows
//    it would address (k_i = 0) start at zero and stay zero;
//  - an extra v channel is zero, so its column of U' = T beta V, of U = U' - W H and of H starts and
//    stays zero, and so does the column of o; the gated RMSNorm then divides the sum of squares by
//    d_v, the true column count, not by D.
// The padded run is therefore the same computation on the same numbers. These copies cost one extra
// pass over the inputs, the outputs and the states; they exist for shape coverage, not speed.
//
// Every copy works on 16-byte units. Each head segment is a multiple of 32 channels, so a unit never
// straddles a head boundary: the channel map below is written per unit.
#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

constexpr int kPadThreads = 256;
constexpr long kPadMaxBlocks = 8192;

int pad_blocks(long n) {
  const long b = (n + kPadThreads - 1) / kPadThreads;
  return (int)(b < 1 ? 1 : (b > kPadMaxBlocks ? kPadMaxBlocks : b));
}

// unit cp of a padded row -> unit of the original row, or -1 (a zero unit)
__device__ __forceinline__ int unit_src(const ChanMap& m, int cp) {
  const int qk = m.n_k * m.D;
  if (cp < 2 * qk) {
    const int part = cp >= qk ? 1 : 0, x = cp - part * qk;
    const int kh = x / m.D, i = x - kh * m.D;
    return i < m.dk ? part * m.n_k * m.dk + kh * m.dk + i : -1;
  }
  const int x = cp - 2 * qk;
  const int h = x / m.D, j = x - h * m.D;
  return j < m.dv ? 2 * m.n_k * m.dk + h * m.dv + j : -1;
}

// unit c of an original row -> its unit in the padded row
__device__ __forceinline__ int unit_dst(const ChanMap& m, int c) {
  const int qk = m.n_k * m.dk;
  if (c < 2 * qk) {
    const int part = c >= qk ? 1 : 0, x = c - part * qk;
    const int kh = x / m.dk, i = x - kh * m.dk;
    return part * m.n_k * m.D + kh * m.D + i;
  }
  const int x = c - 2 * qk;
  const int h = x / m.dv, j = x - h * m.dv;
  return 2 * m.n_k * m.D + h * m.D + j;
}

// dst [rows][Ud] (padded) from src [rows][Us] (original)
__global__ __launch_bounds__(kPadThreads) void pad_units_kernel(const uint4* src, uint4* dst, long rows, int Us, int Ud,
                                                                ChanMap m) {
  const long n = rows * Ud;
  for (long e = blockIdx.x * (long)kPadThreads + threadIdx.x; e < n; e += (long)gridDim.x * kPadThreads) {
    const long r = e / Ud;
    const int sc = unit_src(m, (int)(e - r * Ud));
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (sc >= 0) v = src[r * Us + sc];
    dst[e] = v;
  }
}

// dst [rows][Ud] (original) from src [rows][Us] (padded); with len, rows are [B][Lb] and row (b, t) is
// copied only for t < len[b] (the rest of dst is left as it was)
__global__ __launch_bounds__(kPadThreads) void unpad_units_kernel(const uint4* src, uint4* dst, long rows, int Us,
                                                                  int Ud, ChanMap m, const int32_t* len, int Lb) {
  const long n = rows * Ud;
  for (long e = blockIdx.x * (long)kPadThreads + threadIdx.x; e < n; e += (long)gridDim.x * kPadThreads) {
    const long r = e / Ud;
    if (len) {
      const long b = r / Lb;
      if (r - b * Lb >= len[b]) continue;
    }
    dst[e] = src[r * Us + unit_dst(m, (int)(e - r * Ud))];
  }
}

// dst [mats][D][D] from src [mats][dk][dv] (fp32, in float4 units: dv4 = dv / 4, D4 = D / 4)
__global__ __launch_bounds__(kPadThreads) void pad_state_kernel(const float4* src, float4* dst, long mats, int dk,
                                                                int dv4, int D, int D4) {
  const long per = (long)D * D4, n = mats * per;
  for (long e = blockIdx.x * (long)kPadThreads + threadIdx.x; e < n; e += (long)gridDim.x * kPadThreads) {
    const long mt = e / per;
    const int rem = (int)(e - mt * per), i = rem / D4, j = rem - i * D4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < dk && j < dv4) v = src[(mt * dk + i) * dv4 + j];
    dst[e] = v;
  }
}

// dst [mats][dk][dv] from src [mats][D][D]
__global__ __launch_bounds__(kPadThreads) void unpad_state_kernel(const float4* src, float4* dst, long mats, int dk,
                                                                  int dv4, int D, int D4) {
  const long per = (long)dk * dv4, n = mats * per;
  for (long e = blockIdx.x * (long)kPadThreads + threadIdx.x; e < n; e += (long)gridDim.x * kPadThreads) {
    const long mt = e / per;
    const int rem = (int)(e - mt * per), i = rem / dv4, j = rem - i * dv4;
    dst[e] = src[(mt * D + i) * D4 + j];
  }
}

}  // namespace

hipError_t launch_pad_units(const void* src, void* dst, long rows, int Us, int Ud, const ChanMap& m, hipStream_t st) {
  hipLaunchKernelGGL(pad_units_kernel, dim3(pad_blocks(rows * Ud)), dim3(kPadThreads), 0, st, (const uint4*)src,
                     (uint4*)dst, rows, Us, Ud, m);
  return hipGetLastError();
}

hipError_t launch_unpad_units(const void* src, void* dst, long rows, int Us, int Ud, const ChanMap& m,
                              const int32_t* len, int Lb, hipStream_t st) {
  hipLaunchKernelGGL(unpad_units_kernel, dim3(pad_blocks(rows * Ud)), dim3(kPadThreads), 0, st, (const uint4*)src,
                     (uint4*)dst, rows, Us, Ud, m, len, Lb);
  return hipGetLastError();
}

hipError_t launch_pad_state(const float* src, float* dst, long mats, int dk, int dv, int D, hipStream_t st) {
  hipLaunchKernelGGL(pad_state_kernel, dim3(pad_blocks(mats * D * (D / 4))), dim3(kPadThreads), 0, st,
                     (const float4*)src, (float4*)dst, mats, dk, dv / 4, D, D / 4);
  return hipGetLastError();
}

hipError_t launch_unpad_state(const float* src, float* dst, long mats, int dk, int dv, int D, hipStream_t st) {
  hipLaunchKernelGGL(unpad_state_kernel, dim3(pad_blocks(mats * dk * (dv / 4))), dim3(kPadThreads), 0, st,
                     (const float4*)src, (float4*)dst, mats, dk, dv / 4, D, D / 4);
  return hipGetLastError();
}

}  // namespace gdn
