// Measurement aid, not part of the method: dense f16 MFMA throughput on this GPU, so that the MFMA
// peak a roofline is quoted against can be checked on the machine itself. Every wave keeps two
// independent 32x32x16 accumulations in flight for `iters` rounds (on this part the 16x16x32 form
// needs about sixteen independent chains per wave to reach the same rate); the sums go to `sink` so
// that nothing is optimised away.
#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

constexpr int kProbeChains = 2;
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_probe_kernel(float* sink, int iters) {
  const int tid = threadIdx.x;
  f16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (_Float16)(((tid + e) & 7) * 0.125f);
    b[e] = (_Float16)(((tid * 3 + e) & 7) * 0.0625f);
  }
  f32x16 c[kProbeChains];
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) c[j][e] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kProbeChains; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c[j][e];
  sink[(long)blockIdx.x * 256 + tid] = s;
}

}  // namespace

hipError_t launch_mfma_probe(float* sink, int blocks, int iters, hipStream_t st) {
  timing_before("mfma_probe", st);
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(256), 0, st, sink, iters);
  timing_after(st);
  return hipGetLastError();
}

}  // namespace gdn
