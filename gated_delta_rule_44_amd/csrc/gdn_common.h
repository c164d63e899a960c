// Device-side helpers shared by the libgdn kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kWave = 64;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---- activation storage types -------------------------------------------------------------------
// bf16 is carried as raw uint16_t bits: widening is a shift, narrowing rounds to nearest even.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float((uint32_t)x.bits << 16); }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return bf16_t{(uint16_t)((u >> 16) | 0x40)};
  u += 0x7fffu + ((u >> 16) & 1u);
  return bf16_t{(uint16_t)(u >> 16)};
}

// ---- scalar maths (fp32) --------------------------------------------------------------------------
__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }
__device__ __forceinline__ float sigmoid(float x) { return 1.0f / (1.0f + __expf(-x)); }
// softplus(x) = log(1 + e^x), written as max(x, 0) + log1p(e^-|x|) so it never overflows
__device__ __forceinline__ float softplus(float x) { return fmaxf(x, 0.0f) + log1pf(__expf(-fabsf(x))); }

// ---- wave reductions -----------------------------------------------------------------------------
template <int kWidth>
__device__ __forceinline__ float wave_sum(float v) {
  // sum over aligned groups of kWidth lanes (kWidth a power of two <= 64); every lane gets the sum
#pragma unroll
  for (int off = kWidth / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// ---- MFMA: D(16x16, fp32) += A(16x32, f16) * B(32x16, f16) ---------------------------------------
// Lane l (g = l / 16) supplies A[l % 16][k in group g] and B[k in group g][l % 16], 8 values each, and
// receives D[4g + i][l % 16], i = 0..3. Which 8 k-indices form group g is up to the caller, as long as
// A and B agree; the state-pass kernel uses {4g..4g+3, 16+4g..16+4g+3} so that two stacked 16x16
// accumulator tiles feed the next product's B operand without leaving registers.
__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// hi/lo split of an fp32 value into two f16 values: x ~= hi + lo to about 2^-22 relative
__device__ __forceinline__ void split_f16(float x, _Float16& hi, _Float16& lo) {
  hi = (_Float16)x;
  lo = (_Float16)(x - (float)hi);
}

}  // namespace gdn
