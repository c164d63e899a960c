// Device-side helpers shared by the libgdn kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kWave = 64;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
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
// fp32 -> bf16 rounds to nearest even with NaNs kept quiet: gfx950's v_cvt_pk_bf16_f32, one instruction
// for a pair (the integer-rounding form costs a dozen instructions and a branch per value)
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
  return bf16_t{__builtin_bit_cast(uint16_t, (__bf16)x)};
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// bf16(a) in the low half, bf16(b) in the high half
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// ---- scalar maths (fp32) --------------------------------------------------------------------------
// reciprocals and reciprocal square roots on the hardware rcp / rsq (about 1 ulp) instead of IEEE division
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float rsqrt_fast(float x) { return __builtin_amdgcn_rsqf(x); }
__device__ __forceinline__ float silu(float x) { return x * fast_rcp(1.0f + __expf(-x)); }
__device__ __forceinline__ float sigmoid(float x) { return fast_rcp(1.0f + __expf(-x)); }
// softplus(x) = log(1 + e^x), written as max(x, 0) + log1p(e^-|x|) so it never overflows
__device__ __forceinline__ float softplus(float x) { return fmaxf(x, 0.0f) + log1pf(__expf(-fabsf(x))); }

// One token's log-decay g for the chunk form, floored at -30. The chunk form takes every decay factor as
// e^{gamma_r - gamma_s} of in-chunk sums gamma of g, whose rounding error grows with |gamma|, and a full
// forget (g = -inf) would give -inf - (-inf). With the floor |gamma| stays below 64 * 30, and a factor
// e^g below e^-30 (about 9.4e-14) becomes 9.4e-14: the state keeps at most that fraction of what it held
// before the token instead of less. NaN passes through.
constexpr float kLogDecayFloor = -30.0f;
__device__ __forceinline__ float chunk_log_decay(float g) { return g < kLogDecayFloor ? kLogDecayFloor : g; }

// ---- wave reductions -----------------------------------------------------------------------------
// DPP moves inside 16-lane rows (no LDS round trip): quad_perm [1,0,3,2] and [2,3,0,1], then
// row_half_mirror (lane i <-> 7-i) and row_mirror (lane i <-> 15-i) pair each partial sum with a
// disjoint one, so after four steps every lane holds its row's total.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_sum8(float v) {  // aligned groups of 8 lanes
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  return v;
}
__device__ __forceinline__ float row_sum16(float v) { return row_sum8(v) + dpp<0x140>(row_sum8(v)); }
__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}
// sum over all 64 lanes, the same value in every lane
__device__ __forceinline__ float wave_sum64(float v) {
  v = row_sum16(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}
// sum over aligned groups of kWidth lanes (8, 16, 32 or 64); every lane gets its group's sum
template <int kWidth>
__device__ __forceinline__ float wave_sum(float v) {
  static_assert(kWidth == 8 || kWidth == 16 || kWidth == 32 || kWidth == 64, "group width");
  if (kWidth == 64) return wave_sum64(v);
  if (kWidth == 8) return row_sum8(v);
  v = row_sum16(v);
  if (kWidth == 32) v += __shfl_xor(v, 16, kWave);
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

// x as one rounded fp32 value in a register, opaque to the optimiser (an empty asm, no memory access).
// A hi/lo split converts x to f16 twice, once for the stored high half and once for the residual. Left
// visible, the product that forms x was fused into the residual's conversion only (v_fma_mixlo_f16
// rounds the exact product once, the stored half came from the fp32-rounded one): where the exact
// product lies within half an fp32 ulp of an f16 tie the two high halves then differ, and hi + lo
// misses x by one f16 ulp of the high half.
__device__ __forceinline__ float pin_f32(float x) {
  asm("" : "+v"(x));
  return x;
}

// hi/lo split of an fp32 value into two f16 values: x ~= hi + lo to about 2^-22 relative
__device__ __forceinline__ void split_f16(float x, _Float16& hi, _Float16& lo) {
  x = pin_f32(x);
  hi = (_Float16)x;
  lo = (_Float16)(x - (float)hi);
}

// The same split of two values, with the high halves rounded once, into one register
// (v_cvt_pk_f16_f32), and that register made opaque (an empty asm, no instruction) so that the residuals
// are formed from the stored halves: hipcc then forms each residual x - hi with one v_fma_mix_f32 from the
// f16 half, folding a multiply that produced x into it exactly, and rounds both low halves with one more
// v_cvt_pk_f16_f32 (six instructions for two values where split_f16 takes ten with the multiplies).
__device__ __forceinline__ void split2_f16(float x0, float x1, f16x2& hi, f16x2& lo) {
  uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{x0, x1}, f16x2));
  asm("" : "+v"(hb));
  hi = __builtin_bit_cast(f16x2, hb);
  const f32x2_t back = __builtin_convertvector(hi, f32x2_t);
  lo = __builtin_convertvector(f32x2_t{x0 - back[0], x1 - back[1]}, f16x2);
}

// Streamed 16-byte store through a buffer descriptor over [base, base + range) bytes (offsets past the
// range are dropped by the hardware, never written), with the non-temporal and system-scope cache bits.
// For the write-heavy state streams (decode's in-place state, verify's checkpoints) this measured 4-9%
// faster than a non-temporal global store, and a plain global store slower than both.
constexpr int kCpolStream = 2 | 16;  // nt | sc1
__device__ __forceinline__ void store_stream16(void* base, uint32_t range, uint32_t byte_off, f32x4 v) {
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)range, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), rs, byte_off, 0, kCpolStream);
}

}  // namespace gdn
