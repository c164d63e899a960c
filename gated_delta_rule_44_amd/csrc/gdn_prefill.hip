// Chunked prefill of the gated delta rule (gfx950): two launches, plus a norm pass when one value
// head's columns are split over several workgroups.
//
// Chunk form (chunk of C = 64 tokens, entering state H0 = S0^T, gamma_r = sum_{i<=r} g_i inside the
// chunk; from the recurrence S_t = e^{g_t} S_{t-1}(I - beta_t k_t k_t^T) + beta_t v_t k_t^T by the
// WY/UT-transform treatment of the delta rule):
//   A[r][s] = beta_r e^{gamma_r - gamma_s} k_r.k_s (s < r),  T = (I + A)^-1
//   W = T diag(beta e^gamma) K,   U' = T diag(beta) V,   P[r][s] = e^{gamma_r - gamma_s} q_r.k_s (s <= r)
//   U = U' - W H0,   O = scale (diag(e^gamma) Q H0 + P U),   H_C = e^{gamma_C} H0 + K^T diag(e^{gamma_C - gamma}) U
// Every decay factor is the exponential of a non-positive difference, never e^{gamma_r} e^{-gamma_s}.
//
// Launch 1, chunk_prep_kernel (every chunk in parallel; one workgroup per chunk x key head x sequence):
//   conv + SiLU over [saved tail | chunk], q/k L2 norm, gates with the padding mask, the Gram products
//   K K^T and Q K^T (f16 MFMA, hi/lo-split operands), then for each value head of the GQA group the UT
//   inverse T (fp32: diagonal 16x16 blocks by substitution, off-diagonal blocks on fp32 MFMA), W and U'
//   (f16 MFMA), P~ = scale * P, Q~ = scale diag(e^gamma) Q, K~ = diag(e^{gamma_C - gamma}) K.
//   Each chunk's operands are written as a byte image of exactly what the state pass keeps in LDS
//   (rows padded against bank conflicts, k-index permuted inside 32-blocks), plus U' in MFMA fragment
//   order.
// Launch 2, state_pass_kernel (one workgroup per column slice x value head x sequence, chunks in order):
//   H stays in MFMA accumulators for the whole call; the next chunk's image streams into the other LDS
//   buffer by direct global->LDS loads while this chunk computes U = U' - W H, O^T = H^T Q~^T +
//   U^T P~^T and H = e^{gamma_C} H + K~^T U; the gated RMSNorm is fused when one workgroup owns all
//   d_v columns of the head, otherwise norm_kernel finishes it from the saved partial sums.
//
// Precision: f16 operands with fp32 accumulation, and hi/lo f16 pairs (about 22 mantissa bits) where
// rounding would otherwise show in the output: the Gram products, beta*V, H, U, K~ and P~. With fp32
// activations every operand is split. MFMA flushes f16 subnormals, so the lo half of a split value
// must stay >= 2^-14: operands of unit scale are carried multiplied by 2^8 (exact), and the scales
// are chosen so that every product lands in a consistent domain: the state pass keeps H as 2^16 H,
// U as 2^8 U and O^T as 2^16 O^T, with 2^8 Q~, 2^8 P~, 2^8 K~ and unscaled -W in the image.
#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

constexpr int C64 = kChunk;
constexpr float kS8 = 256.f;              // 2^8 operand scale
constexpr float kInvS8 = 1.f / 256.f;
constexpr float kInvS16 = 1.f / 65536.f;

typedef __attribute__((address_space(3))) void lds_void;

// position of k-index j (0..31) inside its 32-block: the group of lane-group g holds
// {4g..4g+3, 16+4g..16+4g+3}, so that two stacked 16x16 accumulator tiles form one operand
__device__ __forceinline__ int kperm(int j) { return ((j & 15) >> 2) * 8 + ((j >> 4) << 2) + (j & 3); }
__device__ __forceinline__ int pcol(int c) { return (c & ~31) + kperm(c & 31); }

// ---- the per-chunk operand image (identical in the workspace and in the state pass's LDS) --------
// Tiles are f16, row-major and unpadded; the 16-byte groups of each row are XOR-swizzled with the row
// index so that the 16 rows an MFMA operand load touches fall in different LDS banks.
template <int D, bool SPLIT>
struct Img {
  // part A, read first in a chunk (U and the H^T Q~^T term)
  static constexpr int W_HI = 0;                               // [64][D]: -W, row = token
  static constexpr int W_LO = W_HI + C64 * D;
  static constexpr int Q_HI = W_LO + (SPLIT ? C64 * D : 0);    // [64][D]: Q~, always split
  static constexpr int Q_LO = Q_HI + C64 * D;
  static constexpr int A_HALFS = Q_LO + C64 * D;
  // part B, read second (the U^T P~^T term and the state update); offsets relative to part B
  static constexpr int K_HI = 0;                               // [D][64]: K~^T, always split
  static constexpr int K_LO = K_HI + D * C64;
  static constexpr int P_HI = K_LO + D * C64;                  // [64][64]: P~, always split
  static constexpr int P_LO = P_HI + C64 * C64;
  static constexpr int B_HALFS = P_LO + C64 * C64;
  static constexpr int A_BYTES = A_HALFS * 2, B_BYTES = B_HALFS * 2;
  static constexpr int BYTES = A_BYTES + B_BYTES;
  static_assert(A_BYTES % 1024 == 0 && B_BYTES % 1024 == 0, "image parts stream in 1 KB wave loads");
};

// half index of (row, col) in a swizzled tile of NCOLS halfs per row
template <int NCOLS>
__device__ __forceinline__ int swz(int row, int col) {
  constexpr int NG = NCOLS / 8;
  constexpr int M = (NG < 8 ? NG : 8) - 1;
  return row * NCOLS + ((((col >> 3) ^ (row & M))) << 3) + (col & 7);
}

template <int D, bool SPLIT>
struct Rec {
  static constexpr long kImg = 0;
  static constexpr long kUp = Img<D, SPLIT>::BYTES;                // U' fp32, MFMA fragment order
  static constexpr long kGc = kUp + 4L * C64 * D;                  // e^{gamma_C}
  static constexpr long kBytes = ((kGc + 16 + 255) / 256) * 256;
};

template <int D, bool SPLIT>
__device__ __forceinline__ char* rec_ptr(const PrefillArgs& p, int b, int h, int c) {
  return (char*)p.ws + (((long)b * p.n_v + h) * p.n_chunks + c) * Rec<D, SPLIT>::kBytes;
}

// Barrier for LDS reads and writes only. __syncthreads() also fences the direct global->LDS copies
// still in flight (vmcnt), which would serialise the next chunk's prefetch with this chunk's work;
// the buffers those copies fill are not read until the wait at the top of the next chunk.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f16x8 ld16(const _Float16* p) { return *(const f16x8*)p; }

__device__ __forceinline__ void pack_split(f32x4 a, f32x4 b, f16x8& hi, f16x8& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hi[i] = (_Float16)a[i];
    lo[i] = (_Float16)(a[i] - (float)hi[i]);
    hi[4 + i] = (_Float16)b[i];
    lo[4 + i] = (_Float16)(b[i] - (float)hi[4 + i]);
  }
}
__device__ __forceinline__ f16x8 pack_hi(f32x4 a, f32x4 b) {
  f16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = (_Float16)a[i];
    r[4 + i] = (_Float16)b[i];
  }
  return r;
}

// four activations as stored (8 bytes of bf16 or 16 of fp32), widened when used
template <typename ActT>
struct Raw4 {
  typedef uint2 type;
  static __device__ __forceinline__ type load(const ActT* p) { return *(const uint2*)p; }
  static __device__ __forceinline__ float4 widen(type u) {
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
  }
};
template <>
struct Raw4<float> {
  typedef float4 type;
  static __device__ __forceinline__ type load(const float* p) { return *(const float4*)p; }
  static __device__ __forceinline__ float4 widen(type u) { return u; }
};

template <typename ActT>
struct Act4;
template <>
struct Act4<float> {
  static __device__ __forceinline__ float4 load(const float* p) { return *(const float4*)p; }
  static __device__ __forceinline__ void store(float* p, float4 v) { *(float4*)p = v; }
};
template <>
struct Act4<bf16_t> {
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

// -------------------------------------------------------------------------------------------------
template <typename ActT, int D, int R, bool SPLIT>
__global__ __launch_bounds__(256) void chunk_prep_kernel(PrefillArgs p) {
  using I = Img<D, SPLIT>;
  constexpr int CPL = D >= 64 ? D / 64 : 1;   // channels per lane in the conv stage
  constexpr int LDW = D + 8, LDT = C64 + 8, LF = C64 + 1;
  constexpr int SZ_TOK = C64 * LDW * 2;       // f16 [64][LDW] (this kernel's own padded tiles)
  constexpr int SZ_CH = D * LDT * 2;          // f16 [D][LDT]
  constexpr int NKB = SPLIT ? 2 : 1;
  constexpr int R1 = (4 * SZ_TOK > (NKB + 2) * SZ_CH) ? 4 * SZ_TOK : (NKB + 2) * SZ_CH;
  constexpr int OFF_QH = 0, OFF_QL = SZ_TOK, OFF_KH = 2 * SZ_TOK, OFF_KL = 3 * SZ_TOK;  // Gram operands
  constexpr int OFF_KB = 0, OFF_VBH = NKB * SZ_CH, OFF_VBL = OFF_VBH + SZ_CH;            // after the Gram
  constexpr int OFF_KK = R1;
  constexpr int OFF_QK = OFF_KK + C64 * LF * 4;
  constexpr int OFF_A = OFF_QK + C64 * LF * 4;
  constexpr int OFF_TF = OFF_A + C64 * LF * 4;
  constexpr int OFF_T = OFF_TF + C64 * LF * 4;
  constexpr int OFF_X = OFF_T + (SPLIT ? 2 : 1) * C64 * LDT * 2;
  constexpr int OFF_G = OFF_X + 4 * 16 * 17 * 4;
  constexpr int OFF_B = OFF_G + R * C64 * 4;
  constexpr int LDS = OFF_B + R * C64 * 4;
  static_assert(LDS <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) char smem[LDS];
  _Float16* sQh = (_Float16*)(smem + OFF_QH);
  _Float16* sQl = (_Float16*)(smem + OFF_QL);
  _Float16* sKh = (_Float16*)(smem + OFF_KH);
  _Float16* sKl = (_Float16*)(smem + OFF_KL);
  _Float16* sKb = (_Float16*)(smem + OFF_KB);   // (beta e^gamma k)^T, [D][LDT], hi (then lo if SPLIT)
  _Float16* sVbh = (_Float16*)(smem + OFF_VBH); // (beta v)^T hi
  _Float16* sVbl = (_Float16*)(smem + OFF_VBL); // (beta v)^T lo
  float* sKK = (float*)(smem + OFF_KK);
  float* sQK = (float*)(smem + OFF_QK);
  float* sA = (float*)(smem + OFF_A);
  float* sTf = (float*)(smem + OFF_TF);
  _Float16* sT = (_Float16*)(smem + OFF_T);     // T hi [64][LDT] (then lo if SPLIT)
  float* sX = (float*)(smem + OFF_X);
  float* sGam = (float*)(smem + OFF_G);
  float* sBet = (float*)(smem + OFF_B);

  const int c = blockIdx.x, kh = blockIdx.y, b = blockIdx.z;
  const int t0 = c * C64;
  const int len = p.len[b];
  if (t0 >= len) return;  // all padding: the state pass stops before this chunk
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g16 = lane >> 4, r16 = lane & 15;
  const int Lb = p.Lb, C = p.C, n_k = p.n_k;
  const ActT* mixed = (const ActT*)p.mixed + (long)b * Lb * C;
  const ActT* tail = (const ActT*)p.tail + (long)b * 3 * C;
  const ActT* cw = (const ActT*)p.conv_w;

  // ---- 1. gates of the R value heads: wave r, lane = token; inclusive scan of g over the chunk -----
  if (w < R) {
    const int h = kh * R + w;
    const int t = t0 + lane;
    const long gi = ((long)b * Lb + (t < len ? t : len - 1)) * p.n_v + h;  // len >= 1 here
    const float av = to_f32(((const ActT*)p.a)[gi]), bv = to_f32(((const ActT*)p.b)[gi]);
    const float g0 = -__expf(p.A_log[h]) * softplus(av + p.dt_bias[h]);
    const float b0 = sigmoid(bv);
    float g = t < len ? g0 : 0.f;
    const float be = t < len ? b0 : 0.f;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const float o = __shfl_up(g, off, kWave);
      if (lane >= off) g += o;
    }
    sGam[w * C64 + lane] = g;
    sBet[w * C64 + lane] = be;
  }

  // ---- 2. conv + SiLU: wave w owns tokens 16w..16w+15, lane owns channels lane*CPL + j ------------
  // every load below is unconditional from a clamped, in-range address and masked afterwards, so
  // that the compiler issues them all before the first wait
  auto conv16 = [&](int gc_base, float (*y)[CPL]) {
    float x[19][CPL], wt[4][CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int ch = lane * CPL + j;
      const bool ok = ch < D;
      const int gc = gc_base + (ok ? ch : 0);
      const float m = ok ? 1.f : 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) wt[q][j] = m * to_f32(cw[gc * 4 + q]);
#pragma unroll
      for (int i = 0; i < 19; ++i) {
        const int t = t0 + 16 * w - 3 + i;
        const ActT* src = t < 0 ? tail + (long)(t + 3) * C : mixed + (long)(t < Lb ? t : Lb - 1) * C;
        const float v = to_f32(src[gc]);
        x[i][j] = t < Lb ? v : 0.f;
      }
    }
#pragma unroll
    for (int tt = 0; tt < 16; ++tt)
#pragma unroll
      for (int j = 0; j < CPL; ++j)
        y[tt][j] = silu(wt[0][j] * x[tt][j] + wt[1][j] * x[tt + 1][j] + wt[2][j] * x[tt + 2][j] + wt[3][j] * x[tt + 3][j]);
  };
  auto l2norm16 = [&](float (*y)[CPL]) {
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < CPL; ++j) ss += y[tt][j] * y[tt][j];
      ss = wave_sum<kWave>(ss);
      const float rn = rsqrt_fast(ss + p.l2_eps);
#pragma unroll
      for (int j = 0; j < CPL; ++j) y[tt][j] *= rn;
    }
  };
  float qn[16][CPL], kn[16][CPL], vv[R][16][CPL];
  conv16(kh * D, qn);
  conv16(n_k * D + kh * D, kn);
#pragma unroll
  for (int r = 0; r < R; ++r) conv16(2 * n_k * D + (kh * R + r) * D, vv[r]);
  l2norm16(qn);
  l2norm16(kn);
#pragma unroll
  for (int tt = 0; tt < 16; ++tt)
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int ch = lane * CPL + j;
      if (ch < D) {
        const int o = (16 * w + tt) * LDW + ch;
        split_f16(kS8 * qn[tt][j], sQh[o], sQl[o]);   // Gram operands carried as 2^8 q, 2^8 k
        split_f16(kS8 * kn[tt][j], sKh[o], sKl[o]);
      }
    }
  __syncthreads();

  // ---- 3. Gram products K K^T and Q K^T on the lower 16x16 tiles (split operands) ---------------
  for (int job = w; job < 20; job += 4) {
    const int prod = job / 10, tile = job % 10;       // tiles (mt, nt), nt <= mt, in row order
    const int mt = tile >= 6 ? 3 : tile >= 3 ? 2 : tile >= 1 ? 1 : 0;
    const int nt = tile - mt * (mt + 1) / 2;
    const _Float16* ah = prod ? sQh : sKh;
    const _Float16* al = prod ? sQl : sKl;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    f16x8 fah[D / 32], fal[D / 32], fbh[D / 32], fbl[D / 32];
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const int ra = (16 * mt + r16) * LDW + 32 * ks + 8 * g16, rb = (16 * nt + r16) * LDW + 32 * ks + 8 * g16;
      fah[ks] = ld16(ah + ra);
      fal[ks] = ld16(al + ra);
      fbh[ks] = ld16(sKh + rb);
      fbl[ks] = ld16(sKl + rb);
    }
    __builtin_amdgcn_sched_barrier(0);  // the reads go out together, then the MFMAs
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      acc = mfma16(fal[ks], fbh[ks], acc);
      acc = mfma16(fah[ks], fbl[ks], acc);
      acc = mfma16(fah[ks], fbh[ks], acc);
    }
    float* dst = prod ? sQK : sKK;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[(16 * mt + 4 * g16 + i) * LF + 16 * nt + r16] = acc[i];
  }
  __syncthreads();

  // ---- 4. per value head of the group ------------------------------------------------------------
  for (int r = 0; r < R; ++r) {
    const int h = kh * R + r;
    const float* gam = sGam + r * C64;
    const float* bet = sBet + r * C64;
    char* rec = rec_ptr<D, SPLIT>(p, b, h, c);
    _Float16* img = (_Float16*)(rec + Rec<D, SPLIT>::kImg);
    _Float16* imgB = img + I::A_HALFS;
    const float gC = gam[C64 - 1];

    // A (strictly lower, fp32), T's upper blocks cleared
    for (int idx = tid; idx < C64 * C64; idx += 256) {
      const int i = idx >> 6, j = idx & 63;
      sA[i * LF + j] = j < i ? bet[i] * __expf(gam[i] - gam[j]) * (kInvS16 * sKK[i * LF + j]) : 0.f;
      if ((j >> 4) > (i >> 4)) sTf[i * LF + j] = 0.f;
    }
    // B operands of W and U' (channel-major) in LDS; Q~ and K~^T straight into the image
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) {
      const int tl = 16 * w + tt;
      const float eg = __expf(gam[tl]);
      const float bk = bet[tl] * eg, bv = bet[tl], ek = __expf(gC - gam[tl]), sq = p.scale * eg;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int ch = lane * CPL + j;
        if (ch < D) {
          const float kb = kS8 * bk * kn[tt][j];
          if (SPLIT) split_f16(kb, sKb[ch * LDT + tl], sKb[D * LDT + ch * LDT + tl]);
          else sKb[ch * LDT + tl] = (_Float16)kb;
          split_f16(kS8 * bv * vv[r][tt][j], sVbh[ch * LDT + tl], sVbl[ch * LDT + tl]);
          const float qv = kS8 * sq * qn[tt][j];
          const int qo = swz<D>(tl, pcol(ch));
          split_f16(qv, img[I::Q_HI + qo], img[I::Q_LO + qo]);
        }
      }
    }
    // K~^T hi/lo: row = channel, 4-token runs of this wave's 16 tokens land 4 halfs apart
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int ch = lane * CPL + j;
      if (ch < D) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f16x4 hi, lo;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int tl = 16 * w + 4 * q + e;
            const float kv = kS8 * __expf(gC - gam[tl]) * kn[4 * q + e][j];
            hi[e] = (_Float16)kv;
            lo[e] = (_Float16)(kv - (float)hi[e]);
          }
          const int ko = swz<C64>(ch, (w >> 1) * 32 + 8 * q + 4 * (w & 1));
          *(f16x4*)&imgB[I::K_HI + ko] = hi;
          *(f16x4*)&imgB[I::K_LO + ko] = lo;
        }
      }
    }
    __syncthreads();

    // T = (I + A)^-1: diagonal blocks by forward substitution (wave 0, one column per lane)
    if (w == 0) {
      const int blk = lane >> 4, jj = lane & 15;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float s = i == jj ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < i; ++m) s -= sA[(16 * blk + i) * LF + 16 * blk + m] * x[m];
        x[i] = s;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sTf[(16 * blk + i) * LF + 16 * blk + jj] = x[i];
    }
    __syncthreads();
    // off-diagonal blocks by level (i - j = 1, 2, 3): T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj, fp32 MFMA
    float* sXw = sX + w * 16 * 17;
    for (int lvl = 1; lvl < 4; ++lvl) {
      if (w < 4 - lvl) {
        const int j = w, i = w + lvl;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int k = j; k < i; ++k)
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            acc = mfma_f32(sA[(16 * i + r16) * LF + 16 * k + 4 * ks + g16], sTf[(16 * k + 4 * ks + g16) * LF + 16 * j + r16], acc);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) sXw[(4 * g16 + ii) * 17 + r16] = acc[ii];
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          y = mfma_f32(sTf[(16 * i + r16) * LF + 16 * i + 4 * ks + g16], sXw[(4 * ks + g16) * 17 + r16], y);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) sTf[(16 * i + 4 * g16 + ii) * LF + 16 * j + r16] = -y[ii];
      }
      __syncthreads();
    }
    for (int idx = tid; idx < C64 * C64; idx += 256) {
      const int i = idx >> 6, j = idx & 63;
      const float tv = kS8 * sTf[i * LF + j];
      if (SPLIT) split_f16(tv, sT[i * LDT + j], sT[C64 * LDT + i * LDT + j]);
      else sT[i * LDT + j] = (_Float16)tv;
    }
    __syncthreads();

    // W^T = (beta e^gamma K)^T T^T  -> image rows = token (4 consecutive d_k per lane, 8-byte stores)
    // U'  = T (beta V)               -> fragment order
    {
      float* gUp = (float*)(rec + Rec<D, SPLIT>::kUp);
      for (int nt = w; nt < D / 16; nt += 4) {
        // this d-tile's B fragments, reused by the four token tiles
        f16x8 kbh[2], kbl[2], vbh[2], vbl[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int rc = (16 * nt + r16) * LDT + 32 * ks + 8 * g16;
          kbh[ks] = ld16(sKb + rc);
          kbl[ks] = SPLIT ? ld16(sKb + D * LDT + rc) : kbh[ks];
          vbh[ks] = ld16(sVbh + rc);
          vbl[ks] = ld16(sVbl + rc);
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4 aw = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
          f16x8 th[2], tl[2];
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const int rt = (16 * mt + r16) * LDT + 32 * ks + 8 * g16;
            th[ks] = ld16(sT + rt);
            tl[ks] = SPLIT ? ld16(sT + C64 * LDT + rt) : th[ks];
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            if (SPLIT) {
              aw = mfma16(kbl[ks], th[ks], aw);
              aw = mfma16(kbh[ks], tl[ks], aw);
              au = mfma16(tl[ks], vbh[ks], au);
            }
            aw = mfma16(kbh[ks], th[ks], aw);
            au = mfma16(th[ks], vbl[ks], au);
            au = mfma16(th[ks], vbh[ks], au);
          }
          // au = (2^8 T)(2^8 beta V) = 2^16 U'; the state pass takes 2^8 U'
          *(f32x4*)&gUp[((long)(nt * 4 + mt) * kWave + lane) * 4] = au * kInvS8;
          const int wo = swz<D>(16 * mt + r16, 32 * (nt >> 1) + 8 * g16 + 4 * (nt & 1));
          f16x4 hi, lo;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float wv = -kInvS16 * aw[i];   // aw = (2^8 beta e^gamma K)^T (2^8 T)^T = 2^16 W^T
            hi[i] = (_Float16)wv;
            lo[i] = (_Float16)(wv - (float)hi[i]);
          }
          *(f16x4*)&img[I::W_HI + wo] = hi;
          if (SPLIT) *(f16x4*)&img[I::W_LO + wo] = lo;
        }
      }
    }
    // P~ = scale * decay-masked Q K^T (s <= t), 8 permuted columns per 16-byte store
    {
      const int t = tid >> 2;
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const int grp = 2 * (tid & 3) + pp;      // 8-column group: block grp/4, lane-group grp%4
        const int kk = grp >> 2, gg = grp & 3;
        f16x8 hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int s = 32 * kk + (e < 4 ? 4 * gg + e : 16 + 4 * gg + e - 4);
          const float val = s <= t ? p.scale * __expf(gam[t] - gam[s]) * (kInvS8 * sQK[t * LF + s]) : 0.f;
          hi[e] = (_Float16)val;
          lo[e] = (_Float16)(val - (float)hi[e]);
        }
        const int po = swz<C64>(t, 8 * grp);
        *(f16x8*)&imgB[I::P_HI + po] = hi;
        *(f16x8*)&imgB[I::P_LO + po] = lo;
      }
    }
    if (tid == 0) *(float*)(rec + Rec<D, SPLIT>::kGc) = __expf(gC);
    __syncthreads();
  }
}

// -------------------------------------------------------------------------------------------------
// State pass. NW waves x NT 16-column tiles per wave = the workgroup's d_v slice.
template <typename ActT, int D, int NW, int NT, bool SPLIT, bool FUSED>
__global__ __launch_bounds__(64 * NW) void state_pass_kernel(PrefillArgs p) {
  using I = Img<D, SPLIT>;
  constexpr int HM = D / 16, KD = D / 32, CW = NW * 16 * NT, NSPLIT = D / CW;
  static_assert(NSPLIT * CW == D, "column split");
  static_assert(FUSED == (NSPLIT == 1), "the norm is fused exactly when one workgroup owns the head");
  static_assert(NW * C64 * 4 <= I::B_BYTES, "norm exchange fits in a consumed part B");
  // LDS: part A (W, Q~) single-buffered, reloaded as soon as a chunk has used it; part B (K~^T, P~)
  // double-buffered, the next chunk's copy streaming in during the whole current chunk
  __shared__ __attribute__((aligned(1024))) char smem[I::A_BYTES + 2 * I::B_BYTES];

  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g16 = lane >> 4, r16 = lane & 15;
  const int Lb = p.Lb, n_v = p.n_v, C = p.C;
  const int len = p.len[b];
  const int n_real = (len + C64 - 1) / C64;
  const int cb = split * CW + w * 16 * NT;  // first d_v column of this wave

  // direct global->LDS copies, 1 KB per wave instruction (lane i's 16 bytes land at 16 i)
  // (a fixed count per wave, so the compiler can count them when it waits for later loads)
  static_assert((I::A_BYTES / 1024) % NW == 0 && (I::B_BYTES / 1024) % NW == 0, "copies split evenly over waves");
  char* const ldsA = smem;
  auto ldsB = [&](int buf) { return smem + I::A_BYTES + buf * I::B_BYTES; };
  auto prefetch_A = [&](int c) {
    const char* src = rec_ptr<D, SPLIT>(p, b, h, c) + lane * 16;
#pragma unroll
    for (int k = 0; k < I::A_BYTES / 1024 / NW; ++k)
      __builtin_amdgcn_global_load_lds((const void*)(src + (w + k * NW) * 1024), (lds_void*)(ldsA + (w + k * NW) * 1024), 16, 0, 0);
  };
  auto prefetch_B = [&](int c, int buf) {
    const char* src = rec_ptr<D, SPLIT>(p, b, h, c) + I::A_BYTES + lane * 16;
    char* dst = ldsB(buf);
#pragma unroll
    for (int k = 0; k < I::B_BYTES / 1024 / NW; ++k)
      __builtin_amdgcn_global_load_lds((const void*)(src + (w + k * NW) * 1024), (lds_void*)(dst + (w + k * NW) * 1024), 16, 0, 0);
  };
  // U', e^{gamma_C} and (fused norm) z of chunk c, loaded one chunk ahead so that the wait at the top
  // of the loop covers them
  typedef typename Raw4<ActT>::type RawZ;
  auto load_up = [&](int c, f32x4 (*u)[NT], float& gc, RawZ (*zr)[NT]) {
    if (FUSED) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int t = c * C64 + 16 * mt + r16;  // rows past Lb read row Lb-1; their results are never stored
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          zr[mt][nt] = Raw4<ActT>::load((const ActT*)p.z + (((long)b * Lb + (t < Lb ? t : Lb - 1)) * n_v + h) * D + cb + 16 * nt + 4 * g16);
      }
    }
    const char* rec = rec_ptr<D, SPLIT>(p, b, h, c);
    const float* gUp = (const float*)(rec + Rec<D, SPLIT>::kUp);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) u[mt][nt] = *(const f32x4*)&gUp[((long)((cb / 16 + nt) * 4 + mt) * kWave + lane) * 4];
    gc = *(const float*)(rec + Rec<D, SPLIT>::kGc);
  };

  float* st = p.state + ((long)b * n_v + h) * D * D;
  f32x4 H[HM][NT];
#pragma unroll
  for (int hm = 0; hm < HM; ++hm)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) H[hm][nt][i] = 65536.f * st[(long)(16 * hm + 4 * g16 + i) * D + cb + 16 * nt + r16];

  float nw[NT][4];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) nw[nt][i] = p.norm_w[cb + 16 * nt + 4 * g16 + i];

  ActT* out = (ActT*)p.out;
  float* oraw = (float*)((char*)p.ws + p.oraw_off);
  float* sspart = (float*)((char*)p.ws + p.ss_off);

  f32x4 Upn[4][NT];
  float gCn = 0.f;
  RawZ zn[4][NT];
  f32x4 res[4][NT];      // finished rows of the previous chunk, stored at the top of the next iteration
  int res_c = -1;
  auto store_res = [&](int c) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int t = c * C64 + 16 * mt + r16;
      if (t < Lb) {
        const long rowb = ((long)b * Lb + t) * n_v + h;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int col = cb + 16 * nt + 4 * g16;
          const float4 v = make_float4(res[mt][nt][0], res[mt][nt][1], res[mt][nt][2], res[mt][nt][3]);
          if (FUSED) Act4<ActT>::store(out + rowb * D + col, v);
          else *(float4*)(oraw + rowb * D + col) = v;
        }
      }
    }
  };

  if (n_real > 0) {
    prefetch_A(0);
    prefetch_B(0, 0);
    load_up(0, Upn, gCn, zn);
  }
  for (int c = 0; c < n_real; ++c) {
    const int buf = c & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const _Float16* img = (const _Float16*)ldsA;
    const _Float16* imgB = (const _Float16*)ldsB(buf);
    if (res_c >= 0) store_res(res_c);
    f32x4 U[4][NT];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) U[mt][nt] = Upn[mt][nt];
    const float gC = gCn;
    RawZ zr[4][NT];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) zr[mt][nt] = zn[mt][nt];
    if (c + 1 < n_real) {
      prefetch_B(c + 1, buf ^ 1);
      load_up(c + 1, Upn, gCn, zn);
    }

    // H as an operand (rows d_k in the permuted 32-groups), hi/lo
    f16x8 Hb[KD][NT], Hl[KD][NT];
#pragma unroll
    for (int kk = 0; kk < KD; ++kk)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) pack_split(H[2 * kk][nt] * kInvS8, H[2 * kk + 1][nt] * kInvS8, Hb[kk][nt], Hl[kk][nt]);
    // U = U' - W H ; O^T = H^T Q~^T. Operand fragments are loaded a row-block at a time before the
    // MFMAs that use them, so the LDS reads overlap instead of waiting one by one.
    f32x4 OT[4][NT];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) OT[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      f16x8 aw[KD], bq[KD], bql[KD], awl[SPLIT ? KD : 1];
#pragma unroll
      for (int kk = 0; kk < KD; ++kk) {
        const int ro = swz<D>(16 * mt + r16, 32 * kk + 8 * g16);
        aw[kk] = ld16(img + I::W_HI + ro);
        bq[kk] = ld16(img + I::Q_HI + ro);
        bql[kk] = ld16(img + I::Q_LO + ro);
        if (SPLIT) awl[kk] = ld16(img + I::W_LO + ro);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the batch of reads ahead of the MFMAs
#pragma unroll
      for (int kk = 0; kk < KD; ++kk)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if (SPLIT) U[mt][nt] = mfma16(awl[kk], Hb[kk][nt], U[mt][nt]);
          OT[mt][nt] = mfma16(Hb[kk][nt], bql[kk], OT[mt][nt]);
          U[mt][nt] = mfma16(aw[kk], Hl[kk][nt], U[mt][nt]);
          U[mt][nt] = mfma16(aw[kk], Hb[kk][nt], U[mt][nt]);
          OT[mt][nt] = mfma16(Hl[kk][nt], bq[kk], OT[mt][nt]);
          OT[mt][nt] = mfma16(Hb[kk][nt], bq[kk], OT[mt][nt]);
        }
    }
    // every wave is done with part A: the next chunk's copy can stream in now
    lds_barrier();
    if (c + 1 < n_real) prefetch_A(c + 1);
    // U as an operand (tokens in the permuted 32-groups), hi/lo
    f16x8 Uh[2][NT], Ul[2][NT];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) pack_split(U[2 * kk][nt], U[2 * kk + 1][nt], Uh[kk][nt], Ul[kk][nt]);
    // O^T += U^T P~^T
    {
      f16x8 bp[4][2], bpl[4][2];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int ro = swz<C64>(16 * mt + r16, 32 * kk + 8 * g16);
          bp[mt][kk] = ld16(imgB + I::P_HI + ro);
          bpl[mt][kk] = ld16(imgB + I::P_LO + ro);
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            OT[mt][nt] = mfma16(Uh[kk][nt], bpl[mt][kk], OT[mt][nt]);
            OT[mt][nt] = mfma16(Ul[kk][nt], bp[mt][kk], OT[mt][nt]);
            OT[mt][nt] = mfma16(Uh[kk][nt], bp[mt][kk], OT[mt][nt]);
          }
    }
    // H = e^{gamma_C} H + K~^T U, four 16-row blocks of K~^T per batch of loads
    constexpr int KBAT = HM < 4 ? HM : 4;
#pragma unroll
    for (int hb = 0; hb < HM; hb += KBAT) {
      f16x8 akh[KBAT][2], akl[KBAT][2];
#pragma unroll
      for (int q = 0; q < KBAT; ++q)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int ro = swz<C64>(16 * (hb + q) + r16, 32 * kk + 8 * g16);
          akh[q][kk] = ld16(imgB + I::K_HI + ro);
          akl[q][kk] = ld16(imgB + I::K_LO + ro);
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < KBAT; ++q) {
        const int hm = hb + q;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) H[hm][nt][i] *= gC;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            H[hm][nt] = mfma16(akl[q][kk], Uh[kk][nt], H[hm][nt]);
            H[hm][nt] = mfma16(akh[q][kk], Ul[kk][nt], H[hm][nt]);
            H[hm][nt] = mfma16(akh[q][kk], Uh[kk][nt], H[hm][nt]);
          }
      }
    }

    // epilogue: O^T tile (mt, nt) holds token 16mt + r16, columns cb + 16nt + 4g16 .. +3 (as 2^16 O^T)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) OT[mt][nt] = OT[mt][nt] * kInvS16;
    float ssw[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      float ss = 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) ss += OT[mt][nt][i] * OT[mt][nt][i];
      ss += __shfl_xor(ss, 16, kWave);
      ss += __shfl_xor(ss, 32, kWave);
      ssw[mt] = ss;
    }
    if (FUSED) {
      // cross-wave sums through the image this chunk has finished with
      lds_barrier();
      float* sSS = (float*)ldsB(buf);
      if (g16 == 0) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) sSS[w * C64 + 16 * mt + r16] = ssw[mt];
      }
      lds_barrier();
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        float ss = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) ss += sSS[ww * C64 + 16 * mt + r16];
        const float inv = rsqrt_fast(ss / (float)D + p.rms_eps);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const float4 zf = Raw4<ActT>::widen(zr[mt][nt]);
          const float zz[4] = {zf.x, zf.y, zf.z, zf.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) res[mt][nt][i] = nw[nt][i] * (OT[mt][nt][i] * inv) * silu(zz[i]);
        }
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int t = c * C64 + 16 * mt + r16;
        if (g16 == 0 && t < Lb) sspart[(((long)b * Lb + t) * n_v + h) * (NSPLIT * NW) + split * NW + w] = ssw[mt];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) res[mt][nt] = OT[mt][nt];
      }
    }
    res_c = c;
  }
  if (res_c >= 0) store_res(res_c);

  // final state, in place
#pragma unroll
  for (int hm = 0; hm < HM; ++hm)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) st[(long)(16 * hm + 4 * g16 + i) * D + cb + 16 * nt + r16] = H[hm][nt][i] * kInvS16;

  // conv tail: rows len .. len+2 of [old tail | mixed]. Split 0 of value head h owns its v channels;
  // split 0 of the first value head of each GQA group also the q and k channels of its key head.
  if (split == 0) {
    const int R = n_v / p.n_k;
    ActT* tl = (ActT*)p.tail + (long)b * 3 * C;
    const ActT* mx = (const ActT*)p.mixed + (long)b * Lb * C;
    const int kh = h / R;
    const int nch = (h % R == 0) ? 3 * D : D;
    for (int lc = tid; lc < nch; lc += 64 * NW) {
      int gc;
      if (lc < D) gc = 2 * p.n_k * D + h * D + lc;
      else if (lc < 2 * D) gc = kh * D + (lc - D);
      else gc = p.n_k * D + kh * D + (lc - 2 * D);
      ActT v3[3];
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const int src = len + i;  // row of [tail | mixed]
        v3[i] = src < 3 ? tl[(long)src * C + gc] : mx[(long)(src - 3) * C + gc];
      }
#pragma unroll
      for (int i = 0; i < 3; ++i) tl[(long)i * C + gc] = v3[i];
    }
  }
}

// the gated RMSNorm when a head's columns were split: out = w * o / rms(o) * silu(z)
template <typename ActT, int D, int NPART>
__global__ __launch_bounds__(256) void norm_kernel(PrefillArgs p) {
  const long n = (long)p.B * p.Lb * p.n_v * (D / 4);
  const float* oraw = (const float*)((const char*)p.ws + p.oraw_off);
  const float* sspart = (const float*)((const char*)p.ws + p.ss_off);
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    const int cq = (int)(i % (D / 4));
    const long row = i / (D / 4);  // (b, t, h)
    const int bt = (int)(row / p.n_v);
    const int b = bt / p.Lb, t = bt % p.Lb;
    if (t >= p.len[b]) continue;
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NPART; ++k) ss += sspart[row * NPART + k];
    const float inv = rsqrt_fast(ss / (float)D + p.rms_eps);
    const float4 o = *(const float4*)(oraw + row * D + 4 * cq);
    const float4 z = Act4<ActT>::load((const ActT*)p.z + row * D + 4 * cq);
    const float* nw = p.norm_w + 4 * cq;
    const float4 v = make_float4(nw[0] * (o.x * inv) * silu(z.x), nw[1] * (o.y * inv) * silu(z.y),
                                 nw[2] * (o.z * inv) * silu(z.z), nw[3] * (o.w * inv) * silu(z.w));
    Act4<ActT>::store((ActT*)p.out + row * D + 4 * cq, v);
  }
}

// ---- launch configuration --------------------------------------------------------------------------
struct PassCfg {
  int nw, nt, nsplit;
};
PassCfg pass_cfg(int B, int n_v, int D, bool split_all) {
  if (D == 128 && !split_all) return B * n_v < 128 ? PassCfg{2, 1, 4} : PassCfg{4, 2, 1};
  if (D == 64) return PassCfg{4, 1, 1};
  return PassCfg{2, 1, 1};
}

long rec_bytes(int D, bool split_all) {
  if (split_all) return D == 32 ? Rec<32, true>::kBytes : Rec<64, true>::kBytes;
  return D == 32 ? Rec<32, false>::kBytes : D == 64 ? Rec<64, false>::kBytes : Rec<128, false>::kBytes;
}

template <typename ActT, int D, int R, bool SPLIT, int NW, int NT>
hipError_t launch_t(const PrefillArgs& p, hipStream_t st) {
  constexpr int NSPLIT = D / (NW * 16 * NT);
  hipLaunchKernelGGL((chunk_prep_kernel<ActT, D, R, SPLIT>), dim3(p.n_chunks, p.n_k, p.B), dim3(256), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((state_pass_kernel<ActT, D, NW, NT, SPLIT, NSPLIT == 1>), dim3(NSPLIT, p.n_v, p.B),
                     dim3(64 * NW), 0, st, p);
  e = hipGetLastError();
  if (e != hipSuccess || NSPLIT == 1) return e;
  const long n = (long)p.B * p.Lb * p.n_v * (D / 4);
  const long blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  hipLaunchKernelGGL((norm_kernel<ActT, D, NSPLIT * NW>), dim3((unsigned)blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <typename ActT, int D, bool SPLIT, int NW, int NT>
hipError_t launch_r(const PrefillArgs& p, int R, hipStream_t st) {
  switch (R) {
    case 1: return launch_t<ActT, D, 1, SPLIT, NW, NT>(p, st);
    case 2: return launch_t<ActT, D, 2, SPLIT, NW, NT>(p, st);
    case 4: return launch_t<ActT, D, 4, SPLIT, NW, NT>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t prefill_ws_bytes(int B, int n_v, int D, int Lb, int n_chunks, bool split_all) {
  const PassCfg cfg = pass_cfg(B, n_v, D, split_all);
  size_t bytes = (size_t)B * n_v * n_chunks * rec_bytes(D, split_all);
  if (cfg.nsplit > 1) {
    bytes += (size_t)B * Lb * n_v * D * 4;                       // unnormalised o
    bytes += (size_t)B * Lb * n_v * cfg.nsplit * cfg.nw * 4;     // partial sums of squares
    bytes = (bytes + 255) / 256 * 256;
  }
  return bytes;
}

void prefill_ws_layout(PrefillArgs& p, int D, bool split_all) {
  const size_t rec = (size_t)p.B * p.n_v * p.n_chunks * rec_bytes(D, split_all);
  p.oraw_off = (long)rec;
  p.ss_off = (long)(rec + (size_t)p.B * p.Lb * p.n_v * D * 4);
}

hipError_t launch_prefill(const PrefillArgs& p, int act_dtype, int D, int R, hipStream_t st) {
  if (act_dtype == kActBf16) {
    const PassCfg cfg = pass_cfg(p.B, p.n_v, D, false);
    if (D == 32) return launch_r<bf16_t, 32, false, 2, 1>(p, R, st);
    if (D == 64) return launch_r<bf16_t, 64, false, 4, 1>(p, R, st);
    if (D == 128) {
      if (cfg.nsplit == 1) return launch_r<bf16_t, 128, false, 4, 2>(p, R, st);
      return launch_r<bf16_t, 128, false, 2, 1>(p, R, st);
    }
  } else {
    if (D == 32) return launch_r<float, 32, true, 2, 1>(p, R, st);
    if (D == 64) return launch_r<float, 64, true, 4, 1>(p, R, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
