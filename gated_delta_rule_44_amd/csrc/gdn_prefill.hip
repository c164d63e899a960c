// Chunked prefill of the gated delta rule (gfx950), in two launches.
//
// Chunk form (chunk of C = 64 tokens, entering state H0 = S0^T, gamma_r = sum_{i<=r} g_i inside the
// chunk; derived from the recurrence S_t = e^{g_t} S_{t-1}(I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
// the WY/UT-transform treatment of the delta rule):
//   A[r][s] = beta_r e^{gamma_r - gamma_s} k_r.k_s (s < r),  T = (I + A)^-1
//   W = T diag(beta e^gamma) K,   U' = T diag(beta) V,   P[r][s] = e^{gamma_r - gamma_s} q_r.k_s (s <= r)
//   U = U' - W H0,   O = scale (diag(e^gamma) Q H0 + P U),   H_C = e^{gamma_C} H0 + K^T diag(e^{gamma_C - gamma}) U
// Every decay factor is the exponential of a non-positive difference, never a product of e^{gamma_r}
// and e^{-gamma_s}, so strong decays underflow to 0 instead of overflowing.
//
// Launch 1, chunk_prep_kernel (all chunks in parallel; one workgroup per chunk x key head x sequence):
//   conv + SiLU on [saved tail | chunk], q/k L2 norm, gates and the padding mask, the Gram products
//   K K^T and Q K^T on f16 MFMA with hi/lo-split operands (the products whose rounding the output is
//   most sensitive to), then per value head of the GQA group the UT inverse T (fp32, 16x16 blocks),
//   W and U' on f16 MFMA, and the operands of the state pass, written to the workspace.
// Launch 2, state_pass_kernel (one workgroup per value head x sequence, walking the chunks in order):
//   H stays in MFMA accumulator registers for the whole call, each wave owning a slice of d_v
//   columns; per chunk U = U' - W H, O = Q~ H + P~ U and H = e^{gamma_C} H + K~^T U are f16 MFMA
//   products, then the gated RMSNorm epilogue; finally the fp32 state and the conv tail are written
//   back in place.
#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

constexpr int C64 = kChunk;

// workspace record of one (sequence, value head, chunk)
template <int D>
struct Rec {
  static constexpr long kWn = 0;                         // -W       f16 [64][D]
  static constexpr long kQt = kWn + 2L * C64 * D;        // Q~       f16 [64][D]   scale e^gamma q
  static constexpr long kKtT = kQt + 2L * C64 * D;       // K~^T     f16 [D][64]   (e^{gamma_C-gamma} k)^T
  static constexpr long kPt = kKtT + 2L * C64 * D;       // P~       f16 [64][64]  scale P
  static constexpr long kUp = kPt + 2L * C64 * C64;      // U'       fp32, MFMA fragment order
  static constexpr long kGc = kUp + 4L * C64 * D;        // e^{gamma_C}
  static constexpr long kBytes = ((kGc + 16 + 255) / 256) * 256;
};

template <int D>
__device__ __forceinline__ char* rec_ptr(const PrefillArgs& p, int b, int h, int c) {
  return (char*)p.ws + (((long)b * p.n_v + h) * p.n_chunks + c) * Rec<D>::kBytes;
}

// -------------------------------------------------------------------------------------------------
template <typename ActT, int D, int R>
__global__ __launch_bounds__(256) void chunk_prep_kernel(PrefillArgs p) {
  constexpr int CPL = D >= 64 ? D / 64 : 1;   // channels per lane in the conv stage
  constexpr int LD = D + 8;                   // f16 row stride of token-major tiles
  constexpr int LT = C64 + 8;                 // f16 row stride of channel-major / 64-wide tiles
  constexpr int LF = C64 + 1;                 // fp32 row stride of 64x64 matrices
  constexpr int SZ_TOK = C64 * LD * 2;
  constexpr int SZ_CH = D * LT * 2;
  constexpr int OFF_QH = 0, OFF_QL = SZ_TOK, OFF_KH = 2 * SZ_TOK, OFF_KL = 3 * SZ_TOK;
  constexpr int OFF_KT = 0, OFF_VT = SZ_CH, OFF_WS = 2 * SZ_CH;   // reuse after the Gram
  static_assert(OFF_WS + SZ_TOK <= 4 * SZ_TOK, "reuse fits");
  constexpr int OFF_KK = 4 * SZ_TOK;
  constexpr int OFF_QK = OFF_KK + C64 * LF * 4;
  constexpr int OFF_A = OFF_QK + C64 * LF * 4;
  constexpr int OFF_X = OFF_A + C64 * LF * 4;
  constexpr int OFF_T = OFF_X + 16 * 17 * 4;
  constexpr int OFF_G = OFF_T + C64 * LT * 2;
  constexpr int OFF_B = OFF_G + R * C64 * 4;
  constexpr int LDS = OFF_B + R * C64 * 4;
  __shared__ __attribute__((aligned(16))) char smem[LDS];
  _Float16* sQh = (_Float16*)(smem + OFF_QH);
  _Float16* sQl = (_Float16*)(smem + OFF_QL);
  _Float16* sKh = (_Float16*)(smem + OFF_KH);
  _Float16* sKl = (_Float16*)(smem + OFF_KL);
  _Float16* sKT = (_Float16*)(smem + OFF_KT);
  _Float16* sVT = (_Float16*)(smem + OFF_VT);
  _Float16* sWs = (_Float16*)(smem + OFF_WS);
  float* sKK = (float*)(smem + OFF_KK);
  float* sQK = (float*)(smem + OFF_QK);
  float* sA = (float*)(smem + OFF_A);
  float* sX = (float*)(smem + OFF_X);
  _Float16* sT = (_Float16*)(smem + OFF_T);
  float* sGam = (float*)(smem + OFF_G);
  float* sBet = (float*)(smem + OFF_B);

  const int c = blockIdx.x, kh = blockIdx.y, b = blockIdx.z;
  const int t0 = c * C64;
  const int len = p.len[b];
  if (t0 >= len) return;  // all padding: the state pass skips this chunk
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g16 = lane >> 4, r16 = lane & 15;
  const int Lb = p.Lb, C = p.C, n_k = p.n_k;
  const ActT* mixed = (const ActT*)p.mixed + (long)b * Lb * C;
  const ActT* tail = (const ActT*)p.tail + (long)b * 3 * C;
  const ActT* cw = (const ActT*)p.conv_w;

  // ---- 1. conv + SiLU: wave w owns tokens 16w..16w+15, lane owns channels lane*CPL + j ----------
  auto conv16 = [&](int gc_base, float (*y)[CPL]) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int ch = lane * CPL + j;
      if (ch >= D) {
#pragma unroll
        for (int tt = 0; tt < 16; ++tt) y[tt][j] = 0.f;
        continue;
      }
      const int gc = gc_base + ch;
      const float w0 = to_f32(cw[gc * 4 + 0]), w1 = to_f32(cw[gc * 4 + 1]);
      const float w2 = to_f32(cw[gc * 4 + 2]), w3 = to_f32(cw[gc * 4 + 3]);
      float x[19];
#pragma unroll
      for (int i = 0; i < 19; ++i) {
        const int t = t0 + 16 * w - 3 + i;
        x[i] = t < 0 ? to_f32(tail[(long)(t + 3) * C + gc]) : (t < Lb ? to_f32(mixed[(long)t * C + gc]) : 0.f);
      }
#pragma unroll
      for (int tt = 0; tt < 16; ++tt)
        y[tt][j] = silu(w0 * x[tt] + w1 * x[tt + 1] + w2 * x[tt + 2] + w3 * x[tt + 3]);
    }
  };
  auto l2norm16 = [&](float (*y)[CPL]) {
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < CPL; ++j) ss += y[tt][j] * y[tt][j];
      ss = wave_sum<kWave>(ss);
      const float rn = 1.0f / sqrtf(ss + p.l2_eps);
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
  for (int tt = 0; tt < 16; ++tt) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int ch = lane * CPL + j;
      if (ch < D) {
        const int o = (16 * w + tt) * LD + ch;
        split_f16(qn[tt][j], sQh[o], sQl[o]);
        split_f16(kn[tt][j], sKh[o], sKl[o]);
      }
    }
  }
  // gates for the R value heads: wave r, lane = token; inclusive scan of g over the chunk
  if (w < R) {
    const int h = kh * R + w;
    const int t = t0 + lane;
    float g = 0.f, be = 0.f;
    if (t < len) {
      const long gi = ((long)b * Lb + t) * p.n_v + h;
      g = -__expf(p.A_log[h]) * softplus(to_f32(((const ActT*)p.a)[gi]) + p.dt_bias[h]);
      be = sigmoid(to_f32(((const ActT*)p.b)[gi]));
    }
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const float o = __shfl_up(g, off, kWave);
      if (lane >= off) g += o;
    }
    sGam[w * C64 + lane] = g;
    sBet[w * C64 + lane] = be;
  }
  __syncthreads();

  // ---- 2. Gram products K K^T and Q K^T (lower 16x16 tiles), split-f16 operands ----------------
  for (int nt = 0; nt <= w; ++nt) {
    f32x4 kk = {0.f, 0.f, 0.f, 0.f}, qk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const int col = 32 * ks + 8 * g16;
      const int ra = (16 * w + r16) * LD + col, rb = (16 * nt + r16) * LD + col;
      const f16x8 akh = *(const f16x8*)&sKh[ra], akl = *(const f16x8*)&sKl[ra];
      const f16x8 aqh = *(const f16x8*)&sQh[ra], aql = *(const f16x8*)&sQl[ra];
      const f16x8 bkh = *(const f16x8*)&sKh[rb], bkl = *(const f16x8*)&sKl[rb];
      kk = mfma16(akl, bkh, kk);
      kk = mfma16(akh, bkl, kk);
      kk = mfma16(akh, bkh, kk);
      qk = mfma16(aql, bkh, qk);
      qk = mfma16(aqh, bkl, qk);
      qk = mfma16(aqh, bkh, qk);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sKK[(16 * w + 4 * g16 + i) * LF + 16 * nt + r16] = kk[i];
      sQK[(16 * w + 4 * g16 + i) * LF + 16 * nt + r16] = qk[i];
    }
  }
  __syncthreads();

  // ---- 3. per value head of the group ----------------------------------------------------------
  for (int r = 0; r < R; ++r) {
    const int h = kh * R + r;
    const float* gam = sGam + r * C64;
    const float* bet = sBet + r * C64;
    char* rec = rec_ptr<D>(p, b, h, c);

    // A (strictly lower) in fp32
    for (int idx = tid; idx < C64 * C64; idx += 256) {
      const int i = idx >> 6, j = idx & 63;
      sA[i * LF + j] = j < i ? bet[i] * __expf(gam[i] - gam[j]) * sKK[i * LF + j] : 0.f;
    }
    __syncthreads();
    // T = (I + A)^-1 in place: diagonal 16x16 blocks by forward substitution (one column per lane)
    {
      float x[16];
      const int blk = lane >> 4, jj = lane & 15;
      if (w == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float s = i == jj ? 1.f : 0.f;
#pragma unroll
          for (int m = 0; m < i; ++m) s -= sA[(16 * blk + i) * LF + 16 * blk + m] * x[m];
          x[i] = s;
        }
      }
      __syncthreads();
      if (w == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sA[(16 * blk + i) * LF + 16 * blk + jj] = x[i];
      }
      __syncthreads();
    }
    // off-diagonal blocks: T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj, row blocks in order, j ascending
    {
      const int rr = tid >> 4, cc = tid & 15;
      for (int i = 1; i < 4; ++i) {
        for (int j = 0; j < i; ++j) {
          float xs = 0.f;
          for (int k = j; k < i; ++k) {
#pragma unroll
            for (int m = 0; m < 16; ++m) xs += sA[(16 * i + rr) * LF + 16 * k + m] * sA[(16 * k + m) * LF + 16 * j + cc];
          }
          sX[rr * 17 + cc] = xs;
          __syncthreads();
          float ys = 0.f;
#pragma unroll
          for (int m = 0; m < 16; ++m) ys += sA[(16 * i + rr) * LF + 16 * i + m] * sX[m * 17 + cc];
          sA[(16 * i + rr) * LF + 16 * j + cc] = -ys;
          __syncthreads();
        }
      }
    }
    for (int idx = tid; idx < C64 * C64; idx += 256) {
      const int i = idx >> 6, j = idx & 63;
      sT[i * LT + j] = (_Float16)sA[i * LF + j];
    }
    // B operands of W and U' (channel-major), and the state-pass operands Q~ and K~^T
    {
      const float gC = gam[C64 - 1];
      _Float16* gQt = (_Float16*)(rec + Rec<D>::kQt);
      _Float16* gKtT = (_Float16*)(rec + Rec<D>::kKtT);
#pragma unroll
      for (int tt = 0; tt < 16; ++tt) {
        const int tl = 16 * w + tt;
        const float eg = __expf(gam[tl]);
        const float bk = bet[tl] * eg, bv = bet[tl], ek = __expf(gC - gam[tl]), sq = p.scale * eg;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          const int ch = lane * CPL + j;
          if (ch < D) {
            sKT[ch * LT + tl] = (_Float16)(bk * kn[tt][j]);
            sVT[ch * LT + tl] = (_Float16)(bv * vv[r][tt][j]);
            gQt[tl * D + ch] = (_Float16)(sq * qn[tt][j]);
            gKtT[ch * C64 + tl] = (_Float16)(ek * kn[tt][j]);
          }
        }
      }
    }
    __syncthreads();
    // W = T (beta e^gamma K), U' = T (beta V) on MFMA; wave w takes the d-tiles nt = w (mod 4)
    {
      float* gUp = (float*)(rec + Rec<D>::kUp);
      for (int nt = w; nt < D / 16; nt += 4) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4 aw = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const f16x8 at = *(const f16x8*)&sT[(16 * mt + r16) * LT + 32 * ks + 8 * g16];
            const f16x8 bw = *(const f16x8*)&sKT[(16 * nt + r16) * LT + 32 * ks + 8 * g16];
            const f16x8 bu = *(const f16x8*)&sVT[(16 * nt + r16) * LT + 32 * ks + 8 * g16];
            aw = mfma16(at, bw, aw);
            au = mfma16(at, bu, au);
          }
          *(f32x4*)&gUp[((long)(nt * 4 + mt) * kWave + lane) * 4] = au;
#pragma unroll
          for (int i = 0; i < 4; ++i) sWs[(16 * mt + 4 * g16 + i) * LD + 16 * nt + r16] = (_Float16)(-aw[i]);
        }
      }
    }
    __syncthreads();
    {
      _Float16* gWn = (_Float16*)(rec + Rec<D>::kWn);
      for (int v = tid; v < C64 * D / 8; v += 256) {
        const int row = v / (D / 8), cv = v % (D / 8);
        *(f16x8*)&gWn[row * D + cv * 8] = *(const f16x8*)&sWs[row * LD + cv * 8];
      }
      // P~ = scale * decay-masked Q K^T, lower triangle including the diagonal
      _Float16* gPt = (_Float16*)(rec + Rec<D>::kPt);
      const int i = tid >> 2, j0 = (tid & 3) * 16;
      f16x8 v0, v1;
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        const int j = j0 + jj;
        const float val = j <= i ? p.scale * __expf(gam[i] - gam[j]) * sQK[i * LF + j] : 0.f;
        if (jj < 8) v0[jj] = (_Float16)val;
        else v1[jj - 8] = (_Float16)val;
      }
      *(f16x8*)&gPt[i * C64 + j0] = v0;
      *(f16x8*)&gPt[i * C64 + j0 + 8] = v1;
      if (tid == 0) *(float*)(rec + Rec<D>::kGc) = __expf(gam[C64 - 1]);
    }
    __syncthreads();
  }
}

// -------------------------------------------------------------------------------------------------
template <int D>
struct PassShape {
  static constexpr int NW = D == 32 ? 2 : 4;  // waves; wave w owns d_v columns [w*16*NT, (w+1)*16*NT)
  static constexpr int NT = D / (16 * NW);    // 16-column tiles per wave
  static constexpr int HM = D / 16;           // 16-row tiles of H over d_k
  static constexpr int KD = D / 32;           // k-steps over d_k
};

// two 4-wide f16 runs {k0..k0+3, k0+16..k0+19} of a row: the permuted k-group matching two stacked
// 16x16 accumulator tiles
__device__ __forceinline__ f16x8 ld_perm(const _Float16* row, int k0) {
  const f16x4 lo = *(const f16x4*)(row + k0);
  const f16x4 hi = *(const f16x4*)(row + k0 + 16);
  f16x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

__device__ __forceinline__ f16x8 pack_acc(f32x4 a, f32x4 b) {
  f16x8 r;
  r[0] = (_Float16)a[0]; r[1] = (_Float16)a[1]; r[2] = (_Float16)a[2]; r[3] = (_Float16)a[3];
  r[4] = (_Float16)b[0]; r[5] = (_Float16)b[1]; r[6] = (_Float16)b[2]; r[7] = (_Float16)b[3];
  return r;
}

template <typename ActT, int D, int R>
__global__ __launch_bounds__(64 * PassShape<D>::NW) void state_pass_kernel(PrefillArgs p) {
  using S = PassShape<D>;
  constexpr int NW = S::NW, NT = S::NT, HM = S::HM, KD = S::KD, NTH = 64 * NW;
  constexpr int LD = D + 8, LT = C64 + 8;
  __shared__ __attribute__((aligned(16))) _Float16 sW[C64 * LD];
  __shared__ __attribute__((aligned(16))) _Float16 sQ[C64 * LD];
  __shared__ __attribute__((aligned(16))) _Float16 sKT[D * LT];
  __shared__ __attribute__((aligned(16))) _Float16 sP[C64 * LT];
  __shared__ float sSS[NW][C64];

  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g16 = lane >> 4, r16 = lane & 15;
  const int Lb = p.Lb, n_v = p.n_v, C = p.C;
  const int len = p.len[b];
  const int n_real = (len + C64 - 1) / C64;
  const int cb = w * 16 * NT;  // first d_v column of this wave

  float* st = p.state + ((long)b * n_v + h) * D * D;
  f32x4 H[HM][NT];
#pragma unroll
  for (int hm = 0; hm < HM; ++hm)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) H[hm][nt][i] = st[(long)(16 * hm + 4 * g16 + i) * D + cb + 16 * nt + r16];

  const ActT* zin = (const ActT*)p.z;
  ActT* out = (ActT*)p.out;

  for (int c = 0; c < n_real; ++c) {
    const char* rec = rec_ptr<D>(p, b, h, c);
    {
      const _Float16* gWn = (const _Float16*)(rec + Rec<D>::kWn);
      const _Float16* gQt = (const _Float16*)(rec + Rec<D>::kQt);
      const _Float16* gKtT = (const _Float16*)(rec + Rec<D>::kKtT);
      const _Float16* gPt = (const _Float16*)(rec + Rec<D>::kPt);
      for (int v = tid; v < C64 * D / 8; v += NTH) {
        const int row = v / (D / 8), cv = v % (D / 8);
        *(f16x8*)&sW[row * LD + cv * 8] = *(const f16x8*)&gWn[row * D + cv * 8];
        *(f16x8*)&sQ[row * LD + cv * 8] = *(const f16x8*)&gQt[row * D + cv * 8];
      }
      for (int v = tid; v < D * C64 / 8; v += NTH) {
        const int row = v / (C64 / 8), cv = v % (C64 / 8);
        *(f16x8*)&sKT[row * LT + cv * 8] = *(const f16x8*)&gKtT[row * C64 + cv * 8];
      }
      for (int v = tid; v < C64 * C64 / 8; v += NTH) {
        const int row = v / (C64 / 8), cv = v % (C64 / 8);
        *(f16x8*)&sP[row * LT + cv * 8] = *(const f16x8*)&gPt[row * C64 + cv * 8];
      }
    }
    const float gC = *(const float*)(rec + Rec<D>::kGc);
    const float* gUp = (const float*)(rec + Rec<D>::kUp);
    f32x4 U[4][NT];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) U[mt][nt] = *(const f32x4*)&gUp[((long)((w * NT + nt) * 4 + mt) * kWave + lane) * 4];
    __syncthreads();

    // H as the B operand (d_k on the k axis, permuted group {4g.., 16+4g..} of each 32-row block)
    f16x8 Hb[KD][NT];
#pragma unroll
    for (int kk = 0; kk < KD; ++kk)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) Hb[kk][nt] = pack_acc(H[2 * kk][nt], H[2 * kk + 1][nt]);

    // U = U' - W H  and  O = Q~ H
    f32x4 O[4][NT];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) O[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KD; ++kk) {
        const f16x8 aw = ld_perm(&sW[(16 * mt + r16) * LD], 32 * kk + 4 * g16);
        const f16x8 aq = ld_perm(&sQ[(16 * mt + r16) * LD], 32 * kk + 4 * g16);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          U[mt][nt] = mfma16(aw, Hb[kk][nt], U[mt][nt]);
          O[mt][nt] = mfma16(aq, Hb[kk][nt], O[mt][nt]);
        }
      }
    }
    // U as the B operand (tokens on the k axis)
    f16x8 Ub[2][NT];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) Ub[kk][nt] = pack_acc(U[2 * kk][nt], U[2 * kk + 1][nt]);
    // H = e^{gamma_C} H + K~^T U
#pragma unroll
    for (int hm = 0; hm < HM; ++hm) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) H[hm][nt][i] *= gC;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const f16x8 ak = ld_perm(&sKT[(16 * hm + r16) * LT], 32 * kk + 4 * g16);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) H[hm][nt] = mfma16(ak, Ub[kk][nt], H[hm][nt]);
      }
    }
    // O += P~ U
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const f16x8 ap = ld_perm(&sP[(16 * mt + r16) * LT], 32 * kk + 4 * g16);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) O[mt][nt] = mfma16(ap, Ub[kk][nt], O[mt][nt]);
      }

    // gated RMSNorm over the D columns of each token row
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float ss = 0.f;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) ss += O[mt][nt][i] * O[mt][nt][i];
        ss = wave_sum<16>(ss);
        if (r16 == 0) sSS[w][16 * mt + 4 * g16 + i] = ss;
      }
    __syncthreads();
    const int t0 = c * C64;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * mt + 4 * g16 + i;
        float ss = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) ss += sSS[ww][row];
        const float inv = 1.0f / sqrtf(ss / (float)D + p.rms_eps);
        const int t = t0 + row;
        if (t < Lb) {
          const long ob = ((long)b * Lb + t) * n_v * D + (long)h * D;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const int col = cb + 16 * nt + r16;
            const float zz = to_f32(zin[ob + col]);
            out[ob + col] = from_f32<ActT>(p.norm_w[col] * (O[mt][nt][i] * inv) * silu(zz));
          }
        }
      }
    __syncthreads();  // LDS reused by the next chunk
  }

  // final state, in place
#pragma unroll
  for (int hm = 0; hm < HM; ++hm)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) st[(long)(16 * hm + 4 * g16 + i) * D + cb + 16 * nt + r16] = H[hm][nt][i];

  // conv tail: rows len .. len+2 of [old tail | mixed]; value head h owns its v channels, the first
  // value head of each GQA group also the q and k channels of its key head
  {
    ActT* tl = (ActT*)p.tail + (long)b * 3 * C;
    const ActT* mx = (const ActT*)p.mixed + (long)b * Lb * C;
    const int kh = h / R;
    const int nch = (h % R == 0) ? 3 * D : D;
    for (int lc = tid; lc < nch; lc += NTH) {
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

template <typename ActT, int D, int R>
hipError_t launch_prefill_t(const PrefillArgs& p, hipStream_t st) {
  hipLaunchKernelGGL((chunk_prep_kernel<ActT, D, R>), dim3(p.n_chunks, p.n_k, p.B), dim3(256), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((state_pass_kernel<ActT, D, R>), dim3(p.n_v, p.B), dim3(64 * PassShape<D>::NW), 0, st, p);
  return hipGetLastError();
}

template <typename ActT, int D>
hipError_t launch_prefill_d(const PrefillArgs& p, int R, hipStream_t st) {
  switch (R) {
    case 1: return launch_prefill_t<ActT, D, 1>(p, st);
    case 2: return launch_prefill_t<ActT, D, 2>(p, st);
    case 4: return launch_prefill_t<ActT, D, 4>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t prefill_ws_bytes(int B, int n_v, int D, int n_chunks) {
  long rec = D == 32 ? Rec<32>::kBytes : D == 64 ? Rec<64>::kBytes : Rec<128>::kBytes;
  return (size_t)B * n_v * n_chunks * rec;
}

hipError_t launch_prefill(const PrefillArgs& p, int act_dtype, int D, int R, hipStream_t st) {
  if (act_dtype == kActBf16) {
    if (D == 32) return launch_prefill_d<bf16_t, 32>(p, R, st);
    if (D == 64) return launch_prefill_d<bf16_t, 64>(p, R, st);
    if (D == 128) return launch_prefill_d<bf16_t, 128>(p, R, st);
  } else {
    if (D == 32) return launch_prefill_d<float, 32>(p, R, st);
    if (D == 64) return launch_prefill_d<float, 64>(p, R, st);
    if (D == 128) return launch_prefill_d<float, 128>(p, R, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
