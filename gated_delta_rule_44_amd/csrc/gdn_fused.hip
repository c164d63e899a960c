// Fused chunked prefill of the gated delta rule for d_k = d_v = 128 and bf16 activations (gfx950).
//
// One persistent workgroup per (sequence, value head[, segment]) walks its chunks of C = 64 tokens in
// order, with every intermediate of a chunk in LDS or registers; only the projected inputs are read
// from HBM and only the output (and the final state) written. Per chunk, with entering state H = S^T
// (d_k x d_v), gamma the in-chunk cumulative log-decay, beta the write strengths:
//   A[r][s] = beta_r e^{gamma_r - gamma_s} k_r.k_s  (s < r)
//   U = (I + A)^{-1} Y,   Y = diag(beta) (V - diag(e^gamma) K H)
//   O = scale (diag(e^gamma) Q H + P U),  P[t][s] = e^{gamma_t - gamma_s} q_t.k_s (s <= t)
//   H <- e^{gamma_C} H + K^T diag(e^{gamma_C - gamma}) U
// This is the WY/UT chunk form of the recurrence S_t = e^{g_t} S_{t-1} (I - beta_t k_t k_t^T) +
// beta_t v_t k_t^T, o_t = scale S_t q_t: the write vectors u_t of a chunk solve one unit lower
// triangular system. U is found by blocked forward substitution over the four 16-token blocks,
// U_m = T_mm (Y_m - sum_{j<m} A_mj U_j) with T_mm = (I + A_mm)^{-1}, so the full inverse is never formed.
//
// Waves 0-3 ("chain") each own 32 columns of H in fp32 accumulators and run the state-dependent
// products of chunk c: K H, the solve, Q H and P U for O^T, and the state update, all on f16 MFMA.
// Each chain wave also forms its own V from the conv of its 32 value channels (inputs staged in LDS)
// and finishes the gated RMSNorm of its columns (row sums exchanged through LDS).
// Waves 4-7 ("prep") build chunk c + 1 meanwhile: the conv + SiLU of its q and k channels (16 tokens
// per wave), the q/k L2 norms, the gates with the padding mask, the q, k and decayed k^T operand
// fragments, then the Gram products K K^T and K Q^T, the off-diagonal blocks of -A, the decayed P,
// and the four diagonal inverses T_mm by substitution.
// Four workgroup barriers per chunk order the two roles:
//   X..Y   chain: right-hand sides, solve, P U and  prep: conv, norms, gates, operand pairs of c+1
//          state update of c
//   Y..Y1  chain: gated norm + stores of c; v of c+1 prep: q, k, k~ and gates of c+1 to LDS; loads of c+2
//   Y1..Y2 chain: K H and H^T Q^T of c+1             prep: Gram products, A blocks, P of c+1
//   Y2..X  chain: -                                  prep (one wave): T_mm of c+1
//
// Modes: OUT runs a segment of chunks from its entering state and writes the outputs (and, for the
// segment that holds the sequence's last chunk, the final state). MAP_N and MAP_M run a segment
// from H = 0 with the real V and from H = I with V = 0: since a segment maps its entering state
// affinely, H_out = M H_in + N, these give N and M, from which scan_kernel forms every segment's
// entering state; then OUT runs all segments in parallel. A sequence of few heads is thereby spread
// over many CUs.
//
// Precision: MFMA operands are f16 with fp32 accumulation; every operand whose rounding reaches the
// output or state bounds is carried as a hi/lo pair of f16 values (about 22 bits), each product
// being the three terms hi.hi + hi.lo + lo.hi: q and k in the Gram products, H, U, Q, P, k~, T_mm
// and the right-hand sides of the solve. K in K H and the off-diagonal -A blocks of the solve are the
// high half alone: a rounding model of the chunk form puts their cost at a few hundredths of the
// output bound, where a single-f16 U, right-hand side or P costs about twice the bound. To keep low halves above f16's subnormal range (which MFMA flushes), operands
// carry exact power-of-two scales: 2^8 for q, k, H, U, A, T, right-hand sides; 2^16 for P, whose
// entries span many decades. Accumulators: H as 2^16 H, K H and U as 2^16, O^T as 2^24 O^T.
// The scales bound what the operands can hold: |H| and |U| must stay below 255.
#include <mutex>
#include <type_traits>

#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

constexpr int FD = 128;  // head dimension (d_k = d_v)
constexpr int FC = 64;   // chunk
constexpr float kS8 = 256.f, kIS8 = 1.f / 256.f, kS16 = 65536.f, kIS16 = 1.f / 65536.f;
constexpr float kIS24 = 1.f / 16777216.f;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int MODE_OUT = 0, MODE_MAP_N = 1, MODE_MAP_M = 2;

// ---- LDS layout (bytes) ------------------------------------------------------------------------------
// fragment arrays hold 16 bytes (f16x8) or 8 bytes (f16x4) per lane, lane-contiguous, hi and lo halves
// in separate 1 KB (or 512 B) blocks
constexpr int L_Q = 0;                       // q:   [mt 4][kk 4][hl 2][lane] f16x8, 2^8 q (token rows)
constexpr int L_K = L_Q + 32768;             // k:   [mt 4][kk 4][hl 2][lane] f16x8, 2^8 k (token rows)
constexpr int L_KT = L_K + 32768;            // k~:  [hm 8][kb 2][hl 2][lane] f16x8, 2^8 e^{gC-g} k (d rows)
constexpr int L_P = L_KT + 32768;            // P:   [pair 6][hl 2][lane] f16x8, 2^16 scale e^{gt-gs} q.k
constexpr int L_AO = L_P + 6 * 2 * 1024;     // -A:  [pair 6][lane] f16x4, 2^8, hi only (off-diagonal 16 x 16 blocks)
constexpr int L_TI = L_AO + 6 * 512;     // T_mm:[m 4][hl 2][lane] f16x4, 2^8
constexpr int LDA = 20;                      // row stride (floats) of the fp32 16 x 16 blocks (16-byte rows)
constexpr int L_AD = L_TI + 4 * 2 * 512;     // A_mm fp32 [m 4][16][LDA] (strictly lower part)
constexpr int L_TF = L_AD + 4 * 16 * LDA * 4; // T_mm fp32 [m 4][16][LDA]
constexpr int L_G = L_TF + 4 * 16 * LDA * 4;  // beta[64], e^gamma[64], gamma[64], e^{gamma_C}
constexpr int L_SS = L_G + 1024;              // row sums of squares of O: [chain wave 4][token 64]
constexpr int VROWS = FC + 3;                 // staged conv input rows of a chunk (3 halo rows)
constexpr int L_VS = L_SS + 1024;             // v inputs per chain wave: [wave 4][VROWS][32] bf16
constexpr int L_NW = L_VS + 4 * VROWS * 64;  // norm weights [128] fp32
constexpr int L_VT = L_NW + FD * 4;           // conv taps of the head's value channels [128] (4 bf16 each)
constexpr int L_QKT = L_VT + FD * 8;          // per prep lane: taps of its q and k channel pairs [wave 4][lane][4]
constexpr int L_END = L_QKT + 4 * 64 * 4 * 8;
static_assert(L_END <= 160 * 1024, "LDS budget");

__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ f32x4 mfma32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16k(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// hi/lo pairs of 4 or 8 fp32 values (scaled by the caller)
__device__ __forceinline__ void split4v(f32x4 x, f16x4& hi, f16x4& lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    _Float16 h, l;
    split_f16(x[e], h, l);
    hi[e] = h;
    lo[e] = l;
  }
}
__device__ __forceinline__ f16x8 cat8(f16x4 a, f16x4 b) { return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}; }

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf1(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

// fragment-slot position of index j (0..31) inside a 32-block: lane group and element
__device__ __forceinline__ int slot_g(int j) { return (j & 15) >> 2; }
__device__ __forceinline__ int slot_e(int j) { return (j & 16 ? 4 : 0) + (j & 3); }

// Slot of lane (g, c) inside a 1 KB fragment block of the q / k (block (mt, kk)) and k~ (block (hm, kb))
// arrays: rotated within each 16-lane group, so that the prep waves' scattered 4- and 8-byte stores
// spread over the LDS banks while every 16-lane group of a reading wave still covers all 16 positions
__device__ __forceinline__ int qk_slot(int g, int c, int kk) { return 16 * g + ((c + 4 * g + kk) & 15); }
__device__ __forceinline__ int kt_slot(int g, int c, int hm) { return 16 * g + ((c + hm) & 15); }

// pair indices of the lower blocks
__device__ __forceinline__ int pidx(int mt, int kb) { return mt < 2 ? mt : 2 + 2 * (mt - 2) + kb; }   // P: (t tile, s 32-block)
__device__ __forceinline__ int aidx(int mt, int nt) { return mt * (mt - 1) / 2 + nt; }                // -A: (r tile, s tile), nt < mt

struct Unit {
  int b, h, kh, s;      // sequence, value head, key head, segment
  int c0, c1;           // chunks [c0, c1) of this workgroup (empty if c0 >= c1)
  int len;
  bool last;            // holds the sequence's last real chunk
};

template <int MODE>
__device__ __forceinline__ Unit unit_of(const FusedArgs& p) {
  // consecutive units (the value heads of one key head, then sequences) share an XCD, so that the q/k
  // inputs a key head's workgroups both read are fetched once into that XCD's L2 (dispatch assigns
  // workgroup ids to the 8 XCDs round-robin)
  const int nblk = gridDim.x, bid = blockIdx.x;
  const int lid = (nblk & 7) == 0 ? (bid & 7) * (nblk >> 3) + (bid >> 3) : bid;
  Unit u;
  int rest = lid;
  if (MODE == MODE_OUT) {
    u.s = rest % p.nseg;
    rest /= p.nseg;
  } else {
    u.s = rest % (p.nseg - 1);  // the last segment needs no map
    rest /= (p.nseg - 1);
  }
  u.h = rest % p.n_v;
  u.b = rest / p.n_v;
  u.kh = u.h / (p.n_v / p.n_k);
  u.len = p.len[u.b];
  const int n_real = (u.len + FC - 1) / FC;
  u.c0 = u.s * p.seg_chunks;
  u.c1 = min(u.c0 + p.seg_chunks, n_real);
  u.last = u.c0 < u.c1 && u.c1 == n_real;
  return u;
}

// ---------------------------------------------------------------------------------------------------
// ---- the chain role (waves 0-3) -------------------------------------------------------------------
template <int MODE>
__device__ __forceinline__ void chain_role(const FusedArgs& p, const Unit& u, char* smem) {
  constexpr bool OUT = MODE == MODE_OUT;
  constexpr bool WITH_V = MODE != MODE_MAP_M;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g16 = lane >> 4, c16 = lane & 15;
  const int Lb = p.Lb, C = p.C, n_v = p.n_v, n_k = p.n_k;
  const int b = u.b, h = u.h, len = u.len;
  const uint16_t* mixed = (const uint16_t*)p.mixed + (long)b * Lb * C;
  const uint16_t* tail = (const uint16_t*)p.tail + (long)b * 3 * C;
  const f16x8* sQ = (const f16x8*)(smem + L_Q);
  const f16x8* sK = (const f16x8*)(smem + L_K);
  const f16x8* sKT = (const f16x8*)(smem + L_KT);
  const f16x8* sP = (const f16x8*)(smem + L_P);
  const f16x4* sAO = (const f16x4*)(smem + L_AO);
  const f16x4* sTI = (const f16x4*)(smem + L_TI);
  const float* sBeta = (const float*)(smem + L_G);
  const float* sEg = sBeta + 64;
  const float* sEc = sBeta + 192;
  float* sSS = (float*)(smem + L_SS);
  float* sNW = (float*)(smem + L_NW);
  char* stage = smem + L_VS + w * VROWS * 64;
  if (OUT && threadIdx.x < FD) sNW[threadIdx.x] = p.norm_w[threadIdx.x];  // read after the prologue's barriers
  // the value channels' conv taps, staged once (the chunk loop's barriers would otherwise make every chunk
  // wait on a global load of them); read after the prologue's barriers
  uint2* sVT = (uint2*)(smem + L_VT);
  if (threadIdx.x < FD)
    sVT[threadIdx.x] = *(const uint2*)((const uint16_t*)p.conv_w + (long)(2 * n_k * FD + h * FD + threadIdx.x) * 4);

  const int cw0 = 32 * w;   // first H column of this wave
  f32x4 Hacc[8][2];         // 2^16 H[16 hm + 4 g + i][cw0 + 16 n + c]
  f32x4 Oacc[2][4];         // 2^24 O^T[cw0 + 16 n + 4 g + i][token 16 mt + c]
  uint2 zr[2][4];           // z of the output rows (4 bf16)
  u32x4 vpre[5];            // staged v inputs of the next chunk, in flight
  // the entering state: OUT from the saved state (segment 0) or the scan's segment state; MAP_N from
  // zero; MAP_M from the identity
  {
    const float* src = nullptr;
    if (OUT) src = u.s == 0 ? p.state + ((long)b * n_v + h) * FD * FD
                            : p.seg_in + (((long)b * n_v + h) * p.nseg + u.s) * FD * FD;
#pragma unroll
    for (int hm = 0; hm < 8; ++hm)
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * hm + 4 * g16 + i, col = cw0 + 16 * n + c16;
          float v = 0.f;
          if (OUT) v = src[(long)r * FD + col];
          if (MODE == MODE_MAP_M) v = r == col ? 1.f : 0.f;
          Hacc[hm][n][i] = kS16 * v;
        }
  }

  // staged v inputs of chunk c: 67 rows x 32 channels (64 bytes a row), 16 bytes a lane and load
  auto v_load = [&](int c) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      const int r = 16 * k + (lane >> 2);
      const int T = c * FC - 3 + r;  // token of the row (< 0: the saved tail)
      const bool ok = r < VROWS && T < Lb;
      const uint16_t* row = ok ? (T < 0 ? tail + (long)(T + 3) * C : mixed + (long)T * C) : tail;
      vpre[k] = ok ? *(const u32x4*)(row + 2 * n_k * FD + h * FD + cw0 + 8 * (lane & 3)) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto v_stage = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      const int r = 16 * k + (lane >> 2);
      if (r < VROWS) *(u32x4*)(stage + r * 64 + 16 * (lane & 3)) = vpre[k];
    }
  };
  auto z_load = [&](int c) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int T = c * FC + 16 * mt + c16;
      const long row = ((long)b * Lb + (T < Lb ? T : Lb - 1)) * n_v + h;
#pragma unroll
      for (int n = 0; n < 2; ++n) zr[n][mt] = *(const uint2*)((const uint16_t*)p.z + row * FD + cw0 + 16 * n + 4 * g16);
    }
  };

  // the products of chunk c
  // K H (K high half alone) and, for OUT, H^T Q^T of a chunk: they need only its q and k and the state
  // it enters with, so they run while the prep forms the chunk's Gram products. H fragments one 32-row
  // block at a time: rows 32 kk + {4 g .. 4 g + 3, 16 + 4 g .. 16 + 4 g + 3} are accumulator rows of
  // tiles 2 kk and 2 kk + 1.
  f32x4 Z[4][2];            // 2^16 K H, then the right-hand sides of the solve
  auto products_kh = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        Z[mt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
        Oacc[n][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      f16x8 hh[2], hl[2];
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        f16x4 ah, al, bh, bl;
        split4v(Hacc[2 * kk][n] * kIS8, ah, al);
        split4v(Hacc[2 * kk + 1][n] * kIS8, bh, bl);
        hh[n] = cat8(ah, bh);
        hl[n] = cat8(al, bl);
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f16x8 kf = sK[((mt * 4 + kk) * 2) * 64 + qk_slot(g16, c16, kk)];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          Z[mt][n] = mfma32(kf, hl[n], Z[mt][n]);
          Z[mt][n] = mfma32(kf, hh[n], Z[mt][n]);
        }
        if (OUT) {
          const int qs = qk_slot(g16, c16, kk);
          const f16x8 qh = sQ[((mt * 4 + kk) * 2) * 64 + qs], ql = sQ[((mt * 4 + kk) * 2 + 1) * 64 + qs];
#pragma unroll
          for (int n = 0; n < 2; ++n) {
            Oacc[n][mt] = mfma32(hl[n], qh, Oacc[n][mt]);
            Oacc[n][mt] = mfma32(hh[n], ql, Oacc[n][mt]);
            Oacc[n][mt] = mfma32(hh[n], qh, Oacc[n][mt]);
          }
        }
      }
    }
  };

  // the rest of a chunk's products, once its Gram products and T_mm are in LDS
  auto chunk = [&]() __attribute__((always_inline)) {
    // right-hand sides 2^16 Y = beta (2^16 V - e^gamma 2^16 K H); V = conv + SiLU of this wave's value
    // channels at token 16 mt + 4 g + i, column cw0 + 16 n + c, from the staged inputs
    {
      const uint16_t* st = (const uint16_t*)stage;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int t0 = 16 * mt + 4 * g16;
        const float4 be = *(const float4*)(sBeta + t0), eg = *(const float4*)(sEg + t0);
        const float bev[4] = {be.x, be.y, be.z, be.w}, egv[4] = {eg.x, eg.y, eg.z, eg.w};
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          float x[7] = {}, vw[4] = {};
          if (WITH_V) {
            const uint2 tp = sVT[cw0 + 16 * n + c16];  // taps of channel cw0 + 16 n + c
            vw[0] = bf_lo(tp.x); vw[1] = bf_hi(tp.x); vw[2] = bf_lo(tp.y); vw[3] = bf_hi(tp.y);
#pragma unroll
            for (int r = 0; r < 7; ++r) x[r] = bf1(st[(t0 + r) * 32 + 16 * n + c16]);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v = 0.f;
            if (WITH_V) v = silu(vw[0] * x[i] + vw[1] * x[i + 1] + vw[2] * x[i + 2] + vw[3] * x[i + 3]);
            Z[mt][n][i] = bev[i] * (kS16 * v - egv[i] * Z[mt][n][i]);
          }
        }
      }
    }
    // blocked forward substitution: U_m = T_mm (Y_m - sum_{j<m} A_mj U_j), as 2^8 U hi/lo
    f16x4 Uh[4][2], Ul[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int j = 0; j < mt; ++j) {
        const f16x4 ah = sAO[aidx(mt, j) * 64 + lane];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          Z[mt][n] = mfma16k(ah, Ul[j][n], Z[mt][n]);
          Z[mt][n] = mfma16k(ah, Uh[j][n], Z[mt][n]);
        }
      }
      const f16x4 th = sTI[(mt * 2) * 64 + lane], tl = sTI[(mt * 2 + 1) * 64 + lane];
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        f16x4 zh, zl;
        split4v(Z[mt][n] * kIS8, zh, zl);
        f32x4 ua = {0.f, 0.f, 0.f, 0.f};
        ua = mfma16k(tl, zh, ua);
        ua = mfma16k(th, zl, ua);
        ua = mfma16k(th, zh, ua);
        split4v(ua * kIS8, Uh[mt][n], Ul[mt][n]);
      }
    }
    // O^T = 2^24 (scale e^{gamma_t} H^T q_t + U^T P^T): token t = 16 mt + c scales its column in the lane
    if (OUT) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const float f = p.scale * kS8 * sEg[16 * mt + c16];
#pragma unroll
        for (int n = 0; n < 2; ++n) Oacc[n][mt] *= f;
#pragma unroll
        for (int kb = 0; kb <= (mt >> 1); ++kb) {
          const int pi = pidx(mt, kb);
          const f16x8 ph = sP[(pi * 2) * 64 + lane], pl = sP[(pi * 2 + 1) * 64 + lane];
#pragma unroll
          for (int n = 0; n < 2; ++n) {
            const f16x8 uh = cat8(Uh[2 * kb][n], Uh[2 * kb + 1][n]), ul = cat8(Ul[2 * kb][n], Ul[2 * kb + 1][n]);
            Oacc[n][mt] = mfma32(ul, ph, Oacc[n][mt]);
            Oacc[n][mt] = mfma32(uh, pl, Oacc[n][mt]);
            Oacc[n][mt] = mfma32(uh, ph, Oacc[n][mt]);
          }
        }
      }
      // row sums of squares over this wave's 32 columns (token 16 mt + c): over i and n, then lane groups
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        float s = 0.f;
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i) s += Oacc[n][mt][i] * Oacc[n][mt][i];
        s += __shfl_xor(s, 16, kWave);
        s += __shfl_xor(s, 32, kWave);
        if (g16 == 0) sSS[w * 64 + 16 * mt + c16] = s;
      }
    }
    // H = e^{gamma_C} H + K~^T U
    const float ec = sEc[0];
#pragma unroll
    for (int hm = 0; hm < 8; ++hm) {
#pragma unroll
      for (int n = 0; n < 2; ++n) Hacc[hm][n] *= ec;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int ks = kt_slot(g16, c16, hm);
        const f16x8 kh8 = sKT[((hm * 2 + kb) * 2) * 64 + ks], kl8 = sKT[((hm * 2 + kb) * 2 + 1) * 64 + ks];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const f16x8 uh = cat8(Uh[2 * kb][n], Uh[2 * kb + 1][n]), ul = cat8(Ul[2 * kb][n], Ul[2 * kb + 1][n]);
          Hacc[hm][n] = mfma32(kl8, uh, Hacc[hm][n]);
          Hacc[hm][n] = mfma32(kh8, ul, Hacc[hm][n]);
          Hacc[hm][n] = mfma32(kh8, uh, Hacc[hm][n]);
        }
      }
    }
  };

  // the gated RMSNorm of chunk c's rows of this wave's columns, and the store (rows < len only)
  auto norm = [&](int c) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int t = 16 * mt + c16;
      const float tot = (sSS[t] + sSS[64 + t]) + (sSS[128 + t] + sSS[192 + t]);
      const float inv = rsqrt_fast(tot * (kIS24 * kIS24) * (1.f / FD) + p.rms_eps) * kIS24;
      const int T = c * FC + t;
      if (T < len) {
        const long row = ((long)b * Lb + T) * n_v + h;
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const int col = cw0 + 16 * n + 4 * g16;
          const float4 nw = *(const float4*)(sNW + col);
          const uint2 zz = zr[n][mt];
          const float y0 = nw.x * (Oacc[n][mt][0] * inv) * silu(bf_lo(zz.x));
          const float y1 = nw.y * (Oacc[n][mt][1] * inv) * silu(bf_hi(zz.x));
          const float y2 = nw.z * (Oacc[n][mt][2] * inv) * silu(bf_lo(zz.y));
          const float y3 = nw.w * (Oacc[n][mt][3] * inv) * silu(bf_hi(zz.y));
          if (p.out_f32) {
            *(float4*)((float*)p.out + row * FD + col) = make_float4(y0, y1, y2, y3);
          } else {
            uint2 o;
            o.x = pack_bf16x2(y0, y1);
            o.y = pack_bf16x2(y2, y3);
            *(uint2*)((uint16_t*)p.out + row * FD + col) = o;
          }
        }
      }
    }
  };

  // prologue: stage chunk c0's v inputs while the prep builds chunk c0's operands, and form K H and
  // H^T Q^T of chunk c0 beside its Gram products
  if (WITH_V) v_load(u.c0);
  lds_barrier();
  if (WITH_V) v_stage();
  lds_barrier();
  products_kh();
  lds_barrier();
  lds_barrier();
  // Per chunk c: the rest of its products (beside the prep's conv of chunk c + 1); Y; its gated norm and
  // stores (beside the prep's operand writes; z is loaded at the start, the v inputs of chunk c + 1 are
  // loaded before and staged after the norm); Y1; K H and H^T Q^T of chunk c + 1 (beside its Gram
  // products); Y2; X. (Loads are issued after the products so that nothing in flight holds registers
  // through them.)
  for (int c = u.c0; c < u.c1; ++c) {
    chunk();
    lds_barrier();  // Y: chunk c's operands are free
    if (OUT) z_load(c);
    const bool next = c + 1 < u.c1;
    if (WITH_V && next) v_load(c + 1);
    if (OUT) norm(c);
    if (WITH_V && next) v_stage();
    lds_barrier();  // Y1: chunk c + 1's q, k and k~ are in LDS
    if (next) products_kh();
    lds_barrier();  // Y2
    lds_barrier();  // X: chunk c + 1's Gram products and T_mm are ready
  }

  // the exit state
  float* dst = nullptr;
  if (OUT && u.last) dst = p.state + ((long)b * n_v + h) * FD * FD;
  if (MODE == MODE_MAP_N) dst = p.seg_map + ((((long)b * n_v + h) * (p.nseg - 1) + u.s) * 2 + 0) * FD * FD;
  if (MODE == MODE_MAP_M) dst = p.seg_map + ((((long)b * n_v + h) * (p.nseg - 1) + u.s) * 2 + 1) * FD * FD;
  if (dst) {
    bool bad = false;
#pragma unroll
    for (int hm = 0; hm < 8; ++hm)
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = Hacc[hm][n][i] * kIS16;
          bad |= !(fabsf(v) < 255.f);
          dst[(long)(16 * hm + 4 * g16 + i) * FD + cw0 + 16 * n + c16] = v;
        }
    if (p.status && __any(bad) && lane == 0) atomicOr(p.status, 1);
  }
}

// ---- the prep role (waves 4-7) --------------------------------------------------------------------
template <int MODE>
__device__ __forceinline__ void prep_role(const FusedArgs& p, const Unit& u, char* smem) {
  constexpr bool WITH_Q = MODE == MODE_OUT;  // the maps need neither q nor P
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pw = w - 4;                      // tokens 16 pw .. 16 pw + 15 of each chunk
  const int g16 = lane >> 4, c16 = lane & 15;
  const int Lb = p.Lb, C = p.C, n_v = p.n_v, n_k = p.n_k;
  const int b = u.b, h = u.h, kh = u.kh, len = u.len;
  const uint16_t* mixed = (const uint16_t*)p.mixed + (long)b * Lb * C;
  const uint16_t* tail = (const uint16_t*)p.tail + (long)b * 3 * C;
  f16x8* sQ = (f16x8*)(smem + L_Q);
  f16x8* sK = (f16x8*)(smem + L_K);
  f16x8* sKT = (f16x8*)(smem + L_KT);
  f16x8* sP = (f16x8*)(smem + L_P);
  f16x4* sAO = (f16x4*)(smem + L_AO);
  f16x4* sTI = (f16x4*)(smem + L_TI);
  float* sAD = (float*)(smem + L_AD);
  float* sTF = (float*)(smem + L_TF);
  float* sBeta = (float*)(smem + L_G);
  float* sEg = sBeta + 64;
  float* sGam = sBeta + 128;
  float* sEc = sBeta + 192;

  uint32_t xq[19], xk[19];     // q / k inputs of the next chunk: rows 16 pw - 3 .. 16 pw + 15, channel pairs
  uint16_t a_raw = 0, b_raw = 0;  // gate inputs of the next chunk (lane = token)
  // conv taps of the lane's q and k channels 2 lane, 2 lane + 1, staged once in the lane's own LDS slot
  // (the chunk loop's barriers would otherwise make every chunk wait on a global load of them)
  uint2* qtap = (uint2*)(smem + L_QKT) + (pw * 64 + lane) * 4;
  uint2* ktap = qtap + 2;
  {
    const uint2* gq = (const uint2*)((const uint16_t*)p.conv_w + (long)(kh * FD + 2 * lane) * 4);
    const uint2* gk = (const uint2*)((const uint16_t*)p.conv_w + (long)(n_k * FD + kh * FD + 2 * lane) * 4);
    qtap[0] = gq[0];
    qtap[1] = gq[1];
    ktap[0] = gk[0];
    ktap[1] = gk[1];
  }
  auto load = [&](int c) __attribute__((always_inline)) {
    const int T0 = c * FC + 16 * pw - 3;
    // rows T0 .. T0 + 18: T < 0 the saved tail, T >= Lb zero (never read); the row pointer steps by one
    // row and moves from the tail to the call's first row at T = 0 (the first chunk only)
    const uint16_t* row = T0 >= 0 ? mixed + (long)T0 * C : tail + (long)(T0 + 3) * C;
    const int o = kh * FD + 2 * lane;
#pragma unroll
    for (int r = 0; r < 19; ++r) {
      const int T = T0 + r;
      if (T == 0) row = mixed;
      const bool ok = T < Lb;
      xq[r] = ok ? *(const uint32_t*)(row + o) : 0u;
      xk[r] = ok ? *(const uint32_t*)(row + o + n_k * FD) : 0u;
      row += C;
    }
    const int t = c * FC + lane;
    const long gi = ((long)b * Lb + (t < Lb ? t : Lb - 1)) * n_v + h;
    a_raw = ((const uint16_t*)p.a)[gi];
    b_raw = ((const uint16_t*)p.b)[gi];
  };

  // gate parameters of the head, read once (the loop's barriers would make the compiler read them again
  // every chunk, a memory round trip each)
  const float negA = -__expf(p.A_log[h]), dtb = p.dt_bias[h];
  float qn[16][2], kn[16][2];
  float g_gam = 0.f, g_beta = 0.f, g_eg = 0.f, g_ed = 0.f, g_ec = 0.f;
  // conv + SiLU of the lane's q and k channel pairs over the wave's 16 tokens, L2 norms, and the
  // gates of token `lane` (every prep wave forms all 64: each needs the decays of its tokens)
  // one pass: conv + SiLU of a channel pair over the wave's 16 tokens, and the squares' sums per token
  auto conv_pass = [&](const uint32_t (&x)[19], const uint2* tap, float (&y)[16][2], float (&ss)[16]) __attribute__((always_inline)) {
    float wt[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint2 t = tap[j];
      wt[j][0] = bf_lo(t.x); wt[j][1] = bf_hi(t.x); wt[j][2] = bf_lo(t.y); wt[j][3] = bf_hi(t.y);
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      float sq = 0.f;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float a = 0.f;
#pragma unroll
        for (int tp = 0; tp < 4; ++tp) a += wt[j][tp] * (j ? bf_hi(x[t + tp]) : bf_lo(x[t + tp]));
        const float v = silu(a);
        y[t][j] = v;
        sq += v * v;
      }
      ss[t] = sq;
    }
  };
  // sums of 16 values over the 64 lanes: at step m (32, 16, 8, 4) a lane keeps the half of its values
  // selected by its bit m and adds the partner's copy of that half; after four steps lane l holds value
  // (l >> 2) summed over the lanes sharing bits 1..0, and two exchanges complete the sum. Returns
  // 1/sqrt(sum + eps) of value l >> 2.
  auto inv_norms = [&](float (&ss)[16]) __attribute__((always_inline)) {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int m = 32 >> st, half = 8 >> st;
      const bool upper = (lane & m) != 0;
#pragma unroll
      for (int i = 0; i < half; ++i) {
        // (the two values are pinned: left visible, the per-lane choice between them became a per-lane
        // index into ss, lowered to compare-and-select over the whole array)
        const float lo = pin_f32(ss[i]), hi = pin_f32(ss[i + half]);
        const float keep = upper ? hi : lo;
        const float give = upper ? lo : hi;
        ss[i] = keep + __shfl_xor(give, m, kWave);
      }
    }
    float tot = ss[0] + __shfl_xor(ss[0], 2, kWave);
    tot += __shfl_xor(tot, 1, kWave);
    return rsqrt_fast(tot + p.l2_eps);
  };
  auto scale_rows = [&](float (&y)[16][2], float rn) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const float r = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rn), 4 * t));
      y[t][0] *= r;
      y[t][1] *= r;
    }
  };
  // conv + SiLU of the lane's q and k channel pairs over the wave's 16 tokens, L2 norms, and the gates
  // of token `lane` (every prep wave forms all 64: each needs the decays of its tokens)
  auto conv = [&](int c) __attribute__((always_inline)) {
    {
      float ss[16];
      conv_pass(xq, qtap, qn, ss);
      scale_rows(qn, inv_norms(ss));
    }
    {
      float ss[16];
      conv_pass(xk, ktap, kn, ss);
      scale_rows(kn, inv_norms(ss));
    }
    const int t = c * FC + lane;
    const bool real = t < len;
    const float g0 = chunk_log_decay(negA * softplus(bf1(a_raw) + dtb));
    float gm = real ? g0 : 0.f;
    g_beta = real ? sigmoid(bf1(b_raw)) : 0.f;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const float o = __shfl_up(gm, off, kWave);
      if (lane >= off) gm += o;
    }
    g_gam = gm;
    const float gC = __shfl(gm, FC - 1, kWave);
    g_eg = __expf(gm);
    g_ed = __expf(gC - gm);
    g_ec = __expf(gC);
  };

  // hi/lo pairs of the wave's operands, formed before the chain frees the LDS buffers (registers):
  // q and k of token t, channels 2 lane and 2 lane + 1, as f16 pairs; k~ = 2^8 e^{gamma_C - gamma_s} k_s
  // for channel 2 lane + j and the four tokens 4 gq .. 4 gq + 3 of lane group gq, as f16x4
  uint32_t qph[16], qpl[16], kph[16], kpl[16];
  f16x4 kth[2][4], ktl[2][4];
  auto pack = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      f16x2 hp, lp;
      split2_f16(kS8 * kn[t][0], kS8 * kn[t][1], hp, lp);
      kph[t] = __builtin_bit_cast(uint32_t, hp);
      kpl[t] = __builtin_bit_cast(uint32_t, lp);
      if (WITH_Q) {
        split2_f16(kS8 * qn[t][0], kS8 * qn[t][1], hp, lp);
        qph[t] = __builtin_bit_cast(uint32_t, hp);
        qpl[t] = __builtin_bit_cast(uint32_t, lp);
      }
    }
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      float ed[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        ed[e] = kS8 * __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, g_ed), 16 * pw + 4 * gq + e));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        split4v(f32x4{ed[0] * kn[4 * gq][j], ed[1] * kn[4 * gq + 1][j], ed[2] * kn[4 * gq + 2][j], ed[3] * kn[4 * gq + 3][j]},
                kth[j][gq], ktl[j][gq]);
    }
  };

  // the packed operands to LDS: q, k as token rows (row t of token tile pw; channel 2 lane (+1) is
  // index j0 (+1) of 32-block kk: lane group slot_g(j0), elements slot_e(j0), slot_e(j0) + 1), k~ as d
  // rows (channel d is row d % 16 of tile d / 16; token s = 16 pw + t sits in 32-block pw / 2 at index
  // 16 (pw & 1) + t: lane group t / 4, elements 4 (pw & 1) + t % 4); and the gates
  auto write = [&]() __attribute__((always_inline)) {
    const int j0 = (2 * lane) & 31, kk = (2 * lane) >> 5;
    const int sg = slot_g(j0), se = slot_e(j0);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int base = ((pw * 4 + kk) * 2) * 64 + qk_slot(sg, t, kk);
      *(uint32_t*)((_Float16*)&sK[base] + se) = kph[t];
      *(uint32_t*)((_Float16*)&sK[base + 64] + se) = kpl[t];
      if (WITH_Q) {
        *(uint32_t*)((_Float16*)&sQ[base] + se) = qph[t];
        *(uint32_t*)((_Float16*)&sQ[base + 64] + se) = qpl[t];
      }
    }
    const int kb = pw >> 1, eo = 4 * (pw & 1);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int d = 2 * lane + j, hm = d >> 4, cr = d & 15;
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int base = ((hm * 2 + kb) * 2) * 64 + kt_slot(gq, cr, hm);
        *(f16x4*)((_Float16*)&sKT[base] + eo) = kth[j][gq];
        *(f16x4*)((_Float16*)&sKT[base + 64] + eo) = ktl[j][gq];
      }
    }
    if (pw == 0) {
      sBeta[lane] = g_beta;
      sEg[lane] = g_eg;
      sGam[lane] = g_gam;
      if (lane == 0) sEc[0] = g_ec;
    }
  };

  // Gram products of tile (mt, nt), nt <= mt: K K^T and (OUT) K Q^T, both as D = K_nt Y_mt^T so that lane
  // (g, c) holds entry [16 mt + c][16 nt + 4 g + i]: the layout of a 16x16x16 A operand (row 16 mt + c,
  // contraction indices 4 g .. 4 g + 3) and of half a 16x16x32 A operand (elements 4 (nt & 1) .. +3 of
  // 32-block nt / 2). The ten tiles go round-robin over the prep waves.
  auto gram = [&]() __attribute__((always_inline)) {
#pragma unroll 1
    for (int i = 0; i < 3; ++i) {
      const int tile = pw + 4 * i;
      if (tile >= 10) break;
      const int mt = tile >= 6 ? 3 : tile >= 3 ? 2 : tile >= 1 ? 1 : 0;
      const int nt = tile - mt * (mt + 1) / 2;
      f32x4 k0 = {0.f, 0.f, 0.f, 0.f}, k1 = k0, k2 = k0, q0 = k0, q1 = k0, q2 = k0;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int qs = qk_slot(g16, c16, kk);
        const f16x8 xh = sK[((nt * 4 + kk) * 2) * 64 + qs], xl = sK[((nt * 4 + kk) * 2 + 1) * 64 + qs];
        const f16x8 yh = sK[((mt * 4 + kk) * 2) * 64 + qs], yl = sK[((mt * 4 + kk) * 2 + 1) * 64 + qs];
        k0 = mfma32(xl, yh, k0);
        k1 = mfma32(xh, yl, k1);
        k2 = mfma32(xh, yh, k2);
        if (WITH_Q) {
          const f16x8 zh = sQ[((mt * 4 + kk) * 2) * 64 + qs], zl = sQ[((mt * 4 + kk) * 2 + 1) * 64 + qs];
          q0 = mfma32(xl, zh, q0);
          q1 = mfma32(xh, zl, q1);
          q2 = mfma32(xh, zh, q2);
        }
      }
      const int r = 16 * mt + c16;
      const float gr = sGam[r], br = sBeta[r];
      const float4 gs4 = *(const float4*)(sGam + 16 * nt + 4 * g16);
      const float gs[4] = {gs4.x, gs4.y, gs4.z, gs4.w};
      float dec[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) dec[e] = __expf(gr - gs[e]);  // s <= r here for the entries kept
      {
        const f32x4 kk4 = (k2 + (k0 + k1)) * kIS16;  // k_r . k_s
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = 16 * nt + 4 * g16 + e < r ? br * dec[e] * kk4[e] : 0.f;
        if (nt < mt) {
          f16x4 hi;
#pragma unroll
          for (int e = 0; e < 4; ++e) hi[e] = (_Float16)(x[e] * -kS8);
          sAO[aidx(mt, nt) * 64 + lane] = hi;
        } else {
          *(float4*)&sAD[(mt * 16 + c16) * LDA + 4 * g16] = make_float4(x[0], x[1], x[2], x[3]);
        }
      }
      if (WITH_Q) {
        const f32x4 qk4 = (q2 + (q0 + q1)) * kIS16;  // q_r . k_s
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = 16 * nt + 4 * g16 + e <= r ? (p.scale * kS16) * dec[e] * qk4[e] : 0.f;
        f16x4 hi, lo;
        split4v(x, hi, lo);
        const int pi = pidx(mt, nt >> 1), eo = 4 * (nt & 1);
        *(f16x4*)((_Float16*)&sP[(pi * 2) * 64 + lane] + eo) = hi;
        *(f16x4*)((_Float16*)&sP[(pi * 2 + 1) * 64 + lane] + eo) = lo;
        if (nt == mt && (mt & 1) == 0) {  // the upper half of the diagonal 32-block is zero
          const f16x4 z4 = {(_Float16)0.f, (_Float16)0.f, (_Float16)0.f, (_Float16)0.f};
          *(f16x4*)((_Float16*)&sP[(pi * 2) * 64 + lane] + 4) = z4;
          *(f16x4*)((_Float16*)&sP[(pi * 2 + 1) * 64 + lane] + 4) = z4;
        }
      }
    }
  };

  // (one wave) T_mm = (I + A_mm)^{-1} of the four diagonal blocks by forward substitution (lane =
  // block x column), then as 16x16x16 A-operand fragments (row c, columns 4 g .. 4 g + 3), 2^8 hi/lo
  auto tinv = [&]() __attribute__((always_inline)) {
    const int m = lane >> 4, j = lane & 15;
    const float* Am = sAD + m * 16 * LDA;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = i == j ? 1.f : 0.f;
#pragma unroll
      for (int q = 0; q < i; ++q) s -= Am[i * LDA + q] * x[q];
      x[i] = s;
      __builtin_amdgcn_sched_barrier(0);  // row by row: keeps the row loads from all being hoisted at once
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sTF[(m * 16 + i) * LDA + j] = x[i];
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the writes above land before the reads below
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
      const float4 row = *(const float4*)(sTF + (mm * 16 + c16) * LDA + 4 * g16);
      f16x4 hi, lo;
      split4v(f32x4{row.x, row.y, row.z, row.w} * kS8, hi, lo);
      sTI[(mm * 2) * 64 + lane] = hi;
      sTI[(mm * 2 + 1) * 64 + lane] = lo;
    }
  };

  // prologue: chunk c0's operands
  load(u.c0);
  conv(u.c0);
  pack();
  lds_barrier();
  write();
  if (u.c0 + 1 < u.c1) load(u.c0 + 1);
  lds_barrier();
  gram();
  lds_barrier();
  if (pw == 0) tinv();
  lds_barrier();
  for (int c = u.c0; c + 1 < u.c1; ++c) {  // the chain runs chunk c meanwhile
    conv(c + 1);
    pack();
    lds_barrier();  // Y: the chain is done with chunk c's operands
    write();
    if (c + 2 < u.c1) load(c + 2);
    lds_barrier();  // Y1
    gram();
    lds_barrier();  // Y2
    if (pw == 0) tinv();
    lds_barrier();  // X
  }
  // the chain's last chunk: nothing more to build
  lds_barrier();
  lds_barrier();
  lds_barrier();
  lds_barrier();
}

template <int MODE>
__global__ __launch_bounds__(512) void fused_kernel(FusedArgs p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const Unit u = unit_of<MODE>(p);
  if (u.c0 >= u.c1) return;                  // an empty segment: nothing to run or write
  if (MODE != MODE_OUT && u.last) return;    // the last segment's map is never used
  if (threadIdx.x < 256) chain_role<MODE>(p, u, smem);
  else prep_role<MODE>(p, u, smem);
}

// ---------------------------------------------------------------------------------------------------
// Entering state of every segment: H_{s+1} = M_s H_s + N_s, s = 0 .. (last real segment) - 1, from the
// sequence's saved state H_0. One workgroup of 4 waves per (sequence, head, 16-column slice); wave w
// forms row tiles 2 w and 2 w + 1 of the next state. M_s as hi/lo f16 A operands (2^8), H_s as hi/lo B
// operands (2^8), through LDS between steps.
__global__ __launch_bounds__(256) void scan_kernel(FusedArgs p) {
  const int slice = blockIdx.x & 7, hb = blockIdx.x >> 3;
  const int h = hb % p.n_v, b = hb / p.n_v;
  const int len = p.len[b];
  const int n_real = (len + FC - 1) / FC;
  if (n_real == 0) return;
  const int s_last = (n_real - 1) / p.seg_chunks;  // segment of the last real chunk
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g16 = lane >> 4, c16 = lane & 15;
  const int col = 16 * slice + c16;
  __shared__ float sH[FD][17];
  const float* H0 = p.state + ((long)b * p.n_v + h) * FD * FD;
  for (int i = tid; i < FD * 16; i += 256) sH[i >> 4][i & 15] = H0[(long)(i >> 4) * FD + 16 * slice + (i & 15)];
  __syncthreads();
  for (int s = 0; s < s_last; ++s) {
    const float* N = p.seg_map + ((((long)b * p.n_v + h) * (p.nseg - 1) + s) * 2 + 0) * FD * FD;
    const float* M = N + FD * FD;
    // B operand fragments of 2^8 H_s: k-block kk, rows 32 kk + {4 g .. 4 g + 3, 16 + 4 g .. 16 + 4 g + 3}
    f16x8 bh[4], bl[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      f32x4 x0, x1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x0[e] = kS8 * sH[32 * kk + 4 * g16 + e][c16];
        x1[e] = kS8 * sH[32 * kk + 16 + 4 * g16 + e][c16];
      }
      f16x4 h0, l0, h1, l1;
      split4v(x0, h0, l0);
      split4v(x1, h1, l1);
      bh[kk] = cat8(h0, h1);
      bl[kk] = cat8(l0, l1);
    }
    f32x4 acc[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int rt = 2 * w + q;  // row tile of M and of the result
      f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, a2 = a0;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const float* mr = M + (long)(16 * rt + c16) * FD + 32 * kk;
        const float4 m0 = *(const float4*)(mr + 4 * g16), m1 = *(const float4*)(mr + 16 + 4 * g16);
        f16x4 h0, l0, h1, l1;
        split4v(f32x4{m0.x, m0.y, m0.z, m0.w} * kS8, h0, l0);
        split4v(f32x4{m1.x, m1.y, m1.z, m1.w} * kS8, h1, l1);
        const f16x8 ah = cat8(h0, h1), al = cat8(l0, l1);
        a0 = mfma32(al, bh[kk], a0);
        a1 = mfma32(ah, bl[kk], a1);
        a2 = mfma32(ah, bh[kk], a2);
      }
      acc[q] = (a2 + (a0 + a1)) * kIS16;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[q][i] += N[(long)(16 * rt + 4 * g16 + i) * FD + col];
    }
    __syncthreads();  // every wave has read H_s
    float* dst = p.seg_in + (((long)b * p.n_v + h) * p.nseg + s + 1) * FD * FD;
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * (2 * w + q) + 4 * g16 + i;
        sH[r][c16] = acc[q][i];
        dst[(long)r * FD + col] = acc[q][i];
      }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------------------
// conv tail update after a fused prefill: new tail = rows len .. len + 2 of [old tail | mixed], one
// thread per 8 channels of one sequence (reads all three rows before writing)
__global__ __launch_bounds__(256) void tail_kernel(FusedArgs p) {
  const int b = blockIdx.y;
  const int c8 = blockIdx.x * 256 + threadIdx.x;
  if (8 * c8 >= p.C) return;
  const int len = p.len[b];
  const int C = p.C;
  uint16_t* tl = (uint16_t*)p.tail + (long)b * 3 * C + 8 * c8;
  const uint16_t* mx = (const uint16_t*)p.mixed + (long)b * p.Lb * C + 8 * c8;
  u32x4 v[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int r = len + j;  // row of [tail | mixed]
    v[j] = r < 3 ? *(const u32x4*)(tl + (long)r * C) : *(const u32x4*)(mx + (long)(r - 3) * C);
  }
#pragma unroll
  for (int j = 0; j < 3; ++j) *(u32x4*)(tl + (long)j * C) = v[j];
}

}  // namespace

// ---- host side ---------------------------------------------------------------------------------------

// Segments per (sequence, head). A call of few (sequence, head) units is spread over the chip by
// segments: every unit's chunks are cut into S segments of seg_chunks chunks, whose maps (two
// workgroups each, all but the last segment) run in one wave of workgroups, then the scan, then all
// segments at once. The plan is a performance choice only (no workgroup waits for another), made for
// a chip of kPlanCUs CUs so that workspace sizes do not depend on the device.
constexpr int kPlanCUs = 256;

// the largest segment count for B x n_v units and Lb tokens: at least 3 (2 would not pay for the map
// pass), at most one map workgroup per CU, at least 4 chunks per segment; 1 = no segments.
// Non-decreasing in Lb.
int seg_cap(int B, int n_v, int Lb) {
  const int n_chunks = (Lb + FC - 1) / FC;
  const long units = (long)B * n_v;
  const long by_cus = kPlanCUs / (2 * units) + 1;
  long S = by_cus < n_chunks / 4 ? by_cus : n_chunks / 4;
  return S >= 3 ? (int)S : 1;
}

void fused_plan(int B, int n_v, int Lb, int& nseg, int& seg_chunks) {
  const int n_chunks = (Lb + FC - 1) / FC;
  const int S = seg_cap(B, n_v, Lb);
  seg_chunks = (n_chunks + S - 1) / S;
  nseg = (n_chunks + seg_chunks - 1) / seg_chunks;  // <= S
}

// segment maps [B][n_v][S-1][2][D][D] and segment states [B][n_v][S][D][D] for the cap S
size_t fused_ws_bytes(int B, int n_v, int Lb) {
  const int S = seg_cap(B, n_v, Lb);
  if (S <= 1) return 0;
  return (size_t)B * n_v * ((size_t)(S - 1) * 2 + S) * FD * FD * 4;
}

hipError_t launch_fused(FusedArgs p, hipStream_t st) {
  // the dynamic LDS limit of the three instantiations, raised once per device (thread-safe)
  static std::once_flag once[64];
  static hipError_t attr[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::call_once(once[dev], [dev] {
    hipError_t e = hipFuncSetAttribute((const void*)fused_kernel<MODE_OUT>, hipFuncAttributeMaxDynamicSharedMemorySize, L_END);
    if (e == hipSuccess) e = hipFuncSetAttribute((const void*)fused_kernel<MODE_MAP_N>, hipFuncAttributeMaxDynamicSharedMemorySize, L_END);
    if (e == hipSuccess) e = hipFuncSetAttribute((const void*)fused_kernel<MODE_MAP_M>, hipFuncAttributeMaxDynamicSharedMemorySize, L_END);
    attr[dev] = e;
  });
  if (attr[dev] != hipSuccess) return attr[dev];
  const int units = p.B * p.n_v;
  if (p.nseg > 1) {
    p.seg_map = (float*)p.ws;
    p.seg_in = p.seg_map + (size_t)units * (p.nseg - 1) * 2 * FD * FD;
    const int nm = units * (p.nseg - 1);
    timing_before("fused_map", st);
    hipLaunchKernelGGL(fused_kernel<MODE_MAP_N>, dim3(nm), dim3(512), L_END, st, p);
    hipLaunchKernelGGL(fused_kernel<MODE_MAP_M>, dim3(nm), dim3(512), L_END, st, p);
    timing_after(st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    timing_before("fused_scan", st);
    hipLaunchKernelGGL(scan_kernel, dim3(units * 8), dim3(256), 0, st, p);
    timing_after(st);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  timing_before("fused", st);
  hipLaunchKernelGGL(fused_kernel<MODE_OUT>, dim3(units * p.nseg), dim3(512), L_END, st, p);
  timing_after(st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  timing_before("tail", st);
  hipLaunchKernelGGL(tail_kernel, dim3((p.C / 8 + 255) / 256, p.B), dim3(256), 0, st, p);
  timing_after(st);
  return hipGetLastError();
}

}  // namespace gdn
