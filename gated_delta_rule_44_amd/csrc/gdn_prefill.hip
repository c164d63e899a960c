// Chunked prefill of the gated delta rule (gfx950): two launches.
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
//   K K^T and K Q^T (f16 MFMA, hi/lo-split operands), then for each value head of the GQA group the UT
//   inverse T (fp32: diagonal 16x16 blocks by substitution, off-diagonal blocks on fp32 MFMA), W and U'
//   (f16 MFMA), P~ = scale P, Q~ = scale diag(e^gamma) Q and K~ = diag(e^{gamma_C - gamma}) K (with
//   several value heads per key head, q and k once per key head and the decays as per-token factors;
//   see the records below). Every operand the state pass needs is written as a ready MFMA fragment:
//   1 KB blocks in which lane l's 16 bytes are exactly what lane l of the consuming wave loads, so each
//   store and each load is one fully coalesced 1 KB wave access.
// Launch 2, state_pass_kernel (one workgroup per column slice x value head x sequence, chunks in order;
//   eight waves in two roles, one of each on every SIMD; wave w works on token tile w & 3 and owns H
//   row tile w):
//   chain waves 0-3:  U = U' - W H for their token tile (H read as fragments from LDS)
//   output waves 4-7: O^T = H^T Q~^T + U^T P~^T for their token tile
//   every wave:       its row tile of H = e^{gamma_C} H + K~^T U (U read back as fragments from LDS)
//   Only H and U cross waves, through LDS; each wave loads its own fragments of the next chunks into
//   registers while the current chunk computes. The gated RMSNorm: when one workgroup owns all d_v
//   columns of the head it normalises each row at once. When the columns are split over 2 or 4 slices
//   on a long call, each slice posts its partial sum of squares of the row, keeps w o silu(z) of its
//   columns in LDS and scales them by 1/rms a few chunks later, once every slice of the head has
//   posted (chunk_prep marks those sums pending first; all slices of a head are resident together, one
//   workgroup per CU). Otherwise the slices save o and their sums and norm_kernel finishes the rows.
//
// Fragment convention (f16 16x16x32 MFMA, lane l = 16 g + c): a 32-wide k-block is split so that lane
// group g holds k = {4g..4g+3, 16+4g..16+4g+3}. With that grouping the two 16x16 accumulator tiles of a
// 32-row block give, lane by lane, exactly the operand fragment of that block, so results turn into
// operands without moving between lanes.
//
// Precision: f16 operands with fp32 accumulation, and hi/lo f16 pairs (about 22 mantissa bits) where
// rounding would otherwise show in the output: the Gram products, beta*V, H, U, K~, Q~ and P~. With
// fp32 activations every operand is split. MFMA flushes f16 subnormals, so the lo half of a split value
// must stay >= 2^-14: operands of unit scale are carried multiplied by 2^8 (exact), and the scales are
// chosen so that every product lands in a consistent domain: the state pass keeps H as 2^16 H, U as
// 2^8 U and O^T as 2^24 O^T, with 2^16 Q~, 2^16 P~, 2^8 K~, 2^16 U' and 2^8 -W in the record. Q~ and
// P~ hold scale (< 1) and the decays folded in, and -W is small: at 2^8 their lo halves (and the small
// entries of -W) would fall below 2^-14 and flush, which costs about half of a 2e-3 output bound at a
// 4096-token prefill; at these scales the rounding costs a fifth of it.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

constexpr int C64 = kChunk;
constexpr float kS8 = 256.f;              // 2^8 operand scale
constexpr float kInvS8 = 1.f / 256.f;
constexpr float kInvS16 = 1.f / 65536.f;
constexpr float kInvS24 = 1.f / 16777216.f;
// a split head's partial sum of squares not posted yet (a posted sum is >= 0 or NaN, never -1)
constexpr float kSsPending = -1.f;
// bound of a slice's wait for the other slices' sums, in ticks of the 100 MHz constant clock (1 s)
constexpr uint64_t kSpinTicks = 100000000ull;

// Barrier for LDS reads and writes only. __syncthreads() also waits for this wave's outstanding global
// loads and stores (vmcnt), which would stall on the record stores of chunk_prep and serialise the
// register prefetch of the next chunk in the state pass with the current chunk's work.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// k-index (inside a 32-block) of fragment slot e (0..7) of lane group g
__device__ __forceinline__ int kslot(int g, int e) { return e < 4 ? 4 * g + e : 12 + 4 * g + e; }

__device__ __forceinline__ f16x8 ld16(const _Float16* p) { return *(const f16x8*)p; }

// the fragment slots of lane group g from a row of 32 halfs or floats: {4g..4g+3} then {16+4g..16+4g+3}
__device__ __forceinline__ f16x8 frag_row_h(const _Float16* row32, int g) {
  const f16x4 a = *(const f16x4*)(row32 + 4 * g), b = *(const f16x4*)(row32 + 16 + 4 * g);
  return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ void frag_row_f(const float* row32, int g, float (&x)[8]) {
  const float4 a = *(const float4*)(row32 + 4 * g), b = *(const float4*)(row32 + 16 + 4 * g);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

__device__ __forceinline__ void split8(const float (&x)[8], f16x8& hi, f16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    f16x2 h, l;
    split2_f16(x[e], x[e + 1], h, l);
    hi[e] = h[0];
    hi[e + 1] = h[1];
    lo[e] = l[0];
    lo[e + 1] = l[1];
  }
}
__device__ __forceinline__ void split4(f32x4 x, f16x4& hi, f16x4& lo) {
#pragma unroll
  for (int e = 0; e < 4; e += 2) {
    f16x2 h, l;
    split2_f16(x[e], x[e + 1], h, l);
    hi[e] = h[0];
    hi[e + 1] = h[1];
    lo[e] = l[0];
    lo[e + 1] = l[1];
  }
}

// ---- the per-chunk records -----------------------------------------------------------------------
// Fragment blocks of 1 KB: lane l's 16 bytes at 16 l. Token tile mt = 16 tokens, H row tile hm = 16
// rows of d_k, kk = 32-block of the contraction index, hi/lo halves in separate blocks.
// One record per sequence x value head x chunk. With one value head per key head (SH false) it holds
// the decayed Q~ and K~ too. With several (SH true), q and k, which are per key head, go once into a
// key record per sequence x key head x chunk, undecayed, and the value record carries the per-token
// decays instead: the state pass scales the columns of Q H by scale e^{gamma_t} and decays U by
// e^{gamma_C - gamma_t} before the state update.
template <int D, bool SPLIT, bool SH>
struct Rec {
  static constexpr int KD = D / 32, HM = D / 16;
  static constexpr int W_HI = 0;                               // [mt][kk]: 2^8 -W[token][d_k]
  static constexpr int W_LO = W_HI + 4 * KD;                   // (fp32 activations only)
  static constexpr int Q_HI = W_LO + (SPLIT ? 4 * KD : 0);     // [mt][kk]: 2^16 Q~[token][d_k] (SH false)
  static constexpr int Q_LO = Q_HI + 4 * KD;
  static constexpr int P_HI = SH ? Q_HI : Q_LO + 4 * KD;       // [mt][kk]: 2^16 P~[token t][token s]
  static constexpr int P_LO = P_HI + 8;
  static constexpr int K_HI = P_LO + 8;                        // [hm][kk]: 2^8 K~^T[d_k][token] (SH false)
  static constexpr int K_LO = K_HI + 2 * HM;
  static constexpr int UP = SH ? K_HI : K_LO + 2 * HM;         // [mt][nt]: 2^16 U' in accumulator order
  static constexpr int NBLK = UP + 4 * HM;
  static constexpr long kGc = NBLK * 1024L;                    // e^{gamma_C}
  static constexpr long kEg = kGc + 256;                       // SH: 2^8 scale e^{gamma_t}, t = 0..63
  static constexpr long kEd = kEg + 256;                       // SH: e^{gamma_C - gamma_t}
  static constexpr long kBytes = kGc + (SH ? 768 : 256);
};
// the key record (SH): 2^8 q and 2^8 k^T of one key head, hi/lo, as the Q~ / K~ blocks above
template <int D>
struct KeyRec {
  static constexpr int KD = D / 32, HM = D / 16;
  static constexpr int Q_HI = 0, Q_LO = 4 * KD, K_HI = 8 * KD, K_LO = 8 * KD + 2 * HM;
  static constexpr long kBytes = (8 * KD + 4 * HM) * 1024L;
};

template <int D, bool SPLIT, bool SH>
__device__ __forceinline__ char* rec_ptr(const PrefillArgs& p, int b, int h, int c) {
  return (char*)p.ws + (((long)b * p.n_v + h) * p.n_chunks + c) * Rec<D, SPLIT, SH>::kBytes;
}
template <int D>
__device__ __forceinline__ char* key_ptr(const PrefillArgs& p, int b, int vk, int c) {
  return (char*)p.ws + p.key_off + (((long)b * (p.n_v / p.grp) + vk) * p.n_chunks + c) * KeyRec<D>::kBytes;
}
// (the lane offset is an unsigned 32-bit value added to a wave-uniform base, which the compiler can
// encode as a scalar base plus vector offset instead of a per-lane 64-bit address)
// NTS: a non-temporal store, for records too large to stay cached until the state pass reads them
template <bool NTS, typename V>
__device__ __forceinline__ void st_rec(V* dst, V v) {
  if constexpr (NTS) __builtin_nontemporal_store(v, dst);
  else *dst = v;
}
template <bool NTS = false>
__device__ __forceinline__ void put_frag(char* rec, int blk, int lane, f16x8 v) {
  st_rec<NTS>((f16x8*)(rec + blk * 1024 + (uint32_t)(lane * 16)), v);
}
__device__ __forceinline__ f16x8 get_frag(const char* rec, int blk, int lane) {
  return *(const f16x8*)(rec + blk * 1024 + (uint32_t)(lane * 16));
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
    u.x = pack_bf16x2(v.x, v.y);
    u.y = pack_bf16x2(v.z, v.w);
    *(uint2*)p = u;
  }
};

// four output values at element index i of out: fp32 when the call asked for fp32 outputs, else the
// activation type
template <typename ActT>
__device__ __forceinline__ void store_out4(const PrefillArgs& p, long i, float4 v) {
  if (std::is_same<ActT, float>::value || p.out_f32) *(float4*)((float*)p.out + i) = v;
  else Act4<ActT>::store((ActT*)p.out + i, v);
}

// two adjacent activations (4 bytes of bf16 or 8 of fp32), loaded as stored and widened when used
template <typename ActT>
struct Pair {
  typedef uint32_t type;
  static __device__ __forceinline__ type load(const ActT* p) { return *(const uint32_t*)p; }
  static __device__ __forceinline__ float2 widen(type u) {
    return make_float2(__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u));
  }
};
template <>
struct Pair<float> {
  typedef float2 type;
  static __device__ __forceinline__ type load(const float* p) { return *(const float2*)p; }
  static __device__ __forceinline__ float2 widen(type u) { return u; }
};

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// -------------------------------------------------------------------------------------------------
// With a head's columns split over state-pass slices: mark the partial sums of squares of this chunk's
// rows (every value head of key head kh) pending; each slice overwrites its own when it posts it.
// Layout [sequence][value head][token][slice].
__device__ __forceinline__ void mark_sums_pending(const PrefillArgs& p, int b, int vk, int R, int t0, int tid) {
  const int ns = p.nsplit;
  if (ns <= 1 || !p.exchange) return;
  float* ss = (float*)((char*)p.ws + p.ss_off);
  for (int i = tid; i < R * C64 * ns; i += 512) {
    const int hr = i / (C64 * ns), t = t0 + (i / ns) % C64;
    if (t < p.Lb) ss[(((long)b * p.n_v + vk * R + hr) * p.Lb + t) * ns + i % ns] = kSsPending;
  }
}

// -------------------------------------------------------------------------------------------------
template <typename ActT, int D, int R, bool SPLIT>
__global__ __launch_bounds__(512) void chunk_prep_kernel(PrefillArgs p) {
  constexpr bool SH = R > 1;
  using RC = Rec<D, SPLIT, SH>;
  constexpr int NWV = 8, NTH = 64 * NWV;      // two waves per SIMD: one's waits overlap the other's work
  constexpr int TPW = C64 / NWV;              // tokens per wave in the conv stage
  constexpr int KD = D / 32, HM = D / 16;
  constexpr int CPL = D >= 64 ? D / 64 : 1;   // channels per lane in the conv stage (adjacent)
  constexpr int LQ = D + 8;                   // halfs per row, token-major f16 tiles
  constexpr int LT = C64 + 4;                 // floats per row, channel-major fp32 tiles and Gram results
  constexpr int LF = C64 + 1;                 // floats per row, A and T
  constexpr int LDT = C64 + 8;                // halfs per row, T as f16
  constexpr int SZ_TOK = C64 * LQ * 2;
  constexpr int SZ_CHF = D * LT * 4;
  constexpr int SZ_AT = 2 * C64 * LF * 4;
  constexpr int SZ_R1 = cmax(2 * SZ_TOK, SZ_CHF);   // q hi|lo for the Gram, then v^T (fp32) per head
  constexpr int SZ_R2 = cmax(2 * SZ_TOK, SZ_AT);    // k hi|lo for the Gram, then A | T (fp32) per head
  constexpr int OFF_R1 = 0, OFF_R2 = SZ_R1;
  constexpr int OFF_KT = OFF_R2 + SZ_R2;            // k^T fp32 [D][LT]
  constexpr int OFF_KK = OFF_KT + SZ_CHF;           // 2^16 K K^T [r][s]
  constexpr int OFF_QK = OFF_KK + C64 * LT * 4;     // 2^16 Q K^T [t][s]
  constexpr int OFF_T = OFF_QK + C64 * LT * 4;      // 2^8 T as f16 hi (then lo)
  constexpr int OFF_X = OFF_T;                      // level products, only while T is still fp32
  constexpr int OFF_G = OFF_T + (SPLIT ? 2 : 1) * C64 * LDT * 2;
  constexpr int OFF_B = OFF_G + R * C64 * 4;
  constexpr int OFF_E = OFF_B + R * C64 * 4;        // per head: e^{gamma_t}, then e^{gamma_C - gamma_t}
  constexpr int LDS = OFF_E + 2 * C64 * 4;
  static_assert(4 * 16 * 17 * 4 <= (SPLIT ? 2 : 1) * C64 * LDT * 2, "level products fit the T tile");
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(CPL == 1 || (CPL == 2 && D == 128), "channel layout");
  __shared__ __attribute__((aligned(16))) char smem[LDS];
  _Float16* sQh = (_Float16*)(smem + OFF_R1);
  _Float16* sQl = sQh + C64 * LQ;
  float* sVt = (float*)(smem + OFF_R1);
  _Float16* sKh = (_Float16*)(smem + OFF_R2);
  _Float16* sKl = sKh + C64 * LQ;
  float* sA = (float*)(smem + OFF_R2);
  float* sTf = sA + C64 * LF;
  float* sKt = (float*)(smem + OFF_KT);
  float* sKK = (float*)(smem + OFF_KK);
  float* sQK = (float*)(smem + OFF_QK);
  _Float16* sT = (_Float16*)(smem + OFF_T);
  float* sX = (float*)(smem + OFF_X);
  float* sGam = (float*)(smem + OFF_G);
  float* sBet = (float*)(smem + OFF_B);
  float* sEg = (float*)(smem + OFF_E);
  float* sEd = sEg + C64;

  // group vk: value heads vk R .. vk R + R - 1 of key head kh
  const int c = blockIdx.x, vk = blockIdx.y, b = blockIdx.z;
  const int kh = vk * R / (p.n_v / p.n_k);
  const int t0 = c * C64;
  const int len = p.len[b];
  if (t0 >= len) return;  // all padding: the state pass stops before this chunk
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so addresses built on it stay scalar
  mark_sums_pending(p, b, vk, R, t0, tid);
  const int g16 = lane >> 4, r16 = lane & 15;
  const int Lb = p.Lb, C = p.C, n_k = p.n_k;
  const ActT* mixed = (const ActT*)p.mixed + (long)b * Lb * C;
  const ActT* tail = (const ActT*)p.tail + (long)b * 3 * C;
  const ActT* cw = (const ActT*)p.conv_w;

  // ---- 1. every global load of this stage first, then the arithmetic: gate inputs (lane = token),
  // conv inputs and taps of q, k and the R value heads (wave w: rows TPW w - 3 .. TPW w + TPW - 1, lane:
  // channels CPL lane + j, two adjacent channels per load). Addresses are clamped into range and the
  // values masked when widened, so that all loads are in flight before the first wait.
  constexpr int NCV = 2 + R;  // convolutions: q, k, then the value heads
  typedef typename std::conditional<CPL == 2, typename Pair<ActT>::type, ActT>::type XRaw;
  typedef typename Raw4<ActT>::type WRaw;
  const int hg = vk * R + (w < R ? w : 0);
  const int tg = t0 + lane;
  const long gi = ((long)b * Lb + (tg < len ? tg : len - 1)) * p.n_v + hg;  // len >= 1 here
  const ActT a_raw = ((const ActT*)p.a)[gi], b_raw = ((const ActT*)p.b)[gi];
  XRaw xr[NCV][TPW + 3];
  WRaw wr[NCV][CPL];
#pragma unroll
  for (int j = 0; j < NCV; ++j) {
    const int base = j == 0 ? kh * D : j == 1 ? (n_k + kh) * D : (2 * n_k + vk * R + j - 2) * D;
    const int gc = base + (CPL == 2 ? 2 * lane : (lane < D ? lane : 0));
#pragma unroll
    for (int i = 0; i < CPL; ++i) wr[j][i] = Raw4<ActT>::load(cw + (gc + i) * 4);
#pragma unroll
    for (int i = 0; i < TPW + 3; ++i) {
      const int t = t0 + TPW * w - 3 + i;
      const ActT* src = t < 0 ? tail + (long)(t + 3) * C : mixed + (long)(t < Lb ? t : Lb - 1) * C;
      if constexpr (CPL == 2) xr[j][i] = Pair<ActT>::load(src + gc);
      else xr[j][i] = src[gc];
    }
  }

  // ---- 2. gates of the R value heads: wave r, lane = token; inclusive scan of g over the chunk -----
  if (w < R) {
    const float g0 = chunk_log_decay(-__expf(p.A_log[hg]) * softplus(to_f32(a_raw) + p.dt_bias[hg]));
    const float b0 = sigmoid(to_f32(b_raw));
    float g = tg < len ? g0 : 0.f;
    const float be = tg < len ? b0 : 0.f;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const float o = __shfl_up(g, off, kWave);
      if (lane >= off) g += o;
    }
    sGam[w * C64 + lane] = g;
    sBet[w * C64 + lane] = be;
  }

  // ---- 3. conv + SiLU of convolution j: y[tt][i] for token TPW w + tt, channel CPL lane + i ---------
  auto conv = [&](int j, float (*y)[CPL]) {
    float x[TPW + 3][CPL], wt[4][CPL];
    const float m = CPL == 2 || lane < D ? 1.f : 0.f;  // lanes past d (d = 32) produce zeros
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const float4 wf = Raw4<ActT>::widen(wr[j][i]);
      wt[0][i] = m * wf.x; wt[1][i] = m * wf.y; wt[2][i] = m * wf.z; wt[3][i] = m * wf.w;
    }
#pragma unroll
    for (int i = 0; i < TPW + 3; ++i) {
      const bool in = t0 + TPW * w - 3 + i < Lb;
      if constexpr (CPL == 2) {
        const float2 v = Pair<ActT>::widen(xr[j][i]);
        x[i][0] = in ? v.x : 0.f;
        x[i][CPL - 1] = in ? v.y : 0.f;
      } else {
        x[i][0] = in ? to_f32(xr[j][i]) : 0.f;
      }
    }
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
      for (int i = 0; i < CPL; ++i)
        y[tt][i] = silu(wt[0][i] * x[tt][i] + wt[1][i] * x[tt + 1][i] + wt[2][i] * x[tt + 2][i] + wt[3][i] * x[tt + 3][i]);
  };
  auto l2norm = [&](float (*y)[CPL]) {
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < CPL; ++j) ss += y[tt][j] * y[tt][j];
      ss = wave_sum<kWave>(ss);
      const float rn = rsqrt_fast(ss + p.l2_eps);
#pragma unroll
      for (int j = 0; j < CPL; ++j) y[tt][j] *= rn;
    }
  };
  float qn[TPW][CPL], kn[TPW][CPL], vv[R][TPW][CPL];
  conv(0, qn);
  conv(1, kn);
#pragma unroll
  for (int r = 0; r < R; ++r) conv(2 + r, vv[r]);
  l2norm(qn);
  l2norm(kn);
  // token-major 2^8 q, 2^8 k (hi/lo) for the Gram products; channel-major k in fp32
  if (CPL * lane < D) {
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      const int o = (TPW * w + tt) * LQ + CPL * lane;
      _Float16 qh[CPL], ql[CPL], kh_[CPL], kl[CPL];
      if constexpr (CPL == 2) {
        f16x2 h2, l2;
        split2_f16(kS8 * qn[tt][0], kS8 * qn[tt][1], h2, l2);
        qh[0] = h2[0]; qh[1] = h2[1]; ql[0] = l2[0]; ql[1] = l2[1];
        split2_f16(kS8 * kn[tt][0], kS8 * kn[tt][1], h2, l2);
        kh_[0] = h2[0]; kh_[1] = h2[1]; kl[0] = l2[0]; kl[1] = l2[1];
      } else {
        for (int j = 0; j < CPL; ++j) {
          split_f16(kS8 * qn[tt][j], qh[j], ql[j]);
          split_f16(kS8 * kn[tt][j], kh_[j], kl[j]);
        }
      }
      if (CPL == 2) {
        *(f16x2*)&sQh[o] = f16x2{qh[0], qh[CPL - 1]};
        *(f16x2*)&sQl[o] = f16x2{ql[0], ql[CPL - 1]};
        *(f16x2*)&sKh[o] = f16x2{kh_[0], kh_[CPL - 1]};
        *(f16x2*)&sKl[o] = f16x2{kl[0], kl[CPL - 1]};
      } else {
        sQh[o] = qh[0]; sQl[o] = ql[0]; sKh[o] = kh_[0]; sKl[o] = kl[0];
      }
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j)
#pragma unroll
      for (int q = 0; q < TPW / 4; ++q)
        *(float4*)&sKt[(CPL * lane + j) * LT + TPW * w + 4 * q] =
            make_float4(kn[4 * q][j], kn[4 * q + 1][j], kn[4 * q + 2][j], kn[4 * q + 3][j]);
  }
  lds_barrier();

  // ---- 4. Gram products on the lower 16x16 tiles (split operands) --------------------------------
  // K K^T as [r][s] (for A); K Q^T computed as D[s][t] so that each lane ends up with four
  // consecutive s of one row t of Q K^T (for P~). The three split terms go to separate accumulators.
  for (int job = w; job < 20; job += NWV) {
    const int prod = job / 10, tile = job % 10;       // tiles (mt, nt), nt <= mt, in row order
    const int mt = tile >= 6 ? 3 : tile >= 3 ? 2 : tile >= 1 ? 1 : 0;
    const int nt = tile - mt * (mt + 1) / 2;
    // KK: A = K rows 16mt, B = K rows 16nt.  KQ: A = K rows 16nt (s), B = Q rows 16mt (t)
    const _Float16* bh = prod ? sQh : sKh;
    const _Float16* bl = prod ? sQl : sKl;
    const int ra0 = prod ? 16 * nt : 16 * mt, rb0 = prod ? 16 * mt : 16 * nt;
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, a2 = a0;
    f16x8 fah[KD], fal[KD], fbh[KD], fbl[KD];
#pragma unroll
    for (int ks = 0; ks < KD; ++ks) {
      const int ra = (ra0 + r16) * LQ + 32 * ks + 8 * g16, rb = (rb0 + r16) * LQ + 32 * ks + 8 * g16;
      fah[ks] = ld16(sKh + ra);
      fal[ks] = ld16(sKl + ra);
      fbh[ks] = ld16(bh + rb);
      fbl[ks] = ld16(bl + rb);
    }
#pragma unroll
    for (int ks = 0; ks < KD; ++ks) {
      a0 = mfma16(fal[ks], fbh[ks], a0);
      a1 = mfma16(fah[ks], fbl[ks], a1);
      a2 = mfma16(fah[ks], fbh[ks], a2);
    }
    const f32x4 acc = a2 + (a0 + a1);
    if (prod) {
      *(f32x4*)&sQK[(16 * mt + r16) * LT + 16 * nt + 4 * g16] = acc;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) sKK[(16 * mt + 4 * g16 + i) * LT + 16 * nt + r16] = acc[i];
    }
  }
  // rows of 2^8 q as fragments (token tile mt = q & 3, 32-block kk = q >> 2 for q = w, w + 8, ...),
  // kept in registers for every value head
  constexpr int QPW = (4 * KD + NWV - 1) / NWV;
  f16x8 qfh[QPW], qfl[QPW];
#pragma unroll
  for (int i = 0; i < QPW; ++i) {
    const int q = w + NWV * i < 4 * KD ? w + NWV * i : 0;
    const int row = (16 * (q & 3) + r16) * LQ + 32 * (q >> 2);
    qfh[i] = frag_row_h(sQh + row, g16);
    qfl[i] = frag_row_h(sQl + row, g16);
  }
  if constexpr (SH) {
    // the key record: 2^8 q (token tile q & 3, block q >> 2) and 2^8 k^T (row tile idx >> 1, block
    // idx & 1), once for all value heads of the group
    using KR = KeyRec<D>;
    char* krec = key_ptr<D>(p, b, vk, c);
#pragma unroll
    for (int i = 0; i < QPW; ++i) {
      const int q = w + NWV * i;
      if (q < 4 * KD) {
        put_frag(krec, KR::Q_HI + (q & 3) * KD + (q >> 2), lane, qfh[i]);
        put_frag(krec, KR::Q_LO + (q & 3) * KD + (q >> 2), lane, qfl[i]);
      }
    }
    for (int idx = w; idx < 2 * HM; idx += NWV) {
      const int hm = idx >> 1, kk = idx & 1;
      float x[8];
      frag_row_f(sKt + (16 * hm + r16) * LT + 32 * kk, g16, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= kS8;
      f16x8 hi, lo;
      split8(x, hi, lo);
      put_frag(krec, KR::K_HI + hm * 2 + kk, lane, hi);
      put_frag(krec, KR::K_LO + hm * 2 + kk, lane, lo);
    }
  }
  lds_barrier();

  // ---- 5. per value head of the group ------------------------------------------------------------
  for (int r = 0; r < R; ++r) {
    const int h = vk * R + r;
    const float* gam = sGam + r * C64;
    const float* bet = sBet + r * C64;
    char* rec = rec_ptr<D, SPLIT, SH>(p, b, h, c);
    const float gC = gam[C64 - 1];

    // A (strictly lower, fp32), this head's v channel-major, and the
    // per-token decays e^{gamma_t}, e^{gamma_C - gamma_t} (each exponential taken once per head)
    if (tid < C64) {
      sEg[tid] = __expf(gam[tid]);
      sEd[tid] = __expf(gC - gam[tid]);
    }
    // (only the strictly lower part is ever read: rows p and 63 - p share 16 threads, 63 entries a pair)
    static_assert(NTH == 32 * 16 && C64 == 64, "row pairs of the A fill");
    {
      const int pr = tid >> 4, q = tid & 15;
#pragma unroll
      for (int e = q; e < C64 - 1; e += 16) {
        const int i = e < pr ? pr : C64 - 1 - pr;
        const int j = e < pr ? e : e - pr;
        sA[i * LF + j] = bet[i] * __expf(gam[i] - gam[j]) * (kInvS16 * sKK[i * LT + j]);
      }
    }
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {  // compile-time index into vv (a runtime one would go to scratch)
      if (rr != r || CPL * lane >= D) continue;
#pragma unroll
      for (int j = 0; j < CPL; ++j)
#pragma unroll
        for (int q = 0; q < TPW / 4; ++q)
          *(float4*)&sVt[(CPL * lane + j) * LT + TPW * w + 4 * q] =
              make_float4(vv[rr][4 * q][j], vv[rr][4 * q + 1][j], vv[rr][4 * q + 2][j], vv[rr][4 * q + 3][j]);
    }
    lds_barrier();

    // T = (I + A)^-1: diagonal blocks by forward substitution (wave 0, one column per lane); the
    // other waves write the fragments that do not need T meanwhile
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
    {
      // Q~ (token tile q & 3, block q >> 2): 2^16 scale e^{gamma_t} q_t
#pragma unroll
      for (int i = 0; i < QPW; ++i) {
        const int q = w + NWV * i;
        if (!SH && q < 4 * KD) {
          const int mt = q & 3, kk = q >> 2;
          const float fq = kS8 * p.scale * sEg[16 * mt + r16];
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = fq * ((float)qfh[i][e] + (float)qfl[i][e]);
          f16x8 hi, lo;
          split8(x, hi, lo);
          put_frag(rec, RC::Q_HI + mt * KD + kk, lane, hi);
          put_frag(rec, RC::Q_LO + mt * KD + kk, lane, lo);
        }
      }
      // P~ (token tile w & 3, block w >> 2): 2^16 scale e^{gamma_t - gamma_s} q_t.k_s for s <= t, else 0
      {
        const int mt = w & 3, kk = w >> 2;
        const int t = 16 * mt + r16;
        const float gt = gam[t];
        float x[8];
        frag_row_f(sQK + t * LT + 32 * kk, g16, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int s = 32 * kk + kslot(g16, e);
          x[e] = s <= t ? p.scale * __expf(gt - gam[s]) * x[e] : 0.f;
        }
        f16x8 hi, lo;
        split8(x, hi, lo);
        put_frag(rec, RC::P_HI + mt * 2 + kk, lane, hi);
        put_frag(rec, RC::P_LO + mt * 2 + kk, lane, lo);
      }
      // K~^T (row tile idx >> 1, block idx & 1 for idx = w, w + 8, ...): 2^8 e^{gamma_C - gamma_s} k_s;
      // with a key record, the per-token decays instead
      if (SH && tid < C64) {
        *(float*)(rec + RC::kEg + 4 * tid) = kS8 * p.scale * sEg[tid];
        *(float*)(rec + RC::kEd + 4 * tid) = sEd[tid];
      }
      for (int idx = SH ? 2 * HM : w; idx < 2 * HM; idx += NWV) {
        const int hm = idx >> 1, kk = idx & 1;
        float x[8];
        frag_row_f(sKt + (16 * hm + r16) * LT + 32 * kk, g16, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= kS8 * sEd[32 * kk + kslot(g16, e)];
        f16x8 hi, lo;
        split8(x, hi, lo);
        put_frag(rec, RC::K_HI + hm * 2 + kk, lane, hi);
        put_frag(rec, RC::K_LO + hm * 2 + kk, lane, lo);
      }
    }
    lds_barrier();
    // off-diagonal blocks by level (i - j = 1, 2, 3): T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj, fp32 MFMA
    for (int lvl = 1; lvl < 4; ++lvl) {
      if (w < 4 - lvl) {
        float* sXw = sX + w * 16 * 17;
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
      lds_barrier();
    }
    for (int idx = tid; idx < C64 * C64; idx += NTH) {
      const int i = idx >> 6, j = idx & 63;
      const float tv = (j >> 4) > (i >> 4) ? 0.f : kS8 * sTf[i * LF + j];  // T's upper blocks are zero
      if (SPLIT) split_f16(tv, sT[i * LDT + j], sT[C64 * LDT + i * LDT + j]);
      else sT[i * LDT + j] = (_Float16)tv;
    }
    lds_barrier();

    // W and U'. T's row fragments (all four token tiles) serve as the B operand of
    // W^T = (beta e^gamma K)^T T^T and as the A operand of U' = T (beta V); wave w takes d_k tiles
    // j = w, w + 8, ... of W^T and value tiles nt = w, w + 8, ... of U', so that each operand
    // fragment built from K or V is made once.
    if (w < HM) {
      f16x8 th[4][2], tl[4][2];
      float fk[2][8], fv[2][8];  // per-token factors of this lane's fragment slots
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const int rt = (16 * mt + r16) * LDT + 32 * ks;
          th[mt][ks] = frag_row_h(sT + rt, g16);
          tl[mt][ks] = SPLIT ? frag_row_h(sT + C64 * LDT + rt, g16) : th[mt][ks];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int s = 32 * ks + kslot(g16, e);
          fv[ks][e] = kS8 * bet[s];
          fk[ks][e] = fv[ks][e] * sEg[s];
        }
      }
      for (int j = w; j < HM; j += NWV) {
        // W^T tile (j, mt) = (2^8 beta e^gamma K)^T (2^8 T)^T = 2^16 W^T, stored as 2^8 -W; lane (g, c) holds
        // W[16 mt + c][16 j + 4 g + i], half (j & 1) of the fragment of block j >> 1
        f16x8 kbh[2], kbl[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          float x[8];
          frag_row_f(sKt + (16 * j + r16) * LT + 32 * ks, g16, x);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] *= fk[ks][e];
          split8(x, kbh[ks], kbl[ks]);
        }
        f32x4 acc[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) acc[mt] = mfma16(kbh[ks], th[mt][ks], acc[mt]);
          if (SPLIT) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) acc[mt] = mfma16(kbl[ks], th[mt][ks], acc[mt]);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) acc[mt] = mfma16(kbh[ks], tl[mt][ks], acc[mt]);
          }
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f16x4 hi, lo;
          split4(acc[mt] * -kInvS8, hi, lo);
          char* dst = rec + (RC::W_HI + mt * KD + (j >> 1)) * 1024 + (uint32_t)(lane * 16 + 8 * (j & 1));
          *(f16x4*)dst = hi;
          if (SPLIT) *(f16x4*)(dst + 4 * KD * 1024) = lo;
        }
      }
      for (int nt = w; nt < HM; nt += NWV) {
        // U' tile (mt, nt) = (2^8 T)(2^8 beta V) = 2^16 U', stored as is
        f16x8 vh[2], vl[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          float x[8];
          frag_row_f(sVt + (16 * nt + r16) * LT + 32 * ks, g16, x);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] *= fv[ks][e];
          split8(x, vh[ks], vl[ks]);
        }
        f32x4 a0[4], a1[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) a0[mt] = a1[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) a0[mt] = mfma16(th[mt][ks], vl[ks], a0[mt]);
          if (SPLIT) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) a0[mt] = mfma16(tl[mt][ks], vh[ks], a0[mt]);
          }
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) a1[mt] = mfma16(th[mt][ks], vh[ks], a1[mt]);
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          *(f32x4*)(rec + (RC::UP + mt * HM + nt) * 1024 + (uint32_t)(lane * 16)) = a1[mt] + a0[mt];
      }
    }
    if (tid == 0) *(float*)(rec + RC::kGc) = __expf(gC);
    lds_barrier();
  }
}

// -------------------------------------------------------------------------------------------------
// chunk_prep with bf16 activations in less than half the LDS of chunk_prep_kernel (the same records),
// so that two workgroups share a CU and one's memory waits and barriers overlap the other's work.
// k is staged only token-major (K~, the key record and the W operands gather their d-major fragments
// from it); the Gram accumulators stay in registers and become P~ (record) and A (LDS) per value head;
// the W operands of every value head are built while k is staged, and the U' operand of a head waits
// in registers while its T is formed.
template <typename ActT, int D, int R, bool NTS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4, 4))) void chunk_prep2_kernel(PrefillArgs p) {
  constexpr bool SH = R > 1;
  using RC = Rec<D, false, SH>;
  using KR = KeyRec<D>;
  constexpr int NWV = 8;
  constexpr int TPW = C64 / NWV;
  constexpr int KD = D / 32, HM = D / 16;
  constexpr int CPL = D / 64;                 // channels per lane in the conv stage (adjacent)
  constexpr int LQ = D + 8, LT = C64 + 4, LF = C64 + 1, LDT = C64 + 8;
  constexpr int SZ_TOK = C64 * LQ * 2;        // one token-major f16 tile
  constexpr int SZ_AF = C64 * LF * 4;         // one fp32 64 x 64 tile
  constexpr int SZ_RQ = cmax(2 * SZ_TOK, 2 * SZ_AF);                   // q hi|lo, then A | T (fp32)
  constexpr int SZ_RK = cmax(2 * SZ_TOK, cmax(D * LT * 4, C64 * LDT * 2));  // k hi|lo, then v^T, then T (f16)
  constexpr int OFF_RK = SZ_RQ, OFF_G = OFF_RK + SZ_RK;
  constexpr int LDS = OFF_G + 4 * R * C64 * 4;
  static_assert(D == 64 || D == 128, "channel layout");
  static_assert(4 * 16 * 17 * 4 <= C64 * LDT * 2, "level products fit the T tile");
  static_assert(2 * LDS <= 160 * 1024, "two workgroups per CU");
  __shared__ __attribute__((aligned(16))) char smem[LDS];
  _Float16* sQh = (_Float16*)smem;
  _Float16* sQl = sQh + C64 * LQ;
  float* sA = (float*)smem;                    // after the Gram products
  float* sTf = sA + C64 * LF;
  _Float16* sKh = (_Float16*)(smem + OFF_RK);
  _Float16* sKl = sKh + C64 * LQ;
  float* sVt = (float*)(smem + OFF_RK);        // after K~ and the W operand are built
  float* sX = (float*)(smem + OFF_RK);         // level products, after the v operand is built
  _Float16* sT = (_Float16*)(smem + OFF_RK);   // after the levels
  float* sGam = (float*)(smem + OFF_G);
  float* sBet = sGam + R * C64;               // per value head of the group: [r][token]
  float* sEg = sBet + R * C64;
  float* sEd = sEg + R * C64;

  // group vk: value heads vk R .. vk R + R - 1 of key head kh
  const int c = blockIdx.x, vk = blockIdx.y, b = blockIdx.z;
  const int kh = vk * R / (p.n_v / p.n_k);
  const int t0 = c * C64;
  const int len = p.len[b];
  if (t0 >= len) return;  // all padding: the state pass stops before this chunk
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g16 = lane >> 4, r16 = lane & 15;
  mark_sums_pending(p, b, vk, R, t0, tid);
  const int Lb = p.Lb, C = p.C, n_k = p.n_k;
  const ActT* mixed = (const ActT*)p.mixed + (long)b * Lb * C;
  const ActT* tail = (const ActT*)p.tail + (long)b * 3 * C;
  const ActT* cw = (const ActT*)p.conv_w;

  // ---- 1. every global load first: gate inputs (lane = token), conv inputs and taps of q, k and the
  // R value heads (wave w: rows TPW w - 3 .. TPW w + TPW - 1, lane: channels CPL lane + i) ---------
  constexpr int NCV = 2 + R;
  typedef typename std::conditional<CPL == 2, typename Pair<ActT>::type, ActT>::type XRaw;
  typedef typename Raw4<ActT>::type WRaw;
  const int hg = vk * R + (w < R ? w : 0);
  const int tg = t0 + lane;
  const long gi = ((long)b * Lb + (tg < len ? tg : len - 1)) * p.n_v + hg;
  const ActT a_raw = ((const ActT*)p.a)[gi], b_raw = ((const ActT*)p.b)[gi];
  XRaw xr[NCV][TPW + 3];
  WRaw wr[NCV][CPL];
#pragma unroll
  for (int j = 0; j < NCV; ++j) {
    const int gc = (j == 0 ? kh : j == 1 ? n_k + kh : 2 * n_k + vk * R + j - 2) * D + CPL * lane;
#pragma unroll
    for (int i = 0; i < CPL; ++i) wr[j][i] = Raw4<ActT>::load(cw + (gc + i) * 4);
#pragma unroll
    for (int i = 0; i < TPW + 3; ++i) {
      const int t = t0 + TPW * w - 3 + i;
      const ActT* src = t < 0 ? tail + (long)(t + 3) * C : mixed + (long)(t < Lb ? t : Lb - 1) * C;
      if constexpr (CPL == 2) xr[j][i] = Pair<ActT>::load(src + gc);
      else xr[j][i] = src[gc];
    }
  }

  // ---- 2. gates of value head r (wave r, lane = token): inclusive scan of g, the per-token decays ---
  if (w < R) {
    const float g0 = chunk_log_decay(-__expf(p.A_log[hg]) * softplus(to_f32(a_raw) + p.dt_bias[hg]));
    const float b0 = sigmoid(to_f32(b_raw));
    float g = tg < len ? g0 : 0.f;
    const float be = tg < len ? b0 : 0.f;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const float o = __shfl_up(g, off, kWave);
      if (lane >= off) g += o;
    }
    const float gC = __shfl(g, C64 - 1, kWave);
    sGam[w * C64 + lane] = g;
    sBet[w * C64 + lane] = be;
    sEg[w * C64 + lane] = __expf(g);
    sEd[w * C64 + lane] = __expf(gC - g);
  }

  // ---- 3. conv + SiLU (token TPW w + tt, channel CPL lane + i), L2 norms of q and k ---------------
  auto conv = [&](int j, float (*y)[CPL]) {
    float x[TPW + 3][CPL], wt[4][CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const float4 wf = Raw4<ActT>::widen(wr[j][i]);
      wt[0][i] = wf.x; wt[1][i] = wf.y; wt[2][i] = wf.z; wt[3][i] = wf.w;
    }
#pragma unroll
    for (int i = 0; i < TPW + 3; ++i) {
      const bool in = t0 + TPW * w - 3 + i < Lb;
      if constexpr (CPL == 2) {
        const float2 v = Pair<ActT>::widen(xr[j][i]);
        x[i][0] = in ? v.x : 0.f;
        x[i][CPL - 1] = in ? v.y : 0.f;
      } else {
        x[i][0] = in ? to_f32(xr[j][i]) : 0.f;
      }
    }
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
      for (int i = 0; i < CPL; ++i)
        y[tt][i] = silu(wt[0][i] * x[tt][i] + wt[1][i] * x[tt + 1][i] + wt[2][i] * x[tt + 2][i] + wt[3][i] * x[tt + 3][i]);
  };
  auto l2norm = [&](float (*y)[CPL]) {
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < CPL; ++j) ss += y[tt][j] * y[tt][j];
      ss = wave_sum<kWave>(ss);
      const float rn = rsqrt_fast(ss + p.l2_eps);
#pragma unroll
      for (int j = 0; j < CPL; ++j) y[tt][j] *= rn;
    }
  };
  float qn[TPW][CPL], kn[TPW][CPL], vv[R][TPW][CPL];
  conv(0, qn);
  conv(1, kn);
#pragma unroll
  for (int r = 0; r < R; ++r) conv(2 + r, vv[r]);
  l2norm(qn);
  l2norm(kn);
  // token-major 2^8 q and 2^8 k (hi/lo)
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int o = (TPW * w + tt) * LQ + CPL * lane;
    _Float16 qh[CPL], ql[CPL], kh_[CPL], kl[CPL];
    if constexpr (CPL == 2) {
      f16x2 h2, l2;
      split2_f16(kS8 * qn[tt][0], kS8 * qn[tt][1], h2, l2);
      qh[0] = h2[0]; qh[1] = h2[1]; ql[0] = l2[0]; ql[1] = l2[1];
      split2_f16(kS8 * kn[tt][0], kS8 * kn[tt][1], h2, l2);
      kh_[0] = h2[0]; kh_[1] = h2[1]; kl[0] = l2[0]; kl[1] = l2[1];
    } else {
      for (int j = 0; j < CPL; ++j) {
        split_f16(kS8 * qn[tt][j], qh[j], ql[j]);
        split_f16(kS8 * kn[tt][j], kh_[j], kl[j]);
      }
    }
    if constexpr (CPL == 2) {
      *(f16x2*)&sQh[o] = f16x2{qh[0], qh[CPL - 1]};
      *(f16x2*)&sQl[o] = f16x2{ql[0], ql[CPL - 1]};
      *(f16x2*)&sKh[o] = f16x2{kh_[0], kh_[CPL - 1]};
      *(f16x2*)&sKl[o] = f16x2{kl[0], kl[CPL - 1]};
    } else {
      sQh[o] = qh[0]; sQl[o] = ql[0]; sKh[o] = kh_[0]; sKl[o] = kl[0];
    }
  }
  lds_barrier();

  // ---- 4. Gram products (split operands, three accumulators) --------------------------------------
  // D[i][j] = X rows ra0 + i . Y rows rb0 + j over d; lane (g, c) gets i = 4 g + e, j = c
  auto gram = [&](const _Float16* xh, const _Float16* xl, int ra0, const _Float16* yh, const _Float16* yl,
                  int rb0) __attribute__((always_inline)) {
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, a2 = a0;
#pragma unroll
    for (int ks = 0; ks < KD; ++ks) {  // operands one 32-block at a time (registers are the limit here)
      const int ra = (ra0 + r16) * LQ + 32 * ks + 8 * g16, rb = (rb0 + r16) * LQ + 32 * ks + 8 * g16;
      const f16x8 fah = ld16(xh + ra), fal = ld16(xl + ra), fbh = ld16(yh + rb), fbl = ld16(yl + rb);
      a0 = mfma16(fal, fbh, a0);
      a1 = mfma16(fah, fbl, a1);
      a2 = mfma16(fah, fbh, a2);
    }
    return a2 + (a0 + a1);
  };
  // lower 16x16 tiles (mt, nt), nt <= mt, in row order
  auto tile_mt = [](int tile) { return tile >= 6 ? 3 : tile >= 3 ? 2 : tile >= 1 ? 1 : 0; };

  // q: with one value head, Q~ = 2^16 scale e^{gamma_t} q_t into the value record; with several, 2^8 q
  // into the key record (fragment (token tile q & 3, 32-block q >> 2) for q = w, w + 8, ...)
  constexpr int QPW = (4 * KD + NWV - 1) / NWV;
  char* krec = SH ? key_ptr<D>(p, b, vk, c) : nullptr;
  char* rec0 = rec_ptr<D, false, SH>(p, b, vk * R, c);
#pragma unroll
  for (int i = 0; i < QPW; ++i) {
    const int q = w + NWV * i;
    if (q < 4 * KD) {
      const int mt = q & 3, kk = q >> 2;
      const int row = (16 * mt + r16) * LQ + 32 * kk;
      const f16x8 qh = frag_row_h(sQh + row, g16), ql = frag_row_h(sQl + row, g16);
      if constexpr (SH) {
        put_frag<NTS>(krec, KR::Q_HI + mt * KD + kk, lane, qh);
        put_frag<NTS>(krec, KR::Q_LO + mt * KD + kk, lane, ql);
      } else {
        const float fq = kS8 * p.scale * sEg[16 * mt + r16];
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = fq * ((float)qh[e] + (float)ql[e]);
        f16x8 hi, lo;
        split8(x, hi, lo);
        put_frag<NTS>(rec0, RC::Q_HI + mt * KD + kk, lane, hi);
        put_frag<NTS>(rec0, RC::Q_LO + mt * KD + kk, lane, lo);
      }
    }
  }
  // K Q^T tiles of s tiles 2 kk and 2 kk + 1 for the P~ fragment (token tile w & 3, block w >> 2):
  // lane (g, c) of the two accumulators holds exactly that fragment's slots
  const int pmt = w & 3, pkk = w >> 2;
  f32x4 pa = {0.f, 0.f, 0.f, 0.f}, pb = pa;
  if (2 * pkk <= pmt) pa = gram(sKh, sKl, 32 * pkk, sQh, sQl, 16 * pmt);
  if (2 * pkk + 1 <= pmt) pb = gram(sKh, sKl, 32 * pkk + 16, sQh, sQl, 16 * pmt);
  // P~ of every value head: 2^16 scale e^{gamma_t - gamma_s} q_t.k_s for s <= t, else 0
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float* gam = sGam + r * C64;
    const int t = 16 * pmt + r16;
    const float gt = gam[t];
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = pa[e];
      x[4 + e] = pb[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int s = 32 * pkk + kslot(g16, e);
      x[e] = s <= t ? p.scale * __expf(gt - gam[s]) * x[e] : 0.f;
    }
    f16x8 hi, lo;
    split8(x, hi, lo);
    char* rec = rec_ptr<D, false, SH>(p, b, vk * R + r, c);
    put_frag<NTS>(rec, RC::P_HI + pmt * 2 + pkk, lane, hi);
    put_frag<NTS>(rec, RC::P_LO + pmt * 2 + pkk, lane, lo);
  }
  // K K^T tiles, two for the waves without K Q^T tiles: waves 0-3 tiles 0-3, 4: 4-5, 5: 6-7, 6: 8, 7: 9
  const int kt0 = w < 4 ? w : w == 4 ? 4 : w == 5 ? 6 : w + 2;
  const bool two = w == 4 || w == 5;
  f32x4 kka, kkb = {0.f, 0.f, 0.f, 0.f};
  {
    const int mt = tile_mt(kt0), nt = kt0 - mt * (mt + 1) / 2;
    kka = gram(sKh, sKl, 16 * mt, sKh, sKl, 16 * nt);
  }
  if (two) {
    const int mt = tile_mt(kt0 + 1), nt = kt0 + 1 - mt * (mt + 1) / 2;
    kkb = gram(sKh, sKl, 16 * mt, sKh, sKl, 16 * nt);
  }
  lds_barrier();  // q is dead

  // ---- 5. k^T fragments from token-major k: K~ (one value head) or the key record's k; W operands --
  // slots s of this lane for d = 16 hm + r16, hi and lo as staged
  auto k_col = [&](int hm, int kk, f16x8& hi, f16x8& lo) __attribute__((always_inline)) {
    const int d = 16 * hm + r16;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int s = 32 * kk + kslot(g16, e);
      hi[e] = sKh[s * LQ + d];
      lo[e] = sKl[s * LQ + d];
    }
  };
  for (int idx = w; idx < 2 * HM; idx += NWV) {
    const int hm = idx >> 1, kk = idx & 1;
    f16x8 hi, lo;
    k_col(hm, kk, hi, lo);
    if constexpr (SH) {
      put_frag<NTS>(krec, KR::K_HI + hm * 2 + kk, lane, hi);
      put_frag<NTS>(krec, KR::K_LO + hm * 2 + kk, lane, lo);
    } else {  // K~^T: 2^8 e^{gamma_C - gamma_s} k_s
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = sEd[32 * kk + kslot(g16, e)] * ((float)hi[e] + (float)lo[e]);
      split8(x, hi, lo);
      put_frag<NTS>(rec0, RC::K_HI + hm * 2 + kk, lane, hi);
      put_frag<NTS>(rec0, RC::K_LO + hm * 2 + kk, lane, lo);
    }
  }
  // the W operand of wave w (d tile w) for every value head: 2^8 beta_s e^{gamma_s} k_s as f16
  f16x8 kb[R][2];
  if (w < HM) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      f16x8 hi, lo;
      k_col(w, ks, hi, lo);
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int s = r * C64 + 32 * ks + kslot(g16, e);
          kb[r][ks][e] = (_Float16)(sBet[s] * sEg[s] * ((float)hi[e] + (float)lo[e]));
        }
    }
  }
  lds_barrier();  // k is dead

  // ---- 6. per value head of the group ------------------------------------------------------------
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float* gam = sGam + r * C64;
    const float* bet = sBet + r * C64;
    char* rec = rec_ptr<D, false, SH>(p, b, vk * R + r, c);
    // A (strictly lower, fp32) from the K K^T accumulators, into the q region
    auto put_A = [&](int tile, f32x4 acc) __attribute__((always_inline)) {
      const int mt = tile_mt(tile), nt = tile - mt * (mt + 1) / 2;
      const int j = 16 * nt + r16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * mt + 4 * g16 + e;
        if (j < i) sA[i * LF + j] = bet[i] * __expf(gam[i] - gam[j]) * (kInvS16 * acc[e]);
      }
    };
    put_A(kt0, kka);
    if (two) put_A(kt0 + 1, kkb);
    // with a key record: the per-token decays the state pass applies
    if (SH && tid < C64) {
      *(float*)(rec + RC::kEg + 4 * tid) = kS8 * p.scale * sEg[r * C64 + tid];
      *(float*)(rec + RC::kEd + 4 * tid) = sEd[r * C64 + tid];
    }
    // v of this head channel-major, into the k region
#pragma unroll
    for (int j = 0; j < CPL; ++j)
#pragma unroll
      for (int q = 0; q < TPW / 4; ++q)
        *(float4*)&sVt[(CPL * lane + j) * LT + TPW * w + 4 * q] =
            make_float4(vv[r][4 * q][j], vv[r][4 * q + 1][j], vv[r][4 * q + 2][j], vv[r][4 * q + 3][j]);
    lds_barrier();

    // T's diagonal blocks by forward substitution (wave 0, one column per lane); the U' operand of
    // wave w (value tile w): 2^8 beta_s v_s, hi/lo
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
    f16x8 vh[2], vl[2];
    if (w < HM) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        float x[8];
        frag_row_f(sVt + (16 * w + r16) * LT + 32 * ks, g16, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= kS8 * bet[32 * ks + kslot(g16, e)];
        split8(x, vh[ks], vl[ks]);
      }
    }
    lds_barrier();  // v^T is dead: the level products go into its region

    // T's off-diagonal blocks by level (i - j = 1, 2, 3): T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj
    for (int lvl = 1; lvl < 4; ++lvl) {
      if (w < 4 - lvl) {
        float* sXw = sX + w * 16 * 17;
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
      lds_barrier();
    }
    for (int idx = tid; idx < C64 * C64; idx += 64 * NWV) {
      const int i = idx >> 6, j = idx & 63;
      sT[i * LDT + j] = (_Float16)((j >> 4) > (i >> 4) ? 0.f : kS8 * sTf[i * LF + j]);  // upper blocks are zero
    }
    lds_barrier();

    // W^T = (beta e^gamma K)^T T^T (d tile w) and U' = T (beta V) (value tile w), one token tile mt at
    // a time (the operands of the next value head are live here too)
    if (w < HM) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f16x8 th[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) th[ks] = frag_row_h(sT + (16 * mt + r16) * LDT + 32 * ks, g16);
        // W^T tile (w, mt) = 2^16 W^T (stored as 2^8 -W); lane (g, c) holds W[16 mt + c][16 w + 4 g + i], half (w & 1)
        // of the fragment of block w >> 1
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) acc = mfma16(kb[r][ks], th[ks], acc);
        f16x4 hi, lo;
        split4(acc * -kInvS8, hi, lo);
        st_rec<NTS>((f16x4*)(rec + (RC::W_HI + mt * KD + (w >> 1)) * 1024 + (uint32_t)(lane * 16 + 8 * (w & 1))), hi);
        // U' tile (mt, w) = (2^8 T)(2^8 beta V) = 2^16 U', stored as is
        f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          a0 = mfma16(th[ks], vl[ks], a0);
          a1 = mfma16(th[ks], vh[ks], a1);
        }
        st_rec<NTS>((f32x4*)(rec + (RC::UP + mt * HM + w) * 1024 + (uint32_t)(lane * 16)), a1 + a0);
      }
    }
    if (tid == 0) *(float*)(rec + RC::kGc) = __expf(gam[C64 - 1]);
    if (r + 1 < R) lds_barrier();  // T of this head is read; A, T and v of the next head overwrite it
  }
}

// -------------------------------------------------------------------------------------------------
// State pass: 8 waves, a slice of CS = 16 NT value columns of one head. Wave w works on token tile
// w & 3 and owns H row tile w (when w < d_k/16). Waves 0-3 carry the chain: U = U' - W H for their
// token tile. Waves 4-7 carry the output: O^T = H^T Q~^T + U^T P~^T for their token tile. Every wave
// then updates its own H row tile, H = e^{gamma_C} H + K~^T U. Each SIMD runs one chain wave and one
// output wave, so the output work fills the gaps of the chain.
//
// Each wave's fragments of a chunk are loaded straight into registers. Memory latency is longer than
// one chunk of work, so with DB the loop is unrolled by two over two register sets and the loads run
// two chunks ahead: each fragment of chunk c is refilled with chunk c+2 right after its last use.
// The two roles keep separate fragment sets (and run separate copies of the chunk loop), so that the
// registers of one role are never live in the other's code.
template <int KD, int NT, bool SPLIT, typename RawZ>
struct ChainFrags {
  f16x8 w[KD], wl[SPLIT ? KD : 1];  // -W of the token tile
  f32x4 up[NT];                     // U' of the token tile, this slice
  f16x8 k[2], kl[2];                // K~^T of the own H tile
  float gc;                         // e^{gamma_C}
  f32x4 ed;                         // with a key record: e^{gamma_C - gamma_t} of this lane's U rows
  RawZ z[NT];                       // split head: z of the token tile, handed to the output wave
};
template <int KD, int NT, typename RawZ, int NS>
struct OutFrags {
  f16x8 q[KD], ql[KD];              // Q~ of the token tile
  f16x8 p[2], pl[2];                // P~ of the token tile
  f16x8 k[2], kl[2];                // K~^T of the own H tile
  float gc;                         // e^{gamma_C}
  float eg;                         // with a key record: scale e^{gamma_t} of this lane's token
  RawZ z[NT];                       // z of the token tile (gated norm)
  float sums[NS];                   // split head: a pair of the slices' row sums of an earlier chunk, in flight
};

// how the gated RMSNorm of a row is finished: in the epilogue (one workgroup owns the head), by the
// slices' exchange of row sums, or by norm_kernel from the saved unnormalised o and partial sums
constexpr int kNormFused = 0, kNormExchange = 1, kNormPass = 2;

template <typename ActT, int D, int NT, bool SPLIT, int NM, bool DB, bool SH>
__global__ __launch_bounds__(512) void state_pass_kernel(PrefillArgs p) {
  constexpr bool FUSED = NM == kNormFused, XCH = NM == kNormExchange;
  using RC = Rec<D, SPLIT, SH>;
  using KR = KeyRec<D>;
  constexpr int KD = D / 32, HM = D / 16, CS = 16 * NT, NSPLIT = D / CS;
  constexpr int NG = (NT == 2 || NT == 4) ? 2 : 1;  // column tiles per MFMA group (registers cap NT = 8 at 1)
  static_assert(NSPLIT * CS == D, "column split");
  static_assert(HM <= 8, "one H row tile per wave");
  static_assert(FUSED == (NSPLIT == 1), "FUSED: one workgroup owns every column of the head");
  static_assert(NSPLIT == 1 || NSPLIT % 2 == 0, "row sums are read in pairs");
  static_assert(!XCH || (DB && (NT == 2 || NT == 4)), "the row-sum exchange: 32- or 64-column slices, two fragment sets");
  // row-sum exchange: the rows of chunk c are normalised at the end of chunk c + kDelay. With 32
  // columns the row sums are loaded at the start of chunk c + 2 into the fragment set of that chunk
  // and used a whole chunk later (the uncached round trip is longer than one chunk); with 64 columns,
  // where registers are scarce, they are loaded after the state update of chunk c + 2 and used at its
  // end.
  constexpr bool kDeep = NT == 2;
  constexpr int kDelay = kDeep ? 3 : 2, kRing = kDelay + 1;
  typedef typename Raw4<ActT>::type RawZ;
  typedef ChainFrags<KD, NT, SPLIT, RawZ> CF;
  typedef OutFrags<KD, NT, RawZ, 2> OF;
  // H and U as MFMA operand fragments: [32-block][nt][hi, lo][lane], 16 bytes each
  __shared__ f16x8 sH[KD * NT * 2 * kWave];
  __shared__ f16x8 sU[2 * NT * 2 * kWave];
  __shared__ f16x8 sUd[SH ? 2 * NT * 2 * kWave : 1];  // with a key record: diag(e^{gamma_C - gamma}) U

  // workgroups of one head run on one XCD (dispatch goes round-robin over the 8 XCDs), so that the
  // record of a chunk is fetched from HBM once and shared through that XCD's L2
  const int nblk = gridDim.x, bid = blockIdx.x;
  const int lid = (nblk & 7) == 0 ? (bid & 7) * (nblk >> 3) + (bid >> 3) : bid;
  const int split = lid % NSPLIT, hb = lid / NSPLIT;
  const int h = hb % p.n_v, b = hb / p.n_v;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: record addresses stay scalar
  const int tt = w & 3;                      // token tile
  const bool chain = w < 4;                  // chain wave (U) or output wave (O)
  const bool owner = w < HM;                 // owns H row tile w
  const int g16 = lane >> 4, r16 = lane & 15;
  const int Lb = p.Lb, n_v = p.n_v, C = p.C;
  const int len = p.len[b];
  const int n_real = (len + C64 - 1) / C64;
  const int cb = split * CS;

  // single fragments of chunk c (past the end: the last chunk, loaded and unused, branch-free)
  auto rec_of = [&](int c) { return (const char*)rec_ptr<D, SPLIT, SH>(p, b, h, c < n_real ? c : n_real - 1); };
  auto key_of = [&](int c) { return (const char*)key_ptr<D>(p, b, h / p.grp, c < n_real ? c : n_real - 1); };
  auto ld_w = [&](CF& f, int c, int kk) __attribute__((always_inline)) {
    const char* rec = rec_of(c);
    f.w[kk] = get_frag(rec, RC::W_HI + tt * KD + kk, lane);
    if (SPLIT) f.wl[kk] = get_frag(rec, RC::W_LO + tt * KD + kk, lane);
  };
  auto ld_q = [&](OF& f, int c, int kk) __attribute__((always_inline)) {
    if constexpr (SH) {
      const char* rec = key_of(c);
      f.q[kk] = get_frag(rec, KR::Q_HI + tt * KD + kk, lane);
      f.ql[kk] = get_frag(rec, KR::Q_LO + tt * KD + kk, lane);
    } else {
      const char* rec = rec_of(c);
      f.q[kk] = get_frag(rec, RC::Q_HI + tt * KD + kk, lane);
      f.ql[kk] = get_frag(rec, RC::Q_LO + tt * KD + kk, lane);
    }
  };
  auto ld_up = [&](CF& f, int c, int nt) __attribute__((always_inline)) {
    f.up[nt] = *(const f32x4*)(rec_of(c) + (RC::UP + tt * HM + cb / 16 + nt) * 1024 + (uint32_t)(lane * 16));
  };
  auto ld_p = [&](OF& f, int c, int kk) __attribute__((always_inline)) {
    const char* rec = rec_of(c);
    f.p[kk] = get_frag(rec, RC::P_HI + tt * 2 + kk, lane);
    f.pl[kk] = get_frag(rec, RC::P_LO + tt * 2 + kk, lane);
  };
  auto ld_k = [&](auto& f, int c, int kk) __attribute__((always_inline)) {
    const int hm = owner ? w : 0;  // a wave without a tile loads tile 0 and ignores it
    if constexpr (SH) {
      const char* rec = key_of(c);
      f.k[kk] = get_frag(rec, KR::K_HI + hm * 2 + kk, lane);
      f.kl[kk] = get_frag(rec, KR::K_LO + hm * 2 + kk, lane);
    } else {
      const char* rec = rec_of(c);
      f.k[kk] = get_frag(rec, RC::K_HI + hm * 2 + kk, lane);
      f.kl[kk] = get_frag(rec, RC::K_LO + hm * 2 + kk, lane);
    }
  };
  auto ld_gc = [&](auto& f, int c) __attribute__((always_inline)) { f.gc = *(const float*)(rec_of(c) + RC::kGc); };
  // the per-token decays of a record with a key record: rows 16 tt + 4 g16 + i of U (chain), token
  // 16 tt + r16 of O (output)
  auto ld_ed = [&](CF& f, int c) __attribute__((always_inline)) {
    if constexpr (SH) f.ed = *(const f32x4*)(rec_of(c) + RC::kEd + 4 * (16 * tt + 4 * g16));
  };
  auto ld_eg = [&](OF& f, int c) __attribute__((always_inline)) {
    if constexpr (SH) f.eg = *(const float*)(rec_of(c) + RC::kEg + 4 * (16 * tt + r16));
  };
  // z of token 16 tt + r16, columns cb + 16 nt + 4 g16 .. +3: loaded by the output wave when one
  // workgroup owns the head, by the chain wave of the token tile (registers to spare) when it is split
  auto ld_z = [&](auto& f, int c) __attribute__((always_inline)) {
    {
      const int cc = c < n_real ? c : n_real - 1;
      const int t = cc * C64 + 16 * tt + r16;  // rows past Lb read row Lb-1; their results are never stored
      const long row = ((long)b * Lb + (t < Lb ? t : Lb - 1)) * n_v + h;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) f.z[nt] = Raw4<ActT>::load((const ActT*)p.z + row * D + cb + 16 * nt + 4 * g16);
    }
  };
  auto load_all = [&](auto& f, int c) __attribute__((always_inline)) {
    if constexpr (std::is_same<std::decay_t<decltype(f)>, CF>::value) {
#pragma unroll
      for (int kk = 0; kk < KD; ++kk) ld_w(f, c, kk);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) ld_up(f, c, nt);
      ld_ed(f, c);
      if (XCH) ld_z(f, c);
    } else {
#pragma unroll
      for (int kk = 0; kk < KD; ++kk) ld_q(f, c, kk);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) ld_p(f, c, kk);
      ld_eg(f, c);
      if (FUSED) ld_z(f, c);
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) ld_k(f, c, kk);
    ld_gc(f, c);
  };

  // ---- the state: 2^16 H of row tile w, columns cb + 16 nt + r16 ----
  float* st = p.state + ((long)b * n_v + h) * D * D;
  f32x4 Hacc[NT];
  {
    const int hl = owner ? w : 0;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = st[(long)(16 * hl + 4 * g16 + i) * D + cb + 16 * nt + r16];
        Hacc[nt][i] = owner ? 65536.f * v : 0.f;
      }
  }
  // 2^8 H hi/lo into its fragment slots: tile w is half (w & 1) of 32-block w >> 1
  auto put_H = [&]() __attribute__((always_inline)) {
    if (owner) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f16x4 hi, lo;
        split4(Hacc[nt] * kInvS8, hi, lo);
        _Float16* dst = (_Float16*)&sH[(((w >> 1) * NT + nt) * 2) * kWave + lane] + 4 * (w & 1);
        *(f16x4*)dst = hi;
        *(f16x4*)(dst + 8 * kWave) = lo;
      }
    }
  };
  put_H();

  // the norm weights of this slice, read from LDS in the epilogue (registers are the scarce resource)
  __shared__ __attribute__((aligned(16))) float sNW[CS];
  if (tid < CS) sNW[tid] = p.norm_w[cb + tid];
  // split head: w o silu(z) of the last kRing chunks, [chunk % kRing][token tile][nt][lane], until
  // the row's 1/rms is known; z of the last two chunks from the chain waves, [chunk & 1][token tile][nt][lane]
  __shared__ float4 sY[XCH ? kRing * 4 * NT * kWave : 1];
  __shared__ RawZ sZ[XCH ? 2 * 4 * NT * kWave : 1];

  float* sspart = (float*)((char*)p.ws + p.ss_off);
  float* oraw = (float*)((char*)p.ws + p.oraw_off);

  // row-sum exchange: the partial sums of squares that every slice posted for the row of token
  // 16 tt + r16 of chunk cc, [sequence][head][token][slice], read past the caches (agent scope: the
  // slices may sit on different L2s). Lane group g16 loads pair g16 % NP of its row's sums, so a wave
  // reads 16 consecutive rows in one contiguous sweep; finish_rows combines the groups' pairs.
  constexpr int NP = NSPLIT > 1 ? NSPLIT / 2 : 1;
  float* ssrow = sspart + ((long)b * n_v + h) * Lb * NSPLIT;  // this head's rows
  auto load_sums = [&](int cc, float (&sums)[2]) __attribute__((always_inline)) {
    // unconditional (a row past Lb reads row Lb - 1 and is ignored), so that nothing waits here
    const int t = cc * C64 + 16 * tt + r16;
    const uint64_t* src = (const uint64_t*)(ssrow + (long)(t < Lb ? t : Lb - 1) * NSPLIT) + (g16 % NP);
    const uint64_t u = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sums[0] = __uint_as_float((uint32_t)u);
    sums[1] = __uint_as_float((uint32_t)(u >> 32));
  };
  // scale this slice's w o silu(z) of the row by 1/rms and store it. A slice posts chunk c before it
  // waits for chunk c - kDelay and every slice of the head is resident, so a sum still pending
  // arrives; the time bound only guarantees that the kernel ends even if that were not so.
  auto finish_rows = [&](int cc, const float (&in)[2]) __attribute__((always_inline)) {
    const int t = cc * C64 + 16 * tt + r16;
    float sums[2] = {in[0], in[1]};  // a copy: re-reading into the fragment set kept it out of registers
    // the row's total over every slice and whether one is still pending, in all four lane groups
    auto combine = [&](float& tot) __attribute__((always_inline)) {
      tot = sums[0] + sums[1];
      int pend = (sums[0] == kSsPending || sums[1] == kSsPending) ? 1 : 0;
#pragma unroll
      for (int m = 1; m < NP; m *= 2) {
        tot += __shfl_xor(tot, 16 * m, kWave);
        pend |= __shfl_xor(pend, 16 * m, kWave);
      }
      return pend == 0 || t >= Lb;
    };
    float tot;
    bool ready = combine(tot);
    if (!__all(ready)) {
      const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
      do {
        __builtin_amdgcn_s_sleep(2);
        load_sums(cc, sums);
        ready = combine(tot);
      } while (!__all(ready) && __builtin_amdgcn_s_memrealtime() - t_start < kSpinTicks);
    }
    // a row whose sums never all arrived (the bound expired: a slice of the head was not running) is
    // written as NaN and reported through the device status word, never normalised with a missing sum
    float inv = rsqrt_fast(tot / p.rms_n + p.rms_eps);
    if (!ready) inv = __builtin_nanf("");
    if (p.status && !__all(ready) && lane == 0) atomicOr(p.status, 2);
    const long row = ((long)b * Lb + t) * n_v + h;
    if (t < Lb) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float4 y = sY[(((cc % kRing) * 4 + tt) * NT + nt) * kWave + lane];
        store_out4<ActT>(p, row * D + cb + 16 * nt + 4 * g16, make_float4(y.x * inv, y.y * inv, y.z * inv, y.w * inv));
      }
    }
  };

  // f: the fragment set of chunk c; g: the other set (split heads, output waves: its row sums, loaded
  // at the start of chunk c - 1, are those of chunk c - 3)
  auto chunk = [&](int c, auto& f, auto& g, int step) __attribute__((always_inline)) {
    constexpr bool kChain = std::is_same<std::decay_t<decltype(f)>, CF>::value;
    const int cn = c + step;  // the chunk whose fragments refill f
    f32x4 OT[NT];
    // split head, output waves: the row sums of chunk c - 2 (a spill of these with 64 columns would be
    // reloaded behind the whole queue of fragment prefetches, hence the later load there)
    float sums[2];
    if constexpr (!kChain && XCH && kDeep) {
      if (c >= 2) load_sums(c - 2, f.sums);
    }
    lds_barrier();  // H of this chunk is in sH
    if constexpr (kChain) {
      // ---- 2^8 U = 2^-8 (2^16 U' + (2^8 -W)(2^8 H)) (token tile tt); hi*lo and hi*hi terms apart ----
      f32x4 U[NT];
#pragma unroll
      for (int n0 = 0; n0 < NT; n0 += NG) {
        f16x8 hf[KD][NG], hl[KD][NG];
#pragma unroll
        for (int kk = 0; kk < KD; ++kk)
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            hf[kk][g] = sH[((kk * NT + n0 + g) * 2) * kWave + lane];
            hl[kk][g] = sH[((kk * NT + n0 + g) * 2 + 1) * kWave + lane];
          }
        f32x4 ua[NG], ub[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          ua[g] = f.up[n0 + g];
          ub[g] = f32x4{0.f, 0.f, 0.f, 0.f};
          ld_up(f, cn, n0 + g);
        }
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) {
#pragma unroll
          for (int g = 0; g < NG; ++g) ua[g] = mfma16(f.w[kk], hl[kk][g], ua[g]);
#pragma unroll
          for (int g = 0; g < NG; ++g) ub[g] = mfma16(f.w[kk], hf[kk][g], ub[g]);
          if (SPLIT) {
#pragma unroll
            for (int g = 0; g < NG; ++g) ua[g] = mfma16(f.wl[kk], hf[kk][g], ua[g]);
          }
          if (n0 + NG >= NT) ld_w(f, cn, kk);  // last use of this block's W in the chunk
        }
#pragma unroll
        for (int g = 0; g < NG; ++g) U[n0 + g] = (ua[g] + ub[g]) * kInvS8;
      }
      // U hi/lo into its fragment slots: token tile tt is half (tt & 1) of 32-block tt >> 1 (and, with a
      // key record, the decayed U the state update takes)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f16x4 hi, lo;
        split4(U[nt], hi, lo);
        const int slot = (((tt >> 1) * NT + nt) * 2) * kWave + lane;
        _Float16* dst = (_Float16*)&sU[slot] + 4 * (tt & 1);
        *(f16x4*)dst = hi;
        *(f16x4*)(dst + 8 * kWave) = lo;
        if constexpr (SH) {
          split4(U[nt] * f.ed, hi, lo);
          _Float16* dd = (_Float16*)&sUd[slot] + 4 * (tt & 1);
          *(f16x4*)dd = hi;
          *(f16x4*)(dd + 8 * kWave) = lo;
        }
      }
      ld_ed(f, cn);
      if constexpr (XCH) {  // read by the output wave of the token tile after the next barrier
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sZ[(((c & 1) * 4 + tt) * NT + nt) * kWave + lane] = f.z[nt];
        ld_z(f, cn);
      }
    } else {
      // ---- O^T = H^T Q~^T (token tile tt) ----
#pragma unroll
      for (int n0 = 0; n0 < NT; n0 += NG) {
        f16x8 hf[KD][NG], hl[KD][NG];
#pragma unroll
        for (int kk = 0; kk < KD; ++kk)
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            hf[kk][g] = sH[((kk * NT + n0 + g) * 2) * kWave + lane];
            hl[kk][g] = sH[((kk * NT + n0 + g) * 2 + 1) * kWave + lane];
          }
        f32x4 oa[NG], ob[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) oa[g] = ob[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) {
#pragma unroll
          for (int g = 0; g < NG; ++g) oa[g] = mfma16(hf[kk][g], f.ql[kk], oa[g]);
#pragma unroll
          for (int g = 0; g < NG; ++g) ob[g] = mfma16(hf[kk][g], f.q[kk], ob[g]);
#pragma unroll
          for (int g = 0; g < NG; ++g) oa[g] = mfma16(hl[kk][g], f.q[kk], oa[g]);
          if (n0 + NG >= NT) ld_q(f, cn, kk);  // last use of this block's Q~ in the chunk
        }
#pragma unroll
        for (int g = 0; g < NG; ++g) OT[n0 + g] = SH ? (oa[g] + ob[g]) * f.eg : oa[g] + ob[g];
      }
      ld_eg(f, cn);
    }
    lds_barrier();  // U of every token tile is in sU; every wave is done reading sH
    // ---- own H tile: H = e^{gamma_C} H + K~^T U; output waves also O^T += U^T P~^T ----
    if constexpr (!SH) {
      // both products read the same U fragments: interleaved, so that the MFMA pipe stays full
#pragma unroll
      for (int n0 = 0; n0 < NT; n0 += NG) {
        f16x8 uf[2][NG], ul[2][NG];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            uf[kk][g] = sU[((kk * NT + n0 + g) * 2) * kWave + lane];
            ul[kk][g] = sU[((kk * NT + n0 + g) * 2 + 1) * kWave + lane];
          }
#pragma unroll
        for (int g = 0; g < NG; ++g) Hacc[n0 + g] = Hacc[n0 + g] * f.gc;
        if (n0 + NG >= NT) ld_gc(f, cn);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
          for (int term = 0; term < 3; ++term) {
            if (owner) {
#pragma unroll
              for (int g = 0; g < NG; ++g) {
                const f16x8 ka = term == 0 ? f.kl[kk] : f.k[kk];
                const f16x8 ub = term == 1 ? ul[kk][g] : uf[kk][g];
                Hacc[n0 + g] = mfma16(ka, ub, Hacc[n0 + g]);
              }
            }
            if constexpr (!kChain) {
#pragma unroll
              for (int g = 0; g < NG; ++g) {
                const f16x8 ua = term == 1 ? ul[kk][g] : uf[kk][g];
                const f16x8 pb = term == 0 ? f.pl[kk] : f.p[kk];
                OT[n0 + g] = mfma16(ua, pb, OT[n0 + g]);
              }
            }
          }
          if (n0 + NG >= NT) {  // last use of this block's K~ (and P~) in the chunk
            ld_k(f, cn, kk);
            if constexpr (!kChain) ld_p(f, cn, kk);
          }
        }
      }
    } else {
      // the state update takes the decayed U, O^T the plain one: one after the other, so that only one
      // set of U fragments is held at a time
#pragma unroll
      for (int n0 = 0; n0 < NT; n0 += NG) {
        f16x8 df[2][NG], dl[2][NG];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            df[kk][g] = sUd[((kk * NT + n0 + g) * 2) * kWave + lane];
            dl[kk][g] = sUd[((kk * NT + n0 + g) * 2 + 1) * kWave + lane];
          }
#pragma unroll
        for (int g = 0; g < NG; ++g) Hacc[n0 + g] = Hacc[n0 + g] * f.gc;
        if (n0 + NG >= NT) ld_gc(f, cn);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          if (owner) {
#pragma unroll
            for (int term = 0; term < 3; ++term)
#pragma unroll
              for (int g = 0; g < NG; ++g)
                Hacc[n0 + g] = mfma16(term == 0 ? f.kl[kk] : f.k[kk], term == 1 ? dl[kk][g] : df[kk][g], Hacc[n0 + g]);
          }
          if (n0 + NG >= NT) ld_k(f, cn, kk);  // last use of this block's K in the chunk
        }
      }
      if constexpr (!kChain) {
#pragma unroll
        for (int n0 = 0; n0 < NT; n0 += NG) {
          f16x8 uf[2][NG], ul[2][NG];
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int g = 0; g < NG; ++g) {
              uf[kk][g] = sU[((kk * NT + n0 + g) * 2) * kWave + lane];
              ul[kk][g] = sU[((kk * NT + n0 + g) * 2 + 1) * kWave + lane];
            }
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int term = 0; term < 3; ++term)
#pragma unroll
              for (int g = 0; g < NG; ++g)
                OT[n0 + g] = mfma16(term == 1 ? ul[kk][g] : uf[kk][g], term == 0 ? f.pl[kk] : f.p[kk], OT[n0 + g]);
            if (n0 + NG >= NT) ld_p(f, cn, kk);  // last use of this block's P~ in the chunk
          }
        }
      }
    }
    if constexpr (!kChain && XCH && !kDeep) {
      if (c >= 2) load_sums(c - 2, sums);
    }
    put_H();

    // ---- output waves: token 16 tt + r16, columns cb + 16 nt + 4 g16 + i ----
    if constexpr (!kChain) {
      float ss = 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        OT[nt] = OT[nt] * kInvS24;
#pragma unroll
        for (int i = 0; i < 4; ++i) ss += OT[nt][i] * OT[nt][i];
      }
      ss += __shfl_xor(ss, 16, kWave);
      ss += __shfl_xor(ss, 32, kWave);
      const int t = c * C64 + 16 * tt + r16;
      const long row = ((long)b * Lb + t) * n_v + h;
      if constexpr (FUSED) {
        const float inv = rsqrt_fast(ss / p.rms_n + p.rms_eps);
        float4 res[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const float4 zf = Raw4<ActT>::widen(f.z[nt]);
          const float4 nw = *(const float4*)&sNW[16 * nt + 4 * g16];
          res[nt] = make_float4(nw.x * (OT[nt][0] * inv) * silu(zf.x), nw.y * (OT[nt][1] * inv) * silu(zf.y),
                                nw.z * (OT[nt][2] * inv) * silu(zf.z), nw.w * (OT[nt][3] * inv) * silu(zf.w));
        }
        ld_z(f, cn);
        if (t < Lb) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) store_out4<ActT>(p, row * D + cb + 16 * nt + 4 * g16, res[nt]);
        }
      } else if constexpr (XCH) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const float4 zf = Raw4<ActT>::widen(sZ[(((c & 1) * 4 + tt) * NT + nt) * kWave + lane]);
          const float4 nw = *(const float4*)&sNW[16 * nt + 4 * g16];
          sY[((((c % kRing) * 4 + tt) * NT + nt) * kWave) + lane] =
              make_float4(nw.x * OT[nt][0] * silu(zf.x), nw.y * OT[nt][1] * silu(zf.y),
                          nw.z * OT[nt][2] * silu(zf.z), nw.w * OT[nt][3] * silu(zf.w));
        }
        if (t < Lb && g16 == 0)
          __hip_atomic_store(ssrow + (long)t * NSPLIT + split, ss, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if constexpr (kDeep) {
          if (c >= 3) finish_rows(c - 3, g.sums);
        } else {
          if (c >= 2) finish_rows(c - 2, sums);
        }
      } else if (t < Lb) {  // norm pass: this slice's sum of squares ([sequence][token][head][slice]) and o
        if (g16 == 0) sspart[row * NSPLIT + split] = ss;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          *(float4*)(oraw + row * D + cb + 16 * nt + 4 * g16) = make_float4(OT[nt][0], OT[nt][1], OT[nt][2], OT[nt][3]);
      }
    }
  };

  // every wave runs the same number of chunks and barriers, whichever copy of the loop it is in
  auto run = [&](auto& f0, auto& f1) __attribute__((always_inline)) {
    if constexpr (DB) {
      load_all(f0, 0);
      load_all(f1, 1);
      // the loop body has no branch, so the compiler can count the loads still in flight at its top
      // (a conditional second chunk made it wait for all of them)
      int c = 0;
      for (; c + 1 < n_real; c += 2) {
        chunk(c, f0, f1, 2);
        chunk(c + 1, f1, f0, 2);
      }
      if (c < n_real) chunk(c, f0, f1, 2);
    } else {
      load_all(f0, 0);
      for (int c = 0; c < n_real; ++c) chunk(c, f0, f0, 1);
    }
  };
  if (n_real > 0) {
    if (chain) {
      CF f0, f1;
      run(f0, f1);
    } else {
      OF f0, f1;
      run(f0, f1);
      if constexpr (XCH) {  // the rows of the last kDelay chunks: every load in flight before the first use
        static_assert(kDelay <= 3, "tail");
        const int c0 = n_real > kDelay ? n_real - kDelay : 0;
        float s0[2], s1[2], s2[2];
        load_sums(c0, s0);  // a chunk past the end reads valid rows and is not used
        load_sums(c0 + 1, s1);
        if constexpr (kDelay == 3) load_sums(c0 + 2, s2);
        finish_rows(c0, s0);
        if (c0 + 1 < n_real) finish_rows(c0 + 1, s1);
        if constexpr (kDelay == 3) {
          if (c0 + 2 < n_real) finish_rows(c0 + 2, s2);
        }
      }
    }
  }

  // final state, in place; a value outside the range of the 2^8-scaled f16 operand pairs (or not finite)
  // raises the range bit of the device status word
  if (owner) {
    bool bad = false;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = Hacc[nt][i] * kInvS16;
        bad |= !(fabsf(v) < 255.f);
        st[(long)(16 * w + 4 * g16 + i) * D + cb + 16 * nt + r16] = v;
      }
    if (p.status && __any(bad) && lane == 0) atomicOr(p.status, 1);
  }

  // conv tail: rows len .. len+2 of [old tail | mixed]. Split 0 of value head h owns its v channels;
  // split 0 of the first value head of each GQA group also the q and k channels of its key head.
  if (split == 0) {
    const int R = n_v / p.n_k;
    ActT* tl = (ActT*)p.tail + (long)b * 3 * C;
    const ActT* mx = (const ActT*)p.mixed + (long)b * Lb * C;
    const int kh = h / R;
    const int nch = (h % R == 0) ? 3 * D : D;
    for (int lc = tid; lc < nch; lc += 512) {
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

// the gated RMSNorm when a head's columns were split and the state pass left the rows unnormalised:
// out = w * o / rms(o) * silu(z), one thread per 4 columns of one (sequence, token, head) row; the
// slices' partial sums of a row are adjacent, [sequence][token][head][slice]; rows past len are left
// alone
template <typename ActT, int D, int NPART>
__global__ __launch_bounds__(256) void norm_kernel(PrefillArgs p) {
  constexpr int Q = D / 4;
  const float* oraw = (const float*)((const char*)p.ws + p.oraw_off);
  const float* sspart = (const float*)((const char*)p.ws + p.ss_off);
  const int b = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int rr = i / Q, cq = i % Q;
  if (rr >= p.len[b] * p.n_v) return;
  const long row = (long)b * p.Lb * p.n_v + rr;
  const float* sp = sspart + row * NPART;
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < NPART; ++k) ss += sp[k];
  const float inv = rsqrt_fast(ss / p.rms_n + p.rms_eps);
  const float4 o = *(const float4*)(oraw + row * D + 4 * cq);
  const float4 z = Act4<ActT>::load((const ActT*)p.z + row * D + 4 * cq);
  const float4 nw = *(const float4*)(p.norm_w + 4 * cq);
  const float4 v = make_float4(nw.x * (o.x * inv) * silu(z.x), nw.y * (o.y * inv) * silu(z.y),
                               nw.z * (o.z * inv) * silu(z.z), nw.w * (o.w * inv) * silu(z.w));
  store_out4<ActT>(p, row * D + 4 * cq, v);
}

// ---- launch configuration --------------------------------------------------------------------------
// 16-column tiles per state-pass workgroup. A head's chain of chunks is sequential, so the only way
// to spread a short batch over the 256 CUs is to split its value columns: NSPLIT slices per head, the
// largest power of two (at most 8) with NSPLIT B n_v <= 256, the whole head from 129 (sequence, head)
// pairs on. The grid then never exceeds one workgroup per CU: every slice of a head is resident at
// once, which the slices' exchange of row sums for the gated norm relies on.
int pass_nt(int B, int n_v, int D) {
  if (D != 128) return D / 16;
  const long pairs = (long)B * n_v;
  return pairs > 128 ? 8 : pairs > 64 ? 4 : pairs > 32 ? 2 : 1;
}

// A split head finishes its gated norm by the slices' exchange of row sums when its slices are 32 or
// 64 columns wide (2 or 4 per head, which comes with a grid of more than 128 workgroups) and the call
// runs at least 16 chunks. The state pass then streams its records at full bandwidth and the
// exchange's uncached round trips hide behind it, while the norm pass it replaces would move 12 bytes
// per output element. With 16-column slices (8 per head) each chunk is mostly latency and the round
// trips lengthened the chain by more than the norm pass costs; on a short call the last chunks' round
// trip, which nothing hides, costs more than the norm pass too. Those split heads save o and their
// sums for a separate norm pass.
bool pass_exchange(int B, int n_v, int D, int Lb) {
  const int nsplit = D / (16 * pass_nt(B, n_v, D));
  return (nsplit == 2 || nsplit == 4) && Lb >= 16 * kChunk;
}

// The exchange's waits end because every slice of a head is resident at once: the grid (at most 256
// workgroups, one per CU) must fit the device's CUs, which a partitioned or shared device may not
// offer; then the call takes the norm pass, which never waits. CU counts are read once per device.
bool exchange_fits(long grid) { return grid <= device_cus(); }

// bytes of one value record and of one key record (zero without key records)
template <int D, bool SPLIT>
void rec_sizes_t(bool sh, long& vrec, long& krec) {
  vrec = sh ? Rec<D, SPLIT, true>::kBytes : Rec<D, SPLIT, false>::kBytes;
  krec = sh ? KeyRec<D>::kBytes : 0;
}
void rec_sizes(int D, bool split_all, bool sh, long& vrec, long& krec) {
  if (split_all) {
    if (D == 32) rec_sizes_t<32, true>(sh, vrec, krec);
    else rec_sizes_t<64, true>(sh, vrec, krec);
  } else if (D == 32) {
    rec_sizes_t<32, false>(sh, vrec, krec);
  } else if (D == 64) {
    rec_sizes_t<64, false>(sh, vrec, krec);
  } else {
    rec_sizes_t<128, false>(sh, vrec, krec);
  }
}

template <typename ActT, int D, int NT, bool SPLIT, int NM, bool SH>
void launch_pass(const PrefillArgs& p, hipStream_t st) {
  constexpr int NSPLIT = D / (16 * NT);
  hipLaunchKernelGGL((state_pass_kernel<ActT, D, NT, SPLIT, NM, (NT <= 4), SH>), dim3(NSPLIT * p.n_v * p.B), dim3(512), 0, st, p);
}

// The exchanging state pass as a cooperative launch: the runtime starts it only if every workgroup can
// be resident at once (which the slices' waits need), else refuses and nothing runs
template <typename ActT, int D, int NT, bool SPLIT, bool SH>
hipError_t launch_pass_coop(const PrefillArgs& p, hipStream_t st) {
  constexpr int NSPLIT = D / (16 * NT);
  PrefillArgs q = p;
  void* args[] = {&q};
  return hipLaunchCooperativeKernel((const void*)state_pass_kernel<ActT, D, NT, SPLIT, kNormExchange, true, SH>,
                                    dim3(NSPLIT * p.n_v * p.B), dim3(512), args, 0, st);
}

// true while `st` is being captured into a graph (a replay may share the device with other work, so the
// slices' co-residency that the exchange needs is not guaranteed there)
bool capturing(hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return cs != hipStreamCaptureStatusNone;
}

constexpr long kNtRecordBytes = 160L << 20;

template <typename ActT, int D, int R, bool SPLIT, int NT>
hipError_t launch_t(const PrefillArgs& p, hipStream_t st) {
  constexpr int NSPLIT = D / (16 * NT);
  timing_before("chunk_prep", st);
  if constexpr (R <= 2 && !SPLIT && (D == 64 || D == 128)) {
    // the records end at ss_off. Up to 134 MB they were still cached when the state pass read them
    // (non-temporal stores cost 160 -> 207 us at 16 value heads x 4096 tokens); from 201 MB on,
    // non-temporal stores measured 4-6% faster calls (32 value heads x 1-3 sequences x 4096 tokens)
    if (p.ss_off > kNtRecordBytes)
      hipLaunchKernelGGL((chunk_prep2_kernel<ActT, D, R, true>), dim3(p.n_chunks, p.n_v / R, p.B), dim3(512), 0, st, p);
    else
      hipLaunchKernelGGL((chunk_prep2_kernel<ActT, D, R, false>), dim3(p.n_chunks, p.n_v / R, p.B), dim3(512), 0, st, p);
  } else
    hipLaunchKernelGGL((chunk_prep_kernel<ActT, D, R, SPLIT>), dim3(p.n_chunks, p.n_v / R, p.B), dim3(512), 0, st, p);
  timing_after(st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  bool exchanged = false;
  timing_before("state_pass", st);
  if constexpr (NSPLIT == 1) {
    launch_pass<ActT, D, NT, SPLIT, kNormFused, (R > 1)>(p, st);
  } else if constexpr (NSPLIT == 2 || NSPLIT == 4) {
    if (p.exchange && !capturing(st)) {
      exchanged = launch_pass_coop<ActT, D, NT, SPLIT, (R > 1)>(p, st) == hipSuccess;
      if (!exchanged) (void)hipGetLastError();  // refused: the norm pass below, which never waits
    }
    if (!exchanged) launch_pass<ActT, D, NT, SPLIT, kNormPass, (R > 1)>(p, st);
  } else {
    launch_pass<ActT, D, NT, SPLIT, kNormPass, (R > 1)>(p, st);
  }
  timing_after(st);
  e = hipGetLastError();
  if (e != hipSuccess || NSPLIT == 1 || exchanged) return e;
  const long per_seq = (long)p.Lb * p.n_v * (D / 4);  // < 2^31, checked by the caller
  timing_before("norm", st);
  hipLaunchKernelGGL((norm_kernel<ActT, D, NSPLIT>), dim3((unsigned)((per_seq + 255) / 256), p.B), dim3(256), 0, st, p);
  timing_after(st);
  return hipGetLastError();
}

template <typename ActT, int D, bool SPLIT, int NT>
hipError_t launch_r(const PrefillArgs& p, int R, hipStream_t st) {
  switch (R) {
    case 1: return launch_t<ActT, D, 1, SPLIT, NT>(p, st);
    case 2: return launch_t<ActT, D, 2, SPLIT, NT>(p, st);
    case 4: return launch_t<ActT, D, 4, SPLIT, NT>(p, st);
    default: return hipErrorInvalidValue;
  }
}

// fp32 activations at d = 128: groups of one or two value heads (chunk_prep2), the bf16 operands
template <typename ActT, int D, int NT>
hipError_t launch_r12(const PrefillArgs& p, int R, hipStream_t st) {
  switch (R) {
    case 1: return launch_t<ActT, D, 1, false, NT>(p, st);
    case 2: return launch_t<ActT, D, 2, false, NT>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int device_cus() {
  static int cus[64];
  static std::once_flag once[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 0;
  }
  std::call_once(once[dev], [dev] {
    if (hipDeviceGetAttribute(&cus[dev], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
      (void)hipGetLastError();
      cus[dev] = 0;
    }
  });
  return cus[dev];
}

// value heads per chunk_prep workgroup where its grid fills the device
static int natural_group(int n_k, int n_v, int D, bool act_f32) {
  const int R = n_v / n_k;
  if (act_f32 && D == 128) return R % 2 == 0 ? 2 : 1;  // chunk_prep2 only (R <= 2) at this shape
  if (R == 1 || R == 2 || R == 4) return R;
  return R % 4 == 0 ? 4 : R % 2 == 0 ? 2 : 1;
}

// Below this many chunk_prep workgroups the grid leaves CUs idle and one workgroup's latency sets
// chunk_prep's time; a call then runs one value head per workgroup (at 16/32 heads a single chunk
// takes 23 us with two value heads per workgroup and 18 us with one), forming q and k once per head.
constexpr long kSmallPrepGrid = 256;

int prefill_group(int n_k, int n_v, int D, bool act_f32, int B, int n_chunks) {
  const int g = natural_group(n_k, n_v, D, act_f32);
  if (g > 1 && (long)B * n_chunks * (n_v / g) < kSmallPrepGrid) return 1;
  return g;
}

// hi/lo operands throughout (fp32-equivalent) for fp32 activations up to d = 64; from d = 128 the
// records would not fit chunk_prep's LDS, and fp32 activations take the bf16 activations' operands
bool prefill_split_all(int D, bool act_f32) { return act_f32 && D <= 64; }

static size_t records_bytes(int B, int n_v, int D, int n_chunks, bool split_all, int grp) {
  long vrec, krec;
  rec_sizes(D, split_all, grp > 1, vrec, krec);
  return (size_t)B * n_chunks * ((size_t)n_v * vrec + (size_t)(n_v / grp) * krec);
}

size_t prefill_ws_bytes(int B, int n_k, int n_v, int D, int Lb, int n_chunks, bool act_f32) {
  const bool split_all = prefill_split_all(D, act_f32);
  const int nsplit = D / (16 * pass_nt(B, n_v, D));
  const int g = natural_group(n_k, n_v, D, act_f32);
  const int grp = prefill_group(n_k, n_v, D, act_f32, B, n_chunks);
  size_t bytes = records_bytes(B, n_v, D, n_chunks, split_all, grp);
  if (grp == g && g > 1) {
    // the longest call that still takes one value head per workgroup has larger records than a
    // slightly longer call with groups: the size covers both, so that it never shrinks as Lb grows
    const long nc_small = (kSmallPrepGrid - 1) / ((long)B * (n_v / g));
    if (nc_small >= 1) bytes = std::max(bytes, records_bytes(B, n_v, D, (int)nc_small, split_all, 1));
  }
  if (nsplit > 1) {
    // partial sums of squares, and the unnormalised o for a norm pass; the o area is counted even
    // when the slices exchange their sums, so that the size never shrinks as Lb grows (a workspace
    // sized for the longest call serves every shorter one)
    bytes += (size_t)B * Lb * n_v * nsplit * 4;
    bytes += (size_t)B * Lb * n_v * D * 4;
    bytes = (bytes + 255) / 256 * 256;
  }
  return bytes;
}

void prefill_ws_layout(PrefillArgs& p, int D, bool act_f32) {
  const bool split_all = prefill_split_all(D, act_f32);
  long vrec, krec;
  p.grp = prefill_group(p.n_k, p.n_v, D, act_f32, p.B, p.n_chunks);
  rec_sizes(D, split_all, p.grp > 1, vrec, krec);
  p.key_off = (long)p.B * p.n_v * p.n_chunks * vrec;
  const size_t rec = (size_t)p.key_off + (size_t)p.B * (p.n_v / p.grp) * p.n_chunks * krec;
  p.nsplit = D / (16 * pass_nt(p.B, p.n_v, D));
  p.exchange = pass_exchange(p.B, p.n_v, D, p.Lb) && exchange_fits((long)p.nsplit * p.B * p.n_v) ? 1 : 0;
  p.ss_off = (long)rec;
  p.oraw_off = (long)(rec + (size_t)p.B * p.Lb * p.n_v * p.nsplit * 4);
}

hipError_t launch_prefill(const PrefillArgs& p, int act_dtype, int D, int R, hipStream_t st) {
  const int nt = pass_nt(p.B, p.n_v, D);
  if (act_dtype == kActBf16) {
    if (D == 32) return launch_r<bf16_t, 32, false, 2>(p, R, st);
    if (D == 64) return launch_r<bf16_t, 64, false, 4>(p, R, st);
    if (D == 128) {
      if (nt == 8) return launch_r<bf16_t, 128, false, 8>(p, R, st);
      if (nt == 4) return launch_r<bf16_t, 128, false, 4>(p, R, st);
      if (nt == 2) return launch_r<bf16_t, 128, false, 2>(p, R, st);
      return launch_r<bf16_t, 128, false, 1>(p, R, st);
    }
  } else {
    if (D == 32) return launch_r<float, 32, true, 2>(p, R, st);
    if (D == 64) return launch_r<float, 64, true, 4>(p, R, st);
    if (D == 128) {
      if (nt == 8) return launch_r12<float, 128, 8>(p, R, st);
      if (nt == 4) return launch_r12<float, 128, 4>(p, R, st);
      if (nt == 2) return launch_r12<float, 128, 2>(p, R, st);
      return launch_r12<float, 128, 1>(p, R, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
