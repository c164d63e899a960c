// Single-token recurrence for decode and for verify-with-checkpoints (gfx950).
//
// Work item = (key head kh, row bp = b P + p): T tokens one after the other through the conv on the
// channels of key head kh (its q and k channels and the v channels of its value heads, R at a time), the q/k L2
// norm, the gates, one delta-rule step per value head, the gated RMSNorm, and the state/tail stores.
// Decode is T = 1 writing back to the pool row; verify writes each token's state and tail to its
// checkpoint row and leaves the pool untouched. Both run this one kernel, so checkpoint i is bitwise
// what i+1 decode calls produce (the multistate verify of the "mtp/generate.py" page claims the same
// bit-identity against its per-token kernel). A batch-of-paths verify has P rows per sequence b, every
// one starting from b's pool row (that page tiles the cache into one row per candidate path); the P
// workgroups of one (sequence, key head) are n_k apart in the grid and read the same state block,
// which the second and later ones find in the cache.
//
// The step (H = S^T, [d_k][d_v] per value head, k and q L2-normalised):
//   H <- e^g H;  u = beta (v - H^T k);  H <- H + k u^T;  o = scale H^T q
// computed from one read of the old H:  u = beta (v - e^g H_old^T k),
//   o = scale (e^g H_old^T q + (k.q) u),  H_new = e^g H_old + k u^T.
//
// The state is HBM-streamed fp32, read and written exactly once per call. Each value head has its own
// 256 threads (the workgroup is 256 R threads); a thread holds a 4-column x RPT-row block of its head's
// H (d_k rows of d_v columns, each head dim 32, 64 or 128) in registers; column partial sums are reduced across the row groups of a wave with lane shuffles
// and across the head's waves in LDS. The register footprint is kept small (at d = 128 with up to two
// value heads per key head half of a thread's rows wait in LDS, which leaves room for two workgroups
// per CU), so that the waves of different workgroups overlap one's loads with another's arithmetic
// and stores. Keeping the q/k
// channels of a key head in one workgroup is what lets decode update the conv tail in place without a
// race.
#include "gdn_common.h"
#include "gdn_kernels.h"

// No implicit contraction: every fused multiply-add below is written out, so the rounding of a token
// step is fixed by the source and identical wherever the compiler places the code (a verify token is
// bitwise the decode step).
#pragma clang fp contract(off)

namespace gdn {

namespace {

// Barrier for LDS only: __syncthreads() would also wait for the next item's state loads (vmcnt).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int DK, int DV, int R>
struct StepShape {
  static constexpr int HT = 256;                               // threads per value head
  static constexpr int NTH = HT * R;
  static constexpr int QD = DV / 4;                            // column quads per row
  static constexpr int RG = HT / QD;                           // row groups per head
  static constexpr int RPT = DK / RG;                          // rows per thread
  // at d = 128 with up to two value heads per key head, half of each thread's rows live in LDS (32 KB
  // per head, only ever touched by their own thread), so that the kernel fits 128 VGPRs and two
  // workgroups share a CU: one's loads and stores overlap the other's reductions and barriers
  static constexpr bool LH = DK == 128 && DV == 128 && R <= 2;
  static constexpr int RR = LH ? RPT / 2 : RPT;                // rows per thread held in registers
};

template <typename ActT, int DK, int DV, int R, bool GROUPED>
__global__ __launch_bounds__((StepShape<DK, DV, R>::NTH))
__attribute__((amdgpu_waves_per_eu(StepShape<DK, DV, R>::LH ? 2 * StepShape<DK, DV, R>::NTH / 256 : 1)))
void step_kernel(StepArgs p) {
  using S = StepShape<DK, DV, R>;
  constexpr int HT = S::HT, NTH = S::NTH, QD = S::QD, RPT = S::RPT, HW = HT / kWave, RR = S::RR, RL = RPT - RR;
  constexpr int NCH = 2 * DK + R * DV;       // channels owned by an item
  constexpr int CPT = (NCH + NTH - 1) / NTH;
  static_assert(RPT >= 1 && S::RG * RPT == DK, "thread layout");
  static_assert(QD <= kWave && kWave % QD == 0, "a wave holds whole row groups");

  // Two LDS barriers per token. The conv outputs are double-buffered by token parity: token t + 1
  // writes the other buffer before its first barrier, while slower waves may still read token t's;
  // the buffer of token t is written again only after the second barrier of token t + 1, which every
  // wave reaches after its last read of token t. The wave partials are written after the first
  // barrier of their token, which every wave reaches only after it has summed the previous token's.
  __shared__ float sY[2][NCH];               // conv outputs of a token: q | k | v(R heads)
  __shared__ __attribute__((aligned(16))) float sRed[R][HW][2][DV];  // per head, per wave: partial H^T k, H^T q
  __shared__ f32x4 sHL[RL > 0 ? R * S::RG * RL * QD : 1];   // rows RR.. of each thread's block

  const int tid = threadIdx.x, lane = tid % kWave;
  const int r = tid / HT;                    // value head of the group owned by this thread
  const int th = tid % HT;
  const int hw = th / kWave;                 // wave inside the head's threads
  const int cq = th % QD, rg = th / QD;
  const int n_k = p.n_k, n_v = p.n_v, C = p.C;
  const long SZ = (long)n_v * DK * DV;       // state floats per record
  const long TZ = 3L * C;                    // tail elements per record

  const ActT* conv_w = (const ActT*)p.conv_w;
  const ActT* mixed = (const ActT*)p.mixed;
  const ActT* zin = (const ActT*)p.z;
  const ActT* ain = (const ActT*)p.a;
  const ActT* bin = (const ActT*)p.b;
  ActT* out = (ActT*)p.out;

  // pool row of an item: slot[b], read through the constant address space (the slot map is not written
  // during the call), so that it is a scalar load, which no vector-memory wait has to drain
  auto slot_of = [&](int item) {
    const int b = item / n_k / p.P;
    typedef const __attribute__((address_space(4))) int32_t* const_i32;
    return p.slot ? (long)((const_i32)p.slot)[b] : (long)b;
  };
  // row RR + j of this thread's block in LDS
  auto hl_at = [&](int j) -> f32x4& { return sHL[((r * S::RG + rg) * (RL > 0 ? RL : 1) + j) * QD + cq]; };
  // this thread's block of value head h's state in pool row s: rows rg*RPT + i, columns 4 cq .. 4 cq + 3
  auto load_H = [&](f32x4 (&H)[RR], long s, int h) __attribute__((always_inline)) {
    const float* src = p.state_in + s * SZ + (long)h * DK * DV + (long)(rg * RPT) * DV + 4 * cq;
#pragma unroll
    for (int i = 0; i < RR; ++i) H[i] = __builtin_nontemporal_load((const f32x4*)(src + (long)i * DV));
#pragma unroll
    for (int j = 0; j < RL; ++j) hl_at(j) = __builtin_nontemporal_load((const f32x4*)(src + (long)(RR + j) * DV));
  };

  // the conv state of the channels a thread owns in one group of an item: q and k channels of key
  // head kh, v channels of value heads vb .. vb + R - 1 (gc = -1 for an unowned slot), their taps and
  // the three tail rows
  struct Conv {
    int gch[CPT];
    float w0[CPT], w1[CPT], w2[CPT], w3[CPT], t0[CPT], t1[CPT], t2[CPT];
  };
  // per-token activations of one item, loaded ahead of use
  struct TokIn {
    float x[CPT];   // pre-conv inputs of the owned channels
    float av, bv;   // gate inputs of this thread's head
    float z[4];     // z of this thread's output columns (row group 0 only)
  };
  auto load_conv = [&](Conv& cv, int kh, int vb, const ActT* tail_in) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int lc = tid + j * NTH;
      int gc = -1;
      if (lc < DK) gc = kh * DK + lc;
      else if (lc < 2 * DK) gc = n_k * DK + kh * DK + (lc - DK);
      else if (lc < NCH) gc = 2 * n_k * DK + vb * DV + (lc - 2 * DK);
      cv.gch[j] = gc;
      const int gl = gc >= 0 ? gc : 0;  // unconditional loads (a clamped channel for unowned slots)
      cv.w0[j] = to_f32(conv_w[gl * 4 + 0]);
      cv.w1[j] = to_f32(conv_w[gl * 4 + 1]);
      cv.w2[j] = to_f32(conv_w[gl * 4 + 2]);
      cv.w3[j] = to_f32(conv_w[gl * 4 + 3]);
      cv.t0[j] = to_f32(tail_in[0L * C + gl]);
      cv.t1[j] = to_f32(tail_in[1L * C + gl]);
      cv.t2[j] = to_f32(tail_in[2L * C + gl]);
    }
  };
  auto load_tok = [&](TokIn& in, const Conv& cv, long row, int h) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) in.x[j] = to_f32(mixed[row * C + (cv.gch[j] >= 0 ? cv.gch[j] : 0)]);
    in.av = to_f32(ain[row * n_v + h]);
    in.bv = to_f32(bin[row * n_v + h]);
    const long ob = row * (long)n_v * DV + (long)h * DV;
#pragma unroll
    for (int c = 0; c < 4; ++c) in.z[c] = to_f32(zin[ob + 4 * cq + c]);
  };
  float nw[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) nw[c] = p.norm_w[4 * cq + c];

  // One token of value head h (this thread's): conv + SiLU of the owned channels and their tail rows
  // (to tail_to), the q/k norms and gates, the step on H, the new state (to dst, this head's block of
  // a record) and the output row `row`. Decode and verify run this same code, so a verify checkpoint
  // is bitwise what the decode calls produce.
  auto token = [&](f32x4 (&H)[RR], Conv& cv, const TokIn& in, float A, float dtb, int h, long row, ActT* tail_to,
                   float* dst, bool qk_tail, int& par) __attribute__((always_inline)) {
    float* const y = sY[par];
    // ---- conv + SiLU on the owned channels, tail shift
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int gc = cv.gch[j];
      const float x = in.x[j];
      if (gc >= 0) {
        float pre = cv.w0[j] * cv.t0[j];
        pre = fmaf(cv.w1[j], cv.t1[j], pre);
        pre = fmaf(cv.w2[j], cv.t2[j], pre);
        pre = fmaf(cv.w3[j], x, pre);
        y[tid + j * NTH] = silu(pre);
        cv.t0[j] = cv.t1[j];
        cv.t1[j] = cv.t2[j];
        cv.t2[j] = x;
      }
    }
    // tail after this token: decode writes the pool row, verify the checkpoint row
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int gc = cv.gch[j];
      if (gc >= 0 && (qk_tail || tid + j * NTH >= 2 * DK)) {
        tail_to[0L * C + gc] = from_f32<ActT>(cv.t0[j]);
        tail_to[1L * C + gc] = from_f32<ActT>(cv.t1[j]);
        tail_to[2L * C + gc] = from_f32<ActT>(cv.t2[j]);
      }
    }
    const float decay = __expf(A * softplus(in.av + dtb));
    const float beta = sigmoid(in.bv);
    lds_barrier();

    // ---- q/k L2 norm and k.q (every wave computes them, no broadcast needed)
    float sq = 0.f, sk = 0.f, skq = 0.f;
    for (int i = lane; i < DK; i += kWave) {
      const float qv = y[i], kv = y[DK + i];
      sq = fmaf(qv, qv, sq);
      sk = fmaf(kv, kv, sk);
      skq = fmaf(kv, qv, skq);
    }
    sq = wave_sum<kWave>(sq);
    sk = wave_sum<kWave>(sk);
    skq = wave_sum<kWave>(skq);
    const float rq = rsqrt_fast(sq + p.l2_eps);
    const float rk = rsqrt_fast(sk + p.l2_eps);
    const float kq = (skq * rk) * rq;  // k^ . q^

    // column partial sums of H^T k and H^T q over this thread's rows (q and k re-read from LDS
    // where used, which keeps the register footprint to the state blocks)
    float pk[4] = {0.f, 0.f, 0.f, 0.f}, pq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const float qn = y[rg * RPT + i] * rq, kn = y[DK + rg * RPT + i] * rk;
      const f32x4 hv = i < RR ? H[i < RR ? i : 0] : hl_at(i < RR ? 0 : i - RR);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        pk[c] = fmaf(hv[c], kn, pk[c]);
        pq[c] = fmaf(hv[c], qn, pq[c]);
      }
    }
    // across the row groups inside the wave (lanes with the same column quad)
#pragma unroll
    for (int off = QD; off < kWave; off <<= 1) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        pk[c] = pk[c] + __shfl_xor(pk[c], off, kWave);
        pq[c] = pq[c] + __shfl_xor(pq[c], off, kWave);
      }
    }
    if (lane < QD) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        sRed[r][hw][0][4 * cq + c] = pk[c];
        sRed[r][hw][1][4 * cq + c] = pq[c];
      }
    }
    lds_barrier();
    // H^T k and H^T q on this thread's four columns: the head's wave partials, summed in wave order
    f32x4 hk4 = *(const f32x4*)&sRed[r][0][0][4 * cq], hq4 = *(const f32x4*)&sRed[r][0][1][4 * cq];
#pragma unroll
    for (int ww = 1; ww < HW; ++ww) {
      const f32x4 pk4 = *(const f32x4*)&sRed[r][ww][0][4 * cq], pq4 = *(const f32x4*)&sRed[r][ww][1][4 * cq];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        hk4[c] = hk4[c] + pk4[c];
        hq4[c] = hq4[c] + pq4[c];
      }
    }
    float u[4], o[4];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float v = y[2 * DK + r * DV + 4 * cq + c];
      u[c] = beta * (v - decay * hk4[c]);
      o[c] = p.scale * fmaf(kq, u[c], decay * hq4[c]);
      ss = fmaf(o[c], o[c], ss);
    }
    // new state
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const float kn = y[DK + rg * RPT + i] * rk;
      const f32x4 hv = i < RR ? H[i < RR ? i : 0] : hl_at(i < RR ? 0 : i - RR);
      f32x4 nh;
#pragma unroll
      for (int c = 0; c < 4; ++c) nh[c] = fmaf(kn, u[c], decay * hv[c]);
      if (i < RR) H[i < RR ? i : 0] = nh;
      else hl_at(i < RR ? 0 : i - RR) = nh;
      store_stream16(dst, DK * DV * 4, ((rg * RPT + i) * DV + 4 * cq) * 4, nh);
    }
    // gated RMSNorm over the DV columns held by the QD lanes of row group 0
    ss = wave_sum<QD>(ss);
    if (th < QD) {
      const float inv = rsqrt_fast(ss / (float)DV + p.rms_eps);
      const long ob = row * (long)n_v * DV + (long)h * DV;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float yv = nw[c] * (o[c] * inv) * silu(in.z[c]);
        if (p.out_f32) ((float*)p.out)[ob + 4 * cq + c] = yv;
        else out[ob + 4 * cq + c] = from_f32<ActT>(yv);
      }
    }
    par ^= 1;
  };

  int par = 0;  // parity of the token over every token the workgroup runs: selects the conv output buffer
  f32x4 H[RR];
  const int item = blockIdx.x;
  const int kh = item % n_k, bp = item / n_k;  // row: sequence bp / P, path bp % P
  const long s = slot_of(item);
  const ActT* tail_in = (const ActT*)p.tail_in + s * TZ;
  // With more value heads per key head than one workgroup holds (R of the n_v / n_k), the workgroup
  // takes them R at a time, forming q and k again for each group. The q and k channels of the conv
  // tail are written by the last group only: decode updates the tail in place, and every group reads
  // the old rows.
  const int RQ = GROUPED ? n_v / n_k : R, ngroups = GROUPED ? RQ / R : 1;
  for (int grp = 0; grp < ngroups; ++grp) {
    const int h = kh * RQ + grp * R + r;
    const bool qk_tail = grp + 1 == ngroups;
    // The group's small inputs are loaded before its state: loads complete in issue order, so
    // anything issued after the state would wait for all of it.
    Conv cv;
    load_conv(cv, kh, kh * RQ + grp * R, tail_in);
    const float A = -__expf(p.A_log[h]), dtb = p.dt_bias[h];
    TokIn cur;
    load_tok(cur, cv, (long)bp * p.T, h);
    load_H(H, s, h);
    for (int t = 0; t < p.T; ++t) {
      const long row = (long)bp * p.T + t;
      TokIn in = cur;
      if (t + 1 < p.T) load_tok(cur, cv, row + 1, h);  // verify only
      token(H, cv, in, A, dtb, h, row, (ActT*)p.tail_out + (p.verify ? row * TZ : s * TZ),
            p.state_out + (p.verify ? row * SZ : s * SZ) + (long)h * DK * DV, qk_tail, par);
    }
  }
}

// one workgroup per (key head, sequence): many small independent workgroups keep every CU's memory
// pipe busy, one finishing its stores while the next loads
template <typename ActT, int DK, int DV, int R, bool GROUPED>
hipError_t launch_step_r(const StepArgs& p, hipStream_t st) {
  using S = StepShape<DK, DV, R>;
  timing_before(p.verify ? "step_verify" : "step_decode", st);
  hipLaunchKernelGGL((step_kernel<ActT, DK, DV, R, GROUPED>), dim3(p.n_k * p.B * p.P), dim3(S::NTH), 0, st, p);
  timing_after(st);
  return hipGetLastError();
}

// value heads per workgroup pass: the GQA ratio itself where a shape is built for it (1, 2, 4), else its
// largest divisor among 4, 2, 1, the workgroup looping over the groups
template <typename ActT, int DK, int DV>
hipError_t launch_step_d(const StepArgs& p, int ratio, hipStream_t st) {
  switch (ratio) {
    case 1: return launch_step_r<ActT, DK, DV, 1, false>(p, st);
    case 2: return launch_step_r<ActT, DK, DV, 2, false>(p, st);
    case 4: return launch_step_r<ActT, DK, DV, 4, false>(p, st);
    default:
      if (ratio % 4 == 0) return launch_step_r<ActT, DK, DV, 4, true>(p, st);
      if (ratio % 2 == 0) return launch_step_r<ActT, DK, DV, 2, true>(p, st);
      return launch_step_r<ActT, DK, DV, 1, true>(p, st);
  }
}

template <typename ActT, int DK>
hipError_t launch_step_k(const StepArgs& p, int DV, int ratio, hipStream_t st) {
  if (DV == 32) return launch_step_d<ActT, DK, 32>(p, ratio, st);
  if (DV == 64) return launch_step_d<ActT, DK, 64>(p, ratio, st);
  if (DV == 128) return launch_step_d<ActT, DK, 128>(p, ratio, st);
  return hipErrorInvalidValue;
}

template <typename ActT>
hipError_t launch_step_a(const StepArgs& p, int DK, int DV, int ratio, hipStream_t st) {
  if (DK == 32) return launch_step_k<ActT, 32>(p, DV, ratio, st);
  if (DK == 64) return launch_step_k<ActT, 64>(p, DV, ratio, st);
  if (DK == 128) return launch_step_k<ActT, 128>(p, DV, ratio, st);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_step(const StepArgs& p, int act_dtype, int DK, int DV, int ratio, hipStream_t st) {
  return act_dtype == kActBf16 ? launch_step_a<bf16_t>(p, DK, DV, ratio, st) : launch_step_a<float>(p, DK, DV, ratio, st);
}

}  // namespace gdn
