// Single-token recurrence for decode and for verify-with-checkpoints (gfx950).
//
// One workgroup per (key head kh, sequence b) runs T tokens one after the other: the conv on the
// channels of key head kh (its q and k channels and the v channels of its R value heads), the q/k L2
// norm, the gates, one delta-rule step per value head, the gated RMSNorm, and the state/tail stores.
// Decode is T = 1 writing back to the pool row; verify writes each token's state and tail to its
// checkpoint row and leaves the pool untouched. Both run this one kernel, so checkpoint i is bitwise
// what i+1 decode calls produce (the multistate verify of the "mtp/generate.py" page claims the same
// bit-identity against its per-token kernel).
//
// The step (H = S^T, [d_k][d_v] per value head, k and q L2-normalised):
//   H <- e^g H;  u = beta (v - H^T k);  H <- H + k u^T;  o = scale H^T q
// computed from one read of the old H:  u = beta (v - e^g H_old^T k),
//   o = scale (e^g H_old^T q + (k.q) u),  H_new = e^g H_old + k u^T.
// The state is HBM-streamed fp32: each thread holds a 4-column x RPT-row block of H in registers,
// column partial sums are reduced across row groups with lane shuffles, then across waves in LDS.
#include "gdn_common.h"
#include "gdn_kernels.h"

#pragma clang fp contract(off)

namespace gdn {

namespace {

constexpr int kMaxChanPerThread = 6;  // (2*128 + 4*128) / 256 = 3 with R <= 4; room to spare

// 256 threads per workgroup; for R <= 2 the register budget is capped so that two workgroups share
// a CU and one workgroup's state loads overlap the other's arithmetic and stores
template <int D>
struct StepThreads {
  static constexpr int value = 256;
};

template <typename ActT, int D, int R>
__global__ __launch_bounds__(StepThreads<D>::value) __attribute__((amdgpu_waves_per_eu(R <= 2 ? 2 : 1))) void step_kernel(StepArgs p) {
  constexpr int kThreads = StepThreads<D>::value;
  constexpr int QD = D / 4;              // column quads per row
  constexpr int RG = kThreads / QD;      // row groups
  constexpr int RPT = D / RG;            // rows per thread (>= 1 since D*D >= 4*256 for D >= 32)
  constexpr int NCH = 2 * D + R * D;     // channels owned by this workgroup
  constexpr int CPT = (NCH + kThreads - 1) / kThreads;
  static_assert(RPT >= 1 && RG * RPT == D, "thread layout");
  static_assert(CPT <= kMaxChanPerThread, "channels per thread");

  __shared__ float sY[NCH];              // conv outputs of the current token: q | k | v(R heads)
  __shared__ float sRed[kThreads / kWave][2][D];

  const int kh = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int cq = tid % QD, rg = tid / QD;
  const int n_k = p.n_k, n_v = p.n_v, C = p.C;
  const long s = p.slot ? (long)p.slot[b] : (long)b;
  const long SZ = (long)n_v * D * D;      // state floats per record
  const long TZ = 3L * C;                 // tail elements per record

  const ActT* conv_w = (const ActT*)p.conv_w;
  const ActT* mixed = (const ActT*)p.mixed;
  const ActT* zin = (const ActT*)p.z;
  const ActT* ain = (const ActT*)p.a;
  const ActT* bin = (const ActT*)p.b;
  const ActT* tail_in = (const ActT*)p.tail_in + s * TZ;
  ActT* out = (ActT*)p.out;

  // channel ownership, conv weights and tail rows in registers
  int gch[CPT];
  float w0[CPT], w1[CPT], w2[CPT], w3[CPT], t0[CPT], t1[CPT], t2[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int lc = tid + j * kThreads;
    int gc = -1;
    if (lc < D) gc = kh * D + lc;
    else if (lc < 2 * D) gc = n_k * D + kh * D + (lc - D);
    else if (lc < NCH) gc = 2 * n_k * D + kh * R * D + (lc - 2 * D);
    gch[j] = gc;
    const int gl = gc >= 0 ? gc : 0;  // unconditional loads (a clamped channel for unowned slots)
    w0[j] = to_f32(conv_w[gl * 4 + 0]);
    w1[j] = to_f32(conv_w[gl * 4 + 1]);
    w2[j] = to_f32(conv_w[gl * 4 + 2]);
    w3[j] = to_f32(conv_w[gl * 4 + 3]);
    t0[j] = to_f32(tail_in[0L * C + gl]);
    t1[j] = to_f32(tail_in[1L * C + gl]);
    t2[j] = to_f32(tail_in[2L * C + gl]);
  }

  // the R value heads' states in registers
  float4 H[R][RPT];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float* src = p.state_in + s * SZ + (long)(kh * R + r) * D * D;
#pragma unroll
    for (int i = 0; i < RPT; ++i) H[r][i] = *(const float4*)(src + (long)(rg * RPT + i) * D + 4 * cq);
  }

  for (int t = 0; t < p.T; ++t) {
    const long row = (long)b * p.T + t;
    // ---- conv + SiLU on the owned channels, tail shift
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int gc = gch[j];
      const float x = to_f32(mixed[row * C + (gc >= 0 ? gc : 0)]);
      if (gc >= 0) {
        float pre = w0[j] * t0[j];
        pre = pre + w1[j] * t1[j];
        pre = pre + w2[j] * t2[j];
        pre = pre + w3[j] * x;
        sY[tid + j * kThreads] = silu(pre);
        t0[j] = t1[j];
        t1[j] = t2[j];
        t2[j] = x;
      }
    }
    // tail after this token: decode writes the pool row, verify the checkpoint row
    {
      ActT* to = (ActT*)p.tail_out + (p.verify ? row * TZ : s * TZ);
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int gc = gch[j];
        if (gc >= 0) {
          to[0L * C + gc] = from_f32<ActT>(t0[j]);
          to[1L * C + gc] = from_f32<ActT>(t1[j]);
          to[2L * C + gc] = from_f32<ActT>(t2[j]);
        }
      }
    }
    __syncthreads();

    // ---- q/k L2 norm and k.q (every wave computes them, no broadcast needed)
    float sq = 0.f, sk = 0.f, skq = 0.f;
    for (int i = lane; i < D; i += kWave) {
      const float qv = sY[i], kv = sY[D + i];
      sq = sq + qv * qv;
      sk = sk + kv * kv;
      skq = skq + kv * qv;
    }
    sq = wave_sum<kWave>(sq);
    sk = wave_sum<kWave>(sk);
    skq = wave_sum<kWave>(skq);
    const float rq = rsqrt_fast(sq + p.l2_eps);
    const float rk = rsqrt_fast(sk + p.l2_eps);
    const float kq = (skq * rk) * rq;  // k^ . q^

    float kn[RPT], qn[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      qn[i] = sY[rg * RPT + i] * rq;
      kn[i] = sY[D + rg * RPT + i] * rk;
    }

#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int h = kh * R + r;
      const long gi = row * n_v + h;
      const float decay = __expf(-__expf(p.A_log[h]) * softplus(to_f32(ain[gi]) + p.dt_bias[h]));
      const float beta = sigmoid(to_f32(bin[gi]));

      // column partial sums of H^T k and H^T q over this thread's rows
      float pk[4] = {0.f, 0.f, 0.f, 0.f}, pq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const float hv[4] = {H[r][i].x, H[r][i].y, H[r][i].z, H[r][i].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          pk[c] = pk[c] + hv[c] * kn[i];
          pq[c] = pq[c] + hv[c] * qn[i];
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
      __syncthreads();  // sRed free (previous head done)
      if (lane < QD) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          sRed[wave][0][4 * cq + c] = pk[c];
          sRed[wave][1][4 * cq + c] = pq[c];
        }
      }
      __syncthreads();
      float u[4], o[4];
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int col = 4 * cq + c;
        float hk = sRed[0][0][col], hq = sRed[0][1][col];
#pragma unroll
        for (int w = 1; w < kThreads / kWave; ++w) {
          hk = hk + sRed[w][0][col];
          hq = hq + sRed[w][1][col];
        }
        const float v = sY[2 * D + r * D + col];
        u[c] = beta * (v - decay * hk);
        o[c] = p.scale * (decay * hq + kq * u[c]);
        ss = ss + o[c] * o[c];
      }
      // new state
      float* dst = p.state_out + (p.verify ? row * SZ : s * SZ) + (long)h * D * D;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        float4 nh;
        nh.x = decay * H[r][i].x + kn[i] * u[0];
        nh.y = decay * H[r][i].y + kn[i] * u[1];
        nh.z = decay * H[r][i].z + kn[i] * u[2];
        nh.w = decay * H[r][i].w + kn[i] * u[3];
        H[r][i] = nh;
        *(float4*)(dst + (long)(rg * RPT + i) * D + 4 * cq) = nh;
      }
      // gated RMSNorm over the D columns held by the QD lanes of this row group
      ss = wave_sum<QD>(ss);
      if (tid < QD) {
        const float inv = rsqrt_fast(ss / (float)D + p.rms_eps);
        const long ob = row * (long)n_v * D + (long)h * D;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int col = 4 * cq + c;
          const float zz = to_f32(zin[ob + col]);
          out[ob + col] = from_f32<ActT>(p.norm_w[col] * (o[c] * inv) * silu(zz));
        }
      }
    }
    __syncthreads();  // sY reused by the next token
  }
}

template <typename ActT, int D>
hipError_t launch_step_d(const StepArgs& p, int R, hipStream_t st) {
  dim3 grid(p.n_k, p.B), block(StepThreads<D>::value);
  switch (R) {
    case 1: hipLaunchKernelGGL((step_kernel<ActT, D, 1>), grid, block, 0, st, p); break;
    case 2: hipLaunchKernelGGL((step_kernel<ActT, D, 2>), grid, block, 0, st, p); break;
    case 4: hipLaunchKernelGGL((step_kernel<ActT, D, 4>), grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_step(const StepArgs& p, int act_dtype, int D, int R, hipStream_t st) {
  if (act_dtype == kActBf16) {
    if (D == 32) return launch_step_d<bf16_t, 32>(p, R, st);
    if (D == 64) return launch_step_d<bf16_t, 64>(p, R, st);
    if (D == 128) return launch_step_d<bf16_t, 128>(p, R, st);
  } else {
    if (D == 32) return launch_step_d<float, 32>(p, R, st);
    if (D == 64) return launch_step_d<float, 64>(p, R, st);
    if (D == 128) return launch_step_d<float, 128>(p, R, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
