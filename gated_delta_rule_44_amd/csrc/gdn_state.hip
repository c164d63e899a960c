// State-record copy (gather/scatter) and the accepted-prefix rule (gfx950).
//
// A record is {fp32 state [n_v][d_k][d_v], conv tail [3][C_ch]}: fixed size, O(1) in context length
// (the "uni_engine.py" page: copy_cache_ copies the conv and recurrent tables in place, its bridge
// moves only that fixed payload). The copy streams 16-byte vectors, 8 per thread in flight; grid.y
// is the record, grid.x tiles the record's bytes.
#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// kUnroll 16-byte vectors of one range per thread: every load is issued before the first store, and
// whole blocks (all but the last of a range) take the branch-free path so that the compiler does not
// wait on each load separately
__device__ __forceinline__ void copy_range(const u32x4* s, u32x4* d, long n, long base) {
  u32x4 v[kUnroll];
  if (base + (long)(kUnroll - 1) * kThreads < n) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(s + base + (long)u * kThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(v[u], d + base + (long)u * kThreads);
  } else {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const long k = base + (long)u * kThreads;
      if (k < n) d[k] = s[k];
    }
  }
}

__global__ __launch_bounds__(kThreads) void copy_kernel(CopyArgs p) {
  const int i = blockIdx.y;
  const long si = p.src_idx ? (long)p.src_idx[i] : (long)i;
  const long di = p.dst_idx ? (long)p.dst_idx[i] : (long)i;
  const long nstate = p.src_state ? p.state_floats / 4 : 0;   // 16-byte vectors
  const long ntail = p.src_tail ? p.tail_bytes / 16 : 0;
  const long nsb = (nstate + kThreads * kUnroll - 1) / (kThreads * kUnroll);  // blocks of the state part
  if ((long)blockIdx.x < nsb) {
    copy_range((const u32x4*)(p.src_state + si * p.state_floats), (u32x4*)(p.dst_state + di * p.state_floats), nstate,
               (long)blockIdx.x * kThreads * kUnroll + threadIdx.x);
  } else if (ntail > 0) {  // the tail part takes its own block range after the state's
    copy_range((const u32x4*)((const char*)p.src_tail + si * p.tail_bytes), (u32x4*)((char*)p.dst_tail + di * p.tail_bytes),
               ntail, ((long)blockIdx.x - nsb) * kThreads * kUnroll + threadIdx.x);
  }
}

// zeros into record dst_idx[i] (or i): the same tiling as copy_kernel, src pointers unused
__global__ __launch_bounds__(kThreads) void zero_kernel(CopyArgs p) {
  const int i = blockIdx.y;
  const long di = p.dst_idx ? (long)p.dst_idx[i] : (long)i;
  const long nstate = p.dst_state ? p.state_floats / 4 : 0;
  const long ntail = p.dst_tail ? p.tail_bytes / 16 : 0;
  const long nsb = (nstate + kThreads * kUnroll - 1) / (kThreads * kUnroll);
  u32x4* d;
  long n, base;
  if ((long)blockIdx.x < nsb) {
    d = (u32x4*)(p.dst_state + di * p.state_floats);
    n = nstate;
    base = (long)blockIdx.x * kThreads * kUnroll + threadIdx.x;
  } else {
    d = (u32x4*)((char*)p.dst_tail + di * p.tail_bytes);
    n = ntail;
    base = ((long)blockIdx.x - nsb) * kThreads * kUnroll + threadIdx.x;
  }
  const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const long k = base + (long)u * kThreads;
    if (k < n) d[k] = z;
  }
}

// the "mtp/generate.py" page's accept_prefix, one sequence per thread. With P paths per sequence
// (its tree_verify_step) every path's prefix is measured and the first path with the longest one wins.
__global__ void accept_kernel(AcceptArgs p) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= p.B) return;
  const int K = p.K, P = p.P;
  int m = -1, win = 0;
  for (int q = 0; q < P; ++q) {
    const int32_t* dr = p.drafts + ((long)b * P + q) * K;
    const int32_t* pr = p.preds + ((long)b * P + q) * (K + 1);
    int j = 0;
    while (j < K && pr[j] == dr[j]) ++j;
    if (j > m) {
      m = j;
      win = q;
    }
  }
  const int32_t* dr = p.drafts + ((long)b * P + win) * K;
  const int32_t* pr = p.preds + ((long)b * P + win) * (K + 1);
  int32_t* em = p.emitted + (long)b * (K + 1);
  for (int i = 0; i <= K; ++i) em[i] = i < m ? dr[i] : (i == m ? pr[m] : 0);
  p.m[b] = m;
  p.n_emitted[b] = m + 1;
  if (p.path) p.path[b] = win;
  if (p.ckpt_index) p.ckpt_index[b] = (b * P + win) * (K + 1) + m;
}

}  // namespace

hipError_t launch_copy(const CopyArgs& p, hipStream_t st) {
  const long per_block = (long)kThreads * kUnroll;
  const long nstate = p.src_state ? p.state_floats / 4 : 0;
  const long ntail = p.src_tail ? p.tail_bytes / 16 : 0;
  const long blocks = (nstate + per_block - 1) / per_block + (ntail + per_block - 1) / per_block;
  if (blocks <= 0 || p.n <= 0) return hipSuccess;
  timing_before("copy", st);
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks, p.n), dim3(kThreads), 0, st, p);
  timing_after(st);
  return hipGetLastError();
}

hipError_t launch_zero(const CopyArgs& p, hipStream_t st) {
  const long per_block = (long)kThreads * kUnroll;
  const long nstate = p.dst_state ? p.state_floats / 4 : 0;
  const long ntail = p.dst_tail ? p.tail_bytes / 16 : 0;
  const long blocks = (nstate + per_block - 1) / per_block + (ntail + per_block - 1) / per_block;
  if (blocks <= 0 || p.n <= 0) return hipSuccess;
  timing_before("zero", st);
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks, p.n), dim3(kThreads), 0, st, p);
  timing_after(st);
  return hipGetLastError();
}

hipError_t launch_accept(const AcceptArgs& p, hipStream_t st) {
  if (p.B <= 0) return hipSuccess;
  timing_before("accept", st);
  hipLaunchKernelGGL(accept_kernel, dim3((p.B + 127) / 128), dim3(128), 0, st, p);
  timing_after(st);
  return hipGetLastError();
}

}  // namespace gdn
