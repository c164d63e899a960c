// Internal launch interface between the C ABI (gdn_api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

// Optional per-launch timing (gdn_timing_begin / gdn_timing_end): every launch site brackets its kernel
// with these; they record HIP events on the launch stream only while a timing session is open.
void timing_before(const char* kernel, hipStream_t st);
void timing_after(hipStream_t st);

constexpr int kActBf16 = 0;
constexpr int kActF32 = 1;

// ---- decode / verify ------------------------------------------------------------------------------
struct StepArgs {
  const void* conv_w;
  const float* A_log;
  const float* dt_bias;
  const float* norm_w;
  const void* mixed;    // [B*P][T][C]
  const void* z;        // [B*P][T][n_v*d_v]
  const void* a;        // [B*P][T][n_v]
  const void* b;        // [B*P][T][n_v]
  const int32_t* slot;  // [B] or null
  const void* tail_in;  // pool [*][3][C]
  const float* state_in;  // pool [*][n_v][d_k][d_v]
  void* tail_out;       // decode: the pool; verify: [B*P*T][3][C]
  float* state_out;     // decode: the pool; verify: [B*P*T][n_v][d_k][d_v]
  void* out;            // [B*P][T][n_v*d_v]
  int out_f32;          // 1: out is fp32 (always with fp32 activations), 0: the activation type
  int B, T, n_k, n_v, C;
  int P;                // rows per sequence: 1, or the paths of a batch-of-paths verify
  int verify;
  float scale, l2_eps, rms_eps;
};
// head dims DK, DV each in {32, 64, 128}; ratio = n_v / n_k
hipError_t launch_step(const StepArgs& p, int act_dtype, int DK, int DV, int ratio, hipStream_t st);

// ---- standalone conv ------------------------------------------------------------------------------
struct ConvArgs {
  const void* conv_w;   // [C][4]
  const void* mixed;    // [B][Lb][C]
  const int32_t* len;   // [B]
  void* tail;           // [B][3][C] in/out
  void* y;              // [B][Lb][C]
  int B, Lb, C;
};
hipError_t launch_conv(const ConvArgs& p, int act_dtype, hipStream_t st);

// ---- chunked prefill ------------------------------------------------------------------------------
constexpr int kChunk = 64;

struct PrefillArgs {
  const void* conv_w;
  const float* A_log;
  const float* dt_bias;
  const float* norm_w;
  const void* mixed;    // [B][Lb][C]
  const void* z;        // [B][Lb][n_v*D]
  const void* a;        // [B][Lb][n_v]
  const void* b;        // [B][Lb][n_v]
  const int32_t* len;   // [B]
  void* tail;           // [B][3][C] in/out
  float* state;         // [B][n_v][D][D] in/out
  void* out;            // [B][Lb][n_v*D]
  int out_f32;          // 1: out is fp32 (always with fp32 activations), 0: the activation type
  void* ws;             // workspace: value records, key records (n_v > n_k), then (split heads only)
                        // the partial sums of squares of every row, one per slice ([sequence][head]
                        // [token][slice] for the exchange, [sequence][token][head][slice] for a norm
                        // pass), and the unnormalised o for a norm pass
  long key_off, ss_off, oraw_off;  // byte offsets inside ws: key records, partial sums, unnormalised o
  int B, Lb, n_k, n_v, C, n_chunks;
  int grp;              // value heads per chunk_prep workgroup (a divisor of n_v / n_k: 1, 2 or 4)
  int nsplit;           // column slices per head in the state pass (1: the whole head)
  int exchange;         // split heads: 1 = the slices exchange row sums, 0 = a norm pass finishes
  int* status;          // device word: bit 0 set when a final state leaves the operand range (or null)
  float scale, l2_eps, rms_eps;
  float rms_n;          // columns the gated RMSNorm averages over: d_v (below D in a call run on
                        // zero-padded heads, whose extra columns of o are exactly zero)
};
// fp32 activations run every MFMA operand as a hi/lo pair (split_all) up to d = 64; at d = 128 they
// take the bf16 operand precisions
// value heads per chunk_prep workgroup: the GQA ratio n_v / n_k where a kernel is built for it (1, 2,
// 4), else its largest divisor among 4, 2, 1 (each group then forms the shared q and k again); one
// where the grid would be too small to fill the device
int prefill_group(int n_k, int n_v, int D, bool act_f32, int B, int n_chunks);
size_t prefill_ws_bytes(int B, int n_k, int n_v, int D, int Lb, int n_chunks, bool act_f32);
void prefill_ws_layout(PrefillArgs& p, int D, bool act_f32);
hipError_t launch_prefill(const PrefillArgs& p, int act_dtype, int D, int R, hipStream_t st);

// ---- zero-padded heads (prefill with d_k != d_v) --------------------------------------------------
// A row of channels [q: n_k heads of dk | k: n_k heads of dk | v: n_v heads of dv], counted in 16-byte
// units, and its padded form with every head widened to D units (n_k = 0 describes a row of value
// heads only: z, out, norm_w).
struct ChanMap {
  int n_k, n_v, dk, dv, D;
};
// dst [rows][Ud] padded (zero units where the original has none) from src [rows][Us]
hipError_t launch_pad_units(const void* src, void* dst, long rows, int Us, int Ud, const ChanMap& m, hipStream_t st);
// dst [rows][Ud] original from src [rows][Us] padded; with len (rows = [B][Lb]) only rows t < len[b]
hipError_t launch_unpad_units(const void* src, void* dst, long rows, int Us, int Ud, const ChanMap& m,
                              const int32_t* len, int Lb, hipStream_t st);
// fp32 states: [mats][D][D] (zero outside dk x dv) from [mats][dk][dv], and back
hipError_t launch_pad_state(const float* src, float* dst, long mats, int dk, int dv, int D, hipStream_t st);
hipError_t launch_unpad_state(const float* src, float* dst, long mats, int dk, int dv, int D, hipStream_t st);

// ---- fused prefill (d_k = d_v = 128, bf16 activations) ----------------------------------------------
struct FusedArgs {
  const void* conv_w;
  const float* A_log;
  const float* dt_bias;
  const float* norm_w;
  const void* mixed;    // [B][Lb][C]
  const void* z;        // [B][Lb][n_v*128]
  const void* a;        // [B][Lb][n_v]
  const void* b;        // [B][Lb][n_v]
  const int32_t* len;   // [B]
  void* tail;           // [B][3][C] in/out (updated by the last launch of the call)
  float* state;         // [B][n_v][128][128] in/out
  void* out;            // [B][Lb][n_v*128]
  int out_f32;          // 1: out is fp32, 0: bf16
  void* ws;             // segment maps and states (nseg > 1), else unused
  float* seg_map;       // [B][n_v][nseg-1][2][128][128]: N_s, M_s (set by launch_fused)
  float* seg_in;        // [B][n_v][nseg][128][128]: entering state of segment s >= 1 (set by launch_fused)
  int* status;          // device word: bit 0 set when a final state leaves the operand range (or null)
  int B, Lb, n_k, n_v, C;
  int nseg, seg_chunks; // segments per (sequence, head) and chunks per segment
  float scale, l2_eps, rms_eps;
};
// compute units of the current device (read once per device; 0 if unknown)
int device_cus();
// segment plan of a call (nseg = 1: one workgroup per (sequence, head) walks every chunk)
void fused_plan(int B, int n_v, int Lb, int& nseg, int& seg_chunks);
size_t fused_ws_bytes(int B, int n_v, int Lb);
hipError_t launch_fused(FusedArgs p, hipStream_t st);

// ---- state records and accept ---------------------------------------------------------------------
struct CopyArgs {
  float* dst_state;
  void* dst_tail;
  const int32_t* dst_idx;
  const float* src_state;
  const void* src_tail;
  const int32_t* src_idx;
  long state_floats;   // per record
  long tail_bytes;     // per record
  int n;
};
hipError_t launch_copy(const CopyArgs& p, hipStream_t st);
hipError_t launch_zero(const CopyArgs& p, hipStream_t st);  // dst pointers and dst_idx only

struct AcceptArgs {
  const int32_t* drafts;  // [B][P][K]
  const int32_t* preds;   // [B][P][K+1]
  int32_t* m;
  int32_t* emitted;
  int32_t* n_emitted;
  int32_t* ckpt_index;
  int32_t* path;          // winning path per sequence, or null (P = 1)
  int B, K, P;
};
hipError_t launch_accept(const AcceptArgs& p, hipStream_t st);

// ---- measurement aid ------------------------------------------------------------------------------
// blocks x 256 threads, each wave 2 chains x iters f16 MFMAs of 32x32x16; sink [blocks * 256] floats
hipError_t launch_mfma_probe(float* sink, int blocks, int iters, hipStream_t st);

}  // namespace gdn
