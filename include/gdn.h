/*
 * gdn.h — C ABI of libgdn.so: the Gated DeltaNet (gated delta-rule) layer hot path on MI355X (gfx950).
 *
 * The layer (as the "qev_fast/statecache.py" page's CacheQwen35._gdn runs it on one chunk continued
 * from a saved state): a causal depthwise conv1d + SiLU over [saved Kc inputs | chunk], the q|k|v
 * channel split, the gates g = -exp(A_log) * softplus(a + dt_bias) and beta = sigmoid(b) with padding
 * masked to g = 0 and beta = 0, q/k L2-normalised per key head, value head h reading key head
 * h / (n_v / n_k), the delta rule
 *     S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = scale * S_t q_t,
 * the fp32 final state written back in place, and the gated RMSNorm w * o / rms(o) * silu(z).
 *
 * Conventions shared by every entry point
 *  - All pointers are caller-owned DEVICE buffers, contiguous, row-major (last index fastest), of
 *    exactly the shape stated, unless marked "host". The library never allocates or frees device
 *    memory; prefill takes a caller workspace. Buffers updated in place keep their addresses (the
 *    "uni_engine.py" page's copy_cache_: destination storage already materialised, addresses kept).
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the default stream); nothing
 *    synchronises with the host. A non-zero return means nothing was launched, except GDN_EHIP
 *    which reports a launch failure; gdn_last_error() then holds a message (thread-local).
 *  - Activation buffers (mixed, z, a, b, out, conv tails, conv_w, y) have dtype desc->act_dtype:
 *    GDN_BF16 (bfloat16) or GDN_F32. Recurrent states and checkpoints are fp32. A_log, dt_bias and
 *    norm_w are fp32. Lengths, slots and indices are int32.
 *  - Index arrays living on the device (len, slot, *_idx) are not range-checked on the device: an
 *    out-of-range value is undefined behaviour. The Python binding checks host copies first.
 *  - State layout per sequence: [n_v][d_k][d_v] (H = S^T, the layout the statecache.py page's
 *    StateCache allocates). Conv tail per sequence: [Kc][C_ch], Kc = conv_k - 1, oldest row first,
 *    C_ch = 2*n_k*d_k + n_v*d_v with channels ordered [q heads | k heads | v heads], head-major.
 *
 * Status codes: GDN_OK = 0; GDN_EINVAL = -1 (null pointer, non-positive size, inconsistent sizes,
 * workspace too small); GDN_EUNSUPPORTED = -2 (a shape outside the layer's definition: d_k or d_v not
 * in {32, 64, 128}, conv_k != 4 or n_v not a multiple of n_k; the caller falls back, as the
 * statecache.py page's StateCache falls back to the plain path on _NotCached); GDN_EHIP = -3. Every
 * pair of head dims is built, d_k != d_v included (prefill then runs the square kernels at max(d_k,
 * d_v) on zero-padded copies in its workspace, which is exact). Every GQA ratio n_v / n_k is built;
 * ratios other than 1, 2 and 4 run their value heads 4, 2 or 1 at a time (the largest that divides
 * the ratio), forming the shared q and k once per group. Prefill with fp32 activations carries every MFMA operand as a hi/lo pair up to d =
 * 64; at d = 128 it uses the operand precisions of bf16 activations (same output and state bounds).
 *
 * Value range (prefill): the chunked prefill carries the state, the write vectors u and the keys and
 * queries as pairs of f16 values scaled by 2^8 (about 22 bits), so |state| and |u| must stay below 255.
 * Activations of unit scale keep them far below (the saved states of the tests are within |S| < 10). A
 * prefill whose final state leaves that range, or is not finite, sets GDN_STATUS_RANGE in the device
 * status word (gdn_device_status); decode and verify run fp32 throughout and have no such limit.
 *
 * Strong decays (prefill): the chunked form floors each token's log-decay g at -30, so a decay factor
 * below e^-30 (about 9.4e-14) counts as e^-30 and a full forget (a = +inf, g = -inf) keeps that fraction
 * of the state instead of none. Without the floor the in-chunk sums of g would lose accuracy, and a
 * full forget would give NaN. Decode and verify take e^g as it is.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* gdn_stream_t; /* the same handle as hipStream_t */

enum { GDN_OK = 0, GDN_EINVAL = -1, GDN_EUNSUPPORTED = -2, GDN_EHIP = -3 };
enum { GDN_BF16 = 0, GDN_F32 = 1 };
enum { GDN_OUT_ACT = 0 };

/* Layer shape and constants (host struct, read during the call only). */
typedef struct {
  int32_t n_k, n_v;   /* key heads, value heads; n_v % n_k == 0 */
  int32_t d_k, d_v;   /* head dims, each in {32, 64, 128} */
  int32_t conv_k;     /* conv kernel width; must be 4 */
  int32_t act_dtype;  /* GDN_BF16 or GDN_F32 */
  float scale;        /* q scale; <= 0 selects d_k^-1/2 */
  float l2_eps;       /* q/k L2 norm: x / sqrt(sum x^2 + l2_eps) */
  float rms_eps;      /* gated RMSNorm epsilon */
  int32_t out_dtype;  /* dtype of `out` in prefill, decode and verify: GDN_OUT_ACT (0) = the activation
                         dtype, or GDN_F32 = fp32 (with bf16 activations: the output before its bf16
                         rounding) */
} gdn_desc;

/* Layer weights (host struct holding device pointers). */
typedef struct {
  const void* conv_w;   /* [C_ch][conv_k], act dtype; tap conv_k-1 meets the current token */
  const float* A_log;   /* [n_v] */
  const float* dt_bias; /* [n_v] */
  const float* norm_w;  /* [d_v], shared by all value heads */
} gdn_weights;

/* Message for the last non-zero status returned on this thread ("" if none). */
const char* gdn_last_error(void);

/* Library version string. */
const char* gdn_version(void);

/*
 * Conditions found on the device by earlier calls, as bits (host function; synchronizes `stream`,
 * then reads the device's status word, and clears it when `clear` is non-zero). Returns the bits
 * (>= 0) or GDN_EHIP. Bit 0 (GDN_STATUS_RANGE): a prefill's final state left the range its f16
 * operand pairs carry (|state| >= 255 or not finite); that call's state and outputs are not to be
 * trusted. Bit 1 (GDN_STATUS_EXCHANGE): in a prefill whose head columns were split over workgroups
 * that exchange row sums for the gated norm, a workgroup waited in vain for another's sums; the rows
 * concerned were written as NaN. The exchange is only launched cooperatively (the runtime guarantees
 * that every workgroup is resident, or refuses, and the call then finishes the norm in a separate pass)
 * and never under graph capture, so this bit marks a fault, not a case the library expects. Kernels
 * only set bits, so the word collects every call since it was last cleared, on every stream of the
 * device.
 */
enum { GDN_STATUS_RANGE = 1, GDN_STATUS_EXCHANGE = 2 };
int gdn_device_status(int clear, gdn_stream_t stream);

/*
 * Causal conv1d + SiLU over [conv_tail | mixed] (statecache.py page, CacheQwen35._gdn: the conv on
 * [saved conv inputs | chunk], no bias, SiLU, the first Kc outputs dropped; then the tail copy).
 *   mixed     [B][Lb][C_ch]   pre-conv inputs of one padded chunk per sequence
 *   len       [B]             real lengths, 0 <= len[b] <= Lb (device)
 *   conv_tail [B][Kc][C_ch]   in/out: replaced by rows len[b] .. len[b]+Kc-1 of [tail | mixed],
 *                             i.e. the last Kc real inputs, old rows kept when len[b] < Kc
 *   y         [B][Lb][C_ch]   y[t][c] = silu(sum_j conv_w[c][j] * xin[t+j][c]); rows >= len[b] are
 *                             computed like the others and carry no meaning
 * Limits: ceil(C_ch / 1024) * ceil(Lb / 64) * B < 2^31 (GDN_EINVAL otherwise).
 * Must not alias: y with mixed or conv_tail.
 */
int gdn_conv_chunk(const gdn_desc* desc, const void* conv_w, const void* mixed, const int32_t* len,
                   void* conv_tail, void* y, int B, int Lb, gdn_stream_t stream);

/* Bytes of device workspace gdn_prefill_chunk needs for B sequences of Lb padded tokens (0 when the
 * shape is not built). With d_k != d_v it includes zero-padded copies of the call's inputs, conv weights,
 * tail, state and output at max(d_k, d_v). The size never shrinks as Lb grows, so a workspace sized for
 * the longest call serves every shorter one. */
size_t gdn_prefill_workspace_bytes(const gdn_desc* desc, int B, int Lb);

/*
 * One padded chunk per sequence through the whole layer, continued from the saved state
 * (statecache.py page, CacheQwen35._gdn; padding gets g = 0 and beta = 0 so the state stops at the
 * real end, as that page's module text says).
 *   mixed [B][Lb][C_ch], z [B][Lb][n_v*d_v], a and b [B][Lb][n_v]: projected inputs
 *   len   [B] real lengths (device), 0 <= len[b] <= Lb
 *   conv_tail [B][Kc][C_ch] in/out (as gdn_conv_chunk); state [B][n_v][d_k][d_v] fp32 in/out
 *   out   [B][Lb][n_v*d_v] gated-RMSNorm output; rows >= len[b] carry no meaning
 *   ws    device workspace of at least gdn_prefill_workspace_bytes(desc, B, Lb) bytes, 256-aligned;
 *         its contents on entry do not matter and are garbage on return; it serves one call at a
 *         time (calls that may overlap, e.g. on two streams, need workspaces of their own)
 * Limits: B <= 65535, Lb * n_v * max(d_k, d_v) < 2^31 and B * ceil(Lb / 64) * n_v < 2^31 (GDN_EINVAL
 * otherwise).
 * Must not alias: out with any input; state or conv_tail with anything else.
 */
int gdn_prefill_chunk(const gdn_desc* desc, const gdn_weights* w, const void* mixed, const void* z,
                      const void* a, const void* b, const int32_t* len, void* conv_tail, float* state,
                      void* out, int B, int Lb, void* ws, size_t ws_bytes, gdn_stream_t stream);

/*
 * gdn_prefill_chunk for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same call without a workspace argument. The
 * library's own static device scratch of 64 MiB serves as the workspace; nothing is allocated.
 *   Path: the one gdn_prefill_chunk takes when its workspace fits the scratch; otherwise, for d = 128
 *   with bf16 activations, the fused path with segment maps (at most 32 MiB); results of either path
 *   meet the layer's bounds against the oracle.
 *   Errors: GDN_EINVAL, with nothing launched, when the call needs more workspace than the scratch
 *   holds (other shapes with very long calls); otherwise as gdn_prefill_chunk.
 *   Concurrency: every call on one device shares that device's scratch, which keeps the last call's
 *   contents; calls that may overlap on one device (two streams, two threads) race and must be
 *   serialised by the caller.
 */
int gdn_prefill_chunk_noalloc(const gdn_desc* desc, const gdn_weights* w, const void* mixed, const void* z,
                              const void* a, const void* b, const int32_t* len, void* conv_tail, float* state,
                              void* out, int B, int Lb, gdn_stream_t stream);

/*
 * One decode token for each of B sequences: the layer with Lb = len = 1 (the "uni_engine.py" page's
 * decode path, which advances every sequence's conv and recurrent state by one token in place, and the
 * per-token step of the "mtp/generate.py" page's decode loop), in fp32 throughout.
 *   mixed [B][C_ch], z [B][n_v*d_v], a and b [B][n_v]
 *   slot  [B] rows of the pools that sequence b owns (device), or NULL for slot[b] = b; slots must
 *         be distinct
 *   conv_tail_pool [*][Kc][C_ch], state_pool [*][n_v][d_k][d_v]: row slot[b] updated in place
 *   out   [B][n_v*d_v]
 */
int gdn_decode_step(const gdn_desc* desc, const gdn_weights* w, const void* mixed, const void* z,
                    const void* a, const void* b, const int32_t* slot, void* conv_tail_pool,
                    float* state_pool, void* out, int B, gdn_stream_t stream);

/*
 * Verify with per-token checkpoints (the "mtp/generate.py" page: forward_with_hidden_stepwise runs
 * the verify tokens one at a time and snapshots the cache after each; its batched multistate
 * kernel captures the same per-token states in one pass). T tokens per sequence run one at a time,
 * with exactly the decode-step arithmetic, from the pool row slot[b], which is NOT modified.
 *   mixed [B][T][C_ch], z [B][T][n_v*d_v], a and b [B][T][n_v], slot as in gdn_decode_step
 *   ckpt_state [B][T][n_v][d_k][d_v]: state after tokens 0..i (checkpoint i)
 *   ckpt_tail  [B][T][Kc][C_ch]:      conv tail after tokens 0..i
 *   out        [B][T][n_v*d_v]
 * Checkpoint i is bitwise equal to i+1 gdn_decode_step calls on the same inputs.
 */
int gdn_verify_with_checkpoints(const gdn_desc* desc, const gdn_weights* w, const void* mixed,
                                const void* z, const void* a, const void* b, int T, const int32_t* slot,
                                const void* conv_tail_pool, const float* state_pool, float* ckpt_state,
                                void* ckpt_tail, void* out, int B, gdn_stream_t stream);

/*
 * Accepted prefix of a speculative verify (mtp/generate.py page: accept_prefix, and its caller's
 * emitted tokens drafts[:m] + [preds[m]]). Integer work, bit-exact.
 *   drafts [B][K], preds [B][K+1] (device)
 *   m [B]          longest prefix length with preds[j] == drafts[j], j < K
 *   emitted [B][K+1]  drafts[:m], then preds[m], then zeros
 *   n_emitted [B]  m + 1
 *   ckpt_index [B] b*(K+1) + m: the verify checkpoint row (of [B*(K+1)] records when the verify
 *                  ran T = K+1 tokens) to restore; may be NULL
 */
int gdn_accept(const int32_t* drafts, const int32_t* preds, int B, int K, int32_t* m, int32_t* emitted,
               int32_t* n_emitted, int32_t* ckpt_index, gdn_stream_t stream);

/*
 * Batch-of-paths (tree) verify (mtp/generate.py page, tree_verify_step: P candidate paths per
 * sequence, the cache tiled into one row per path, every row an ordinary linear sequence). Row
 * bp = b*P + p runs path p of sequence b: T tokens one at a time from pool row slot[b] (or b), which
 * every path of b shares and which is read, never written; the kernel is the one
 * gdn_verify_with_checkpoints runs, so each row is bitwise that call on the row's tokens.
 *   mixed [B][P][T][C_ch], z [B][P][T][n_v*d_v], a and b [B][P][T][n_v]
 *   ckpt_state [B][P][T][n_v][d_k][d_v], ckpt_tail [B][P][T][Kc][C_ch]: record bp*T + t holds the
 *              state and tail after token t of row bp
 *   out [B][P][T][n_v*d_v]
 * Limits: B * P <= 65535. Checkpoints must not alias the pools (GDN_EINVAL).
 */
int gdn_verify_paths(const gdn_desc* desc, const gdn_weights* w, const void* mixed, const void* z,
                     const void* a, const void* b, int T, int P, const int32_t* slot,
                     const void* conv_tail_pool, const float* state_pool, float* ckpt_state, void* ckpt_tail,
                     void* out, int B, gdn_stream_t stream);

/*
 * Winner of a batch-of-paths verify (mtp/generate.py page, tree_verify_step): every path's accepted
 * prefix as in gdn_accept; the winner is the first path with the longest one (ties go to the earlier
 * path). Integer work, bit-exact.
 *   drafts [B][P][K], preds [B][P][K+1] (device)
 *   m [B], path [B]   the winner's prefix length and index
 *   emitted [B][K+1]  the winner's drafts[:m], then its preds[m], then zeros; n_emitted [B] = m + 1
 *   ckpt_index [B]    (b*P + path)*(K+1) + m: the checkpoint record of gdn_verify_paths (run with
 *                     T = K+1) to commit with gdn_state_copy; may be NULL
 * Limits: B * P * (K+1) < 2^31.
 */
int gdn_accept_paths(const int32_t* drafts, const int32_t* preds, int B, int P, int K, int32_t* m, int32_t* path,
                     int32_t* emitted, int32_t* n_emitted, int32_t* ckpt_index, gdn_stream_t stream);

/*
 * Copy n fixed-size state records {fp32 state [n_v][d_k][d_v], conv tail [Kc][C_ch]} — O(1) in
 * context length (uni_engine.py page: copy_cache_, cache_payload_bytes, the bridge). Record i goes
 * from src row src_idx[i] (or i when src_idx is NULL) to dst row dst_idx[i] (or i). Either tail
 * pointer pair may be NULL to copy states only; both state pointers may be NULL to copy tails only.
 * Destination rows must be distinct and must not overlap source rows read by the same call.
 * Commit after verify = gdn_state_copy from the checkpoint records (src_idx = ckpt_index) into the
 * pools (dst_idx = slot).
 */
int gdn_state_copy(const gdn_desc* desc, float* dst_state, void* dst_tail, const int32_t* dst_idx,
                   const float* src_state, const void* src_tail, const int32_t* src_idx, int n,
                   gdn_stream_t stream);

/* Bytes of one state record: n_v*d_k*d_v*4 + Kc*C_ch*sizeof(act) (uni_engine.py page,
 * cache_payload_bytes per sequence per layer). */
size_t gdn_state_record_bytes(const gdn_desc* desc);

/*
 * Prefix-state cache ("qev_fast/statecache.py" page, StateCache): host bookkeeping only, no HIP call.
 * A checkpoint is the fp32 state and conv tail of one sequence after the first `pos` tokens of an
 * earlier row, held in one slot of a caller-owned record pool (slots 0 .. slots-1; one slot may hold a
 * record per GDN layer). For each new row the cache finds the deepest checkpoint whose tokens the row
 * shares, and books checkpoints at the chunk ends the page places: multiples of `stride`, p - tail and
 * p (p = the row's checkpointable prefix, min(p_state, n) rounded down to `align`), no chunk longer than
 * `max_chunk`. With more checkpoints than slots, the least recently used ones go (starting a row from a
 * checkpoint counts as a use). Rows with p < min_prefix take the plain path: no lookup, no checkpoints.
 * Only the recurrent state is cached; the attention K / V of the page's cache belongs to other layers.
 *
 * gdn_pcache_row plans and books one row (ids: its n tokens, host memory). It writes
 *   info[4]       = {restore slot or -1 (start from zero), c0 = tokens the restore covers, p, n_bounds}
 *   bounds[i]     chunk ends in (c0, p], ascending: run [c0, bounds[0]), [bounds[0], bounds[1]), ...,
 *                 then [p, n); after the chunk ending at bounds[i], copy the state into snap_slot[i]
 *                 (-1: that checkpoint was evicted at once, skip the copy)
 *   ckpt[1 + cap] (may be NULL) the restored checkpoint's number, then the new checkpoints' numbers
 *                 (numbers count checkpoints in the order they are made; -1 for none / evicted)
 * and returns n_bounds, or GDN_EINVAL (nothing booked) for bad arguments or n_bounds > cap. The restore
 * must be issued before the snapshots: the restored slot may be handed to a new checkpoint of the row.
 * The plan holds for GPU work issued in order on one stream. Not thread-safe.
 * gdn_pcache_stats copies the GDN_PCACHE_NSTATS counters; gdn_pcache_alive writes the numbers of the
 * live checkpoints (ascending, at most cap) and returns how many there are.
 */
typedef struct gdn_pcache gdn_pcache;
enum {
  GDN_PCACHE_ROWS = 0,          /* rows that looked the cache up */
  GDN_PCACHE_HITS,              /* ... that found a checkpoint at p */
  GDN_PCACHE_PARTIAL,           /* ... that found one before p */
  GDN_PCACHE_COLD,              /* ... that found none */
  GDN_PCACHE_PLAIN,             /* rows too short to checkpoint */
  GDN_PCACHE_TOKENS_REUSED,
  GDN_PCACHE_TOKENS_COMPUTED,
  GDN_PCACHE_CKPTS_MADE,
  GDN_PCACHE_EVICTED,
  GDN_PCACHE_ROWS_KEPT,         /* rows whose token ids are kept: those with a live checkpoint (a gauge) */
  GDN_PCACHE_NSTATS
};
int gdn_pcache_create(int slots, int stride, int tail, int align, int max_chunk, int min_prefix, gdn_pcache** out);
void gdn_pcache_destroy(gdn_pcache* cache);
int gdn_pcache_row(gdn_pcache* cache, const int32_t* ids, int n, int p_state, int cap, int32_t* info, int32_t* bounds,
                   int32_t* snap_slot, int64_t* ckpt);
int gdn_pcache_stats(const gdn_pcache* cache, int64_t* stats);
int gdn_pcache_alive(const gdn_pcache* cache, int cap, int64_t* nums);

/*
 * Zero n state records {fp32 state [n_v][d_k][d_v], conv tail [Kc][C_ch]}: record idx[i] (or i when idx
 * is NULL) of each pool. Either pool may be NULL. The start of a row that no checkpoint covers.
 */
int gdn_state_zero(const gdn_desc* desc, float* state, void* tail, const int32_t* idx, int n, gdn_stream_t stream);

/*
 * Per-launch timing, for measurement (not part of the method). gdn_timing_begin opens a session on the
 * calling thread: until gdn_timing_end, every kernel the library launches from this thread is
 * bracketed by two HIP events recorded on the launch stream (at most `capacity` launches, 1..65536;
 * later ones are not timed). The events are created here, on the host side of the runtime; no
 * device memory is allocated and nothing synchronises until the end.
 * gdn_timing_end waits for the recorded events, writes the first `cap` launches in launch order as
 * (static kernel name, milliseconds) into kernels[] and ms[] (either may be NULL), closes the session
 * and returns the number of launches recorded, or a negative status (GDN_EINVAL: no open session,
 * GDN_EHIP: an event failed). Kernel names: "conv", "chunk_prep", "state_pass", "norm", "zero",
 * "step_decode", "step_verify", "copy", "accept", "mfma_probe".
 */
int gdn_timing_begin(int capacity);
/*
 * MFMA throughput probe, for measurement (not part of the method): blocks x 256 threads, every wave
 * issuing 2 independent chains of `iters` f16 32x32x16 MFMAs (2 * 32 * 32 * 16 FLOP each), so a run
 * does blocks * 4 * 2 * iters * 32768 FLOP. sink: device buffer of blocks * 256 floats (written).
 * Time it with the timing session (kernel name "mfma_probe") or the caller's events.
 */
int gdn_mfma_probe(float* sink, int blocks, int iters, gdn_stream_t stream);
int gdn_timing_end(const char** kernels, float* ms, int cap);

#ifdef __cplusplus
}
#endif
#endif /* GDN_H */
