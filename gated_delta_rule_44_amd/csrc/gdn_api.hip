// The C ABI of libgdn.so (declared in include/gdn.h): argument checks, then kernel launches on the
// caller's stream. Nothing here allocates device memory; only gdn_timing_end (a measurement aid)
// synchronises with the host.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include <new>

#include "gdn.h"
#include "gdn_kernels.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) {
    g_err[0] = 0;
    return GDN_OK;
  }
  return fail(GDN_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

long conv_channels(const gdn_desc* d) { return 2L * d->n_k * d->d_k + (long)d->n_v * d->d_v; }

// shape checks shared by the layer entry points
int check_desc(const gdn_desc* d) {
  if (!d) return fail(GDN_EINVAL, "desc is NULL");
  if (d->n_k <= 0 || d->n_v <= 0) return fail(GDN_EINVAL, "n_k=%d n_v=%d must be positive", d->n_k, d->n_v);
  if (d->act_dtype != GDN_BF16 && d->act_dtype != GDN_F32) return fail(GDN_EINVAL, "act_dtype=%d", d->act_dtype);
  if (d->conv_k != 4) return fail(GDN_EUNSUPPORTED, "conv_k=%d (only 4 is built)", d->conv_k);
  if (d->n_v % d->n_k) return fail(GDN_EUNSUPPORTED, "n_v=%d is not a multiple of n_k=%d", d->n_v, d->n_k);
  if (d->d_k != 32 && d->d_k != 64 && d->d_k != 128)
    return fail(GDN_EUNSUPPORTED, "d_k=%d (built: 32, 64, 128)", d->d_k);
  if (d->d_v != 32 && d->d_v != 64 && d->d_v != 128)
    return fail(GDN_EUNSUPPORTED, "d_v=%d (built: 32, 64, 128)", d->d_v);
  if (!(d->l2_eps >= 0.f) || !(d->rms_eps >= 0.f)) return fail(GDN_EINVAL, "negative or NaN epsilon");
  if (d->out_dtype != GDN_OUT_ACT && d->out_dtype != GDN_F32) return fail(GDN_EINVAL, "out_dtype=%d", d->out_dtype);
  return GDN_OK;
}

// fp32 outputs: with fp32 activations always, with bf16 ones when the caller asks for them
int out_f32(const gdn_desc* d) { return d->act_dtype == GDN_F32 || d->out_dtype == GDN_F32 ? 1 : 0; }

// Prefill path. The fused kernel (one workgroup per (sequence, value head) walking its chunks, nothing
// staged in HBM) serves d_k = d_v = 128 with bf16 activations once the units fill most of the chip:
// measured on 16/32 heads, it is level with the two-launch path at 192 units (6 x 4096 tokens) and
// 12% faster at 256 (8 x 8192); with fewer units the two-launch path, which spreads a head's state
// pass over several CUs, is faster. GDN_PREFILL_PATH in the environment overrides the choice for
// tests and comparisons: "fused" (with segment maps and a scan for few units) or "two_phase".
constexpr long kFusedMinUnits = 192;
bool fused_built(const gdn_desc* d) { return d->d_k == 128 && d->d_v == 128 && d->act_dtype == GDN_BF16; }
bool use_fused(const gdn_desc* d, int B) {
  if (!fused_built(d)) return false;
  const char* e = getenv("GDN_PREFILL_PATH");
  if (e && strcmp(e, "fused") == 0) return true;
  if (e && strcmp(e, "two_phase") == 0) return false;
  return (long)B * d->n_v >= kFusedMinUnits;
}

float q_scale(const gdn_desc* d) { return d->scale > 0.f ? d->scale : 1.0f / sqrtf((float)d->d_k); }

int check_weights(const gdn_weights* w) {
  if (!w) return fail(GDN_EINVAL, "weights is NULL");
  if (!w->conv_w || !w->A_log || !w->dt_bias || !w->norm_w) return fail(GDN_EINVAL, "a weight pointer is NULL");
  if (!aligned16(w->conv_w)) return fail(GDN_EINVAL, "conv_w must be 16-byte aligned");
  return GDN_OK;
}

// ---- per-launch timing session (diagnostics) ----
struct TimedLaunch {
  const char* kernel;
  hipEvent_t start, stop;
};
thread_local TimedLaunch* t_launch = nullptr;  // open session: capacity t_cap, t_used recorded
thread_local int t_cap = 0, t_used = 0;

}  // namespace

// Device status word: kernels set bits in it (atomic OR) for conditions found on the device, which
// gdn_device_status reports. Bit 0: a prefill's exit state (final state or segment map) left the range
// its f16 operands can hold (|H| >= 255, or not finite).
__device__ int gdn_status_word;

// Workspace of gdn_prefill_chunk_noalloc: a file-scope device array (each device that loads the library
// holds its own copy until the process ends). Host code only ever uses its device address, looked up
// per device with hipGetSymbolAddress: the array's name on the host is a host-side stand-in.
constexpr size_t kScratchBytes = 64ull << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
// the word's device address on the current device (each device holds its own copy), looked up once
int* status_ptr() {
  static int* ptr[64];
  static std::once_flag once[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::call_once(once[dev], [dev] {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(gdn_status_word)) != hipSuccess) {
      (void)hipGetLastError();
      p = nullptr;
    }
    ptr[dev] = (int*)p;
  });
  return ptr[dev];
}
}  // namespace

namespace {
// the scratch array's address on the current device, looked up once per device (with that device current)
void* scratch_ptr() {
  static void* ptr[64];
  static std::once_flag once[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::call_once(once[dev], [dev] {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      p = nullptr;
    }
    ptr[dev] = p;
  });
  return ptr[dev];
}
}  // namespace

namespace {

// ---- prefill with d_k != d_v: the square kernels at D = max(d_k, d_v) on zero-padded copies ----
// Workspace: the padded inputs, weights, conv tail, state and output, then the square call's own.
struct PadLayout {
  int D;
  long Cp;
  size_t mixed, z, out, tail, state, conv_w, norm_w, inner, total;
};

PadLayout pad_layout(const gdn_desc* d, int B, int Lb) {
  PadLayout L{};
  L.D = d->d_k > d->d_v ? d->d_k : d->d_v;
  L.Cp = (2L * d->n_k + d->n_v) * L.D;
  const size_t act = d->act_dtype == GDN_BF16 ? 2 : 4, oel = out_f32(d) ? 4 : act;
  const size_t rows = (size_t)B * Lb;
  size_t off = 0;
  auto take = [&off](size_t n) {
    const size_t o = off;
    off += (n + 255) / 256 * 256;
    return o;
  };
  L.mixed = take(rows * L.Cp * act);
  L.z = take(rows * d->n_v * L.D * act);
  L.out = take(rows * d->n_v * L.D * oel);
  L.tail = take((size_t)B * (d->conv_k - 1) * L.Cp * act);
  L.state = take((size_t)B * d->n_v * L.D * L.D * 4);
  L.conv_w = take((size_t)L.Cp * d->conv_k * act);
  L.norm_w = take((size_t)L.D * 4);
  L.inner = off;
  const int n_chunks = (Lb + gdn::kChunk - 1) / gdn::kChunk;
  L.total = off + gdn::prefill_ws_bytes(B, d->n_k, d->n_v, L.D, Lb, n_chunks, d->act_dtype == GDN_F32);
  return L;
}

// Copies in, the square two-launch prefill, copies out, all on `stream`. The RMSNorm averages over
// the d_v real columns (the padded columns of o are exactly zero). Output rows past a sequence's length
// are left unwritten, as in the square call.
int prefill_padded(const gdn_desc* d, const gdn_weights* w, const void* mixed, const void* z, const void* a,
                   const void* b, const int32_t* len, void* conv_tail, float* state, void* out, int B, int Lb,
                   void* ws, gdn_stream_t stream) {
  const hipStream_t st = (hipStream_t)stream;
  const PadLayout L = pad_layout(d, B, Lb);
  char* base = (char*)ws;
  const int act = d->act_dtype == GDN_BF16 ? 2 : 4, oel = out_f32(d) ? 4 : act, Kc = d->conv_k - 1;
  const int ga = 16 / act;              // activation channels per 16-byte unit
  const int gw = 16 / (act * d->conv_k);  // conv_w channels per unit (all conv_k taps of a channel)
  const int go = 16 / oel;              // output channels per unit
  const gdn::ChanMap chan{d->n_k, d->n_v, d->d_k / ga, d->d_v / ga, L.D / ga};
  const gdn::ChanMap vchan{0, d->n_v, 0, d->d_v / ga, L.D / ga};
  const gdn::ChanMap wchan{d->n_k, d->n_v, d->d_k / gw, d->d_v / gw, L.D / gw};
  const gdn::ChanMap nchan{0, 1, 0, d->d_v / 4, L.D / 4};
  const gdn::ChanMap ochan{0, d->n_v, 0, d->d_v / go, L.D / go};
  const int C = (int)conv_channels(d), Cp = (int)L.Cp;
  const long rows = (long)B * Lb, mats = (long)B * d->n_v;
  hipError_t e = hipSuccess;
  auto ok = [&e](hipError_t r) {
    if (e == hipSuccess) e = r;
    return e == hipSuccess;
  };
  if (ok(gdn::launch_pad_units(mixed, base + L.mixed, rows, C / ga, Cp / ga, chan, st)) &&
      ok(gdn::launch_pad_units(z, base + L.z, rows, d->n_v * d->d_v / ga, d->n_v * L.D / ga, vchan, st)) &&
      ok(gdn::launch_pad_units(conv_tail, base + L.tail, (long)B * Kc, C / ga, Cp / ga, chan, st)) &&
      ok(gdn::launch_pad_state(state, (float*)(base + L.state), mats, d->d_k, d->d_v, L.D, st)) &&
      ok(gdn::launch_pad_units(w->conv_w, base + L.conv_w, 1, C / gw, Cp / gw, wchan, st)) &&
      ok(gdn::launch_pad_units(w->norm_w, base + L.norm_w, 1, d->d_v / 4, L.D / 4, nchan, st))) {
    gdn::PrefillArgs p{};
    p.conv_w = base + L.conv_w; p.A_log = w->A_log; p.dt_bias = w->dt_bias; p.norm_w = (const float*)(base + L.norm_w);
    p.mixed = base + L.mixed; p.z = base + L.z; p.a = a; p.b = b; p.len = len; p.tail = base + L.tail;
    p.state = (float*)(base + L.state); p.out = base + L.out;
    p.ws = base + L.inner; p.B = B; p.Lb = Lb; p.n_k = d->n_k; p.n_v = d->n_v; p.C = Cp;
    p.out_f32 = out_f32(d);
    p.status = status_ptr();
    p.n_chunks = (Lb + gdn::kChunk - 1) / gdn::kChunk;
    p.scale = q_scale(d); p.l2_eps = d->l2_eps; p.rms_eps = d->rms_eps; p.rms_n = (float)d->d_v;
    gdn::prefill_ws_layout(p, L.D, d->act_dtype == GDN_F32);
    if (ok(gdn::launch_prefill(p, d->act_dtype, L.D, p.grp, st)) &&
        ok(gdn::launch_unpad_state((const float*)(base + L.state), state, mats, d->d_k, d->d_v, L.D, st)) &&
        ok(gdn::launch_unpad_units(base + L.tail, conv_tail, (long)B * Kc, Cp / ga, C / ga, chan, nullptr, 0, st)))
      ok(gdn::launch_unpad_units(base + L.out, out, rows, d->n_v * L.D / go, d->n_v * d->d_v / go, ochan, len, Lb,
                                 st));
  }
  return hip_status(e, "gdn_prefill_chunk");
}
}  // namespace

namespace gdn {
void timing_before(const char* kernel, hipStream_t st) {
  if (!t_launch || t_used >= t_cap) return;
  t_launch[t_used].kernel = kernel;
  (void)hipEventRecord(t_launch[t_used].start, st);
}
void timing_after(hipStream_t st) {
  if (!t_launch || t_used >= t_cap) return;
  (void)hipEventRecord(t_launch[t_used].stop, st);
  ++t_used;
}
}  // namespace gdn

extern "C" {

int gdn_timing_begin(int capacity) {
  if (t_launch) return fail(GDN_EINVAL, "gdn_timing_begin: a session is already open");
  if (capacity <= 0 || capacity > 65536) return fail(GDN_EINVAL, "gdn_timing_begin: capacity=%d", capacity);
  TimedLaunch* rec = new (std::nothrow) TimedLaunch[capacity];
  if (!rec) return fail(GDN_EINVAL, "gdn_timing_begin: out of host memory");
  for (int i = 0; i < capacity; ++i) {
    hipError_t e = hipEventCreate(&rec[i].start);
    if (e == hipSuccess) e = hipEventCreate(&rec[i].stop);
    if (e != hipSuccess) {
      for (int j = 0; j < i; ++j) {
        (void)hipEventDestroy(rec[j].start);
        (void)hipEventDestroy(rec[j].stop);
      }
      delete[] rec;
      return hip_status(e, "gdn_timing_begin");
    }
  }
  t_launch = rec;
  t_cap = capacity;
  t_used = 0;
  g_err[0] = 0;
  return GDN_OK;
}

int gdn_timing_end(const char** kernels, float* ms, int cap) {
  if (!t_launch) return fail(GDN_EINVAL, "gdn_timing_end: no open session");
  hipError_t err = hipSuccess;
  const int n = t_used;
  for (int i = 0; i < n; ++i) {
    float t = 0.f;
    hipError_t e = hipEventSynchronize(t_launch[i].stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&t, t_launch[i].start, t_launch[i].stop);
    if (e != hipSuccess && err == hipSuccess) err = e;
    if (i < cap) {
      if (kernels) kernels[i] = t_launch[i].kernel;
      if (ms) ms[i] = t;
    }
  }
  for (int i = 0; i < t_cap; ++i) {
    (void)hipEventDestroy(t_launch[i].start);
    (void)hipEventDestroy(t_launch[i].stop);
  }
  delete[] t_launch;
  t_launch = nullptr;
  t_cap = t_used = 0;
  if (err != hipSuccess) return hip_status(err, "gdn_timing_end");
  g_err[0] = 0;
  return n;
}


const char* gdn_last_error(void) { return g_err; }

int gdn_device_status(int clear, gdn_stream_t stream) {
  int* ptr = status_ptr();
  if (!ptr) return fail(GDN_EHIP, "gdn_device_status: no device status word on this device");
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  int v = 0;
  if (e == hipSuccess) e = hipMemcpy(&v, ptr, sizeof(int), hipMemcpyDeviceToHost);
  if (e == hipSuccess && clear) {
    const int zero = 0;
    e = hipMemcpy(ptr, &zero, sizeof(int), hipMemcpyHostToDevice);
  }
  if (e != hipSuccess) return hip_status(e, "gdn_device_status");
  g_err[0] = 0;
  return v;
}

const char* gdn_version(void) { return "gdn-mi355x 0.1 (gfx950)"; }

size_t gdn_state_record_bytes(const gdn_desc* d) {
  if (check_desc(d)) return 0;
  const size_t act = d->act_dtype == GDN_BF16 ? 2 : 4;
  return (size_t)d->n_v * d->d_k * d->d_v * 4 + (size_t)(d->conv_k - 1) * conv_channels(d) * act;
}

int gdn_conv_chunk(const gdn_desc* d, const void* conv_w, const void* mixed, const int32_t* len, void* conv_tail,
                   void* y, int B, int Lb, gdn_stream_t stream) {
  if (int rc = check_desc(d)) return rc;
  if (!conv_w || !mixed || !len || !conv_tail || !y) return fail(GDN_EINVAL, "gdn_conv_chunk: NULL pointer");
  if (B <= 0 || Lb <= 0) return fail(GDN_EINVAL, "gdn_conv_chunk: B=%d Lb=%d must be positive", B, Lb);
  if (!aligned16(conv_w) || !aligned16(mixed) || !aligned16(conv_tail) || !aligned16(y))
    return fail(GDN_EINVAL, "gdn_conv_chunk: buffers must be 16-byte aligned");
  if (y == mixed || y == conv_tail) return fail(GDN_EINVAL, "gdn_conv_chunk: y aliases an input");
  if ((conv_channels(d) + 1023) / 1024 * ((Lb + 63L) / 64) * B >= (1L << 31))
    return fail(GDN_EINVAL, "gdn_conv_chunk: ceil(C/1024) * ceil(Lb/64) * B must stay below 2^31");
  gdn::ConvArgs p{conv_w, mixed, len, conv_tail, y, B, Lb, (int)conv_channels(d)};
  return hip_status(gdn::launch_conv(p, d->act_dtype, (hipStream_t)stream), "gdn_conv_chunk");
}

size_t gdn_prefill_workspace_bytes(const gdn_desc* d, int B, int Lb) {
  if (check_desc(d) || B <= 0 || Lb <= 0) return 0;
  if (d->d_k != d->d_v) return pad_layout(d, B, Lb).total;
  if (use_fused(d, B)) return gdn::fused_ws_bytes(B, d->n_v, Lb);
  const int n_chunks = (Lb + gdn::kChunk - 1) / gdn::kChunk;
  return gdn::prefill_ws_bytes(B, d->n_k, d->n_v, d->d_k, Lb, n_chunks, d->act_dtype == GDN_F32);
}

// the checks and launches of a prefill call; fused: take the fused path whatever the size
static int prefill_impl(const gdn_desc* d, const gdn_weights* w, const void* mixed, const void* z, const void* a,
                        const void* b, const int32_t* len, void* conv_tail, float* state, void* out, int B, int Lb,
                        void* ws, size_t ws_bytes, gdn_stream_t stream, bool fused) {
  if (int rc = check_desc(d)) return rc;
  if (int rc = check_weights(w)) return rc;
  if (!mixed || !z || !a || !b || !len || !conv_tail || !state || !out || !ws)
    return fail(GDN_EINVAL, "gdn_prefill_chunk: NULL pointer");
  if (B <= 0 || Lb <= 0) return fail(GDN_EINVAL, "gdn_prefill_chunk: B=%d Lb=%d must be positive", B, Lb);
  if (B > 65535) return fail(GDN_EINVAL, "gdn_prefill_chunk: B=%d exceeds 65535", B);
  // (heads of different key and value dims run padded to the larger: D = max(d_k, d_v))
  const long dmax = d->d_k > d->d_v ? d->d_k : d->d_v;
  if ((long)Lb * d->n_v * dmax >= (1L << 31))
    return fail(GDN_EINVAL, "gdn_prefill_chunk: Lb * n_v * max(d_k, d_v) = %ld must stay below 2^31",
                (long)Lb * d->n_v * dmax);
  if ((long)B * ((Lb + gdn::kChunk - 1) / gdn::kChunk) * d->n_v >= (1L << 31))
    return fail(GDN_EINVAL, "gdn_prefill_chunk: B * chunks * n_v must stay below 2^31");
  const size_t need = fused ? gdn::fused_ws_bytes(B, d->n_v, Lb) : gdn_prefill_workspace_bytes(d, B, Lb);
  if (ws_bytes < need) return fail(GDN_EINVAL, "gdn_prefill_chunk: workspace %zu bytes < %zu needed", ws_bytes, need);
  if (((uintptr_t)ws & 255u) != 0) return fail(GDN_EINVAL, "gdn_prefill_chunk: workspace must be 256-byte aligned");
  if (!aligned16(state) || !aligned16(mixed) || !aligned16(z) || !aligned16(out) || !aligned16(conv_tail) ||
      !aligned16(w->norm_w))
    return fail(GDN_EINVAL, "gdn_prefill_chunk: buffers must be 16-byte aligned");
  if (out == mixed || out == z || (void*)state == out || conv_tail == out)
    return fail(GDN_EINVAL, "gdn_prefill_chunk: out aliases another buffer");
  if (d->d_k != d->d_v) return prefill_padded(d, w, mixed, z, a, b, len, conv_tail, state, out, B, Lb, ws, stream);
  if (fused || use_fused(d, B)) {
    gdn::FusedArgs f{};
    f.conv_w = w->conv_w; f.A_log = w->A_log; f.dt_bias = w->dt_bias; f.norm_w = w->norm_w;
    f.mixed = mixed; f.z = z; f.a = a; f.b = b; f.len = len; f.tail = conv_tail; f.state = state; f.out = out;
    f.out_f32 = out_f32(d); f.ws = ws; f.status = status_ptr();
    f.B = B; f.Lb = Lb; f.n_k = d->n_k; f.n_v = d->n_v; f.C = (int)conv_channels(d);
    gdn::fused_plan(B, d->n_v, Lb, f.nseg, f.seg_chunks);
    f.scale = q_scale(d); f.l2_eps = d->l2_eps; f.rms_eps = d->rms_eps;
    if ((long)B * d->n_v * f.nseg >= (1L << 31)) return fail(GDN_EINVAL, "gdn_prefill_chunk: grid too large");
    return hip_status(gdn::launch_fused(f, (hipStream_t)stream), "gdn_prefill_chunk");
  }
  gdn::PrefillArgs p{};
  p.conv_w = w->conv_w; p.A_log = w->A_log; p.dt_bias = w->dt_bias; p.norm_w = w->norm_w;
  p.mixed = mixed; p.z = z; p.a = a; p.b = b; p.len = len; p.tail = conv_tail; p.state = state; p.out = out;
  p.ws = ws; p.B = B; p.Lb = Lb; p.n_k = d->n_k; p.n_v = d->n_v; p.C = (int)conv_channels(d);
  p.out_f32 = out_f32(d);
  p.status = status_ptr();
  p.n_chunks = (Lb + gdn::kChunk - 1) / gdn::kChunk;
  p.scale = q_scale(d); p.l2_eps = d->l2_eps; p.rms_eps = d->rms_eps; p.rms_n = (float)d->d_v;
  gdn::prefill_ws_layout(p, d->d_k, d->act_dtype == GDN_F32);
  return hip_status(gdn::launch_prefill(p, d->act_dtype, d->d_k, p.grp, (hipStream_t)stream),
                    "gdn_prefill_chunk");
}

int gdn_prefill_chunk(const gdn_desc* d, const gdn_weights* w, const void* mixed, const void* z, const void* a,
                      const void* b, const int32_t* len, void* conv_tail, float* state, void* out, int B, int Lb,
                      void* ws, size_t ws_bytes, gdn_stream_t stream) {
  return prefill_impl(d, w, mixed, z, a, b, len, conv_tail, state, out, B, Lb, ws, ws_bytes, stream, false);
}

int gdn_prefill_chunk_noalloc(const gdn_desc* d, const gdn_weights* w, const void* mixed, const void* z, const void* a,
                              const void* b, const int32_t* len, void* conv_tail, float* state, void* out, int B,
                              int Lb, gdn_stream_t stream) {
  if (int rc = check_desc(d)) return rc;
  if (B <= 0 || Lb <= 0) return fail(GDN_EINVAL, "gdn_prefill_chunk_noalloc: B=%d Lb=%d must be positive", B, Lb);
  // the call's own path if its workspace fits the scratch; else, where it is built, the fused path,
  // whose segment workspace never exceeds half the scratch
  const size_t need = gdn_prefill_workspace_bytes(d, B, Lb);
  bool fused = false;
  if (need > kScratchBytes) {
    if (!fused_built(d) || gdn::fused_ws_bytes(B, d->n_v, Lb) > kScratchBytes)
      return fail(GDN_EINVAL,
                  "gdn_prefill_chunk_noalloc: the call needs %zu bytes of workspace, more than the %zu-byte static "
                  "scratch; use gdn_prefill_chunk with a workspace", need, (size_t)kScratchBytes);
    fused = true;
  }
  void* ws = scratch_ptr();
  if (!ws) return fail(GDN_EHIP, "gdn_prefill_chunk_noalloc: no device address for the static scratch");
  return prefill_impl(d, w, mixed, z, a, b, len, conv_tail, state, out, B, Lb, ws, kScratchBytes, stream, fused);
}

static int step_common(const gdn_desc* d, const gdn_weights* w, const void* mixed, const void* z, const void* a,
                       const void* b, int T, const int32_t* slot, const void* tail_in, const float* state_in,
                       void* tail_out, float* state_out, void* out, int B, int P, int verify, gdn_stream_t stream,
                       const char* name) {
  if (int rc = check_desc(d)) return rc;
  if (int rc = check_weights(w)) return rc;
  if (!mixed || !z || !a || !b || !tail_in || !state_in || !tail_out || !state_out || !out)
    return fail(GDN_EINVAL, "%s: NULL pointer", name);
  if (B <= 0 || T <= 0 || P <= 0) return fail(GDN_EINVAL, "%s: B=%d T=%d P=%d must be positive", name, B, T, P);
  if ((long)B * P > 65535) return fail(GDN_EINVAL, "%s: B*P=%ld exceeds 65535", name, (long)B * P);
  if (!aligned16(state_in) || !aligned16(state_out)) return fail(GDN_EINVAL, "%s: states must be 16-byte aligned", name);
  gdn::StepArgs p{};
  p.conv_w = w->conv_w; p.A_log = w->A_log; p.dt_bias = w->dt_bias; p.norm_w = w->norm_w;
  p.mixed = mixed; p.z = z; p.a = a; p.b = b; p.slot = slot; p.tail_in = tail_in; p.state_in = state_in;
  p.tail_out = tail_out; p.state_out = state_out; p.out = out;
  p.B = B; p.T = T; p.P = P; p.n_k = d->n_k; p.n_v = d->n_v; p.C = (int)conv_channels(d); p.verify = verify;
  p.out_f32 = out_f32(d);
  p.scale = q_scale(d); p.l2_eps = d->l2_eps; p.rms_eps = d->rms_eps;
  return hip_status(gdn::launch_step(p, d->act_dtype, d->d_k, d->d_v, d->n_v / d->n_k, (hipStream_t)stream), name);
}

int gdn_decode_step(const gdn_desc* d, const gdn_weights* w, const void* mixed, const void* z, const void* a,
                    const void* b, const int32_t* slot, void* conv_tail_pool, float* state_pool, void* out, int B,
                    gdn_stream_t stream) {
  return step_common(d, w, mixed, z, a, b, 1, slot, conv_tail_pool, state_pool, conv_tail_pool, state_pool, out, B,
                     1, 0, stream, "gdn_decode_step");
}

int gdn_verify_with_checkpoints(const gdn_desc* d, const gdn_weights* w, const void* mixed, const void* z,
                                const void* a, const void* b, int T, const int32_t* slot, const void* conv_tail_pool,
                                const float* state_pool, float* ckpt_state, void* ckpt_tail, void* out, int B,
                                gdn_stream_t stream) {
  if (ckpt_state == state_pool || ckpt_tail == conv_tail_pool)
    return fail(GDN_EINVAL, "gdn_verify_with_checkpoints: checkpoints alias the pools");
  return step_common(d, w, mixed, z, a, b, T, slot, conv_tail_pool, state_pool, ckpt_tail, ckpt_state, out, B, 1, 1,
                     stream, "gdn_verify_with_checkpoints");
}

int gdn_verify_paths(const gdn_desc* d, const gdn_weights* w, const void* mixed, const void* z, const void* a,
                     const void* b, int T, int P, const int32_t* slot, const void* conv_tail_pool,
                     const float* state_pool, float* ckpt_state, void* ckpt_tail, void* out, int B,
                     gdn_stream_t stream) {
  if (ckpt_state == state_pool || ckpt_tail == conv_tail_pool)
    return fail(GDN_EINVAL, "gdn_verify_paths: checkpoints alias the pools");
  return step_common(d, w, mixed, z, a, b, T, slot, conv_tail_pool, state_pool, ckpt_tail, ckpt_state, out, B, P, 1,
                     stream, "gdn_verify_paths");
}

int gdn_accept(const int32_t* drafts, const int32_t* preds, int B, int K, int32_t* m, int32_t* emitted,
               int32_t* n_emitted, int32_t* ckpt_index, gdn_stream_t stream) {
  if (!drafts || !preds || !m || !emitted || !n_emitted) return fail(GDN_EINVAL, "gdn_accept: NULL pointer");
  if (B <= 0 || K < 0) return fail(GDN_EINVAL, "gdn_accept: B=%d K=%d", B, K);
  if ((long)B * (K + 1) >= (1L << 31)) return fail(GDN_EINVAL, "gdn_accept: B*(K+1) must stay below 2^31");
  gdn::AcceptArgs p{drafts, preds, m, emitted, n_emitted, ckpt_index, nullptr, B, K, 1};
  return hip_status(gdn::launch_accept(p, (hipStream_t)stream), "gdn_accept");
}

int gdn_accept_paths(const int32_t* drafts, const int32_t* preds, int B, int P, int K, int32_t* m, int32_t* path,
                     int32_t* emitted, int32_t* n_emitted, int32_t* ckpt_index, gdn_stream_t stream) {
  if (!drafts || !preds || !m || !path || !emitted || !n_emitted)
    return fail(GDN_EINVAL, "gdn_accept_paths: NULL pointer");
  if (B <= 0 || P <= 0 || K < 0) return fail(GDN_EINVAL, "gdn_accept_paths: B=%d P=%d K=%d", B, P, K);
  if ((long)B * P * (K + 1) >= (1L << 31))
    return fail(GDN_EINVAL, "gdn_accept_paths: B*P*(K+1) must stay below 2^31");
  gdn::AcceptArgs p{drafts, preds, m, emitted, n_emitted, ckpt_index, path, B, K, P};
  return hip_status(gdn::launch_accept(p, (hipStream_t)stream), "gdn_accept_paths");
}

int gdn_state_copy(const gdn_desc* d, float* dst_state, void* dst_tail, const int32_t* dst_idx,
                   const float* src_state, const void* src_tail, const int32_t* src_idx, int n, gdn_stream_t stream) {
  if (int rc = check_desc(d)) return rc;
  if (n <= 0) return fail(GDN_EINVAL, "gdn_state_copy: n=%d must be positive", n);
  if (n > 65535) return fail(GDN_EINVAL, "gdn_state_copy: n=%d exceeds 65535", n);
  if ((!dst_state) != (!src_state)) return fail(GDN_EINVAL, "gdn_state_copy: state pointers must both be set or both NULL");
  if ((!dst_tail) != (!src_tail)) return fail(GDN_EINVAL, "gdn_state_copy: tail pointers must both be set or both NULL");
  if (!dst_state && !dst_tail) return fail(GDN_EINVAL, "gdn_state_copy: nothing to copy");
  if ((dst_state && (dst_state == src_state)) || (dst_tail && (dst_tail == src_tail)))
    return fail(GDN_EINVAL, "gdn_state_copy: dst aliases src");
  if (!aligned16(dst_state) || !aligned16(src_state) || !aligned16(dst_tail) || !aligned16(src_tail))
    return fail(GDN_EINVAL, "gdn_state_copy: buffers must be 16-byte aligned");
  const long act = d->act_dtype == GDN_BF16 ? 2 : 4;
  gdn::CopyArgs p{};
  p.dst_state = dst_state; p.dst_tail = dst_tail; p.dst_idx = dst_idx;
  p.src_state = src_state; p.src_tail = src_tail; p.src_idx = src_idx;
  p.state_floats = (long)d->n_v * d->d_k * d->d_v;
  p.tail_bytes = (long)(d->conv_k - 1) * conv_channels(d) * act;
  p.n = n;
  if (p.tail_bytes % 16) return fail(GDN_EUNSUPPORTED, "gdn_state_copy: tail record of %ld bytes", p.tail_bytes);
  return hip_status(gdn::launch_copy(p, (hipStream_t)stream), "gdn_state_copy");
}

int gdn_mfma_probe(float* sink, int blocks, int iters, gdn_stream_t stream) {
  if (!sink || blocks <= 0 || iters <= 0) return fail(GDN_EINVAL, "gdn_mfma_probe: sink=%p blocks=%d iters=%d",
                                                      (void*)sink, blocks, iters);
  return hip_status(gdn::launch_mfma_probe(sink, blocks, iters, (hipStream_t)stream), "gdn_mfma_probe");
}

int gdn_state_zero(const gdn_desc* d, float* state, void* tail, const int32_t* idx, int n, gdn_stream_t stream) {
  if (int rc = check_desc(d)) return rc;
  if (n <= 0 || n > 65535) return fail(GDN_EINVAL, "gdn_state_zero: n=%d (1..65535)", n);
  if (!state && !tail) return fail(GDN_EINVAL, "gdn_state_zero: nothing to zero");
  if (!aligned16(state) || !aligned16(tail)) return fail(GDN_EINVAL, "gdn_state_zero: buffers must be 16-byte aligned");
  const long act = d->act_dtype == GDN_BF16 ? 2 : 4;
  gdn::CopyArgs p{};
  p.dst_state = state; p.dst_tail = tail; p.dst_idx = idx;
  p.state_floats = (long)d->n_v * d->d_k * d->d_v;
  p.tail_bytes = (long)(d->conv_k - 1) * conv_channels(d) * act;
  p.n = n;
  if (p.tail_bytes % 16) return fail(GDN_EUNSUPPORTED, "gdn_state_zero: tail record of %ld bytes", p.tail_bytes);
  return hip_status(gdn::launch_zero(p, (hipStream_t)stream), "gdn_state_zero");
}

}  // extern "C"
