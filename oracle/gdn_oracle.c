/*
 * Gated DeltaNet layer: plain fp64 CPU oracle. TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the package's smoke() entry and the benchmark's CPU-baseline leg may load this
 * library. It shares no code, header or table with the HIP path: it is the slow, obviously correct
 * statement of what the layer computes, token by token, in double precision.
 *
 * Sources (pages, and the function on each page):
 *  - "qev_fast/statecache.py" (squad-0.8b), CacheQwen35._gdn: the layer's call sequence — conv over
 *    [saved conv inputs | chunk] with SiLU and no bias, the tail copy of the last Kc real inputs,
 *    the q|k|v channel split, the gates, the padding mask (g = 0, beta = 0), the GQA repeat of q/k
 *    over value heads, the delta rule with in-kernel q/k L2 norm from the saved state, the fp32
 *    state write-back, and the gated RMSNorm.
 *  - The recurrence itself, S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *    o_t = S_t q_t, with g = -exp(A_log) softplus(a + dt_bias) and beta = sigmoid(b), is the
 *    layer's definition; the state is stored as H = S^T, [d_k][d_v] per head, as the page's
 *    StateCache.__init__ allocates it.
 *  - "mtp/generate.py" (sparkle mlx_streaming), forward_with_hidden_stepwise and accept_prefix:
 *    per-token verify checkpoints and the accepted-prefix rule.
 *
 * Readings where the pages are silent: q is scaled by `scale` (default d_k^-1/2); the L2 norm is
 * x / sqrt(sum x^2 + l2_eps); conv tap K-1 multiplies the current token; softplus is log(1 + e^x);
 * the gated norm is w * o / sqrt(mean(o^2) + eps) * silu(z).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int n_k, n_v, d_k, d_v, conv_k;
  double scale, l2_eps, rms_eps;
} oracle_dims;

static double silu(double x) { return x / (1.0 + exp(-x)); }
static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }
static double softplus(double x) { return log1p(exp(x)); }

static int conv_dim(const oracle_dims* d) { return 2 * d->n_k * d->d_k + d->n_v * d->d_v; }

/*
 * Causal depthwise conv1d + SiLU over xin = [tail (Kc rows) | x (L rows)] for one sequence.
 *   y[t][c] = silu( sum_{j<K} w[c][j] * xin[t + j][c] ),  t = 0 .. L-1
 * so tap K-1 meets the current token x[t]. Afterwards tail = xin[len .. len+Kc-1]: the last Kc real
 * inputs, with old tail rows kept when len < Kc (statecache.py page, CacheQwen35._gdn tail copy).
 */
void oracle_conv(int C, int K, int L, int len, const double* w, double* tail, const double* x, double* y) {
  const int Kc = K - 1;
  double* xin = (double*)malloc(sizeof(double) * (size_t)(Kc + L) * C);
  memcpy(xin, tail, sizeof(double) * (size_t)Kc * C);
  memcpy(xin + (size_t)Kc * C, x, sizeof(double) * (size_t)L * C);
  for (int t = 0; t < L; ++t)
    for (int c = 0; c < C; ++c) {
      double s = 0.0;
      for (int j = 0; j < K; ++j) s += w[(size_t)c * K + j] * xin[(size_t)(t + j) * C + c];
      y[(size_t)t * C + c] = silu(s);
    }
  for (int r = 0; r < Kc; ++r)
    for (int c = 0; c < C; ++c) tail[(size_t)r * C + c] = xin[(size_t)(len + r) * C + c];
  free(xin);
}

/* g = -exp(A_log) * softplus(a + dt_bias) * m_t,  beta = sigmoid(b) * m_t,  m_t = [t < len]. */
void oracle_gates(int n_v, int L, int len, const double* A_log, const double* dt_bias, const double* a,
                  const double* b, double* g, double* beta) {
  for (int t = 0; t < L; ++t) {
    const double m = t < len ? 1.0 : 0.0;
    for (int h = 0; h < n_v; ++h) {
      const size_t i = (size_t)t * n_v + h;
      g[i] = -exp(A_log[h]) * softplus(a[i] + dt_bias[h]) * m;
      beta[i] = sigmoid(b[i]) * m;
    }
  }
}

/*
 * The gated delta rule for one sequence, token by token, with q/k L2-normalised per key head and
 * value head h reading key head h / (n_v / n_k) (repeat_interleave over heads).
 *   q, k: [L][n_k][d_k] (raw); v: [L][n_v][d_v]; g, beta: [L][n_v]; H: [n_v][d_k][d_v] in/out;
 *   o: [L][n_v][d_v].
 * Per token, with H = S^T:  H <- e^g H;  u = beta (v - H^T k);  H <- H + k u^T;  o = scale H^T q.
 * That is S_t = e^{g_t} S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T and o_t = scale S_t q_t.
 */
void oracle_delta_rule(const oracle_dims* d, int L, const double* q, const double* k, const double* v,
                       const double* g, const double* beta, double* H, double* o, int nthreads) {
  const int nk = d->n_k, nv = d->n_v, dk = d->d_k, dv = d->d_v, r = d->n_v / d->n_k;
  (void)nthreads;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
  for (int h = 0; h < nv; ++h) {
    const int kh = h / r;
    double* Hh = H + (size_t)h * dk * dv;
    double* qn = (double*)malloc(sizeof(double) * dk);
    double* kn = (double*)malloc(sizeof(double) * dk);
    double* u = (double*)malloc(sizeof(double) * dv);
    for (int t = 0; t < L; ++t) {
      const double* qt = q + ((size_t)t * nk + kh) * dk;
      const double* kt = k + ((size_t)t * nk + kh) * dk;
      const double* vt = v + ((size_t)t * nv + h) * dv;
      double sq = 0.0, sk = 0.0;
      for (int i = 0; i < dk; ++i) { sq += qt[i] * qt[i]; sk += kt[i] * kt[i]; }
      const double rq = 1.0 / sqrt(sq + d->l2_eps), rk = 1.0 / sqrt(sk + d->l2_eps);
      for (int i = 0; i < dk; ++i) { qn[i] = qt[i] * rq; kn[i] = kt[i] * rk; }
      const double decay = exp(g[(size_t)t * nv + h]);
      const double bt = beta[(size_t)t * nv + h];
      for (int i = 0; i < dk * dv; ++i) Hh[i] *= decay;
      for (int j = 0; j < dv; ++j) {
        double hk = 0.0;
        for (int i = 0; i < dk; ++i) hk += Hh[(size_t)i * dv + j] * kn[i];
        u[j] = bt * (vt[j] - hk);
      }
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) Hh[(size_t)i * dv + j] += kn[i] * u[j];
      double* ot = o + ((size_t)t * nv + h) * dv;
      for (int j = 0; j < dv; ++j) {
        double s = 0.0;
        for (int i = 0; i < dk; ++i) s += Hh[(size_t)i * dv + j] * qn[i];
        ot[j] = d->scale * s;
      }
    }
    free(qn); free(kn); free(u);
  }
}

/* out = w * o / sqrt(mean(o^2) + eps) * silu(z), per row of length dv. */
void oracle_gated_rmsnorm(long rows, int dv, const double* o, const double* z, const double* w, double eps,
                          double* out) {
  for (long r = 0; r < rows; ++r) {
    const double* orow = o + (size_t)r * dv;
    double ss = 0.0;
    for (int j = 0; j < dv; ++j) ss += orow[j] * orow[j];
    const double inv = 1.0 / sqrt(ss / dv + eps);
    for (int j = 0; j < dv; ++j)
      out[(size_t)r * dv + j] = w[j] * (orow[j] * inv) * silu(z[(size_t)r * dv + j]);
  }
}

/*
 * The whole layer for B sequences of L (padded) tokens each, continuing from (tail, H):
 *   mixed [B][L][C_ch], z [B][L][n_v*d_v], a/b [B][L][n_v], lens [B];
 *   tail [B][Kc][C_ch] in/out, H [B][n_v][d_k][d_v] in/out, out [B][L][n_v*d_v];
 *   o_pre (optional, may be NULL) receives the pre-norm o.
 * Positions t >= lens[b] are padding: g = beta = 0 (the state stops at the real end) and they do not
 * enter the tail. Their outputs are computed like any other but carry no meaning.
 */
int oracle_layer_forward(const oracle_dims* d, int B, int L, const int* lens, const double* conv_w,
                         const double* A_log, const double* dt_bias, const double* norm_w, const double* mixed,
                         const double* z, const double* a, const double* b, double* tail, double* H, double* out,
                         double* o_pre, int nthreads) {
  if (d->n_k <= 0 || d->n_v % d->n_k != 0 || d->conv_k < 1 || L < 0 || B < 0) return -1;
  const int C = conv_dim(d), Kc = d->conv_k - 1, nk = d->n_k, nv = d->n_v, dk = d->d_k, dv = d->d_v;
  for (int s = 0; s < B; ++s) {
    const int len = lens[s];
    if (len < 0 || len > L) return -1;
    double* y = (double*)malloc(sizeof(double) * (size_t)L * C);
    double* q = (double*)malloc(sizeof(double) * (size_t)L * nk * dk);
    double* k = (double*)malloc(sizeof(double) * (size_t)L * nk * dk);
    double* v = (double*)malloc(sizeof(double) * (size_t)L * nv * dv);
    double* g = (double*)malloc(sizeof(double) * (size_t)L * nv);
    double* be = (double*)malloc(sizeof(double) * (size_t)L * nv);
    double* o = (double*)malloc(sizeof(double) * (size_t)L * nv * dv);
    oracle_conv(C, d->conv_k, L, len, conv_w, tail + (size_t)s * Kc * C, mixed + (size_t)s * L * C, y);
    /* split [q | k | v] along channels, head-major within each */
    for (int t = 0; t < L; ++t) {
      const double* yt = y + (size_t)t * C;
      memcpy(q + (size_t)t * nk * dk, yt, sizeof(double) * nk * dk);
      memcpy(k + (size_t)t * nk * dk, yt + nk * dk, sizeof(double) * nk * dk);
      memcpy(v + (size_t)t * nv * dv, yt + 2 * nk * dk, sizeof(double) * nv * dv);
    }
    oracle_gates(nv, L, len, A_log, dt_bias, a + (size_t)s * L * nv, b + (size_t)s * L * nv, g, be);
    oracle_delta_rule(d, L, q, k, v, g, be, H + (size_t)s * nv * dk * dv, o, nthreads);
    if (o_pre) memcpy(o_pre + (size_t)s * L * nv * dv, o, sizeof(double) * (size_t)L * nv * dv);
    oracle_gated_rmsnorm((long)L * nv, dv, o, z + (size_t)s * L * nv * dv, norm_w, d->rms_eps,
                         out + (size_t)s * L * nv * dv);
    free(y); free(q); free(k); free(v); free(g); free(be); free(o);
  }
  return 0;
}

/*
 * Verify with per-token checkpoints: T tokens per sequence run one at a time from (tail0, H0), which
 * are left untouched; after token i the state and tail are recorded as checkpoint i
 * (mtp/generate.py page, forward_with_hidden_stepwise: one-token steps, a snapshot after each).
 *   ckpt_H [B][T][n_v][d_k][d_v], ckpt_tail [B][T][Kc][C_ch], out [B][T][n_v*d_v].
 */
int oracle_verify(const oracle_dims* d, int B, int T, const double* conv_w, const double* A_log,
                  const double* dt_bias, const double* norm_w, const double* mixed, const double* z, const double* a,
                  const double* b, const double* tail0, const double* H0, double* ckpt_H, double* ckpt_tail,
                  double* out, int nthreads) {
  const int C = conv_dim(d), Kc = d->conv_k - 1, nv = d->n_v;
  const size_t hsz = (size_t)nv * d->d_k * d->d_v, tsz = (size_t)Kc * C;
  double* Hs = (double*)malloc(sizeof(double) * hsz);
  double* ts = (double*)malloc(sizeof(double) * tsz);
  const int one = 1;
  for (int s = 0; s < B; ++s) {
    memcpy(Hs, H0 + s * hsz, sizeof(double) * hsz);
    memcpy(ts, tail0 + s * tsz, sizeof(double) * tsz);
    for (int i = 0; i < T; ++i) {
      const size_t row = (size_t)s * T + i;
      int rc = oracle_layer_forward(d, 1, 1, &one, conv_w, A_log, dt_bias, norm_w, mixed + row * C,
                                    z + row * nv * d->d_v, a + row * nv, b + row * nv, ts, Hs,
                                    out + row * nv * d->d_v, NULL, nthreads);
      if (rc) { free(Hs); free(ts); return rc; }
      memcpy(ckpt_H + row * hsz, Hs, sizeof(double) * hsz);
      memcpy(ckpt_tail + row * tsz, ts, sizeof(double) * tsz);
    }
  }
  free(Hs); free(ts);
  return 0;
}

/*
 * Accepted prefix (mtp/generate.py page, accept_prefix, and the emitted-token assembly of its
 * caller): m = length of the longest prefix with preds[j] == drafts[j], j < K; the emitted tokens
 * are drafts[:m] followed by preds[m]; the checkpoint to restore is m (state after m+1 tokens).
 */
void oracle_accept(int B, int K, const int* drafts, const int* preds, int* m, int* emitted, int* n_emitted) {
  for (int s = 0; s < B; ++s) {
    int j = 0;
    while (j < K && preds[(size_t)s * (K + 1) + j] == drafts[(size_t)s * K + j]) ++j;
    m[s] = j;
    for (int i = 0; i <= K; ++i) emitted[(size_t)s * (K + 1) + i] = 0;
    for (int i = 0; i < j; ++i) emitted[(size_t)s * (K + 1) + i] = drafts[(size_t)s * K + i];
    emitted[(size_t)s * (K + 1) + j] = preds[(size_t)s * (K + 1) + j];
    n_emitted[s] = j + 1;
  }
}

/*
 * Winner of a batch-of-paths verify (mtp/generate.py page, tree_verify_step): every one of the P
 * paths of a sequence gets its accepted prefix m_p by the rule of oracle_accept, and the winner is
 * the first path with the largest m_p (a later path wins only by matching strictly more drafts). The
 * emitted tokens are the winner's, formed as in oracle_accept.
 * drafts [B][P][K], preds [B][P][K+1]; m, path, n_emitted [B]; emitted [B][K+1].
 */
void oracle_accept_paths(int B, int P, int K, const int* drafts, const int* preds, int* m, int* path, int* emitted,
                         int* n_emitted) {
  for (int s = 0; s < B; ++s) {
    int best = 0, best_m = -1;
    for (int p = 0; p < P; ++p) {
      const int* dr = drafts + ((size_t)s * P + p) * K;
      const int* pr = preds + ((size_t)s * P + p) * (K + 1);
      int j = 0;
      while (j < K && pr[j] == dr[j]) ++j;
      if (j > best_m) {
        best_m = j;
        best = p;
      }
    }
    oracle_accept(1, K, drafts + ((size_t)s * P + best) * K, preds + ((size_t)s * P + best) * (K + 1), m + s,
                  emitted + (size_t)s * (K + 1), n_emitted + s);
    path[s] = best;
  }
}
