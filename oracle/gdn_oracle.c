/*
 * gdn_oracle.c -- plain, slow, f64 CPU oracle for the gated-delta-rule (GDN)
 * linear-attention layer: the prepare step (causal depthwise conv + SiLU,
 * q/k/v split, per-head L2 norm, decay / write gates) and the token-by-token
 * gated delta rule recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code, header or helper with the HIP kernels.
 *
 * Every function computes in double precision from inputs that are already
 * exact doubles (the Python wrapper upcasts f32/bf16/f16 values exactly).
 * Rounding to a storage dtype happens only in gdn_oracle_round(), which the
 * wrapper calls at the points where the library stores a tensor.
 *
 * Sources (the semantics, restated in our own code, no listing copied):
 *   [P1] vllm.cpp src/vt/cpu/cpu_ops.cpp
 *   [P2] vllm.cpp src/vllm/model_executor/models/qwen3_5.cpp
 *   [P3] ferrum-kernels 0.8.0 src/ferrum_kernels/backend/cpu.rs
 * cited by page and function name.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared (no fused multiply-add, so
 * the result does not depend on how the compiler contracts expressions; the
 * same policy [P1] FusedChainInterpKernel states for its reference loops).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------------- */
/* Scalar functions.                                                       */
/* ---------------------------------------------------------------------- */

/* logistic function; [P1] Sigmoid, [P3] sigmoid */
static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* x * sigmoid(x); [P1] SiluGate, [P3] silu */
static double silu(double x) { return x / (1.0 + exp(-x)); }

/* ln(1 + e^x) written without overflow.  The pages switch to the identity
 * above x = 20 ([P1] GdnGBetaKernel, [P3] softplus); the exact function
 * differs from that by less than e^-20, so the oracle keeps the exact one. */
static double softplus(double x) { return fmax(x, 0.0) + log1p(exp(-fabs(x))); }

/* ---------------------------------------------------------------------- */
/* A tiny parallel-for over independent items.  Each item writes only its  */
/* own outputs, so the result is identical for every thread count          */
/* ([P1] file header: parallel work partitions outputs only).              */
/* ---------------------------------------------------------------------- */
typedef void (*item_fn)(void* ctx, int64_t item);
typedef struct {
  item_fn fn;
  void* ctx;
  int64_t begin, end;
} span_t;

static void* run_span(void* p) {
  span_t* s = (span_t*)p;
  for (int64_t i = s->begin; i < s->end; ++i) s->fn(s->ctx, i);
  return NULL;
}

static void parallel_for(int64_t n, int nthreads, item_fn fn, void* ctx) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (n < nthreads) nthreads = (int)(n > 0 ? n : 1);
  if (nthreads == 1) {
    for (int64_t i = 0; i < n; ++i) fn(ctx, i);
    return;
  }
  pthread_t th[256];
  span_t sp[256];
  for (int t = 0; t < nthreads; ++t) {
    sp[t].fn = fn;
    sp[t].ctx = ctx;
    sp[t].begin = n * t / nthreads;
    sp[t].end = n * (t + 1) / nthreads;
    pthread_create(&th[t], NULL, run_span, &sp[t]);
  }
  for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* ---------------------------------------------------------------------- */
/* Step a1: causal depthwise conv over each sequence + SiLU.               */
/* [P1] CausalConv1dFwdKernel (varlen, initial conv state, write-back of   */
/* the last K-1 raw inputs), [P3] linear_attention_prepare_varlen_f32.     */
/* ---------------------------------------------------------------------- */
typedef struct {
  int64_t Cc;
  int K, N;
  const int32_t* cu;
  const double* x;      /* [T, x_stride], channel c at column c          */
  int64_t x_stride;
  const double* w;      /* [Cc, K]                                        */
  const double* hist;   /* [N, Cc, K-1] conv history entering each seq    */
  const uint8_t* has_init;
  double* y;            /* [T, Cc] silu(conv)                             */
  double* hist_out;     /* [N, Cc, K-1] history leaving each sequence     */
} conv_ctx;

/* Raw input seen at token p (global index) by sequence s, channel c.
 * Inside the sequence it is x; before its start it is the conv history
 * (column K-1-d holds the input d tokens before the start), or zero when
 * the sequence has no initial state. */
static double conv_tap(const conv_ctx* c, int64_t s, int64_t ch, int64_t p) {
  const int64_t start = c->cu[s];
  if (p >= start) return c->x[p * c->x_stride + ch];
  if (!c->has_init[s]) return 0.0;
  const int64_t before = start - p; /* 1 .. K-1 */
  return c->hist[(s * c->Cc + ch) * (c->K - 1) + (c->K - 1) - before];
}

static void conv_item(void* vctx, int64_t item) {
  const conv_ctx* c = (const conv_ctx*)vctx;
  const int64_t s = item / c->Cc, ch = item % c->Cc;
  const int K = c->K;
  for (int64_t t = c->cu[s]; t < c->cu[s + 1]; ++t) {
    double acc = 0.0;
    for (int j = 0; j < K; ++j) acc += c->w[ch * K + j] * conv_tap(c, s, ch, t - (K - 1) + j);
    c->y[t * c->Cc + ch] = silu(acc);
  }
  /* the new history holds the last K-1 raw inputs, oldest first; a sequence
   * shorter than K-1 keeps the tail of the old history in front of it */
  for (int j = 0; j < K - 1; ++j)
    c->hist_out[(s * c->Cc + ch) * (K - 1) + j] = conv_tap(c, s, ch, c->cu[s + 1] - (K - 1) + j);
}

void gdn_oracle_conv_silu(int64_t Cc, int K, int N, const int32_t* cu, const double* x,
                          int64_t x_stride, const double* w, const double* hist,
                          const uint8_t* has_init, double* y, double* hist_out, int nthreads) {
  conv_ctx c = {Cc, K, N, cu, x, x_stride, w, hist, has_init, y, hist_out};
  parallel_for((int64_t)N * Cc, nthreads, conv_item, &c);
}

/* ---------------------------------------------------------------------- */
/* Steps a2 + a3: split the conv output into per-head q, k, v and          */
/* L2-normalise q and k over the head dim with eps inside the root of the  */
/* plain sum of squares.  [P1] GdnConvSplitKernel, L2NormKernel,           */
/* GdnPostConvKernel; [P3] linear_attention_prepare_f32.                   */
/* ---------------------------------------------------------------------- */
void gdn_oracle_split_l2(int64_t T, int Hk, int Hv, int Dk, int Dv, const double* y, int l2norm,
                         double eps, double* q, double* k, double* v) {
  const int64_t key_dim = (int64_t)Hk * Dk, value_dim = (int64_t)Hv * Dv;
  const int64_t Cc = 2 * key_dim + value_dim;
  for (int64_t t = 0; t < T; ++t) {
    const double* row = y + t * Cc;
    for (int h = 0; h < Hk; ++h) {
      double qs = 0.0, ks = 0.0;
      for (int d = 0; d < Dk; ++d) {
        const double qv = row[h * Dk + d], kv = row[key_dim + h * Dk + d];
        qs += qv * qv;
        ks += kv * kv;
      }
      const double qi = l2norm ? 1.0 / sqrt(qs + eps) : 1.0;
      const double ki = l2norm ? 1.0 / sqrt(ks + eps) : 1.0;
      for (int d = 0; d < Dk; ++d) {
        q[(t * Hk + h) * Dk + d] = row[h * Dk + d] * qi;
        k[(t * Hk + h) * Dk + d] = row[key_dim + h * Dk + d] * ki;
      }
    }
    for (int64_t e = 0; e < value_dim; ++e) v[t * value_dim + e] = row[2 * key_dim + e];
  }
}

/* ---------------------------------------------------------------------- */
/* Step a4: per value head, decay log-gate g = -exp(A_log) *               */
/* softplus(a + dt_bias) and write strength beta = sigmoid(b).             */
/* [P1] GdnGBetaKernel, [P3] linear_attention_prepare_f32.                 */
/* ---------------------------------------------------------------------- */
void gdn_oracle_gates(int64_t T, int Hv, const double* a, int64_t a_stride, const double* b,
                      int64_t b_stride, const double* A_log, const double* dt_bias, double* g,
                      double* beta) {
  for (int64_t t = 0; t < T; ++t)
    for (int h = 0; h < Hv; ++h) {
      g[t * Hv + h] = -exp(A_log[h]) * softplus(a[t * a_stride + h] + dt_bias[h]);
      beta[t * Hv + h] = sigmoid(b[t * b_stride + h]);
    }
}

/* ---------------------------------------------------------------------- */
/* Steps a5 / a6 (their common definition): the gated delta rule, one     */
/* token at a time, per (sequence, value head).  For value head h the      */
/* key/query head is h / (Hv/Hk).  Per token:                              */
/*   S <- exp(g) S ;  u = S k ;  delta = beta (v - u) ;                    */
/*   S <- S + delta k^T ;  o = S (scale q)                                 */
/* with S the [Dv, Dk] state (Dk contiguous).  [P1] GdnHeadTokenStep,      */
/* GdnPrefillKernel, GdnDecodeKernel; [P3] recurrent_gated_delta_rule_f32, */
/* recurrent_gated_delta_rule_varlen_f32.                                  */
/* ---------------------------------------------------------------------- */
typedef struct {
  int Hk, Hv, Dk, Dv, N;
  const int32_t* cu;
  const double *q, *k, *v, *g, *beta;
  double scale;
  int l2norm;
  double eps;
  const double* state_in; /* [N, Hv, Dv, Dk] */
  const uint8_t* has_init;
  double* out;       /* [T, Hv, Dv] */
  double* state_out; /* [N, Hv, Dv, Dk] */
} rec_ctx;

static void rec_item(void* vctx, int64_t item) {
  const rec_ctx* c = (const rec_ctx*)vctx;
  const int64_t s = item / c->Hv;
  const int h = (int)(item % c->Hv);
  const int Dk = c->Dk, Dv = c->Dv, Hk = c->Hk, Hv = c->Hv;
  const int kh = h / (Hv / Hk);
  double* S = c->state_out + (s * Hv + h) * (int64_t)Dv * Dk;
  const double* S0 = c->state_in + (s * Hv + h) * (int64_t)Dv * Dk;
  for (int64_t e = 0; e < (int64_t)Dv * Dk; ++e) S[e] = c->has_init[s] ? S0[e] : 0.0;
  double* kk = (double*)malloc(sizeof(double) * (size_t)Dk);
  double* qq = (double*)malloc(sizeof(double) * (size_t)Dk);
  for (int64_t t = c->cu[s]; t < c->cu[s + 1]; ++t) {
    const double* kr = c->k + (t * Hk + kh) * Dk;
    const double* qr = c->q + (t * Hk + kh) * Dk;
    double kn = 0.0, qn = 0.0;
    for (int d = 0; d < Dk; ++d) {
      kn += kr[d] * kr[d];
      qn += qr[d] * qr[d];
    }
    const double ki = c->l2norm ? 1.0 / sqrt(kn + c->eps) : 1.0;
    const double qi = c->l2norm ? 1.0 / sqrt(qn + c->eps) : 1.0;
    for (int d = 0; d < Dk; ++d) {
      kk[d] = kr[d] * ki;
      qq[d] = qr[d] * qi * c->scale;
    }
    const double decay = exp(c->g[t * Hv + h]);
    const double bt = c->beta[t * Hv + h];
    for (int e = 0; e < Dv; ++e) {
      double* row = S + (int64_t)e * Dk;
      for (int d = 0; d < Dk; ++d) row[d] *= decay;
      double u = 0.0;
      for (int d = 0; d < Dk; ++d) u += row[d] * kk[d];
      const double delta = bt * (c->v[(t * Hv + h) * Dv + e] - u);
      for (int d = 0; d < Dk; ++d) row[d] += delta * kk[d];
      double o = 0.0;
      for (int d = 0; d < Dk; ++d) o += row[d] * qq[d];
      c->out[(t * Hv + h) * Dv + e] = o;
    }
  }
  free(kk);
  free(qq);
}

void gdn_oracle_recurrence(int Hk, int Hv, int Dk, int Dv, int N, const int32_t* cu,
                           const double* q, const double* k, const double* v, const double* g,
                           const double* beta, double scale, int l2norm, double eps,
                           const double* state_in, const uint8_t* has_init, double* out,
                           double* state_out, int nthreads) {
  rec_ctx c = {Hk, Hv, Dk, Dv, N, cu, q, k, v, g, beta, scale, l2norm, eps,
               state_in, has_init, out, state_out};
  parallel_for((int64_t)N * Hv, nthreads, rec_item, &c);
}

/* ---------------------------------------------------------------------- */
/* KDA: the gated delta rule with one log-decay per key channel instead of */
/* one per head.  g is [T, Hv, Dk]; per token, for value head h:           */
/*   S[:, d] <- exp(g[t,h,d]) S[:, d] ;  u = S k ;  delta = beta (v - u) ; */
/*   S <- S + delta k^T ;  o = S (scale q)                                 */
/* i.e. the state's Dk columns decay independently ([P1] KdaHeadTokenStep, */
/* KdaGatedDeltaRuleKernel).  q and k are used as given unless l2norm.     */
/* ---------------------------------------------------------------------- */
static void kda_item(void* vctx, int64_t item) {
  const rec_ctx* c = (const rec_ctx*)vctx;
  const int64_t s = item / c->Hv;
  const int h = (int)(item % c->Hv);
  const int Dk = c->Dk, Dv = c->Dv, Hk = c->Hk, Hv = c->Hv;
  const int kh = h / (Hv / Hk);
  double* S = c->state_out + (s * Hv + h) * (int64_t)Dv * Dk;
  const double* S0 = c->state_in + (s * Hv + h) * (int64_t)Dv * Dk;
  for (int64_t e = 0; e < (int64_t)Dv * Dk; ++e) S[e] = c->has_init[s] ? S0[e] : 0.0;
  double* kk = (double*)malloc(sizeof(double) * (size_t)Dk);
  double* qq = (double*)malloc(sizeof(double) * (size_t)Dk);
  double* dec = (double*)malloc(sizeof(double) * (size_t)Dk);
  for (int64_t t = c->cu[s]; t < c->cu[s + 1]; ++t) {
    const double* kr = c->k + (t * Hk + kh) * Dk;
    const double* qr = c->q + (t * Hk + kh) * Dk;
    double kn = 0.0, qn = 0.0;
    for (int d = 0; d < Dk; ++d) {
      kn += kr[d] * kr[d];
      qn += qr[d] * qr[d];
    }
    const double ki = c->l2norm ? 1.0 / sqrt(kn + c->eps) : 1.0;
    const double qi = c->l2norm ? 1.0 / sqrt(qn + c->eps) : 1.0;
    for (int d = 0; d < Dk; ++d) {
      kk[d] = kr[d] * ki;
      qq[d] = qr[d] * qi * c->scale;
      dec[d] = exp(c->g[(t * Hv + h) * Dk + d]);
    }
    const double bt = c->beta[t * Hv + h];
    for (int e = 0; e < Dv; ++e) {
      double* row = S + (int64_t)e * Dk;
      for (int d = 0; d < Dk; ++d) row[d] *= dec[d];
      double u = 0.0;
      for (int d = 0; d < Dk; ++d) u += row[d] * kk[d];
      const double delta = bt * (c->v[(t * Hv + h) * Dv + e] - u);
      for (int d = 0; d < Dk; ++d) row[d] += delta * kk[d];
      double o = 0.0;
      for (int d = 0; d < Dk; ++d) o += row[d] * qq[d];
      c->out[(t * Hv + h) * Dv + e] = o;
    }
  }
  free(kk);
  free(qq);
  free(dec);
}

void gdn_oracle_kda_recurrence(int Hk, int Hv, int Dk, int Dv, int N, const int32_t* cu,
                               const double* q, const double* k, const double* v, const double* g,
                               const double* beta, double scale, int l2norm, double eps,
                               const double* state_in, const uint8_t* has_init, double* out,
                               double* state_out, int nthreads) {
  rec_ctx c = {Hk, Hv, Dk, Dv, N, cu, q, k, v, g, beta, scale, l2norm, eps,
               state_in, has_init, out, state_out};
  parallel_for((int64_t)N * Hv, nthreads, kda_item, &c);
}

/* ---------------------------------------------------------------------- */
/* KDA gate, per (token, value head, key channel):                         */
/*   g = -exp(A_log[h]) * softplus(g_raw + dt_bias[h][d])                  */
/* with softplus(x) = ln(1 + e^x); dt_bias may be absent (zero).           */
/* [P1] KdaChunkPrefillKernel.                                             */
/* ---------------------------------------------------------------------- */
void gdn_oracle_kda_gate(int64_t T, int Hv, int Dk, const double* g_raw, const double* A_log,
                         const double* dt_bias, double* g) {
  for (int64_t t = 0; t < T; ++t)
    for (int h = 0; h < Hv; ++h)
      for (int d = 0; d < Dk; ++d) {
        const int64_t i = (t * Hv + h) * Dk + d;
        const double x = g_raw[i] + (dt_bias ? dt_bias[h * Dk + d] : 0.0);
        g[i] = -exp(A_log[h]) * softplus(x);
      }
}

/* ---------------------------------------------------------------------- */
/* Mamba2 / SSD (not the delta rule): per sequence and head h, with group  */
/* g = h / (H/G) and the [P, N] state S:                                   */
/*   S <- exp(A[h] dt[t,h]) S + dt[t,h] x[t,h,:] B[t,g,:]^T                */
/*   y[t,h,p] = sum_n S[p,n] C[t,g,n] + D x[t,h,p];  y *= silu(z[t,h,p])   */
/* dt is taken as given (see gdn_oracle_mamba2_dt); D is per head (D_per_p */
/* = 0) or per (head, p), and may be absent, as may z.  [P1]              */
/* Mamba2ChunkScanKernel (what its five stages compute),                   */
/* Mamba2StateUpdateKernel.                                                */
/* ---------------------------------------------------------------------- */
typedef struct {
  int H, P, G, N, Nseq;
  const int32_t* cu;
  const double *x, *dt, *A, *B, *C, *D, *z;
  int D_per_p;
  const double* state_in; /* [Nseq, H, P, N] */
  const uint8_t* has_init;
  double* out;       /* [T, H, P] */
  double* state_out; /* [Nseq, H, P, N] */
} ssd_ctx;

static void ssd_item(void* vctx, int64_t item) {
  const ssd_ctx* c = (const ssd_ctx*)vctx;
  const int64_t s = item / c->H;
  const int h = (int)(item % c->H);
  const int H = c->H, P = c->P, G = c->G, N = c->N;
  const int g = h / (H / G);
  double* S = c->state_out + (s * H + h) * (int64_t)P * N;
  const double* S0 = c->state_in + (s * H + h) * (int64_t)P * N;
  for (int64_t e = 0; e < (int64_t)P * N; ++e) S[e] = c->has_init[s] ? S0[e] : 0.0;
  for (int64_t t = c->cu[s]; t < c->cu[s + 1]; ++t) {
    const double dt = c->dt[t * H + h];
    const double da = exp(c->A[h] * dt);
    const double* xr = c->x + (t * H + h) * P;
    const double* Br = c->B + (t * G + g) * N;
    const double* Cr = c->C + (t * G + g) * N;
    for (int p = 0; p < P; ++p) {
      double* row = S + (int64_t)p * N;
      double y = 0.0;
      for (int n = 0; n < N; ++n) {
        row[n] = da * row[n] + dt * xr[p] * Br[n];
        y += row[n] * Cr[n];
      }
      if (c->D) y += (c->D_per_p ? c->D[h * P + p] : c->D[h]) * xr[p];
      if (c->z) y *= silu(c->z[(t * H + h) * P + p]);
      c->out[(t * H + h) * P + p] = y;
    }
  }
}

void gdn_oracle_mamba2(int H, int P, int G, int N, int Nseq, const int32_t* cu, const double* x,
                       const double* dt, const double* A, const double* B, const double* C,
                       const double* D, int D_per_p, const double* z, const double* state_in,
                       const uint8_t* has_init, double* out, double* state_out, int nthreads) {
  ssd_ctx c = {H, P, G, N, Nseq, cu, x, dt, A, B, C, D, z, D_per_p, state_in, has_init, out, state_out};
  parallel_for((int64_t)Nseq * H, nthreads, ssd_item, &c);
}

/* Mamba2 step size: dt = clamp(softplus(dt_raw + dt_bias[h]), dt_min,     */
/* dt_max), the softplus optional and the identity above 20 as the pages   */
/* guard it; dt_bias may be absent.  [P1] Mamba2ChunkScanKernel stage 1,   */
/* SoftplusGuarded.                                                        */
void gdn_oracle_mamba2_dt(int64_t T, int H, const double* dt_raw, const double* dt_bias, int use_softplus,
                          double dt_min, double dt_max, double* dt) {
  for (int64_t t = 0; t < T; ++t)
    for (int h = 0; h < H; ++h) {
      double d = dt_raw[t * H + h] + (dt_bias ? dt_bias[h] : 0.0);
      if (use_softplus) d = d <= 20.0 ? log1p(exp(d)) : d;
      d = fmin(fmax(d, dt_min), dt_max);
      dt[t * H + h] = d;
    }
}

/* ---------------------------------------------------------------------- */
/* Gated RMS norm of the output, the layer's epilogue.  For each row r of  */
/* D values (one (token, value head) pair):                                */
/*   out[r][j] = x[r][j] / sqrt(ms + eps) * w[j] * act(z[r][j]),           */
/*   ms = (sum_j x[r][j]^2) / D,                                           */
/* act = silu, or the logistic function when sigmoid_gate is set: the norm */
/* is taken before the gate, with one group per row.  [P1]                 */
/* RmsNormGatedKernel; [P3] gated_rms_norm_f32.  x, z and out are dense    */
/* [rows][D]; the caller lays the gate out from wherever it lives.         */
/* ---------------------------------------------------------------------- */
void gdn_oracle_gated_rmsnorm(int64_t rows, int D, const double* x, const double* z, const double* w,
                              double eps, int sigmoid_gate, double* out) {
  for (int64_t r = 0; r < rows; ++r) {
    const double* xr = x + r * D;
    const double* zr = z + r * D;
    double sumsq = 0.0;
    for (int j = 0; j < D; ++j) sumsq += xr[j] * xr[j];
    const double inv = 1.0 / sqrt(sumsq / (double)D + eps);
    for (int j = 0; j < D; ++j) {
      const double act = sigmoid_gate ? sigmoid(zr[j]) : silu(zr[j]);
      out[r * D + j] = xr[j] * inv * w[j] * act;
    }
  }
}

/* ---------------------------------------------------------------------- */
/* Rounding to a storage dtype, round-to-nearest-even, straight from the   */
/* double value (no intermediate float).  [P1] LoadF32/StoreF32 round at   */
/* every store; [P2] GatherStateF32/ScatterStateF32 round the compressed   */
/* state cache once at the cache boundary.                                 */
/* dtype: 0 = f32, 1 = bf16, 2 = f16.                                      */
/* ---------------------------------------------------------------------- */
static double round_binary(double x, int sig_bits, int min_exp, double max_finite) {
  /* sig_bits significant bits (with the leading one); min_exp is the exponent
   * of the smallest normal (2^min_exp); below it the spacing stays
   * 2^(min_exp - sig_bits + 1) (subnormals). */
  if (isnan(x) || isinf(x) || x == 0.0) return x;
  int e;
  frexp(x, &e); /* |x| = m 2^e, m in [0.5, 1): leading bit is 2^(e-1) */
  int lead = e - 1;
  if (lead < min_exp) lead = min_exp;
  const double quantum = ldexp(1.0, lead - (sig_bits - 1));
  const double r = nearbyint(x / quantum) * quantum; /* default mode: ties to even */
  if (fabs(r) > max_finite) return x > 0 ? INFINITY : -INFINITY;
  return r;
}

void gdn_oracle_round(const double* x, double* y, int64_t n, int dtype) {
  for (int64_t i = 0; i < n; ++i) {
    if (dtype == 0)
      y[i] = (double)(float)x[i];
    else if (dtype == 1) /* bf16: 8 significant bits, f32 exponent range */
      y[i] = round_binary(x[i], 8, -126, ldexp(255.0, 120));
    else /* f16: 11 significant bits, smallest normal 2^-14, max 65504 */
      y[i] = round_binary(x[i], 11, -14, 65504.0);
  }
}
