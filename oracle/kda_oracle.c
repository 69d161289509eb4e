/*
 * kda_oracle.c -- plain, slow, fp64 CPU oracle for the KDA forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this library.  The product
 * path (libkda.so and its Python binding) never routes through it, and it
 * shares no code, header, table or helper with the HIP path.
 *
 * What it computes: the token-by-token gated delta rule with per-channel
 * log-decay, one independent recurrence per (batch, head).
 *
 *   "From Numerical Stability to Load Balancing ..." section 2.1: a
 *   fixed-shape state matrix S is decayed by a per-step factor and then
 *   receives key/value outer products.  The pages name the delta rule (Delta
 *   networks in "Architecting Long-Context LLMs ..." section 2.1, Delta
 *   Net-like in "Architecture Analysis ..." section 2.1, delta-rule-based
 *   models in "From Numerical Stability ..." section 1) but never write it
 *   out; the reading used here is the plainest one consistent with a
 *   per-key-channel decay:
 *
 *     g_t   = gate(w_t)                          (dk values, one per key channel)
 *     S     = Diag(exp(g_t)) S                   (forget: row c of S scaled by e^{g_tc})
 *     u_t   = beta_t (v_t - S^T k_t)             (delta-rule prediction error)
 *     S     = S + k_t u_t^T                      (write)
 *     o_t   = S^T q_t                            (read, inclusive of token t)
 *
 *   gate: bounded   g = g_min * sigmoid(w)  ("Architecting ..." section 2.2;
 *                   "Architecture Analysis ..." section 2.2 pseudo-code;
 *                   "Demystifying ..." Breakthrough 1 part 2;
 *                   "From Numerical Stability ..." section 2.2)
 *         unbounded g = -softplus(w)        (the conventional form the same
 *                   sections contrast against), selected by g_min = -INFINITY.
 *
 *   S starts at S0 (zeros when S0 is NULL).  No q scaling, no normalisation:
 *   inputs are used exactly as given.
 *
 * Per-chunk spans (for predicting which chunks overflow): the chunk-local sum
 * of g over a chunk of `chunk` tokens, minimised over key channels
 * ("From Numerical Stability ..." section 2.2: a 16-token tile spans at least
 * 16 * g_min; "Demystifying ..." Breakthrough 1 part 2: the cumulative decay of
 * an L = 16 chunk is at least exp(-80)).
 *
 * Layouts (row-major, float64): q, k, w [B,H,T,dk]; v [B,H,T,dv]; beta [B,H,T];
 * S0, S_final [B,H,dk,dv]; o [B,H,T,dv]; spans [B,H,ceil(T/chunk)].
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* sigmoid(w) = 1 / (1 + e^{-w}) evaluated without overflow for either sign */
static double sigmoid(double w) {
  if (w >= 0.0) return 1.0 / (1.0 + exp(-w));
  double e = exp(w);
  return e / (1.0 + e);
}

/* softplus(w) = log(1 + e^{w}) = max(w, 0) + log1p(e^{-|w|}) */
static double softplus(double w) {
  return (w > 0.0 ? w : 0.0) + log1p(exp(-fabs(w)));
}

double kda_oracle_gate(double w, double g_min) {
  if (isinf(g_min) && g_min < 0.0) return -softplus(w);
  return g_min * sigmoid(w);
}

/* out[i] = gate(w[i]) for i < n */
int kda_oracle_gate_array(const double* w, int64_t n, double g_min, double* out) {
  if (n < 0 || (n > 0 && (!w || !out))) return -1;
  if (isnan(g_min) || g_min > 0.0) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = kda_oracle_gate(w[i], g_min);
  return 0;
}

typedef struct {
  const double *q, *k, *v, *w, *beta, *S0;
  double g_min;
  int64_t B, H, T, dk, dv;
  double *o, *S_final;
  int64_t next;        /* next (b,h) index to process */
  pthread_mutex_t lock;
} job_t;

static void run_head(const job_t* J, int64_t bh) {
  const int64_t T = J->T, dk = J->dk, dv = J->dv;
  const double* q = J->q + bh * T * dk;
  const double* k = J->k + bh * T * dk;
  const double* v = J->v + bh * T * dv;
  const double* w = J->w + bh * T * dk;
  const double* beta = J->beta + bh * T;
  double* o = J->o + bh * T * dv;
  double* S = J->S_final + bh * dk * dv;
  double* g = (double*)malloc(sizeof(double) * dk);
  double* kS = (double*)malloc(sizeof(double) * dv);
  double* u = (double*)malloc(sizeof(double) * dv);

  if (J->S0) memcpy(S, J->S0 + bh * dk * dv, sizeof(double) * dk * dv);
  else memset(S, 0, sizeof(double) * dk * dv);

  for (int64_t t = 0; t < T; ++t) {
    const double* qt = q + t * dk;
    const double* kt = k + t * dk;
    const double* vt = v + t * dv;
    const double* wt = w + t * dk;
    /* forget: row c of S decays by e^{g_tc} */
    for (int64_t c = 0; c < dk; ++c) {
      g[c] = kda_oracle_gate(wt[c], J->g_min);
      double d = exp(g[c]);
      double* row = S + c * dv;
      for (int64_t j = 0; j < dv; ++j) row[j] *= d;
    }
    /* prediction S^T k_t with the decayed state */
    for (int64_t j = 0; j < dv; ++j) kS[j] = 0.0;
    for (int64_t c = 0; c < dk; ++c) {
      const double kc = kt[c];
      const double* row = S + c * dv;
      for (int64_t j = 0; j < dv; ++j) kS[j] += kc * row[j];
    }
    /* delta-rule error, then the rank-one write */
    for (int64_t j = 0; j < dv; ++j) u[j] = beta[t] * (vt[j] - kS[j]);
    for (int64_t c = 0; c < dk; ++c) {
      const double kc = kt[c];
      double* row = S + c * dv;
      for (int64_t j = 0; j < dv; ++j) row[j] += kc * u[j];
    }
    /* read with the updated state */
    double* ot = o + t * dv;
    for (int64_t j = 0; j < dv; ++j) ot[j] = 0.0;
    for (int64_t c = 0; c < dk; ++c) {
      const double qc = qt[c];
      const double* row = S + c * dv;
      for (int64_t j = 0; j < dv; ++j) ot[j] += qc * row[j];
    }
  }
  free(g); free(kS); free(u);
}

static void* worker(void* arg) {
  job_t* J = (job_t*)arg;
  for (;;) {
    pthread_mutex_lock(&J->lock);
    int64_t bh = J->next++;
    pthread_mutex_unlock(&J->lock);
    if (bh >= J->B * J->H) break;
    run_head(J, bh);
  }
  return NULL;
}

/* Returns 0 on success, -1 on bad arguments. nthreads <= 0 means one thread. */
int kda_oracle_f64(const double* q, const double* k, const double* v, const double* w,
                   const double* beta, const double* S0, double g_min,
                   int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                   double* o, double* S_final, int nthreads) {
  if (B < 1 || H < 1 || T < 0 || dk < 1 || dv < 1 || !S_final) return -1;
  if (T > 0 && (!q || !k || !v || !w || !beta || !o)) return -1;
  if (isnan(g_min) || g_min > 0.0) return -1;
  job_t J;
  J.q = q; J.k = k; J.v = v; J.w = w; J.beta = beta; J.S0 = S0; J.g_min = g_min;
  J.B = B; J.H = H; J.T = T; J.dk = dk; J.dv = dv; J.o = o; J.S_final = S_final;
  J.next = 0;
  pthread_mutex_init(&J.lock, NULL);
  int64_t n = nthreads < 1 ? 1 : nthreads;
  if (n > B * H) n = B * H;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * n);
  for (int64_t i = 1; i < n; ++i) pthread_create(&th[i], NULL, worker, &J);
  worker(&J);
  for (int64_t i = 1; i < n; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&J.lock);
  return 0;
}

/* ---------------------------------------------------------------- backward (adjoint of the recurrence)
 *
 * Gradients of a scalar loss L with dL/do = dO and dL/dS_final = dSf (NULL: zero), by reverse-mode
 * differentiation of the token recurrence above, one step at a time from the last token back:
 *
 *   o_t = S_t^T q_t                 dq_t  = S_t do_t;          dS_t += q_t do_t^T
 *   S_t = S' + k_t u^T              dk_t += dS_t u;            du    = dS_t^T k_t;       dS' = dS_t
 *   u   = beta_t (v_t - S'^T k_t)   dbeta_t = du . (v_t - S'^T k_t);  dv_t = beta_t du;
 *                                   z = -beta_t du:  dS' += k_t z^T;  dk_t += S' z
 *   S'  = Diag(e^{g_t}) S_{t-1}     dS_{t-1} = Diag(e^{g_t}) dS';  dg_tc = sum_j dS'[c][j] S'[c][j]
 *   g_t = gate(w_t)                 dw_tc = dg_tc gate'(w_tc):  g_min sigma (1 - sigma), or -sigma
 *
 * and dS0 = dS_0 at the end.  The forward states S_0 .. S_T of each head are kept ((T + 1) dk dv
 * doubles per head in flight), so this is for the small sizes the tests use.
 */

/* d gate / d w */
static double gate_deriv(double w, double g_min) {
  const double s = sigmoid(w);
  if (isinf(g_min) && g_min < 0.0) return -s;
  return g_min * s * (1.0 - s);
}

typedef struct {
  const double *q, *k, *v, *w, *beta, *S0, *dO, *dSf;
  double g_min;
  int64_t B, H, T, dk, dv;
  double *dq, *dk_, *dv_, *dw, *dbeta, *dS0;
  int64_t next;
  int failed;
  pthread_mutex_t lock;
} bjob_t;

static int run_head_bwd(const bjob_t* J, int64_t bh) {
  const int64_t T = J->T, dk = J->dk, dv = J->dv, n = dk * dv;
  const double* q = J->q + bh * T * dk;
  const double* k = J->k + bh * T * dk;
  const double* v = J->v + bh * T * dv;
  const double* w = J->w + bh * T * dk;
  const double* beta = J->beta + bh * T;
  const double* dO = J->dO + bh * T * dv;
  double* hist = (double*)malloc(sizeof(double) * n * (T + 1));   /* S_0 .. S_T */
  double* Sp = (double*)malloc(sizeof(double) * n);                /* S' of the step being undone */
  double* dS = (double*)malloc(sizeof(double) * n);
  double* eg = (double*)malloc(sizeof(double) * dk);
  double* kS = (double*)malloc(sizeof(double) * dv);
  double* u = (double*)malloc(sizeof(double) * dv);
  double* du = (double*)malloc(sizeof(double) * dv);
  if (!hist || !Sp || !dS || !eg || !kS || !u || !du) {
    free(hist); free(Sp); free(dS); free(eg); free(kS); free(u); free(du);
    return -1;
  }
  /* forward, keeping every state */
  if (J->S0) memcpy(hist, J->S0 + bh * n, sizeof(double) * n);
  else memset(hist, 0, sizeof(double) * n);
  for (int64_t t = 0; t < T; ++t) {
    const double* Sprev = hist + t * n;
    double* S = hist + (t + 1) * n;
    for (int64_t c = 0; c < dk; ++c) {
      const double d = exp(kda_oracle_gate(w[t * dk + c], J->g_min));
      for (int64_t j = 0; j < dv; ++j) S[c * dv + j] = d * Sprev[c * dv + j];
    }
    for (int64_t j = 0; j < dv; ++j) kS[j] = 0.0;
    for (int64_t c = 0; c < dk; ++c)
      for (int64_t j = 0; j < dv; ++j) kS[j] += k[t * dk + c] * S[c * dv + j];
    for (int64_t j = 0; j < dv; ++j) u[j] = beta[t] * (v[t * dv + j] - kS[j]);
    for (int64_t c = 0; c < dk; ++c)
      for (int64_t j = 0; j < dv; ++j) S[c * dv + j] += k[t * dk + c] * u[j];
  }
  /* backward */
  if (J->dSf) memcpy(dS, J->dSf + bh * n, sizeof(double) * n);
  else memset(dS, 0, sizeof(double) * n);
  for (int64_t t = T - 1; t >= 0; --t) {
    const double* Sprev = hist + t * n;
    const double* St = hist + (t + 1) * n;
    const double* qt = q + t * dk;
    const double* kt = k + t * dk;
    const double* dot = dO + t * dv;
    double* dqt = J->dq + (bh * T + t) * dk;
    double* dkt = J->dk_ + (bh * T + t) * dk;
    double* dvt = J->dv_ + (bh * T + t) * dv;
    double* dwt = J->dw + (bh * T + t) * dk;
    /* recompute this step's S' and u */
    for (int64_t c = 0; c < dk; ++c) {
      eg[c] = exp(kda_oracle_gate(w[t * dk + c], J->g_min));
      for (int64_t j = 0; j < dv; ++j) Sp[c * dv + j] = eg[c] * Sprev[c * dv + j];
    }
    for (int64_t j = 0; j < dv; ++j) kS[j] = 0.0;
    for (int64_t c = 0; c < dk; ++c)
      for (int64_t j = 0; j < dv; ++j) kS[j] += kt[c] * Sp[c * dv + j];
    for (int64_t j = 0; j < dv; ++j) u[j] = beta[t] * (v[t * dv + j] - kS[j]);
    /* read */
    for (int64_t c = 0; c < dk; ++c) {
      double a = 0.0;
      for (int64_t j = 0; j < dv; ++j) a += St[c * dv + j] * dot[j];
      dqt[c] = a;
      for (int64_t j = 0; j < dv; ++j) dS[c * dv + j] += qt[c] * dot[j];
    }
    /* write */
    for (int64_t c = 0; c < dk; ++c) {
      double a = 0.0;
      for (int64_t j = 0; j < dv; ++j) a += dS[c * dv + j] * u[j];
      dkt[c] = a;
    }
    for (int64_t j = 0; j < dv; ++j) {
      double a = 0.0;
      for (int64_t c = 0; c < dk; ++c) a += dS[c * dv + j] * kt[c];
      du[j] = a;
    }
    /* delta-rule error (dS now stands for dS') */
    double db = 0.0;
    for (int64_t j = 0; j < dv; ++j) {
      db += du[j] * (v[t * dv + j] - kS[j]);
      dvt[j] = beta[t] * du[j];
      du[j] = -beta[t] * du[j];   /* z */
    }
    J->dbeta[bh * T + t] = db;
    for (int64_t c = 0; c < dk; ++c) {
      double a = 0.0;
      for (int64_t j = 0; j < dv; ++j) {
        a += Sp[c * dv + j] * du[j];
        dS[c * dv + j] += kt[c] * du[j];
      }
      dkt[c] += a;
    }
    /* forget */
    for (int64_t c = 0; c < dk; ++c) {
      double a = 0.0;
      for (int64_t j = 0; j < dv; ++j) {
        a += dS[c * dv + j] * Sp[c * dv + j];
        dS[c * dv + j] *= eg[c];
      }
      dwt[c] = a * gate_deriv(w[t * dk + c], J->g_min);
    }
  }
  if (J->dS0) memcpy(J->dS0 + bh * n, dS, sizeof(double) * n);
  free(hist); free(Sp); free(dS); free(eg); free(kS); free(u); free(du);
  return 0;
}

static void* bworker(void* arg) {
  bjob_t* J = (bjob_t*)arg;
  for (;;) {
    pthread_mutex_lock(&J->lock);
    int64_t bh = J->next++;
    pthread_mutex_unlock(&J->lock);
    if (bh >= J->B * J->H) break;
    if (run_head_bwd(J, bh) != 0) {
      pthread_mutex_lock(&J->lock);
      J->failed = 1;
      pthread_mutex_unlock(&J->lock);
    }
  }
  return NULL;
}

/* Gradients [same layouts as the inputs]; dSf and dS0 may be NULL.  Returns 0, or -1 on bad
 * arguments or when the state history does not fit in memory. */
int kda_oracle_bwd_f64(const double* q, const double* k, const double* v, const double* w,
                       const double* beta, const double* S0, double g_min,
                       int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                       const double* dO, const double* dSf,
                       double* dq, double* dk_out, double* dv_out, double* dw, double* dbeta, double* dS0,
                       int nthreads) {
  if (B < 1 || H < 1 || T < 0 || dk < 1 || dv < 1) return -1;
  if (T > 0 && (!q || !k || !v || !w || !beta || !dO || !dq || !dk_out || !dv_out || !dw || !dbeta)) return -1;
  if (isnan(g_min) || g_min > 0.0) return -1;
  bjob_t J;
  J.q = q; J.k = k; J.v = v; J.w = w; J.beta = beta; J.S0 = S0; J.dO = dO; J.dSf = dSf;
  J.g_min = g_min; J.B = B; J.H = H; J.T = T; J.dk = dk; J.dv = dv;
  J.dq = dq; J.dk_ = dk_out; J.dv_ = dv_out; J.dw = dw; J.dbeta = dbeta; J.dS0 = dS0;
  J.next = 0; J.failed = 0;
  pthread_mutex_init(&J.lock, NULL);
  int64_t nt = nthreads < 1 ? 1 : nthreads;
  if (nt > B * H) nt = B * H;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nt);
  for (int64_t i = 1; i < nt; ++i) pthread_create(&th[i], NULL, bworker, &J);
  bworker(&J);
  for (int64_t i = 1; i < nt; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&J.lock);
  return J.failed ? -1 : 0;
}

/* spans[b,h,n] = min over key channels c of the sum of g over the tokens of chunk n. */
int kda_oracle_spans_f64(const double* w, double g_min, int64_t B, int64_t H, int64_t T,
                         int64_t dk, int64_t chunk, double* spans) {
  if (B < 1 || H < 1 || T < 0 || dk < 1 || chunk < 1 || !spans) return -1;
  if (T > 0 && !w) return -1;
  if (isnan(g_min) || g_min > 0.0) return -1;
  const int64_t NC = (T + chunk - 1) / chunk;
  double* acc = (double*)malloc(sizeof(double) * dk);
  for (int64_t bh = 0; bh < B * H; ++bh) {
    for (int64_t n = 0; n < NC; ++n) {
      for (int64_t c = 0; c < dk; ++c) acc[c] = 0.0;
      const int64_t t1 = (n + 1) * chunk < T ? (n + 1) * chunk : T;
      for (int64_t t = n * chunk; t < t1; ++t)
        for (int64_t c = 0; c < dk; ++c) acc[c] += kda_oracle_gate(w[(bh * T + t) * dk + c], g_min);
      double m = acc[0];
      for (int64_t c = 1; c < dk; ++c) m = acc[c] < m ? acc[c] : m;
      spans[bh * NC + n] = m;
    }
  }
  free(acc);
  return 0;
}
