/*
 * kda_ref.c - fp64 CPU oracle for Kimi Delta Attention (KDA).
 *
 * TEST INFRASTRUCTURE ONLY (see kda_ref.h).  A plain, slow, obviously correct
 * token-by-token recurrence; no chunking, blocking or reordering.
 *
 * Source of each step (page "[Paper Review] Kimi K3: Open Frontier
 * Intelligence", section "Method / Architecture" -> "Kimi Delta Attention
 * (KDA)"):
 *   - the per-head recurrence: Diag(alpha_t) decays the prior state per key
 *     channel, (I - beta_t k_t k_t^T) erases the key direction, then k_t v_t^T
 *     is written with strength beta_t (the update paragraph; its displayed
 *     equation was lost in extraction, so the form used is the pinned one:
 *     S_t = (I - beta k k^T) Diag(alpha) S_{t-1} + beta k v^T, o_t = S_t^T q_t);
 *   - q and k are L2-normalised (the projections paragraph);
 *   - the log-decay is a scaled sigmoid bounded below by g_min = -5 (the
 *     "Lower-bounded decay" paragraph), read as g = -5 * sigmoid(a) with the
 *     per-head log-scale A_h at its initial value 0;
 *   - the output passes a full-rank sigmoid gate (the "Full-rank gate"
 *     paragraph), channel-wise over dv.
 */
#include "kda_ref.h"

#include <math.h>
#include <pthread.h>
#include <stdatomic.h>
#include <stdlib.h>
#include <string.h>

/* Logistic function; sigmoid(-inf) = 0 and sigmoid(+inf) = 1 exactly. */
static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

typedef struct {
  int32_t num_seqs, H, dk, dv;
  const int64_t* cu;
  const double *q, *k, *v, *a, *b, *gate, *s0;
  double *o, *s_final;
  atomic_long next;
} fwd_job;

/* One token of the recurrence for one head.  S is dk x dv (row = key channel),
 * updated in place; y receives the gated output row.  Work buffers:
 * qh, kh, alpha (dk), u (dv). */
static void kda_ref_token(int32_t dk, int32_t dv, double* S, const double* q, const double* k,
                          const double* v, const double* a, double b, const double* gate,
                          double* y, double* qh, double* kh, double* alpha, double* u) {
  /* L2 normalisation of q and k over the key channels. */
  double sq = 0.0, sk = 0.0;
  for (int32_t c = 0; c < dk; ++c) {
    sq += q[c] * q[c];
    sk += k[c] * k[c];
  }
  double rq = 1.0 / sqrt(sq + KDA_REF_EPS), rk = 1.0 / sqrt(sk + KDA_REF_EPS);
  for (int32_t c = 0; c < dk; ++c) {
    qh[c] = q[c] * rq;
    kh[c] = k[c] * rk;
  }
  /* Retention per key channel and write strength per token. */
  for (int32_t c = 0; c < dk; ++c) alpha[c] = exp(KDA_REF_GMIN * sigmoid(a[c]));
  double beta = sigmoid(b);

  /* S' = Diag(alpha) S. */
  for (int32_t c = 0; c < dk; ++c)
    for (int32_t j = 0; j < dv; ++j) S[(size_t)c * dv + j] *= alpha[c];
  /* u = beta (v - S'^T kh): the delta-rule correction. */
  for (int32_t j = 0; j < dv; ++j) {
    double w = 0.0;
    for (int32_t c = 0; c < dk; ++c) w += kh[c] * S[(size_t)c * dv + j];
    u[j] = beta * (v[j] - w);
  }
  /* S = S' + kh u^T  (== (I - beta kh kh^T) S' + beta kh v^T). */
  for (int32_t c = 0; c < dk; ++c)
    for (int32_t j = 0; j < dv; ++j) S[(size_t)c * dv + j] += kh[c] * u[j];
  /* o = S^T qh, then the output gate. */
  for (int32_t j = 0; j < dv; ++j) {
    double acc = 0.0;
    for (int32_t c = 0; c < dk; ++c) acc += qh[c] * S[(size_t)c * dv + j];
    y[j] = gate ? sigmoid(gate[j]) * acc : acc;
  }
}

static void* fwd_worker(void* p) {
  fwd_job* J = (fwd_job*)p;
  const int32_t H = J->H, dk = J->dk, dv = J->dv;
  double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
  double* wk = (double*)malloc(sizeof(double) * (size_t)(3 * dk + dv));
  if (!S || !wk) abort();
  double *qh = wk, *kh = wk + dk, *alpha = wk + 2 * dk, *u = wk + 3 * dk;
  const long total = (long)J->num_seqs * H;
  for (;;) {
    long item = atomic_fetch_add(&J->next, 1);
    if (item >= total) break;
    int32_t n = (int32_t)(item / H), h = (int32_t)(item % H);
    size_t soff = ((size_t)n * H + h) * (size_t)dk * dv;
    if (J->s0)
      memcpy(S, J->s0 + soff, sizeof(double) * (size_t)dk * dv);
    else
      memset(S, 0, sizeof(double) * (size_t)dk * dv);
    for (int64_t t = J->cu[n]; t < J->cu[n + 1]; ++t) {
      size_t th = (size_t)t * H + h;
      kda_ref_token(dk, dv, S, J->q + th * dk, J->k + th * dk, J->v + th * dv, J->a + th * dk,
                    J->b[th], J->gate ? J->gate + th * dv : NULL, J->o + th * dv, qh, kh, alpha,
                    u);
    }
    if (J->s_final) memcpy(J->s_final + soff, S, sizeof(double) * (size_t)dk * dv);
  }
  free(S);
  free(wk);
  return NULL;
}

static int run_threads(void* (*fn)(void*), void* job, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 512) nthreads = 512;
  pthread_t th[512];
  int started = 0;
  for (int t = 1; t < nthreads; ++t) {
    if (pthread_create(&th[t], NULL, fn, job) != 0) break;
    ++started;
  }
  fn(job);
  for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
  return 0;
}

int kda_ref_fwd(int32_t num_seqs, const int64_t* cu_seqlens, int32_t H, int32_t dk, int32_t dv,
                const double* q, const double* k, const double* v, const double* a,
                const double* b, const double* gate, const double* s0, double* o,
                double* s_final, int nthreads) {
  if (num_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0 || !cu_seqlens) return -1;
  if (cu_seqlens[0] != 0) return -1;
  for (int32_t n = 0; n < num_seqs; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
  if (cu_seqlens[num_seqs] > 0 && (!q || !k || !v || !a || !b || !o)) return -1;
  fwd_job J = {num_seqs, H, dk, dv, cu_seqlens, q, k, v, a, b, gate, s0, o, s_final, 0};
  return run_threads(fwd_worker, &J, nthreads);
}

typedef struct {
  int32_t num_seqs, H, dk, dv;
  const double *q, *k, *v, *a, *b, *gate;
  double *state, *o;
  atomic_long next;
} dec_job;

static void* dec_worker(void* p) {
  dec_job* J = (dec_job*)p;
  const int32_t H = J->H, dk = J->dk, dv = J->dv;
  double* wk = (double*)malloc(sizeof(double) * (size_t)(3 * dk + dv));
  if (!wk) abort();
  double *qh = wk, *kh = wk + dk, *alpha = wk + 2 * dk, *u = wk + 3 * dk;
  const long total = (long)J->num_seqs * H;
  for (;;) {
    long item = atomic_fetch_add(&J->next, 1);
    if (item >= total) break;
    size_t th = (size_t)item;
    kda_ref_token(dk, dv, J->state + th * (size_t)dk * dv, J->q + th * dk, J->k + th * dk,
                  J->v + th * dv, J->a + th * dk, J->b[th], J->gate ? J->gate + th * dv : NULL,
                  J->o + th * dv, qh, kh, alpha, u);
  }
  free(wk);
  return NULL;
}

int kda_ref_decode_step(int32_t num_seqs, int32_t H, int32_t dk, int32_t dv, const double* q,
                        const double* k, const double* v, const double* a, const double* b,
                        const double* gate, double* state, double* o, int nthreads) {
  if (num_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
  if (num_seqs > 0 && (!q || !k || !v || !a || !b || !state || !o)) return -1;
  dec_job J = {num_seqs, H, dk, dv, q, k, v, a, b, gate, state, o, 0};
  return run_threads(dec_worker, &J, nthreads);
}

/* ---- Segment transitions ------------------------------------------------
 * Page "[Paper Review] Kimi K3...", section "Infrastructure: how to actually
 * run trillion-scale", KDA co-design item: a segment's effect on the state is
 * a cumulative transition plus a locally generated state.  Written out from
 * the recurrence: each token applies S -> F_t S + beta_t kh_t v_t^T with the
 * dk x dk factor F_t = (I - beta_t kh_t kh_t^T) Diag(alpha_t), so a segment
 * maps a start state S0 to M S0 + S_loc with M = F_last ... F_first and S_loc
 * the state reached from S0 = 0.  Here F_t is formed as a dense matrix and
 * multiplied in, the plainest form of that definition. */
typedef struct {
  int32_t num_seqs, H, dk, dv;
  const int64_t* cu;
  const double *k, *v, *a, *b;
  double* trans;
  atomic_long next;
} trans_job;

static void* trans_worker(void* p) {
  trans_job* J = (trans_job*)p;
  const int32_t H = J->H, dk = J->dk, dv = J->dv, w = dv + dk;
  double* X = (double*)malloc(sizeof(double) * (size_t)dk * w);  /* [S_loc | M] */
  double* Y = (double*)malloc(sizeof(double) * (size_t)dk * w);
  double* F = (double*)malloc(sizeof(double) * (size_t)dk * dk);
  double* kh = (double*)malloc(sizeof(double) * (size_t)dk);
  if (!X || !Y || !F || !kh) abort();
  const long total = (long)J->num_seqs * H;
  for (;;) {
    long item = atomic_fetch_add(&J->next, 1);
    if (item >= total) break;
    int32_t n = (int32_t)(item / H), h = (int32_t)(item % H);
    /* S_loc = 0, M = I. */
    for (int32_t r = 0; r < dk; ++r)
      for (int32_t j = 0; j < w; ++j) X[(size_t)r * w + j] = (j - dv == r) ? 1.0 : 0.0;
    for (int64_t t = J->cu[n]; t < J->cu[n + 1]; ++t) {
      size_t th = (size_t)t * H + h;
      const double* k = J->k + th * dk;
      const double* v = J->v + th * dv;
      const double* a = J->a + th * dk;
      double sk = 0.0;
      for (int32_t c = 0; c < dk; ++c) sk += k[c] * k[c];
      double rk = 1.0 / sqrt(sk + KDA_REF_EPS);
      for (int32_t c = 0; c < dk; ++c) kh[c] = k[c] * rk;
      double beta = sigmoid(J->b[th]);
      /* F = (I - beta kh kh^T) Diag(alpha), alpha = exp(g_min sigmoid(a)). */
      for (int32_t r = 0; r < dk; ++r)
        for (int32_t c = 0; c < dk; ++c)
          F[(size_t)r * dk + c] = ((r == c ? 1.0 : 0.0) - beta * kh[r] * kh[c]) *
                                  exp(KDA_REF_GMIN * sigmoid(a[c]));
      /* [S_loc | M] <- F [S_loc | M] + [beta kh v^T | 0]. */
      for (int32_t r = 0; r < dk; ++r)
        for (int32_t j = 0; j < w; ++j) {
          double acc = j < dv ? beta * kh[r] * v[j] : 0.0;
          for (int32_t c = 0; c < dk; ++c) acc += F[(size_t)r * dk + c] * X[(size_t)c * w + j];
          Y[(size_t)r * w + j] = acc;
        }
      memcpy(X, Y, sizeof(double) * (size_t)dk * w);
    }
    memcpy(J->trans + (size_t)item * dk * w, X, sizeof(double) * (size_t)dk * w);
  }
  free(X);
  free(Y);
  free(F);
  free(kh);
  return NULL;
}

int kda_ref_segment_transition(int32_t num_seqs, const int64_t* cu_seqlens, int32_t H,
                               int32_t dk, int32_t dv, const double* k, const double* v,
                               const double* a, const double* b, double* trans, int nthreads) {
  if (num_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0 || !cu_seqlens) return -1;
  if (cu_seqlens[0] != 0) return -1;
  for (int32_t n = 0; n < num_seqs; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
  if (num_seqs > 0 && !trans) return -1;
  if (cu_seqlens[num_seqs] > 0 && (!k || !v || !a || !b)) return -1;
  trans_job J = {num_seqs, H, dk, dv, cu_seqlens, k, v, a, b, trans, 0};
  return run_threads(trans_worker, &J, nthreads);
}

/* ---- Backward (reverse mode) --------------------------------------------
 * Gradients of L = sum_t <dy_t, y_t> + <dS_final, S_final> with respect to
 * every input of kda_ref_fwd, by the chain rule applied to the same token
 * recurrence in reverse order.  With S' = Diag(alpha) S_{t-1},
 * w = S'^T kh, u = beta (v - w), S_t = S' + kh u^T, o = S_t^T qh,
 * y = sigmoid(gate) o, and dS the adjoint of S_t:
 *   dgate = dy o sigmoid'(gate),  do = dy sigmoid(gate),  dS += qh do^T
 *   dqh = S_t do,  du = dS^T kh,  dkh = dS u - beta S' du
 *   dv = beta du,  dbeta = du . (v - w)
 *   dS' = dS - beta kh du^T,  dalpha_c = sum_j dS'_cj S_{t-1,cj}
 *   dS_{t-1} = Diag(alpha) dS'
 * then through the input maps: qh = q r (r = (|q|^2 + eps)^-1/2),
 * dq = r dqh - r^3 (q . dqh) q (same for k); alpha = exp(-5 sigmoid(a)),
 * da = dalpha alpha (-5) sigmoid(a)(1 - sigmoid(a)); db = dbeta beta (1 - beta).
 * The states of a sequence are all kept (slow and simple: test sizes). */
typedef struct {
  int32_t num_seqs, H, dk, dv;
  const int64_t* cu;
  const double *q, *k, *v, *a, *b, *gate, *s0, *dy, *dsf;
  double *dq, *dk_, *dv_, *da, *db, *dgate, *ds0;
  atomic_long next;
} bwd_job;

static void* bwd_worker(void* p) {
  bwd_job* J = (bwd_job*)p;
  const int32_t H = J->H, dk = J->dk, dv = J->dv;
  const size_t SS = (size_t)dk * dv;
  double* vec = (double*)malloc(sizeof(double) * (size_t)(8 * dk + 8 * dv));
  double* dS = (double*)malloc(sizeof(double) * SS);
  double* dSp = (double*)malloc(sizeof(double) * SS);
  if (!vec || !dS || !dSp) abort();
  double *qh = vec, *kh = vec + dk, *alpha = vec + 2 * dk, *dqh = vec + 3 * dk,
         *dkh = vec + 4 * dk, *dalpha = vec + 5 * dk;
  double *w = vec + 8 * dk, *u = w + dv, *o = u + dv, *dO = o + dv, *du = dO + dv;
  const long total = (long)J->num_seqs * H;
  for (;;) {
    long item = atomic_fetch_add(&J->next, 1);
    if (item >= total) break;
    int32_t n = (int32_t)(item / H), h = (int32_t)(item % H);
    const int64_t t0 = J->cu[n], L = J->cu[n + 1] - t0;
    double* S = (double*)malloc(sizeof(double) * SS * (size_t)(L + 1));  /* S_0 .. S_L */
    if (!S) abort();
    const size_t soff = ((size_t)n * H + h) * SS;
    if (J->s0) memcpy(S, J->s0 + soff, sizeof(double) * SS);
    else memset(S, 0, sizeof(double) * SS);
    /* forward, keeping every state */
    for (int64_t t = 0; t < L; ++t) {
      size_t th = (size_t)(t0 + t) * H + h;
      const double *k = J->k + th * dk, *v = J->v + th * dv, *a = J->a + th * dk;
      double sk = 0.0;
      for (int32_t c = 0; c < dk; ++c) sk += k[c] * k[c];
      double rk = 1.0 / sqrt(sk + KDA_REF_EPS), beta = sigmoid(J->b[th]);
      double* Sp = S + SS * (size_t)t;
      double* Sn = S + SS * (size_t)(t + 1);
      for (int32_t c = 0; c < dk; ++c) {
        kh[c] = k[c] * rk;
        alpha[c] = exp(KDA_REF_GMIN * sigmoid(a[c]));
      }
      for (int32_t j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int32_t c = 0; c < dk; ++c) acc += kh[c] * alpha[c] * Sp[(size_t)c * dv + j];
        u[j] = beta * (v[j] - acc);
      }
      for (int32_t c = 0; c < dk; ++c)
        for (int32_t j = 0; j < dv; ++j)
          Sn[(size_t)c * dv + j] = alpha[c] * Sp[(size_t)c * dv + j] + kh[c] * u[j];
    }
    if (J->dsf) memcpy(dS, J->dsf + soff, sizeof(double) * SS);
    else memset(dS, 0, sizeof(double) * SS);
    for (int64_t t = L - 1; t >= 0; --t) {
      size_t th = (size_t)(t0 + t) * H + h;
      const double *q = J->q + th * dk, *k = J->k + th * dk, *v = J->v + th * dv,
                   *a = J->a + th * dk, *dy = J->dy + th * dv;
      const double* gt = J->gate ? J->gate + th * dv : NULL;
      const double *Sp = S + SS * (size_t)t, *Sn = S + SS * (size_t)(t + 1);
      double sq = 0.0, sk = 0.0;
      for (int32_t c = 0; c < dk; ++c) {
        sq += q[c] * q[c];
        sk += k[c] * k[c];
      }
      const double rq = 1.0 / sqrt(sq + KDA_REF_EPS), rk = 1.0 / sqrt(sk + KDA_REF_EPS);
      const double beta = sigmoid(J->b[th]);
      for (int32_t c = 0; c < dk; ++c) {
        qh[c] = q[c] * rq;
        kh[c] = k[c] * rk;
        alpha[c] = exp(KDA_REF_GMIN * sigmoid(a[c]));
      }
      /* output and gate */
      for (int32_t j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int32_t c = 0; c < dk; ++c) acc += qh[c] * Sn[(size_t)c * dv + j];
        o[j] = acc;
        const double sg = gt ? sigmoid(gt[j]) : 1.0;
        if (J->dgate) J->dgate[th * dv + j] = gt ? dy[j] * acc * sg * (1.0 - sg) : 0.0;
        dO[j] = dy[j] * sg;
      }
      for (int32_t c = 0; c < dk; ++c)
        for (int32_t j = 0; j < dv; ++j) dS[(size_t)c * dv + j] += qh[c] * dO[j];
      for (int32_t c = 0; c < dk; ++c) {
        double acc = 0.0;
        for (int32_t j = 0; j < dv; ++j) acc += Sn[(size_t)c * dv + j] * dO[j];
        dqh[c] = acc;
      }
      /* w, u of this token (recomputed from S_{t-1}) */
      for (int32_t j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int32_t c = 0; c < dk; ++c) acc += kh[c] * alpha[c] * Sp[(size_t)c * dv + j];
        w[j] = acc;
        u[j] = beta * (v[j] - acc);
      }
      double dbeta = 0.0;
      for (int32_t j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int32_t c = 0; c < dk; ++c) acc += dS[(size_t)c * dv + j] * kh[c];
        du[j] = acc;
        J->dv_[th * dv + j] = beta * acc;
        dbeta += acc * (v[j] - w[j]);
      }
      for (int32_t c = 0; c < dk; ++c) {
        double acc = 0.0;
        for (int32_t j = 0; j < dv; ++j)
          acc += dS[(size_t)c * dv + j] * u[j] -
                 beta * alpha[c] * Sp[(size_t)c * dv + j] * du[j];
        dkh[c] = acc;
      }
      for (int32_t c = 0; c < dk; ++c) {
        double acc = 0.0;
        for (int32_t j = 0; j < dv; ++j) {
          const double d = dS[(size_t)c * dv + j] - beta * kh[c] * du[j];
          dSp[(size_t)c * dv + j] = d;
          acc += d * Sp[(size_t)c * dv + j];
        }
        dalpha[c] = acc;
      }
      for (int32_t c = 0; c < dk; ++c)
        for (int32_t j = 0; j < dv; ++j)
          dS[(size_t)c * dv + j] = alpha[c] * dSp[(size_t)c * dv + j];
      /* through the input maps */
      double qd = 0.0, kd = 0.0;
      for (int32_t c = 0; c < dk; ++c) {
        qd += q[c] * dqh[c];
        kd += k[c] * dkh[c];
      }
      for (int32_t c = 0; c < dk; ++c) {
        J->dq[th * dk + c] = rq * dqh[c] - rq * rq * rq * qd * q[c];
        J->dk_[th * dk + c] = rk * dkh[c] - rk * rk * rk * kd * k[c];
        const double sa = sigmoid(a[c]);
        J->da[th * dk + c] = dalpha[c] * alpha[c] * KDA_REF_GMIN * sa * (1.0 - sa);
      }
      J->db[th] = dbeta * beta * (1.0 - beta);
    }
    if (J->ds0) memcpy(J->ds0 + soff, dS, sizeof(double) * SS);
    free(S);
  }
  free(vec);
  free(dS);
  free(dSp);
  return NULL;
}

int kda_ref_bwd(int32_t num_seqs, const int64_t* cu_seqlens, int32_t H, int32_t dk, int32_t dv,
                const double* q, const double* k, const double* v, const double* a,
                const double* b, const double* gate, const double* s0, const double* dy,
                const double* d_sfinal, double* dq, double* dk_out, double* dv_out, double* da,
                double* db, double* dgate, double* ds0, int nthreads) {
  if (num_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0 || !cu_seqlens) return -1;
  if (cu_seqlens[0] != 0) return -1;
  for (int32_t n = 0; n < num_seqs; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
  if (cu_seqlens[num_seqs] > 0 &&
      (!q || !k || !v || !a || !b || !dy || !dq || !dk_out || !dv_out || !da || !db))
    return -1;
  bwd_job J = {num_seqs, H, dk, dv, cu_seqlens, q, k, v, a, b, gate, s0, dy, d_sfinal,
               dq, dk_out, dv_out, da, db, dgate, ds0, 0};
  return run_threads(bwd_worker, &J, nthreads);
}
