/*
 * kda_oracle.c -- plain, sequential fp64 CPU oracle for the gated delta rule
 * (Kimi Delta Attention).  TEST INFRASTRUCTURE ONLY: it exists so that tests,
 * the smoke check and the benchmark's CPU baseline can check the GPU library
 * against an obviously correct reference.  Nothing in the product path may
 * call it, and it shares no code, header or build flag with the GPU library.
 *
 * What it computes, per sequence n and head h, token by token in causal order
 * (state S is dk x dv, row r = key channel r; column-vector notation):
 *
 *   fade     S <- Diag(alpha_t) S,  alpha_t = exp(g_t)  (per key channel)
 *   read     w  = S^T k_t            (what the faded memory returns at k_t)
 *   correct  u  = beta_t (v_t - w)   (the delta; ADDITIVE mode: u = v_t)
 *   write    S <- S + k_t u^T
 *   output   o_t = S^T q_t           (read after the write)
 *
 * Sources (pages, sections):
 *  - fade then read then correct, against the faded state:
 *    dev.to "From GPT-2 to Kimi K3: How Language Models Learned to Manage
 *    Memory", block 4 (Gated DeltaNet) and block 5 (one retention factor per
 *    key channel, i.e. per row of S).
 *  - the per-channel update S_t = Diag(alpha)(...)S + beta k v^T with the
 *    write undecayed at its own step: engineermaxxing "From GPT-2 to Kimi K3:
 *    one memory, seven eviction policies", ch. 06b; the decay-first ordering
 *    of the same page's code listing and of the dev.to page is followed (for
 *    a scalar gate both orders agree, ch. 05c).
 *  - read/write/subtract steps and read-after-write output with no
 *    normaliser: heqinghuang "From GPT2 to Kimi3, Explained", section 09.
 *  - ADDITIVE mode (delta term disabled, gated linear attention):
 *    engineermaxxing ch. 02b (additive stamp) and ch. 05b (scalar decay on
 *    the additive memory); with per-channel gates this is the same fade.
 *  - no incoming state means a zero state: heqinghuang section 09.
 *
 * Independent (sequence, head) pairs are spread over POSIX threads; each
 * recurrence is strictly serial.  Compiled with plain gcc -O2, no fast-math.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_MODE_DELTA = 0, ORACLE_MODE_ADDITIVE = 1 };

typedef struct {
  int mode, num_heads, dk, dv, num_seqs;
  const int32_t* cu_seqlens;
  const double *q, *k, *v, *g, *beta, *s0;
  double *o, *s_final;
  int next_task; /* shared work counter */
  pthread_mutex_t lock;
  int failed;
} oracle_job;

/* One (sequence, head) recurrence.  Layouts: q,k,g [T,H,dk]; v,o [T,H,dv];
 * beta [T,H]; s0, s_final [N,H,dk,dv]. */
static int run_one(oracle_job* J, int n, int h) {
  const int H = J->num_heads, dk = J->dk, dv = J->dv;
  double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
  double* a = (double*)malloc(sizeof(double) * (size_t)dk);
  double* w = (double*)malloc(sizeof(double) * (size_t)dv);
  double* u = (double*)malloc(sizeof(double) * (size_t)dv);
  if (!S || !a || !w || !u) {
    free(S); free(a); free(w); free(u);
    return -1;
  }
  const size_t sbase = ((size_t)n * H + h) * (size_t)dk * dv;
  if (J->s0) memcpy(S, J->s0 + sbase, sizeof(double) * (size_t)dk * dv);
  else memset(S, 0, sizeof(double) * (size_t)dk * dv);

  for (int32_t t = J->cu_seqlens[n]; t < J->cu_seqlens[n + 1]; ++t) {
    const double* qt = J->q + ((size_t)t * H + h) * dk;
    const double* kt = J->k + ((size_t)t * H + h) * dk;
    const double* gt = J->g + ((size_t)t * H + h) * dk;
    const double* vt = J->v + ((size_t)t * H + h) * dv;
    const double bt = J->beta[(size_t)t * H + h];
    double* ot = J->o + ((size_t)t * H + h) * dv;

    /* fade: row r of S scaled by alpha_t[r] = exp(g_t[r]) */
    for (int r = 0; r < dk; ++r) a[r] = exp(gt[r]);
    for (int r = 0; r < dk; ++r)
      for (int c = 0; c < dv; ++c) S[(size_t)r * dv + c] *= a[r];

    /* read the faded state at the key: w = S^T k */
    for (int c = 0; c < dv; ++c) w[c] = 0.0;
    for (int r = 0; r < dk; ++r)
      for (int c = 0; c < dv; ++c) w[c] += kt[r] * S[(size_t)r * dv + c];

    /* the correction written at this key */
    if (J->mode == ORACLE_MODE_ADDITIVE)
      for (int c = 0; c < dv; ++c) u[c] = vt[c];
    else
      for (int c = 0; c < dv; ++c) u[c] = bt * (vt[c] - w[c]);

    /* write: S += k u^T */
    for (int r = 0; r < dk; ++r)
      for (int c = 0; c < dv; ++c) S[(size_t)r * dv + c] += kt[r] * u[c];

    /* output read after the write: o = S^T q */
    for (int c = 0; c < dv; ++c) ot[c] = 0.0;
    for (int r = 0; r < dk; ++r)
      for (int c = 0; c < dv; ++c) ot[c] += qt[r] * S[(size_t)r * dv + c];
  }
  if (J->s_final) memcpy(J->s_final + sbase, S, sizeof(double) * (size_t)dk * dv);
  free(S); free(a); free(w); free(u);
  return 0;
}

static void* worker(void* arg) {
  oracle_job* J = (oracle_job*)arg;
  const int total = J->num_seqs * J->num_heads;
  for (;;) {
    pthread_mutex_lock(&J->lock);
    int task = J->next_task++;
    pthread_mutex_unlock(&J->lock);
    if (task >= total) break;
    if (run_one(J, task / J->num_heads, task % J->num_heads) != 0) {
      pthread_mutex_lock(&J->lock);
      J->failed = 1;
      pthread_mutex_unlock(&J->lock);
    }
  }
  return NULL;
}

/* Runs the recurrence for every (sequence, head).  Returns 0 on success,
 * -1 on a bad argument or allocation failure.  nthreads <= 0 means 1. */
int kda_oracle_run(int mode, int num_heads, int dk, int dv, int num_seqs,
                   const int32_t* cu_seqlens, const double* q, const double* k,
                   const double* v, const double* g, const double* beta,
                   const double* s0, double* o, double* s_final, int nthreads) {
  if (num_heads <= 0 || dk <= 0 || dv <= 0 || num_seqs < 0 || !cu_seqlens) return -1;
  if (mode != ORACLE_MODE_DELTA && mode != ORACLE_MODE_ADDITIVE) return -1;
  if (num_seqs == 0) return 0;
  for (int n = 0; n < num_seqs; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
  oracle_job J;
  memset(&J, 0, sizeof(J));
  J.mode = mode; J.num_heads = num_heads; J.dk = dk; J.dv = dv; J.num_seqs = num_seqs;
  J.cu_seqlens = cu_seqlens; J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta;
  J.s0 = s0; J.o = o; J.s_final = s_final;
  pthread_mutex_init(&J.lock, NULL);
  if (nthreads <= 1) {
    worker(&J);
  } else {
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    int started = 0;
    for (int i = 0; i < nthreads; ++i)
      if (pthread_create(&th[i], NULL, worker, &J) == 0) ++started;
    if (started == 0) worker(&J);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    free(th);
  }
  pthread_mutex_destroy(&J.lock);
  return J.failed ? -1 : 0;
}

/* ------------------------------------------------------------------ gradients
 *
 * The pages give no gradient formulas (they motivate the chunked form by
 * training, heqinghuang section 10, engineermaxxing ch. 04, but stop at the
 * forward pass).  The backward pass below is reverse-mode differentiation of
 * the five steps above, taken token by token in reverse causal order; for the
 * state cotangent G = dL/dS after a token's write and the output cotangent do:
 *
 *   output   dq = S do;            G += q do^T
 *   write    dS_a = G;             dk = G u;      du = G^T k
 *   correct  DELTA: dbeta = du . (v - w);  dv = beta du;  dw = -beta du
 *            ADDITIVE: dv = du;  dw = 0  (dbeta = 0)
 *   read     dS_a += k dw^T;       dk += S_a dw
 *   fade     dg[r] = sum_c dS_a[r,c] S_a[r,c];   G <- Diag(alpha) dS_a
 *
 * where S_a is the faded state the token read and wrote.  After the first
 * token G is dL/dS0.  The states a token needs are recomputed by the forward
 * steps above from a copy of the state taken every kSeg tokens (the same
 * operations in the same order, so the recomputed states equal the forward
 * ones bit for bit).
 */
enum { kSeg = 64 };

typedef struct {
  int mode, num_heads, dk, dv, num_seqs;
  const int32_t* cu_seqlens;
  const double *q, *k, *v, *g, *beta, *s0, *d_o, *ds_final;
  double *dq, *dk_out, *dv_out, *dg, *dbeta, *ds0;
  int next_task;
  pthread_mutex_t lock;
  int failed;
} oracle_bwd_job;

/* One forward token step on S in place; leaves the faded state in Sa (when
 * not NULL), the read in w and the correction in u. */
static void fwd_token(int mode, int dk, int dv, double* S, double* Sa, double* w, double* u,
                      const double* kt, const double* vt, const double* gt, double bt) {
  for (int r = 0; r < dk; ++r) {
    const double a = exp(gt[r]);
    for (int c = 0; c < dv; ++c) S[(size_t)r * dv + c] *= a;
  }
  if (Sa) memcpy(Sa, S, sizeof(double) * (size_t)dk * dv);
  for (int c = 0; c < dv; ++c) w[c] = 0.0;
  for (int r = 0; r < dk; ++r)
    for (int c = 0; c < dv; ++c) w[c] += kt[r] * S[(size_t)r * dv + c];
  if (mode == ORACLE_MODE_ADDITIVE)
    for (int c = 0; c < dv; ++c) u[c] = vt[c];
  else
    for (int c = 0; c < dv; ++c) u[c] = bt * (vt[c] - w[c]);
  for (int r = 0; r < dk; ++r)
    for (int c = 0; c < dv; ++c) S[(size_t)r * dv + c] += kt[r] * u[c];
}

static int bwd_one(oracle_bwd_job* J, int n, int h) {
  const int H = J->num_heads, dk = J->dk, dv = J->dv;
  const size_t ss = (size_t)dk * dv;
  const int32_t t0 = J->cu_seqlens[n], t1 = J->cu_seqlens[n + 1];
  const int32_t L = t1 - t0;
  const int nseg = (L + kSeg - 1) / kSeg;
  double* ck = (double*)malloc(sizeof(double) * ss * (size_t)(nseg > 0 ? nseg : 1));
  double* Sbuf = (double*)malloc(sizeof(double) * ss * (kSeg + 1));
  double* Sa = (double*)malloc(sizeof(double) * ss);
  double* G = (double*)malloc(sizeof(double) * ss);
  double* w = (double*)malloc(sizeof(double) * dv);
  double* u = (double*)malloc(sizeof(double) * dv);
  double* du = (double*)malloc(sizeof(double) * dv);
  double* dw = (double*)malloc(sizeof(double) * dv);
  if (!ck || !Sbuf || !Sa || !G || !w || !u || !du || !dw) {
    free(ck); free(Sbuf); free(Sa); free(G); free(w); free(u); free(du); free(dw);
    return -1;
  }
  const size_t sbase = ((size_t)n * H + h) * ss;
  /* forward pass keeping the state at the start of every segment */
  double* S = Sbuf;
  if (J->s0) memcpy(S, J->s0 + sbase, sizeof(double) * ss);
  else memset(S, 0, sizeof(double) * ss);
  for (int32_t t = t0; t < t1; ++t) {
    if ((t - t0) % kSeg == 0) memcpy(ck + (size_t)((t - t0) / kSeg) * ss, S, sizeof(double) * ss);
    const size_t th = (size_t)t * H + h;
    fwd_token(J->mode, dk, dv, S, NULL, w, u, J->k + th * dk, J->v + th * dv, J->g + th * dk,
              J->beta[th]);
  }
  /* reverse pass */
  if (J->ds_final) memcpy(G, J->ds_final + sbase, sizeof(double) * ss);
  else memset(G, 0, sizeof(double) * ss);
  for (int sg = nseg - 1; sg >= 0; --sg) {
    const int32_t a = t0 + sg * kSeg, b = (a + kSeg < t1) ? a + kSeg : t1;
    /* Sbuf[i] = state before token a + i */
    memcpy(Sbuf, ck + (size_t)sg * ss, sizeof(double) * ss);
    for (int32_t t = a; t < b; ++t) {
      const size_t th = (size_t)t * H + h;
      double* Sn = Sbuf + (size_t)(t - a + 1) * ss;
      memcpy(Sn, Sbuf + (size_t)(t - a) * ss, sizeof(double) * ss);
      fwd_token(J->mode, dk, dv, Sn, NULL, w, u, J->k + th * dk, J->v + th * dv, J->g + th * dk,
                J->beta[th]);
    }
    for (int32_t t = b - 1; t >= a; --t) {
      const size_t th = (size_t)t * H + h;
      const double *qt = J->q + th * dk, *kt = J->k + th * dk, *vt = J->v + th * dv;
      const double *gt = J->g + th * dk, *dot = J->d_o + th * dv;
      const double bt = J->beta[th];
      double *dqt = J->dq + th * dk, *dkt = J->dk_out + th * dk, *dvt = J->dv_out + th * dv;
      double* dgt = J->dg + th * dk;
      /* recompute the token: faded state Sa, read w, correction u, state after St */
      double* St = Sbuf + (size_t)(t - a + 1) * ss;
      memcpy(Sa, Sbuf + (size_t)(t - a) * ss, sizeof(double) * ss);
      fwd_token(J->mode, dk, dv, Sa, NULL, w, u, kt, vt, gt, bt);  /* Sa now = St */
      memcpy(Sa, Sbuf + (size_t)(t - a) * ss, sizeof(double) * ss);
      for (int r = 0; r < dk; ++r) {
        const double al = exp(gt[r]);
        for (int c = 0; c < dv; ++c) Sa[(size_t)r * dv + c] *= al;
      }
      /* output */
      for (int r = 0; r < dk; ++r) {
        double x = 0.0;
        for (int c = 0; c < dv; ++c) x += St[(size_t)r * dv + c] * dot[c];
        dqt[r] = x;
      }
      for (int r = 0; r < dk; ++r)
        for (int c = 0; c < dv; ++c) G[(size_t)r * dv + c] += qt[r] * dot[c];
      /* write: dS_a = G (kept in G), dk = G u, du = G^T k */
      for (int r = 0; r < dk; ++r) {
        double x = 0.0;
        for (int c = 0; c < dv; ++c) x += G[(size_t)r * dv + c] * u[c];
        dkt[r] = x;
      }
      for (int c = 0; c < dv; ++c) du[c] = 0.0;
      for (int r = 0; r < dk; ++r)
        for (int c = 0; c < dv; ++c) du[c] += G[(size_t)r * dv + c] * kt[r];
      /* correct */
      if (J->mode == ORACLE_MODE_ADDITIVE) {
        for (int c = 0; c < dv; ++c) { dvt[c] = du[c]; dw[c] = 0.0; }
        J->dbeta[th] = 0.0;
      } else {
        double db = 0.0;
        for (int c = 0; c < dv; ++c) {
          db += du[c] * (vt[c] - w[c]);
          dvt[c] = bt * du[c];
          dw[c] = -bt * du[c];
        }
        J->dbeta[th] = db;
      }
      /* read: dS_a += k dw^T, dk += S_a dw */
      for (int r = 0; r < dk; ++r) {
        double x = 0.0;
        for (int c = 0; c < dv; ++c) {
          G[(size_t)r * dv + c] += kt[r] * dw[c];
          x += Sa[(size_t)r * dv + c] * dw[c];
        }
        dkt[r] += x;
      }
      /* fade */
      for (int r = 0; r < dk; ++r) {
        const double al = exp(gt[r]);
        double x = 0.0;
        for (int c = 0; c < dv; ++c) {
          x += G[(size_t)r * dv + c] * Sa[(size_t)r * dv + c];
          G[(size_t)r * dv + c] *= al;
        }
        dgt[r] = x;
      }
    }
  }
  if (J->ds0) memcpy(J->ds0 + sbase, G, sizeof(double) * ss);
  free(ck); free(Sbuf); free(Sa); free(G); free(w); free(u); free(du); free(dw);
  return 0;
}

static void* bwd_worker(void* arg) {
  oracle_bwd_job* J = (oracle_bwd_job*)arg;
  const int total = J->num_seqs * J->num_heads;
  for (;;) {
    pthread_mutex_lock(&J->lock);
    int task = J->next_task++;
    pthread_mutex_unlock(&J->lock);
    if (task >= total) break;
    if (bwd_one(J, task / J->num_heads, task % J->num_heads) != 0) {
      pthread_mutex_lock(&J->lock);
      J->failed = 1;
      pthread_mutex_unlock(&J->lock);
    }
  }
  return NULL;
}

/* Gradients of a scalar loss L through the recurrence, given dL/do (d_o,
 * [T,H,dv]) and dL/dS_final (ds_final, [N,H,dk,dv], NULL = 0).  Writes
 * dq, dk, dg [T,H,dk], dv [T,H,dv], dbeta [T,H] and ds0 [N,H,dk,dv]
 * (dL/dS0; may be NULL).  Returns 0, or -1 on a bad argument or allocation
 * failure. */
int kda_oracle_bwd(int mode, int num_heads, int dk, int dv, int num_seqs,
                   const int32_t* cu_seqlens, const double* q, const double* k,
                   const double* v, const double* g, const double* beta, const double* s0,
                   const double* d_o, const double* ds_final, double* dq, double* dk_out,
                   double* dv_out, double* dg, double* dbeta, double* ds0, int nthreads) {
  if (num_heads <= 0 || dk <= 0 || dv <= 0 || num_seqs < 0 || !cu_seqlens) return -1;
  if (mode != ORACLE_MODE_DELTA && mode != ORACLE_MODE_ADDITIVE) return -1;
  if (num_seqs == 0) return 0;
  for (int n = 0; n < num_seqs; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
  oracle_bwd_job J;
  memset(&J, 0, sizeof(J));
  J.mode = mode; J.num_heads = num_heads; J.dk = dk; J.dv = dv; J.num_seqs = num_seqs;
  J.cu_seqlens = cu_seqlens; J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.s0 = s0;
  J.d_o = d_o; J.ds_final = ds_final; J.dq = dq; J.dk_out = dk_out; J.dv_out = dv_out;
  J.dg = dg; J.dbeta = dbeta; J.ds0 = ds0;
  pthread_mutex_init(&J.lock, NULL);
  if (nthreads <= 1) {
    bwd_worker(&J);
  } else {
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    int started = 0;
    for (int i = 0; i < nthreads; ++i)
      if (pthread_create(&th[i], NULL, bwd_worker, &J) == 0) ++started;
    if (started == 0) bwd_worker(&J);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    free(th);
  }
  pthread_mutex_destroy(&J.lock);
  return J.failed ? -1 : 0;
}
