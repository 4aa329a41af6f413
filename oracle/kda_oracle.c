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
