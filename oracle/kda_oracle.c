/*
 * kda_oracle.c -- plain, slow, fp64 CPU oracle for the KDA forward pass.
 * TEST INFRASTRUCTURE ONLY (see kda_oracle.h for the definitions it follows).
 *
 * One task = one (b, h, block of value columns).  The value columns of the
 * state evolve independently given (k, beta, alpha): in Eq. 1 every column j
 * of S_t depends only on column j of S_{t-1} and on v_t[j].  Splitting the
 * columns over threads therefore changes no arithmetic.
 */
#include "kda_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define COLS_PER_TASK 16

/* Eq. 5 (reading notes, section 2): g = g_min * sigmoid(exp(A) * z). */
static double gate_logit_to_logdecay(double z, double A, double g_min) {
  double x = exp(A) * z;
  double s = 1.0 / (1.0 + exp(-x));
  return g_min * s;
}

int kda_oracle_gate(const double* z, const double* A, double g_min, long B,
                    long T, long H, long dk, long chunk, double* G) {
  if (!z || !A || !G || B < 0 || T < 0 || H <= 0 || dk <= 0 || chunk <= 0)
    return -1;
  for (long b = 0; b < B; ++b)
    for (long h = 0; h < H; ++h)
      for (long c = 0; c < dk; ++c) {
        double run = 0.0;
        for (long t = 0; t < T; ++t) {
          if (t % chunk == 0) run = 0.0;
          long i = ((b * T + t) * H + h) * dk + c;
          run += gate_logit_to_logdecay(z[i], A[h * dk + c], g_min);
          G[i] = run;
        }
      }
  return 0;
}

typedef struct {
  const double *q, *k, *v, *beta, *g, *z, *A, *S_in;
  double *o, *S_out;
  double g_min, scale;
  long B, T, H, dk, dv;
  int from_z;
  long ntasks;
  long next; /* shared task counter */
  pthread_mutex_t lock;
} job_t;

/* o_t[j0 + j] = scale * sum_c S[c][j] q_t[c] for the task's columns. */
static void read_output(const job_t* J, const double* S, const double* qt,
                        long row, long j0, long nc) {
  if (!J->o) return;
  double* ot = J->o + row * J->dv;
  for (long j = 0; j < nc; ++j) {
    double acc = 0.0;
    for (long c = 0; c < J->dk; ++c) acc += S[c * nc + j] * qt[c];
    ot[j0 + j] = J->scale * acc;
  }
}

/* One (b, h, column block) run of Eq. 1 over all T tokens. */
static void run_task(job_t* J, long task) {
  const long dk = J->dk, dv = J->dv, H = J->H, T = J->T;
  const long nblk = (dv + COLS_PER_TASK - 1) / COLS_PER_TASK;
  const long b = task / (H * nblk);
  const long h = (task / nblk) % H;
  const long j0 = (task % nblk) * COLS_PER_TASK;
  const long j1 = j0 + COLS_PER_TASK < dv ? j0 + COLS_PER_TASK : dv;
  const long nc = j1 - j0;

  double* S = (double*)calloc((size_t)(dk * nc), sizeof(double)); /* S[c][j-j0] */
  double* alpha = (double*)malloc((size_t)dk * sizeof(double));
  double* read = (double*)malloc((size_t)nc * sizeof(double));
  if (J->S_in) {
    const double* Si = J->S_in + (b * H + h) * dk * dv;
    for (long c = 0; c < dk; ++c)
      for (long j = j0; j < j1; ++j) S[c * nc + (j - j0)] = Si[c * dv + j];
  }
  for (long t = 0; t < T; ++t) {
    const long row = (b * T + t) * H + h;
    const double* kt = J->k + row * dk;
    const double* qt = J->q + row * dk;
    const double* vt = J->v + row * dv;
    const double bt = J->beta[row];
    /* retention alpha_t = exp(g_t), g_t per key channel */
    for (long c = 0; c < dk; ++c) {
      double g = J->from_z
                     ? gate_logit_to_logdecay(J->z[row * dk + c], J->A[h * dk + c], J->g_min)
                     : J->g[row * dk + c];
      alpha[c] = exp(g);
    }
    /* 1. decay: D = Diag(alpha_t) S_{t-1}  (scales each key row) */
    for (long c = 0; c < dk; ++c)
      for (long j = 0; j < nc; ++j) S[c * nc + j] *= alpha[c];
    /* 2. correction read: read_j = sum_c k_t[c] * D[c][j] */
    for (long j = 0; j < nc; ++j) {
      double acc = 0.0;
      for (long c = 0; c < dk; ++c) acc += kt[c] * S[c * nc + j];
      read[j] = acc;
    }
    /* 3. S_t = D - beta k (x) read + beta k (x) v */
    for (long c = 0; c < dk; ++c)
      for (long j = 0; j < nc; ++j)
        S[c * nc + j] = S[c * nc + j] - bt * kt[c] * read[j] + bt * kt[c] * vt[j0 + j];
    /* 4. read after the update: o_t = scale * S_t^T q_t */
    read_output(J, S, qt, row, j0, nc);
  }
  if (J->S_out) {
    double* So = J->S_out + (b * H + h) * dk * dv;
    for (long c = 0; c < dk; ++c)
      for (long j = j0; j < j1; ++j) So[c * dv + j] = S[c * nc + (j - j0)];
  }
  free(S);
  free(alpha);
  free(read);
}

static void* worker(void* arg) {
  job_t* J = (job_t*)arg;
  for (;;) {
    pthread_mutex_lock(&J->lock);
    long task = J->next++;
    pthread_mutex_unlock(&J->lock);
    if (task >= J->ntasks) break;
    run_task(J, task);
  }
  return NULL;
}

static int run_job(job_t* J, int nthreads) {
  const long nblk = (J->dv + COLS_PER_TASK - 1) / COLS_PER_TASK;
  J->ntasks = J->B * J->H * nblk;
  J->next = 0;
  if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > J->ntasks) nthreads = (int)(J->ntasks > 0 ? J->ntasks : 1);
  pthread_mutex_init(&J->lock, NULL);
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  int started = 0;
  for (int i = 1; i < nthreads; ++i)
    if (pthread_create(&th[started], NULL, worker, J) == 0) ++started;
  worker(J); /* the calling thread works too */
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&J->lock);
  return 0;
}

static int check_common(const double* q, const double* k, const double* v,
                        const double* beta, long B, long T, long H, long dk,
                        long dv) {
  if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
  if (B * T > 0 && (!q || !k || !v || !beta)) return -1;
  return 0;
}

int kda_oracle_recurrence(const double* q, const double* k, const double* v,
                          const double* beta, const double* g,
                          const double* S_in, double* o, double* S_out, long B,
                          long T, long H, long dk, long dv, double scale,
                          int nthreads) {
  if (check_common(q, k, v, beta, B, T, H, dk, dv)) return -1;
  if (B * T > 0 && !g) return -1;
  job_t J;
  memset(&J, 0, sizeof J);
  J.q = q; J.k = k; J.v = v; J.beta = beta; J.g = g; J.S_in = S_in;
  J.o = o; J.S_out = S_out; J.scale = scale;
  J.B = B; J.T = T; J.H = H; J.dk = dk; J.dv = dv; J.from_z = 0;
  return run_job(&J, nthreads);
}

int kda_oracle_forward_z(const double* q, const double* k, const double* v,
                         const double* beta, const double* z, const double* A,
                         double g_min, const double* S_in, double* o,
                         double* S_out, long B, long T, long H, long dk,
                         long dv, double scale, int nthreads) {
  if (check_common(q, k, v, beta, B, T, H, dk, dv)) return -1;
  if (B * T > 0 && (!z || !A)) return -1;
  job_t J;
  memset(&J, 0, sizeof J);
  J.q = q; J.k = k; J.v = v; J.beta = beta; J.z = z; J.A = A; J.g_min = g_min;
  J.S_in = S_in; J.o = o; J.S_out = S_out; J.scale = scale;
  J.B = B; J.T = T; J.H = H; J.dk = dk; J.dv = dv; J.from_z = 1;
  return run_job(&J, nthreads);
}
