/*
 * CPU oracle for the Gated DeltaNet prefill forward -- TEST INFRASTRUCTURE ONLY.
 * (Loaded only by the tests, the smoke check and the benchmark's CPU-baseline leg.)
 *
 * The recurrence, from "Simple math to speed up GDN prefill" (veitner), section
 * Reminder, state-transition equation:
 *   S_t = S_{t-1} alpha_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  S in R^{dv x dk}.
 * Expanding the product gives the same map as a rank-1 update:
 *   S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T.
 * Each row i of S (a dv index) only involves row i of S_{t-1} and entry i of v_t,
 * so rows evolve independently and are computed here in parallel blocks.
 * The read o_t = S_t q_t happens after the write (awehrs.io "NRM training kernels",
 * General implementation item 4: at level 0 a token sees its own write).
 * Gates (pymllm gdn_chunkwise page, Module Contents, parameters a, b, A_log, dt_bias):
 *   alpha = exp(-exp(A_log) softplus(a + dt_bias)),  beta = sigmoid(b).
 * q and k arrive un-normalised (same page, parameter q) and are L2-normalised here:
 *   x / sqrt(sum x^2 + eps).
 * A value head hv reads q/k head hv / (HV/H) (contiguous groups).
 */
#include "gdn_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

static double load_val(int in_dtype, const void* p, int64_t i) {
  if (in_dtype == 1) {
    uint32_t bits = ((uint32_t)((const uint16_t*)p)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
  }
  return (double)((const float*)p)[i];
}

static double softplus_d(double x) {
  /* log(1 + e^x) without overflow */
  return (x > 0 ? x : 0.0) + log1p(exp(-fabs(x)));
}

void gdn_oracle_gates(double a, double b, double A_log, double dt_bias, double* alpha,
                      double* beta, double* g) {
  double gg = -exp(A_log) * softplus_d(a + dt_bias);
  *g = gg;
  *alpha = exp(gg);
  *beta = 1.0 / (1.0 + exp(-b));
}

typedef struct {
  int in_dtype;
  const void *q, *k, *v;
  const float *a, *b, *A_log, *dt_bias;
  const int64_t* cu;
  int64_t batch;
  int H, HV, dk, dv;
  const int32_t* heads;
  int n_heads;
  int row_lo, row_hi;
  double* S;
  double* out;
  double eps;
  int fp32_arith;
  int row_block;
  int64_t n_items;
  int64_t next; /* shared work counter, guarded by mu */
  pthread_mutex_t mu;
} job_t;

/* One work item: sequence bi, selected head hj, rows [r0, r1) of the state. fp64. */
static void run_item_f64(job_t* J, int64_t bi, int hj, int r0, int r1) {
  const int dk = J->dk, dv = J->dv, H = J->H, HV = J->HV;
  const int hv = J->heads[hj];
  const int h = hv / (HV / H);
  const int nrows = J->row_hi - J->row_lo;
  double* S = J->S + ((bi * J->n_heads + hj) * (int64_t)nrows) * dk;
  double* qn = (double*)malloc(sizeof(double) * dk);
  double* kn = (double*)malloc(sizeof(double) * dk);
  for (int64_t t = J->cu[bi]; t < J->cu[bi + 1]; ++t) {
    const int64_t qk_off = (t * H + h) * (int64_t)dk;
    double sq = 0, sk = 0;
    for (int j = 0; j < dk; ++j) {
      qn[j] = load_val(J->in_dtype, J->q, qk_off + j);
      kn[j] = load_val(J->in_dtype, J->k, qk_off + j);
      sq += qn[j] * qn[j];
      sk += kn[j] * kn[j];
    }
    const double rq = 1.0 / sqrt(sq + J->eps), rk = 1.0 / sqrt(sk + J->eps);
    for (int j = 0; j < dk; ++j) {
      qn[j] *= rq;
      kn[j] *= rk;
    }
    double alpha, beta, g;
    gdn_oracle_gates(J->a[t * HV + hv], J->b[t * HV + hv], J->A_log[hv], J->dt_bias[hv],
                     &alpha, &beta, &g);
    for (int r = r0; r < r1; ++r) {
      double* Sr = S + (int64_t)(r - J->row_lo) * dk;
      const double vr = load_val(J->in_dtype, J->v, (t * HV + hv) * (int64_t)dv + r);
      double sk_dot = 0;
      for (int j = 0; j < dk; ++j) sk_dot += Sr[j] * kn[j];
      const double d = beta * (vr - alpha * sk_dot);
      double o = 0;
      for (int j = 0; j < dk; ++j) {
        Sr[j] = alpha * Sr[j] + d * kn[j];
        o += Sr[j] * qn[j];
      }
      J->out[(t * J->n_heads + hj) * (int64_t)nrows + (r - J->row_lo)] = o;
    }
  }
  free(qn);
  free(kn);
}

/* The same loop with every operation in fp32 (to measure the fp32 rounding floor). */
static void run_item_f32(job_t* J, int64_t bi, int hj, int r0, int r1) {
  const int dk = J->dk, dv = J->dv, H = J->H, HV = J->HV;
  const int hv = J->heads[hj];
  const int h = hv / (HV / H);
  const int nrows = J->row_hi - J->row_lo;
  double* S = J->S + ((bi * J->n_heads + hj) * (int64_t)nrows) * dk;
  float* qn = (float*)malloc(sizeof(float) * dk);
  float* kn = (float*)malloc(sizeof(float) * dk);
  float* Sf = (float*)malloc(sizeof(float) * dk * (size_t)(r1 - r0));
  for (int r = r0; r < r1; ++r)
    for (int j = 0; j < dk; ++j)
      Sf[(size_t)(r - r0) * dk + j] = (float)S[(int64_t)(r - J->row_lo) * dk + j];
  for (int64_t t = J->cu[bi]; t < J->cu[bi + 1]; ++t) {
    const int64_t qk_off = (t * H + h) * (int64_t)dk;
    float sq = 0, sk = 0;
    for (int j = 0; j < dk; ++j) {
      qn[j] = (float)load_val(J->in_dtype, J->q, qk_off + j);
      kn[j] = (float)load_val(J->in_dtype, J->k, qk_off + j);
      sq += qn[j] * qn[j];
      sk += kn[j] * kn[j];
    }
    const float rq = 1.0f / sqrtf(sq + (float)J->eps), rk = 1.0f / sqrtf(sk + (float)J->eps);
    for (int j = 0; j < dk; ++j) {
      qn[j] *= rq;
      kn[j] *= rk;
    }
    const float x = J->a[t * HV + hv] + J->dt_bias[hv];
    const float sp = (x > 0 ? x : 0.0f) + log1pf(expf(-fabsf(x)));
    const float alpha = expf(-expf(J->A_log[hv]) * sp);
    const float beta = 1.0f / (1.0f + expf(-J->b[t * HV + hv]));
    for (int r = r0; r < r1; ++r) {
      float* Sr = Sf + (size_t)(r - r0) * dk;
      const float vr = (float)load_val(J->in_dtype, J->v, (t * HV + hv) * (int64_t)dv + r);
      float sk_dot = 0;
      for (int j = 0; j < dk; ++j) sk_dot += Sr[j] * kn[j];
      const float d = beta * (vr - alpha * sk_dot);
      float o = 0;
      for (int j = 0; j < dk; ++j) {
        Sr[j] = alpha * Sr[j] + d * kn[j];
        o += Sr[j] * qn[j];
      }
      J->out[(t * J->n_heads + hj) * (int64_t)nrows + (r - J->row_lo)] = (double)o;
    }
  }
  for (int r = r0; r < r1; ++r)
    for (int j = 0; j < dk; ++j)
      S[(int64_t)(r - J->row_lo) * dk + j] = (double)Sf[(size_t)(r - r0) * dk + j];
  free(qn);
  free(kn);
  free(Sf);
}

static void* worker(void* arg) {
  job_t* J = (job_t*)arg;
  const int nrows = J->row_hi - J->row_lo;
  const int nblk = (nrows + J->row_block - 1) / J->row_block;
  for (;;) {
    pthread_mutex_lock(&J->mu);
    int64_t it = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (it >= J->n_items) break;
    const int64_t bi = it / ((int64_t)J->n_heads * nblk);
    const int hj = (int)((it / nblk) % J->n_heads);
    const int blk = (int)(it % nblk);
    const int r0 = J->row_lo + blk * J->row_block;
    int r1 = r0 + J->row_block;
    if (r1 > J->row_hi) r1 = J->row_hi;
    if (J->fp32_arith)
      run_item_f32(J, bi, hj, r0, r1);
    else
      run_item_f64(J, bi, hj, r0, r1);
  }
  return NULL;
}

int gdn_oracle_recurrence(int in_dtype, const void* q, const void* k, const void* v,
                          const float* a, const float* b, const float* A_log,
                          const float* dt_bias, const int64_t* cu_seqlens, int64_t batch,
                          int H, int HV, int dk, int dv, const int32_t* heads, int n_heads,
                          int row_lo, int row_hi, double* S, double* out, double eps,
                          int fp32_arith, int nthreads) {
  if (!q || !k || !v || !a || !b || !A_log || !dt_bias || !cu_seqlens || !heads || !S || !out)
    return -1;
  if (batch < 0 || H <= 0 || HV <= 0 || HV % H != 0 || dk <= 0 || dv <= 0 || n_heads < 0 ||
      row_lo < 0 || row_hi > dv || row_lo > row_hi || (in_dtype != 0 && in_dtype != 1))
    return -1;
  for (int j = 0; j < n_heads; ++j)
    if (heads[j] < 0 || heads[j] >= HV) return -1;
  for (int64_t i = 0; i < batch; ++i)
    if (cu_seqlens[i + 1] < cu_seqlens[i]) return -1;
  if (row_hi == row_lo || n_heads == 0 || batch == 0) return 0;

  job_t J;
  memset(&J, 0, sizeof J);
  J.in_dtype = in_dtype;
  J.q = q;
  J.k = k;
  J.v = v;
  J.a = a;
  J.b = b;
  J.A_log = A_log;
  J.dt_bias = dt_bias;
  J.cu = cu_seqlens;
  J.batch = batch;
  J.H = H;
  J.HV = HV;
  J.dk = dk;
  J.dv = dv;
  J.heads = heads;
  J.n_heads = n_heads;
  J.row_lo = row_lo;
  J.row_hi = row_hi;
  J.S = S;
  J.out = out;
  J.eps = eps;
  J.fp32_arith = fp32_arith;
  J.row_block = 16;
  const int nrows = row_hi - row_lo;
  J.n_items = batch * (int64_t)n_heads * ((nrows + J.row_block - 1) / J.row_block);
  J.next = 0;
  pthread_mutex_init(&J.mu, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > J.n_items) nthreads = (int)J.n_items;
  pthread_t th[256];
  for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, &J);
  worker(&J);
  for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
  pthread_mutex_destroy(&J.mu);
  return 0;
}
