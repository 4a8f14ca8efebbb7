/*
 * ssm_oracle.c -- plain, slow, fp64 CPU oracle for the Mamba selective scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with
 * the HIP library; it includes only the C standard library and pthreads.
 *
 * Sources (web pages; cited by title and section/equation):
 *   [SPEC]      "ТЕХНИЧЕСКОЕ ЗАДАНИЕ: Реализовать selective scan (Mamba)"
 *               (aivaro.ru practice task 53), Stage 1 items 3-4.
 *   [EXPLAINED] "Mamba CUDA 实现解析" (mamba-code-explained README),
 *               eqs. (2), (4)-(7).
 *   [BLELLOCH]  "从顺序到并行用PyTorch实现Blelloch算法加速Mamba状态空间模型"
 *               (lpnh.cn news 821471), section 4.1.
 *   [CUTILE]    "Прорыв в оптимизации SSM-моделей" (aikraft.ru digest of the
 *               cuTile Mamba-2 forward kernels), "Технические детали".
 *
 * What is computed is the plain definition: a sequential loop over time in
 * double precision, one independent row at a time.  Every parallel, chunked
 * or scan-based method reaches this same result up to rounding order, since
 * the combine operator of [EXPLAINED] eq. (10) is associative.
 *
 * Inputs arrive as float32 arrays (bf16 inputs are passed already widened,
 * which is exact); every operation below is done in double.
 *
 * Readings where the pages are silent or disagree (each also listed in the
 * design notes of the repository):
 *   - B-bar = delta * B (the simplified discretisation of [EXPLAINED] eq. (5),
 *     [SPEC] Stage 1, [BLELLOCH] 4.1), with the undefined factor mu = 1.
 *   - delta_bias is added before softplus.
 *   - output order: y = (C.h + D*u) * silu(z)  ([SPEC] Stage 1 reference).
 *   - the state starts at zero unless an initial state v_0 is given: the
 *     closed form of [EXPLAINED] eqs. (8)-(9) carries a v_0 term, and with it
 *     a sequence can be scanned in pieces, each piece starting from the
 *     state the previous one ended with.
 *   - Mamba-2 output: y = C.h + D*x (skip connection by analogy with
 *     [EXPLAINED] eq. (2)); its recurrence is the one [CUTILE] states.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* softplus(x) = log(1 + e^x), written in the overflow-free form
 * max(x,0) + log1p(e^{-|x|}) ([SPEC] Stage 1: delta_t = softplus(Delta_t)). */
static double softplus_d(double x) {
  return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));
}

/* silu(z) = z * sigmoid(z) ([SPEC] Stage 1 reference: y *= silu(z)). */
static double silu_d(double z) { return z / (1.0 + exp(-z)); }

/* ------------------------------------------------------------------------ */
/* Mamba-1: diagonal A[d,n]; B and C shared over the channels of a group.    */
/* With one group every channel reads the same B and C; with ngroups = dim  */
/* each channel has its own, the per-channel form of the [SPEC] reference   */
/* kernel (B and C indexed by batch, channel and step).                     */
/* ------------------------------------------------------------------------ */

typedef struct {
  const float *u, *delta, *A, *B, *C, *D, *z, *delta_bias;
  const double *h0; /* initial state [batch, dim, dstate] or NULL (zero) */
  int delta_softplus;
  int64_t batch, dim, dstate, seqlen, ngroups;
  const int64_t *rows;
  int64_t nrows;
  double *y, *last_state;
  int64_t row_begin, row_end; /* slice of the row list for one worker */
} mamba1_job;

static void mamba1_one_row(const mamba1_job *j, int64_t out_index, int64_t row,
                           double *h) {
  const int64_t N = j->dstate, L = j->seqlen;
  const int64_t b = row / j->dim, d = row % j->dim;
  const float *u = j->u + row * L;          /* u, delta, z: [batch, dim, seqlen] */
  const float *dl = j->delta + row * L;
  const float *z = j->z ? j->z + row * L : NULL;
  const float *A = j->A + d * N;            /* A: [dim, dstate] */
  /* B, C: [batch, ngroups, dstate, seqlen]; channel d is in group
   * d / (dim / ngroups) */
  const int64_t g = d / (j->dim / j->ngroups);
  const float *B = j->B + (b * j->ngroups + g) * N * L;
  const float *C = j->C + (b * j->ngroups + g) * N * L;
  const double Dd = j->D ? (double)j->D[d] : 0.0;
  const double bias = j->delta_bias ? (double)j->delta_bias[d] : 0.0;

  /* initial state v_0 ([EXPLAINED] eqs. (8)-(9)); zero when not given */
  for (int64_t n = 0; n < N; ++n) h[n] = j->h0 ? j->h0[row * N + n] : 0.0;
  for (int64_t t = 0; t < L; ++t) {
    /* step size: delta_t = softplus(Delta_t + bias) */
    double dt = (double)dl[t] + bias;
    if (j->delta_softplus) dt = softplus_d(dt);
    const double ut = (double)u[t];
    double yt = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      /* [EXPLAINED] eqs. (5)-(7): a = exp(delta*A[n]), b = delta*B[n],
       * v_k = a_k v_{k-1} + b_k u_k */
      const double a = exp(dt * (double)A[n]);
      const double bu = dt * (double)B[n * L + t] * ut;
      h[n] = a * h[n] + bu;
      /* readout y_t = sum_n C_t[n] h_t[n]  ([SPEC] Stage 1 reference) */
      yt += (double)C[n * L + t] * h[n];
    }
    yt += Dd * ut; /* D skip: y_k = C x_k + D u_k  ([EXPLAINED] eq. (2)) */
    if (z) yt *= silu_d((double)z[t]);
    if (j->y) j->y[out_index * L + t] = yt;
  }
  if (j->last_state)
    for (int64_t n = 0; n < N; ++n) j->last_state[out_index * N + n] = h[n];
}

static void *mamba1_worker(void *arg) {
  const mamba1_job *j = (const mamba1_job *)arg;
  double *h = (double *)malloc(sizeof(double) * (size_t)j->dstate);
  if (!h) return (void *)1;
  for (int64_t i = j->row_begin; i < j->row_end; ++i) {
    const int64_t row = j->rows ? j->rows[i] : i;
    mamba1_one_row(j, i, row, h);
  }
  free(h);
  return NULL;
}

/* Returns 0 on success, -1 on invalid arguments, -2 on thread/alloc failure.
 * B, C: [batch, ngroups, dstate, seqlen], ngroups dividing dim;
 * rows: optional list of flat row indices b*dim+d (NULL = all rows in order);
 * h0: initial state [batch, dim, dstate] (nullable = zero);
 * y: [nrows, seqlen] (nullable); last_state: [nrows, dstate] (nullable). */
int oracle_selective_scan_grouped_f64(const float *u, const float *delta,
                                      const float *A, const float *B,
                                      const float *C, const float *D,
                                      const float *z, const float *delta_bias,
                                      int delta_softplus, const double *h0,
                                      int64_t batch, int64_t dim, int64_t dstate,
                                      int64_t seqlen, int64_t ngroups,
                                      const int64_t *rows, int64_t nrows,
                                      double *y, double *last_state,
                                      int nthreads) {
  if (!u || !delta || !A || !B || !C) return -1;
  if (batch <= 0 || dim <= 0 || dstate <= 0 || seqlen <= 0) return -1;
  if (ngroups <= 0 || dim % ngroups != 0) return -1;
  if (!rows) nrows = batch * dim;
  if (nrows < 0) return -1;
  if (rows)
    for (int64_t i = 0; i < nrows; ++i)
      if (rows[i] < 0 || rows[i] >= batch * dim) return -1;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > nrows) nthreads = nrows > 0 ? (int)nrows : 1;

  mamba1_job jobs[256];
  pthread_t tids[256];
  int started[256];
  int rc = 0;
  for (int w = 0; w < nthreads; ++w) {
    mamba1_job *j = &jobs[w];
    j->u = u; j->delta = delta; j->A = A; j->B = B; j->C = C; j->D = D;
    j->z = z; j->delta_bias = delta_bias; j->delta_softplus = delta_softplus;
    j->h0 = h0;
    j->batch = batch; j->dim = dim; j->dstate = dstate; j->seqlen = seqlen;
    j->ngroups = ngroups;
    j->rows = rows; j->nrows = nrows; j->y = y; j->last_state = last_state;
    j->row_begin = nrows * w / nthreads;
    j->row_end = nrows * (w + 1) / nthreads;
    started[w] = 0;
  }
  for (int w = 1; w < nthreads; ++w)
    started[w] = pthread_create(&tids[w], NULL, mamba1_worker, &jobs[w]) == 0;
  for (int w = 1; w < nthreads; ++w)
    if (!started[w]) rc = -2;
  if (rc == 0 && mamba1_worker(&jobs[0]) != NULL) rc = -2;
  for (int w = 1; w < nthreads; ++w) {
    if (!started[w]) continue;
    void *ret = NULL;
    pthread_join(tids[w], &ret);
    if (ret != NULL) rc = -2;
  }
  return rc;
}

/* One group: B, C [batch, dstate, seqlen]. */
int oracle_selective_scan_h0_f64(const float *u, const float *delta,
                                 const float *A, const float *B, const float *C,
                                 const float *D, const float *z,
                                 const float *delta_bias, int delta_softplus,
                                 const double *h0, int64_t batch, int64_t dim,
                                 int64_t dstate, int64_t seqlen,
                                 const int64_t *rows, int64_t nrows, double *y,
                                 double *last_state, int nthreads) {
  return oracle_selective_scan_grouped_f64(u, delta, A, B, C, D, z, delta_bias,
                                           delta_softplus, h0, batch, dim,
                                           dstate, seqlen, 1, rows, nrows, y,
                                           last_state, nthreads);
}

/* Zero initial state. */
int oracle_selective_scan_f64(const float *u, const float *delta,
                              const float *A, const float *B, const float *C,
                              const float *D, const float *z,
                              const float *delta_bias, int delta_softplus,
                              int64_t batch, int64_t dim, int64_t dstate,
                              int64_t seqlen, const int64_t *rows,
                              int64_t nrows, double *y, double *last_state,
                              int nthreads) {
  return oracle_selective_scan_h0_f64(u, delta, A, B, C, D, z, delta_bias,
                                      delta_softplus, NULL, batch, dim, dstate,
                                      seqlen, rows, nrows, y, last_state,
                                      nthreads);
}

/* ------------------------------------------------------------------------ */
/* Mamba-1 backward: gradients of the forward above with respect to every    */
/* input, by reverse-mode differentiation of the sequential loop.            */
/*                                                                          */
/* Forward (per row, 0-based t), as above:                                  */
/*   s_t = delta[t] + bias;  dt_t = softplus(s_t) or s_t                     */
/*   a_t[n] = exp(dt_t A[n]);  h_t[n] = a_t[n] h_{t-1}[n] + dt_t B_t[n] u_t  */
/*   yh_t = sum_n C_t[n] h_t[n] + D u_t;  y_t = yh_t silu(z_t) or yh_t       */
/* Backward, with g_t = dy_t and lam[n] = dL/dh_t[n] carried backwards:      */
/*   dyh_t = g_t silu(z_t);  dz_t = g_t yh_t silu'(z_t)                      */
/*   lam[n] = C_t[n] dyh_t + a_{t+1}[n] lam[n]     (lam = dlast at t = L)    */
/*   dC_t[n] += dyh_t h_t[n];  dD += dyh_t u_t;  du_t = dyh_t D + ...        */
/*   from h_t = a h_{t-1} + dt B u:                                          */
/*     ddt_t += sum_n lam[n] (a_t[n] A[n] h_{t-1}[n] + B_t[n] u_t)           */
/*     dA[n] += lam[n] a_t[n] dt_t h_{t-1}[n]                                 */
/*     dB_t[n] += lam[n] dt_t u_t;  du_t += sum_n lam[n] dt_t B_t[n]         */
/*   ds_t = ddt_t sigmoid(s_t) (softplus) or ddt_t;  ddelta_t = ds_t;        */
/*   dbias += ds_t;  dh0[n] = a_0[n] lam[n] after t = 0.                      */
/* silu'(z) = sigmoid(z) (1 + z (1 - sigmoid(z))).                           */
/* ------------------------------------------------------------------------ */

typedef struct {
  const float *u, *delta, *A, *B, *C, *D, *z, *delta_bias;
  const double *h0, *dy, *dlast;
  int delta_softplus;
  int64_t batch, dim, dstate, seqlen, ngroups;
  /* per-row outputs (disjoint between workers) */
  double *du, *ddelta, *dz, *dh0;
  /* this worker's private accumulators for the shared-parameter gradients */
  double *dA, *dB, *dC, *dD, *dbias;
  int64_t row_begin, row_end;
} mamba1_bwd_job;

static double sigmoid_d(double x) { return 1.0 / (1.0 + exp(-x)); }

static void *mamba1_bwd_worker(void *arg) {
  const mamba1_bwd_job *j = (const mamba1_bwd_job *)arg;
  const int64_t N = j->dstate, L = j->seqlen;
  double *hs = (double *)malloc(sizeof(double) * (size_t)((L + 1) * N)); /* h_{-1..L-1} */
  double *dts = (double *)malloc(sizeof(double) * (size_t)L);
  double *lam = (double *)malloc(sizeof(double) * (size_t)N);
  if (!hs || !dts || !lam) {
    free(hs); free(dts); free(lam);
    return (void *)1;
  }
  for (int64_t row = j->row_begin; row < j->row_end; ++row) {
    const int64_t b = row / j->dim, d = row % j->dim;
    const float *u = j->u + row * L, *dl = j->delta + row * L;
    const float *z = j->z ? j->z + row * L : NULL;
    const float *A = j->A + d * N;
    /* channel d reads group g's B and C (and accumulates into its dB, dC) */
    const int64_t bg = b * j->ngroups + d / (j->dim / j->ngroups);
    const float *B = j->B + bg * N * L, *C = j->C + bg * N * L;
    const double Dd = j->D ? (double)j->D[d] : 0.0;
    const double bias = j->delta_bias ? (double)j->delta_bias[d] : 0.0;
    const double *dy = j->dy + row * L;
    /* forward, keeping every state: hs[(t+1)*N + n] = h_t[n], hs[n] = h_{-1} */
    for (int64_t n = 0; n < N; ++n) hs[n] = j->h0 ? j->h0[row * N + n] : 0.0;
    for (int64_t t = 0; t < L; ++t) {
      double dt = (double)dl[t] + bias;
      if (j->delta_softplus) dt = softplus_d(dt);
      dts[t] = dt;
      for (int64_t n = 0; n < N; ++n) {
        const double a = exp(dt * (double)A[n]);
        hs[(t + 1) * N + n] = a * hs[t * N + n] + dt * (double)B[n * L + t] * (double)u[t];
      }
    }
    /* backward */
    for (int64_t n = 0; n < N; ++n) lam[n] = j->dlast ? j->dlast[row * N + n] : 0.0;
    for (int64_t t = L - 1; t >= 0; --t) {
      const double dt = dts[t], ut = (double)u[t];
      const double *h = hs + (t + 1) * N, *hp = hs + t * N;
      double yh = Dd * ut;
      for (int64_t n = 0; n < N; ++n) yh += (double)C[n * L + t] * h[n];
      double dyh = dy[t];
      if (z) {
        const double zt = (double)z[t], sg = sigmoid_d(zt);
        dyh = dy[t] * zt * sg;
        j->dz[row * L + t] = dy[t] * yh * sg * (1.0 + zt * (1.0 - sg));
      }
      j->dD[d] += dyh * ut;
      double du = dyh * Dd, ddt = 0.0;
      for (int64_t n = 0; n < N; ++n) {
        /* lam currently holds a_{t+1} lam_{t+1} (or dlast); add the readout */
        lam[n] += (double)C[n * L + t] * dyh;
        j->dC[(bg * N + n) * L + t] += dyh * h[n];
        const double a = exp(dt * (double)A[n]);
        const double bt = (double)B[n * L + t];
        ddt += lam[n] * (a * (double)A[n] * hp[n] + bt * ut);
        j->dA[d * N + n] += lam[n] * a * dt * hp[n];
        j->dB[(bg * N + n) * L + t] += lam[n] * dt * ut;
        du += lam[n] * dt * bt;
        lam[n] *= a; /* now dL/dh_{t-1} */
      }
      double ds = ddt;
      if (j->delta_softplus) ds *= sigmoid_d((double)dl[t] + bias);
      j->ddelta[row * L + t] = ds;
      j->dbias[d] += ds;
      j->du[row * L + t] = du;
    }
    if (j->dh0)
      for (int64_t n = 0; n < N; ++n) j->dh0[row * N + n] = lam[n];
  }
  free(hs); free(dts); free(lam);
  return NULL;
}

/* Gradients of oracle_selective_scan_grouped_f64's outputs (y, last_state)
 * with upstream gradients dy [batch, dim, seqlen] and dlast [batch, dim,
 * dstate] (nullable = zero).  B, C and dB, dC: [batch, ngroups, dstate,
 * seqlen], channel d in group d / (dim / ngroups).  Outputs (all written,
 * float64): du, ddelta, dz (dz only when z is given, else may be NULL)
 * [batch, dim, seqlen]; dA [dim, dstate]; dB, dC; dD, ddelta_bias [dim];
 * dh0 [batch, dim, dstate] (nullable).  Shared-parameter gradients are
 * summed per worker and then over workers in a fixed order.  Returns 0, -1
 * (arguments) or -2. */
int oracle_selective_scan_bwd_grouped_f64(
    const float *u, const float *delta, const float *A, const float *B, const float *C,
    const float *D, const float *z, const float *delta_bias, int delta_softplus,
    const double *h0, const double *dy, const double *dlast, int64_t batch, int64_t dim,
    int64_t dstate, int64_t seqlen, int64_t ngroups, double *du, double *ddelta, double *dA,
    double *dB, double *dC, double *dD, double *dz, double *ddelta_bias, double *dh0,
    int nthreads) {
  if (!u || !delta || !A || !B || !C || !dy) return -1;
  if (!du || !ddelta || !dA || !dB || !dC || !dD || !ddelta_bias) return -1;
  if (z && !dz) return -1;
  if (batch <= 0 || dim <= 0 || dstate <= 0 || seqlen <= 0) return -1;
  if (ngroups <= 0 || dim % ngroups != 0) return -1;
  const int64_t rows = batch * dim, N = dstate, L = seqlen;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  if ((int64_t)nthreads > rows) nthreads = (int)rows;
  const size_t nA = (size_t)(dim * N), nBC = (size_t)(batch * ngroups * N * L), nd = (size_t)dim;
  const size_t per = nA + 2 * nBC + 2 * nd;
  double *acc = (double *)calloc((size_t)nthreads * per, sizeof(double));
  if (!acc) return -2;
  mamba1_bwd_job jobs[64];
  pthread_t tids[64];
  int started[64];
  int rc = 0;
  for (int w = 0; w < nthreads; ++w) {
    mamba1_bwd_job *j = &jobs[w];
    double *base = acc + (size_t)w * per;
    j->u = u; j->delta = delta; j->A = A; j->B = B; j->C = C; j->D = D; j->z = z;
    j->delta_bias = delta_bias; j->h0 = h0; j->dy = dy; j->dlast = dlast;
    j->delta_softplus = delta_softplus;
    j->batch = batch; j->dim = dim; j->dstate = dstate; j->seqlen = seqlen;
    j->ngroups = ngroups;
    j->du = du; j->ddelta = ddelta; j->dz = dz; j->dh0 = dh0;
    j->dA = base; j->dB = base + nA; j->dC = base + nA + nBC;
    j->dD = base + nA + 2 * nBC; j->dbias = base + nA + 2 * nBC + nd;
    j->row_begin = rows * w / nthreads;
    j->row_end = rows * (w + 1) / nthreads;
    started[w] = 0;
  }
  for (int w = 1; w < nthreads; ++w)
    started[w] = pthread_create(&tids[w], NULL, mamba1_bwd_worker, &jobs[w]) == 0;
  for (int w = 1; w < nthreads; ++w)
    if (!started[w]) rc = -2;
  if (rc == 0 && mamba1_bwd_worker(&jobs[0]) != NULL) rc = -2;
  for (int w = 1; w < nthreads; ++w) {
    if (!started[w]) continue;
    void *ret = NULL;
    pthread_join(tids[w], &ret);
    if (ret != NULL) rc = -2;
  }
  if (rc == 0) {
    memset(dA, 0, nA * sizeof(double));
    memset(dB, 0, nBC * sizeof(double));
    memset(dC, 0, nBC * sizeof(double));
    memset(dD, 0, nd * sizeof(double));
    memset(ddelta_bias, 0, nd * sizeof(double));
    for (int w = 0; w < nthreads; ++w) {
      const mamba1_bwd_job *j = &jobs[w];
      for (size_t i = 0; i < nA; ++i) dA[i] += j->dA[i];
      for (size_t i = 0; i < nBC; ++i) dB[i] += j->dB[i];
      for (size_t i = 0; i < nBC; ++i) dC[i] += j->dC[i];
      for (size_t i = 0; i < nd; ++i) dD[i] += j->dD[i];
      for (size_t i = 0; i < nd; ++i) ddelta_bias[i] += j->dbias[i];
    }
  }
  free(acc);
  return rc;
}

/* One group: B, C, dB, dC [batch, dstate, seqlen]. */
int oracle_selective_scan_bwd_f64(const float *u, const float *delta,
                                  const float *A, const float *B, const float *C,
                                  const float *D, const float *z,
                                  const float *delta_bias, int delta_softplus,
                                  const double *h0, const double *dy,
                                  const double *dlast, int64_t batch,
                                  int64_t dim, int64_t dstate, int64_t seqlen,
                                  double *du, double *ddelta, double *dA,
                                  double *dB, double *dC, double *dD,
                                  double *dz, double *ddelta_bias, double *dh0,
                                  int nthreads) {
  return oracle_selective_scan_bwd_grouped_f64(u, delta, A, B, C, D, z, delta_bias,
                                               delta_softplus, h0, dy, dlast, batch, dim,
                                               dstate, seqlen, 1, du, ddelta, dA, dB, dC, dD,
                                               dz, ddelta_bias, dh0, nthreads);
}

/* ------------------------------------------------------------------------ */
/* Mamba-2 (SSD): scalar A per head, B and C per group, state [P, N].       */
/* h_t = exp(A_h dt_t) h_{t-1} + dt_t B_t x_t^T   ([CUTILE], recurrence)     */
/* y_t = C_t . h_t + D_h x_t                                               */
/* ------------------------------------------------------------------------ */

typedef struct {
  const float *x, *dt, *A, *B, *C, *D, *dt_bias;
  const double *init; /* initial state [b, h, P, N] or NULL (zero) */
  int dt_softplus;
  int64_t batch, seqlen, nheads, headdim, dstate, ngroups;
  double *y, *final_state;
  int64_t pair_begin, pair_end; /* (b, h) pairs handled by one worker */
} ssd_job;

static void *ssd_worker(void *arg) {
  const ssd_job *j = (const ssd_job *)arg;
  const int64_t L = j->seqlen, H = j->nheads, P = j->headdim, N = j->dstate,
                G = j->ngroups;
  double *S = (double *)malloc(sizeof(double) * (size_t)(P * N));
  if (!S) return (void *)1;
  for (int64_t pair = j->pair_begin; pair < j->pair_end; ++pair) {
    const int64_t b = pair / H, h = pair % H;
    const int64_t g = h / (H / G); /* heads are split evenly over groups */
    const double Ah = (double)j->A[h];
    const double Dh = j->D ? (double)j->D[h] : 0.0;
    const double bias = j->dt_bias ? (double)j->dt_bias[h] : 0.0;
    if (j->init) /* the state entering the sequence (zero when not given) */
      memcpy(S, j->init + (b * H + h) * P * N, sizeof(double) * (size_t)(P * N));
    else
      memset(S, 0, sizeof(double) * (size_t)(P * N));
    for (int64_t t = 0; t < L; ++t) {
      double dt = (double)j->dt[(b * L + t) * H + h] + bias; /* dt: [b, L, h] */
      if (j->dt_softplus) dt = softplus_d(dt);
      const double alpha = exp(dt * Ah);
      const float *x = j->x + ((b * L + t) * H + h) * P;  /* x: [b, L, h, P] */
      const float *Bt = j->B + ((b * L + t) * G + g) * N; /* B, C: [b, L, g, N] */
      const float *Ct = j->C + ((b * L + t) * G + g) * N;
      for (int64_t p = 0; p < P; ++p) {
        const double xp = (double)x[p];
        double *Sp = S + p * N;
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) {
          Sp[n] = alpha * Sp[n] + dt * (double)Bt[n] * xp;
          acc += (double)Ct[n] * Sp[n];
        }
        if (j->y) j->y[((b * L + t) * H + h) * P + p] = acc + Dh * xp;
      }
    }
    if (j->final_state) /* final_state: [b, h, P, N] */
      memcpy(j->final_state + (b * H + h) * P * N, S,
             sizeof(double) * (size_t)(P * N));
  }
  free(S);
  return NULL;
}

/* init: initial state [b, h, P, N] (nullable = zero). */
int oracle_ssd_h0_f64(const float *x, const float *dt, const float *A,
                      const float *B, const float *C, const float *D,
                      const float *dt_bias, int dt_softplus,
                      const double *init, int64_t batch, int64_t seqlen,
                      int64_t nheads, int64_t headdim, int64_t dstate,
                      int64_t ngroups, double *y, double *final_state,
                      int nthreads) {
  if (!x || !dt || !A || !B || !C) return -1;
  if (batch <= 0 || seqlen <= 0 || nheads <= 0 || headdim <= 0 ||
      dstate <= 0 || ngroups <= 0 || nheads % ngroups != 0)
    return -1;
  const int64_t npairs = batch * nheads;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > npairs) nthreads = (int)npairs;

  ssd_job jobs[256];
  pthread_t tids[256];
  int started[256];
  int rc = 0;
  for (int w = 0; w < nthreads; ++w) {
    ssd_job *j = &jobs[w];
    j->x = x; j->dt = dt; j->A = A; j->B = B; j->C = C; j->D = D;
    j->dt_bias = dt_bias; j->dt_softplus = dt_softplus; j->init = init;
    j->batch = batch; j->seqlen = seqlen; j->nheads = nheads;
    j->headdim = headdim; j->dstate = dstate; j->ngroups = ngroups;
    j->y = y; j->final_state = final_state;
    j->pair_begin = npairs * w / nthreads;
    j->pair_end = npairs * (w + 1) / nthreads;
    started[w] = 0;
  }
  for (int w = 1; w < nthreads; ++w)
    started[w] = pthread_create(&tids[w], NULL, ssd_worker, &jobs[w]) == 0;
  for (int w = 1; w < nthreads; ++w)
    if (!started[w]) rc = -2;
  if (rc == 0 && ssd_worker(&jobs[0]) != NULL) rc = -2;
  for (int w = 1; w < nthreads; ++w) {
    if (!started[w]) continue;
    void *ret = NULL;
    pthread_join(tids[w], &ret);
    if (ret != NULL) rc = -2;
  }
  return rc;
}

/* Zero initial state. */
int oracle_ssd_f64(const float *x, const float *dt, const float *A,
                   const float *B, const float *C, const float *D,
                   const float *dt_bias, int dt_softplus, int64_t batch,
                   int64_t seqlen, int64_t nheads, int64_t headdim,
                   int64_t dstate, int64_t ngroups, double *y,
                   double *final_state, int nthreads) {
  return oracle_ssd_h0_f64(x, dt, A, B, C, D, dt_bias, dt_softplus, NULL, batch,
                           seqlen, nheads, headdim, dstate, ngroups, y,
                           final_state, nthreads);
}
