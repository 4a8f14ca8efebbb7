/* Host-side sanitizer driver for the oracle (test infrastructure only):
 * runs every exported oracle routine on small seeded inputs with several
 * worker threads, plus the invalid-argument paths, so that an
 * AddressSanitizer / UndefinedBehaviorSanitizer build (or a ThreadSanitizer
 * build) of ssm_oracle.c sees every code path.  Exit status 0 when every
 * call returned what it should; the sanitizers abort on their own. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_selective_scan_grouped_f64(const float *u, const float *delta, const float *A,
                                      const float *B, const float *C, const float *D,
                                      const float *z, const float *delta_bias, int delta_softplus,
                                      const double *h0, int64_t batch, int64_t dim,
                                      int64_t dstate, int64_t seqlen, int64_t ngroups,
                                      const int64_t *rows, int64_t nrows, double *y,
                                      double *last_state, int nthreads);
int oracle_selective_scan_bwd_grouped_f64(
    const float *u, const float *delta, const float *A, const float *B, const float *C,
    const float *D, const float *z, const float *delta_bias, int delta_softplus,
    const double *h0, const double *dy, const double *dlast, int64_t batch, int64_t dim,
    int64_t dstate, int64_t seqlen, int64_t ngroups, double *du, double *ddelta, double *dA,
    double *dB, double *dC, double *dD, double *dz, double *ddelta_bias, double *dh0,
    int nthreads);
int oracle_ssd_h0_f64(const float *x, const float *dt, const float *A, const float *B,
                      const float *C, const float *D, const float *dt_bias, int dt_softplus,
                      const double *init, int64_t batch, int64_t seqlen, int64_t nheads,
                      int64_t headdim, int64_t dstate, int64_t ngroups, double *y,
                      double *final_state, int nthreads);

static uint64_t state = 12345;
static double next_uniform(void) {  /* splitmix64 -> [0, 1) */
  uint64_t z = (state += 0x9e3779b97f4a7c15ULL);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  z ^= z >> 31;
  return (double)(z >> 11) * (1.0 / 9007199254740992.0);
}
static float *randf(size_t n, double lo, double hi) {
  float *p = malloc(n * sizeof(float));
  for (size_t i = 0; i < n; ++i) p[i] = (float)(lo + (hi - lo) * next_uniform());
  return p;
}
static double *randd(size_t n) {
  double *p = malloc(n * sizeof(double));
  for (size_t i = 0; i < n; ++i) p[i] = 2.0 * next_uniform() - 1.0;
  return p;
}
static double *outd(size_t n) { return calloc(n, sizeof(double)); }
static int fails = 0;
static void expect(int got, int want, const char *what) {
  if (got != want) {
    fprintf(stderr, "%s: returned %d, expected %d\n", what, got, want);
    ++fails;
  }
}
static void expect_finite(const double *p, size_t n, const char *what) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(p[i])) {
      fprintf(stderr, "%s: non-finite entry %zu\n", what, i);
      ++fails;
      return;
    }
}

int main(void) {
  const int64_t b = 2, d = 6, n = 5, L = 37, G = 3;
  const size_t rowsz = (size_t)(b * d * L), bcs = (size_t)(b * G * n * L);
  float *u = randf(rowsz, -1, 1), *dl = randf(rowsz, -1, 1), *z = randf(rowsz, -2, 2);
  float *A = randf((size_t)(d * n), -4, -0.5), *B = randf(bcs, -1, 1), *C = randf(bcs, -1, 1);
  float *D = randf((size_t)d, -1, 1), *bias = randf((size_t)d, -3, -1);
  double *h0 = randd((size_t)(b * d * n)), *dy = randd(rowsz), *dlast = randd((size_t)(b * d * n));
  double *y = outd(rowsz), *ls = outd((size_t)(b * d * n));
  const int64_t rows[3] = {11, 0, 5};

  /* forward: groups, per channel, one group; row subset; no optional inputs */
  expect(oracle_selective_scan_grouped_f64(u, dl, A, B, C, D, z, bias, 1, h0, b, d, n, L, G, NULL,
                                           0, y, ls, 4), 0, "fwd grouped");
  expect_finite(y, rowsz, "fwd y");
  expect(oracle_selective_scan_grouped_f64(u, dl, A, B, C, NULL, NULL, NULL, 1, NULL, b, d, n, L,
                                           1, rows, 3, y, ls, 3), 0, "fwd rows");
  float *Bc = randf((size_t)(b * d * n * L), -1, 1), *Cc = randf((size_t)(b * d * n * L), -1, 1);
  expect(oracle_selective_scan_grouped_f64(u, dl, A, Bc, Cc, D, z, bias, 0, h0, b, d, n, L, d,
                                           NULL, 0, y, NULL, 2), 0, "fwd per channel");
  expect(oracle_selective_scan_grouped_f64(u, dl, A, B, C, D, z, bias, 1, h0, b, d, n, L, 4, NULL,
                                           0, y, ls, 1), -1, "fwd bad ngroups");
  expect(oracle_selective_scan_grouped_f64(NULL, dl, A, B, C, D, z, bias, 1, h0, b, d, n, L, G,
                                           NULL, 0, y, ls, 1), -1, "fwd null u");

  /* backward: groups with everything, per channel without optional inputs */
  double *du = outd(rowsz), *ddl = outd(rowsz), *dz = outd(rowsz), *dA = outd((size_t)(d * n));
  double *dB = outd((size_t)(b * d * n * L)), *dC = outd((size_t)(b * d * n * L));
  double *dD = outd((size_t)d), *dbias = outd((size_t)d), *dh0 = outd((size_t)(b * d * n));
  expect(oracle_selective_scan_bwd_grouped_f64(u, dl, A, B, C, D, z, bias, 1, h0, dy, dlast, b, d,
                                               n, L, G, du, ddl, dA, dB, dC, dD, dz, dbias, dh0, 4),
         0, "bwd grouped");
  expect_finite(du, rowsz, "bwd du");
  expect_finite(dA, (size_t)(d * n), "bwd dA");
  expect(oracle_selective_scan_bwd_grouped_f64(u, dl, A, Bc, Cc, NULL, NULL, NULL, 0, NULL, dy,
                                               NULL, b, d, n, L, d, du, ddl, dA, dB, dC, dD, NULL,
                                               dbias, NULL, 3), 0, "bwd per channel");
  expect(oracle_selective_scan_bwd_grouped_f64(u, dl, A, B, C, D, z, bias, 1, h0, dy, dlast, b, d,
                                               n, L, G, du, ddl, dA, dB, dC, dD, NULL, dbias, dh0,
                                               1), -1, "bwd z without dz");

  /* SSD: heads over groups, initial state, softplus on and off */
  const int64_t H = 4, P = 3, N = 6, g2 = 2, Ls = 29;
  float *x = randf((size_t)(b * Ls * H * P), -1, 1), *dt = randf((size_t)(b * Ls * H), -1, 1);
  float *As = randf((size_t)H, -8, -1), *Bs = randf((size_t)(b * Ls * g2 * N), -1, 1);
  float *Cs = randf((size_t)(b * Ls * g2 * N), -1, 1), *Ds = randf((size_t)H, -1, 1);
  float *dtb = randf((size_t)H, -3, -1);
  double *init = randd((size_t)(b * H * P * N)), *ys = outd((size_t)(b * Ls * H * P));
  double *fs = outd((size_t)(b * H * P * N));
  expect(oracle_ssd_h0_f64(x, dt, As, Bs, Cs, Ds, dtb, 1, init, b, Ls, H, P, N, g2, ys, fs, 4), 0,
         "ssd");
  expect_finite(ys, (size_t)(b * Ls * H * P), "ssd y");
  expect(oracle_ssd_h0_f64(x, dt, As, Bs, Cs, NULL, NULL, 0, NULL, b, Ls, H, P, N, 1, ys, NULL, 2),
         0, "ssd plain");
  expect(oracle_ssd_h0_f64(x, dt, As, Bs, Cs, Ds, dtb, 1, init, b, Ls, H, P, N, 3, ys, fs, 1), -1,
         "ssd bad ngroups");

  free(u); free(dl); free(z); free(A); free(B); free(C); free(D); free(bias); free(h0); free(dy);
  free(dlast); free(y); free(ls); free(Bc); free(Cc); free(du); free(ddl); free(dz); free(dA);
  free(dB); free(dC); free(dD); free(dbias); free(dh0); free(x); free(dt); free(As); free(Bs);
  free(Cs); free(Ds); free(dtb); free(init); free(ys); free(fs);
  if (fails) {
    fprintf(stderr, "%d check(s) failed\n", fails);
    return 1;
  }
  printf("oracle driver: all calls as expected\n");
  return 0;
}
