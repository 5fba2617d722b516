/*
 * Host driver for a sanitizer build of the oracle (AddressSanitizer and
 * UndefinedBehaviorSanitizer): every entry point of oracle/ssm_oracle.c on
 * small seeded inputs, including the edge cases (empty sequence, one step,
 * one state, absent optional arguments, both input and delta modes, ragged
 * conv widths), and every argument check.  Test infrastructure: built and run
 * by tests/test_oracle_sanitize.py, never part of the product.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int ssm_oracle_scan_f64(const double*, const double*, const double*, const double*, const double*, const double*,
                        const double*, const double*, const double*, double*, double*, int64_t, int64_t, int64_t,
                        int64_t, int, int);
int ssm_oracle_update_f64(double*, const double*, const double*, const double*, const double*, const double*,
                          const double*, const double*, const double*, double*, int64_t, int64_t, int64_t, int, int);
int ssm_oracle_conv1d_f64(const double*, const double*, const double*, const double*, double*, double*, int64_t,
                          int64_t, int64_t, int64_t, int);
int ssm_oracle_scan_bwd_f64(const double*, const double*, const double*, const double*, const double*,
                            const double*, const double*, const double*, const double*, const double*, const double*,
                            double*, double*, double*, double*, double*, double*, double*, double*, double*, int64_t,
                            int64_t, int64_t, int64_t, int, int);
int ssm_oracle_ssd_f64(const double*, const double*, const double*, const double*, const double*, const double*,
                       const double*, const double*, const double*, double*, double*, int64_t, int64_t, int64_t,
                       int64_t, int64_t, int64_t, int);

static uint64_t rng_state = 88172645463325252ull;
static double urand(void) { /* xorshift64, uniform in [-1, 1) */
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return (double)(rng_state >> 11) / (double)(1ull << 52) - 1.0;
}
/* Exactly n doubles on the heap (so that any overrun is caught), or NULL for n == 0. */
static double* buf(int64_t n, double lo, double hi) {
  if (n == 0) return NULL;
  double* p = (double*)malloc((size_t)n * sizeof(double));
  for (int64_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * 0.5 * (urand() + 1.0);
  return p;
}
static int fails = 0;
#define CHECK(cond)                                              \
  do {                                                           \
    if (!(cond)) {                                               \
      fprintf(stderr, "check failed line %d: %s\n", __LINE__, #cond); \
      ++fails;                                                   \
    }                                                            \
  } while (0)

static void scan_case(int64_t b, int64_t L, int64_t d, int64_t n, int opt, int im, int dm) {
  double *x = buf(b * L * d, -1, 1), *dl = buf(b * L * d, dm ? -2 : 1e-3, dm ? 1 : 0.2), *A = buf(d * n, -4, -0.1);
  double *B = buf(b * L * n, -1, 1), *C = buf(b * L * n, -1, 1), *D = opt ? buf(d, -1, 1) : NULL;
  double *z = opt ? buf(b * L * d, -2, 2) : NULL, *h0 = opt ? buf(b * d * n, -1, 1) : NULL;
  double *dtb = dm ? buf(d, -3, -1) : NULL, *y = buf(b * L * d, 0, 0), *hl = buf(b * d * n, 0, 0);
  if (b * L * d > 0) CHECK(ssm_oracle_scan_f64(x, dl, A, B, C, D, z, h0, dtb, y, hl, b, L, d, n, im, dm) == 0);
  double *dy = buf(b * L * d, -1, 1), *dhl = opt ? buf(b * d * n, -1, 1) : NULL;
  double *dx = buf(b * L * d, 0, 0), *ddl = buf(b * L * d, 0, 0), *dA = buf(d * n, 0, 0);
  double *dB = buf(b * L * n, 0, 0), *dC = buf(b * L * n, 0, 0), *dD = opt ? buf(d, 0, 0) : NULL;
  double *dz = opt ? buf(b * L * d, 0, 0) : NULL, *dh0 = buf(b * d * n, 0, 0), *ddtb = dm ? buf(d, 0, 0) : NULL;
  if (b * L * d > 0)
    CHECK(ssm_oracle_scan_bwd_f64(x, dl, A, B, C, D, z, h0, dtb, dy, dhl, dx, ddl, dA, dB, dC, dD, dz, dh0, ddtb, b, L,
                                  d, n, im, dm) == 0);
  if (b * d > 0 && L > 0) {
    double* h = buf(b * d * n, -1, 1);
    CHECK(ssm_oracle_update_f64(h, x, dl, A, B, C, D, z, dtb, y, b, d, n, im, dm) == 0);
    free(h);
  }
  double* ptrs[] = {x, dl, A, B, C, D, z, h0, dtb, y, hl, dy, dhl, dx, ddl, dA, dB, dC, dD, dz, dh0, ddtb};
  for (size_t i = 0; i < sizeof(ptrs) / sizeof(ptrs[0]); ++i) free(ptrs[i]);
}

int main(void) {
  const int64_t shapes[][4] = {{1, 1, 1, 1}, {2, 7, 3, 4}, {1, 0, 2, 2}, {3, 9, 5, 16}, {1, 33, 2, 3}};
  for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s)
    for (int opt = 0; opt < 2; ++opt)
      for (int im = 0; im < 2; ++im)
        for (int dm = 0; dm < 2; ++dm) scan_case(shapes[s][0], shapes[s][1], shapes[s][2], shapes[s][3], opt, im, dm);
  /* conv: every width, with and without bias, carried state, SiLU */
  for (int64_t K = 1; K <= 4; ++K)
    for (int opt = 0; opt < 2; ++opt) {
      const int64_t b = 2, L = 11, d = 3;
      double *x = buf(b * L * d, -1, 1), *w = buf(d * K, -1, 1), *bias = opt ? buf(d, -1, 1) : NULL;
      double *si = (opt && K > 1) ? buf(b * d * (K - 1), -1, 1) : NULL, *y = buf(b * L * d, 0, 0);
      double* so = K > 1 ? buf(b * d * (K - 1), 0, 0) : NULL;
      CHECK(ssm_oracle_conv1d_f64(x, w, bias, si, y, so, b, L, d, K, opt) == 0);
      free(x); free(w); free(bias); free(si); free(y); free(so);
    }
  /* SSD form: groups, optional inputs, both delta modes */
  for (int opt = 0; opt < 2; ++opt)
    for (int dm = 0; dm < 2; ++dm) {
      const int64_t b = 2, L = 9, H = 4, P = 3, G = 2, N = 5;
      double *x = buf(b * L * H * P, -1, 1), *dt = buf(b * L * H, dm ? -2 : 1e-3, dm ? 1 : 0.2), *A = buf(H, -4, -1);
      double *B = buf(b * L * G * N, -1, 1), *C = buf(b * L * G * N, -1, 1), *D = opt ? buf(H, -1, 1) : NULL;
      double *z = opt ? buf(b * L * H * P, -2, 2) : NULL, *h0 = opt ? buf(b * H * P * N, -1, 1) : NULL;
      double *dtb = dm ? buf(H, -3, -1) : NULL, *y = buf(b * L * H * P, 0, 0), *hl = buf(b * H * P * N, 0, 0);
      CHECK(ssm_oracle_ssd_f64(x, dt, A, B, C, D, z, h0, dtb, y, hl, b, L, H, P, G, N, dm) == 0);
      free(x); free(dt); free(A); free(B); free(C); free(D); free(z); free(h0); free(dtb); free(y); free(hl);
    }
  /* argument checks return an error without touching memory */
  double one = 1.0, out = 0.0;
  CHECK(ssm_oracle_scan_f64(NULL, &one, &one, &one, &one, NULL, NULL, NULL, NULL, &out, NULL, 1, 1, 1, 1, 0, 0) != 0);
  CHECK(ssm_oracle_scan_f64(&one, &one, &one, &one, &one, NULL, NULL, NULL, NULL, &out, NULL, 1, 1, 1, 0, 0, 0) != 0);
  CHECK(ssm_oracle_scan_f64(&one, &one, &one, &one, &one, NULL, NULL, NULL, NULL, &out, NULL, 1, 1, 1, 1, 2, 0) != 0);
  CHECK(ssm_oracle_conv1d_f64(&one, &one, NULL, NULL, &out, NULL, 1, 1, 1, 0, 0) != 0);
  CHECK(ssm_oracle_ssd_f64(&one, &one, &one, &one, &one, NULL, NULL, NULL, NULL, &out, NULL, 1, 1, 3, 1, 2, 1, 0) != 0);
  if (fails) {
    fprintf(stderr, "%d checks failed\n", fails);
    return 1;
  }
  printf("oracle sanitizer driver ok\n");
  return 0;
}
