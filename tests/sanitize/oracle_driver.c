/* Drives every entry point of oracle/s6_oracle.c on small seeded inputs, edge
 * cases included, for a build with AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_sanitizers.py).  Exit status 0 when every call returns its
 * documented code and every result is finite. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int s6_oracle_scan(int64_t, int64_t, int64_t, int64_t, const double*, const double*, const double*, const double*,
                   const double*, const double*, const double*, const double*, int, const double*, double*, double*,
                   int);
int s6_oracle_step(int64_t, int64_t, int64_t, double*, const double*, const double*, const double*, const double*,
                   const double*, const double*, const double*, const double*, int, double*, int);
int s6_oracle_scan_bwd(int64_t, int64_t, int64_t, int64_t, const double*, const double*, const double*, const double*,
                       const double*, const double*, const double*, const double*, int, const double*, const double*,
                       const double*, double*, double*, double*, double*, double*, double*, double*, double*, double*,
                       int);
int s6_oracle_scan_complex(int64_t, int64_t, int64_t, int64_t, const double*, const double*, const double*,
                           const double*, const double*, const double*, const double*, const double*, int,
                           const double*, double*, double*, int);
int s6_oracle_max_threads(void);

static uint64_t rng = 88172645463325252ull;
static double urand(void) {  /* xorshift64, uniform in [-1, 1) */
  rng ^= rng << 13;
  rng ^= rng >> 7;
  rng ^= rng << 17;
  return (double)(rng >> 11) / 4503599627370496.0 - 1.0;
}
static double* fill(size_t n, double lo, double hi) {
  double* p = malloc((n ? n : 1) * sizeof(double));
  for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * (urand() + 1.0) / 2.0;
  return p;
}
static int finite_all(const double* p, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(p[i])) return 0;
  return 1;
}

static int fails = 0;
#define CHECK(cond)                                              \
  do {                                                           \
    if (!(cond)) {                                               \
      fprintf(stderr, "check failed line %d: %s\n", __LINE__, #cond); \
      ++fails;                                                   \
    }                                                            \
  } while (0)

static void one(int64_t batch, int64_t L, int64_t D, int64_t N, int with_h0, int with_z, int nthreads) {
  const size_t tok = (size_t)(batch * L * D), bc = (size_t)(batch * L * N), st = (size_t)(batch * D * N);
  double *u = fill(tok, -1, 1), *delta = fill(tok, -4, -2), *z = fill(tok, -2, 2);
  double *B = fill(bc, -1, 1), *C = fill(bc, -1, 1), *bias = fill((size_t)D, -5, -2), *dsk = fill((size_t)D, -1, 1);
  double *A = fill((size_t)(D * N), -8, -0.5), *h0 = fill(st, -1, 1);
  double *out = fill(tok, 0, 0), *last = fill(st, 0, 0);
  CHECK(s6_oracle_scan(batch, L, D, N, u, delta, bias, A, B, C, dsk, with_z ? z : NULL, 1, with_h0 ? h0 : NULL, out,
                       last, nthreads) == 0);
  CHECK(finite_all(out, tok) && finite_all(last, st));
  /* backward */
  double *dout = fill(tok, -1, 1), *dlast = fill(st, -1, 1);
  double *du = fill(tok, 0, 0), *ddelta = fill(tok, 0, 0), *dz = fill(tok, 0, 0), *dB = fill(bc, 0, 0),
         *dC = fill(bc, 0, 0), *dA = fill((size_t)(D * N), 0, 0), *dD = fill((size_t)D, 0, 0),
         *dbias = fill((size_t)D, 0, 0), *dh0 = fill(st, 0, 0);
  CHECK(s6_oracle_scan_bwd(batch, L, D, N, u, delta, bias, A, B, C, dsk, with_z ? z : NULL, 1, with_h0 ? h0 : NULL,
                           dout, dlast, du, ddelta, dA, dB, dC, dD, with_z ? dz : NULL, dbias, dh0, nthreads) == 0);
  CHECK(finite_all(du, tok) && finite_all(dA, (size_t)(D * N)) && finite_all(dh0, st));
  /* complex A: (re, im) pairs for A, h0 and last_state */
  double *Ac = fill((size_t)(2 * D * N), -2, 2), *h0c = fill(2 * st, -1, 1), *lastc = fill(2 * st, 0, 0);
  for (int64_t i = 0; i < D * N; ++i) Ac[2 * i] = -fabs(Ac[2 * i]) - 0.1;
  CHECK(s6_oracle_scan_complex(batch, L, D, N, u, delta, bias, Ac, B, C, dsk, with_z ? z : NULL, 1,
                               with_h0 ? h0c : NULL, out, lastc, nthreads) == 0);
  CHECK(finite_all(out, tok) && finite_all(lastc, 2 * st));
  /* decode step on the first token of each row */
  if (L > 0) {
    double *state = fill(st, -1, 1), *su = fill((size_t)(batch * D), -1, 1), *sd = fill((size_t)(batch * D), -4, -2);
    double *sB = fill((size_t)(batch * N), -1, 1), *sC = fill((size_t)(batch * N), -1, 1), *so = fill((size_t)(batch * D), 0, 0);
    CHECK(s6_oracle_step(batch, D, N, state, su, sd, bias, A, sB, sC, dsk, NULL, 1, so, nthreads) == 0);
    CHECK(finite_all(state, st) && finite_all(so, (size_t)(batch * D)));
    free(state); free(su); free(sd); free(sB); free(sC); free(so);
  }
  free(u); free(delta); free(z); free(B); free(C); free(bias); free(dsk); free(A); free(h0); free(out); free(last);
  free(dout); free(dlast); free(du); free(ddelta); free(dz); free(dB); free(dC); free(dA); free(dD); free(dbias);
  free(dh0); free(Ac); free(h0c); free(lastc);
}

int main(void) {
  const int nt = s6_oracle_max_threads() > 4 ? 4 : s6_oracle_max_threads();
  for (int64_t N = 1; N <= 16; N *= 2) one(2, 37, 5, N, N % 2, 1, nt);
  one(1, 1, 3, 16, 1, 0, 1);   /* one token, no gate */
  one(3, 0, 4, 8, 1, 1, nt);   /* empty sequence: last_state = h0 */
  one(2, 5, 0, 4, 0, 1, nt);   /* no channels */
  one(1, 300, 2, 16, 0, 1, nt);
  /* arguments the oracle rejects */
  double x = 0.0;
  CHECK(s6_oracle_scan(1, 4, 1, 0, &x, &x, NULL, &x, &x, &x, NULL, NULL, 1, NULL, &x, NULL, 1) == 1);
  CHECK(s6_oracle_scan(1, 4, 1, 4, NULL, &x, NULL, &x, &x, &x, NULL, NULL, 1, NULL, &x, NULL, 1) == 1);
  CHECK(s6_oracle_step(-1, 1, 4, &x, &x, &x, NULL, &x, &x, &x, NULL, NULL, 1, &x, 1) == 1);
  if (fails) {
    fprintf(stderr, "%d checks failed\n", fails);
    return 1;
  }
  printf("oracle driver: all checks passed\n");
  return 0;
}
