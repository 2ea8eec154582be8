/*
 * oracle_driver.c -- runs the fp64 oracle's C functions (oracle/ssd_oracle.c:
 * the recurrence, its adjoint and the diagonal selective scan) on small
 * deterministic inputs, with packed sequences (empty ones included), initial
 * states present and absent, and a few invalid arguments.  Built with
 * AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py,
 * so that an out-of-bounds access or undefined operation in the oracle ends
 * the run with an error.  Exit status 0 when every call returned what it
 * should and every output is finite.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int ssd_oracle_recurrence(const double *x, const double *dt, const double *A, const double *B, const double *C,
                          const int64_t *cu_seqlens, int64_t nseq, int64_t H, int64_t P, int64_t N, int64_t G,
                          const double *init_state, double *y, double *final_state, int nthreads);
int ssd_oracle_backward(const double *x, const double *dt, const double *A, const double *B, const double *C,
                        const int64_t *cu_seqlens, int64_t nseq, int64_t H, int64_t P, int64_t N, int64_t G,
                        const double *init_state, const double *dy, const double *dfinal, double *dx,
                        double *ddt, double *dA, double *dB, double *dC, double *dinit, int nthreads);
int ssd_oracle_selective_scan(const double *x, const double *delta, const double *A, const double *B,
                              const double *C, int64_t nbatch, int64_t T, int64_t D, int64_t N, double *y,
                              double *final_state, int nthreads);

static uint64_t rng = 88172645463325252ull;
static double urand(void) {  /* xorshift64, uniform in [0, 1) */
  rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
  return (double)(rng >> 11) / 9007199254740992.0;
}
static double *arr(size_t n, double lo, double hi) {
  double *a = malloc((n ? n : 1) * sizeof(double));
  for (size_t i = 0; i < n; ++i) a[i] = lo + (hi - lo) * urand();
  return a;
}
static int finite_all(const double *a, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(a[i])) return 0;
  return 1;
}

int main(void) {
  int bad = 0;
  const int64_t H = 4, P = 8, N = 5, G = 2;
  const int64_t cu[] = {0, 7, 7, 8, 40, 40, 63};  /* six sequences, two of them empty */
  const int64_t S = 6, T = 63;
  double *x = arr(T * H * P, -1, 1), *dt = arr(T * H, 0.001, 0.2), *A = arr(H, -3, -0.1);
  double *B = arr(T * G * N, -1, 1), *C = arr(T * G * N, -1, 1), *h0 = arr(S * H * P * N, -1, 1);
  double *y = arr(T * H * P, 0, 0), *fs = arr(S * H * P * N, 0, 0);
  for (int with_init = 0; with_init < 2; ++with_init) {
    if (ssd_oracle_recurrence(x, dt, A, B, C, cu, S, H, P, N, G, with_init ? h0 : NULL, y, fs, 1) != 0) ++bad;
    if (!finite_all(y, T * H * P) || !finite_all(fs, S * H * P * N)) ++bad;
    if (ssd_oracle_recurrence(x, dt, A, B, C, cu, S, H, P, N, G, with_init ? h0 : NULL, y, NULL, 2) != 0) ++bad;
  }
  double *dy = arr(T * H * P, -1, 1), *dfin = arr(S * H * P * N, -1, 1);
  double *dx = arr(T * H * P, 0, 0), *ddt = arr(T * H, 0, 0), *dA = arr(S * H, 0, 0);
  double *dB = arr(T * H * N, 0, 0), *dC = arr(T * H * N, 0, 0), *dinit = arr(S * H * P * N, 0, 0);
  for (int opt = 0; opt < 4; ++opt) {
    const double *i0 = (opt & 1) ? h0 : NULL, *df = (opt & 2) ? dfin : NULL;
    if (ssd_oracle_backward(x, dt, A, B, C, cu, S, H, P, N, G, i0, dy, df, dx, ddt, dA, dB, dC,
                            (opt & 1) ? dinit : NULL, 1) != 0) ++bad;
    if (!finite_all(dx, T * H * P) || !finite_all(ddt, T * H) || !finite_all(dA, S * H) ||
        !finite_all(dB, T * H * N) || !finite_all(dC, T * H * N)) ++bad;
  }
  /* a sequence longer than the adjoint's checkpoint interval */
  {
    const int64_t cl[] = {0, 200};
    double *xl = arr(200 * H * P, -1, 1), *dtl = arr(200 * H, 0.001, 0.1), *Bl = arr(200 * G * N, -1, 1);
    double *Cl = arr(200 * G * N, -1, 1), *dyl = arr(200 * H * P, -1, 1);
    double *dxl = arr(200 * H * P, 0, 0), *ddtl = arr(200 * H, 0, 0), *dAl = arr(H, 0, 0);
    double *dBl = arr(200 * H * N, 0, 0), *dCl = arr(200 * H * N, 0, 0);
    if (ssd_oracle_backward(xl, dtl, A, Bl, Cl, cl, 1, H, P, N, G, NULL, dyl, NULL, dxl, ddtl, dAl, dBl, dCl, NULL,
                            1) != 0) ++bad;
    free(xl); free(dtl); free(Bl); free(Cl); free(dyl); free(dxl); free(ddtl); free(dAl); free(dBl); free(dCl);
  }
  /* invalid arguments: refused, nothing read past the arrays */
  const int64_t cu_bad[] = {1, 5};
  if (ssd_oracle_recurrence(x, dt, A, B, C, cu_bad, 1, H, P, N, G, NULL, y, NULL, 1) != -1) ++bad;
  if (ssd_oracle_recurrence(x, dt, A, B, C, cu, S, 3, P, N, G, NULL, y, NULL, 1) != -1) ++bad;
  if (ssd_oracle_backward(x, dt, A, B, C, cu, S, H, P, N, 3, NULL, dy, NULL, dx, ddt, dA, dB, dC, NULL, 1) != -1)
    ++bad;
  /* selective scan */
  {
    const int64_t b = 2, Ts = 33, D = 6, Ns = 7;
    double *xs = arr(b * Ts * D, -1, 1), *de = arr(b * Ts * D, 0.001, 0.1), *As = arr(D * Ns, -4, -0.5);
    double *Bs = arr(b * Ts * Ns, -1, 1), *Cs = arr(b * Ts * Ns, -1, 1), *ys = arr(b * Ts * D, 0, 0);
    double *fss = arr(b * D * Ns, 0, 0);
    if (ssd_oracle_selective_scan(xs, de, As, Bs, Cs, b, Ts, D, Ns, ys, fss, 1) != 0) ++bad;
    if (ssd_oracle_selective_scan(xs, de, As, Bs, Cs, b, 0, D, Ns, ys, NULL, 1) != 0) ++bad;
    if (!finite_all(ys, b * Ts * D) || !finite_all(fss, b * D * Ns)) ++bad;
    if (ssd_oracle_selective_scan(xs, de, As, Bs, Cs, b, Ts, 0, Ns, ys, NULL, 1) != -1) ++bad;
    free(xs); free(de); free(As); free(Bs); free(Cs); free(ys); free(fss);
  }
  free(x); free(dt); free(A); free(B); free(C); free(h0); free(y); free(fs);
  free(dy); free(dfin); free(dx); free(ddt); free(dA); free(dB); free(dC); free(dinit);
  printf("oracle driver: %d failed checks\n", bad);
  return bad ? 1 : 0;
}
