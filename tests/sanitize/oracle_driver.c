/* Runs every entry point of the float64 oracle (oracle/oracle.c) on small
 * seeded inputs -- optional inputs present and absent, reset flags, one
 * step, one state, ragged lengths -- with each buffer allocated to exactly
 * its documented size, so that AddressSanitizer and
 * UndefinedBehaviorSanitizer see any access outside it.  Prints "oracle ok"
 * and exits 0 when no sanitizer fired and every result is finite. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_scan_fwd(const double*, const double*, const double*, const double*, const double*,
                     const double*, const double*, const double*, const double*,
                     const unsigned char*, int, int, int64_t, int64_t, int64_t, int64_t, int64_t,
                     int64_t, double*, double*);
void oracle_state_update(double*, const double*, const double*, const double*, const double*,
                         const double*, const double*, const double*, const double*, int, int,
                         int64_t, int64_t, int64_t, int64_t, int64_t, double*);
void oracle_scan_bwd(const double*, const double*, const double*, const double*, const double*,
                     const double*, const double*, const double*, const double*, const double*,
                     const unsigned char*, int, int, int64_t, int64_t, int64_t, int64_t, int64_t,
                     int64_t, double*, double*, double*, double*, double*, double*, double*,
                     double*, double*);
void oracle_conv1d_silu_fwd(const double*, const double*, const double*, const unsigned char*,
                            int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, double*);
void oracle_conv1d_silu_bwd(const double*, const double*, const double*, const unsigned char*,
                            const double*, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t,
                            double*, double*, double*);
void oracle_scan_fwd_complex(const double*, const double*, const double*, const double*,
                             const double*, const double*, const double*, const double*,
                             const double*, const unsigned char*, int, int, int64_t, int64_t,
                             int64_t, int64_t, int64_t, int64_t, double*, double*);
void oracle_scan_bwd_complex(const double*, const double*, const double*, const double*,
                             const double*, const double*, const double*, const double*,
                             const double*, const double*, const unsigned char*, int, int,
                             int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, double*,
                             double*, double*, double*, double*, double*, double*, double*,
                             double*);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static double rnd(void) { /* xorshift64*, uniform in [-1, 1) */
  g_state ^= g_state >> 12; g_state ^= g_state << 25; g_state ^= g_state >> 27;
  return (double)((g_state * 2685821657736338717ull) >> 11) / 4503599627370496.0 - 1.0;
}
static double* vec(int64_t n) {
  double* p = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) p[i] = rnd();
  return p;
}
static int g_bad = 0;
static void finite(const double* p, int64_t n, const char* what) {
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(p[i])) { fprintf(stderr, "%s[%lld] not finite\n", what, (long long)i); ++g_bad; return; }
}

static void run(int64_t Bt, int64_t D, int64_t N, int64_t L, int full, int disc, int softplus) {
  const int64_t CT = Bt * D * L, BNL = Bt * N * L, DN = D * N, BDN = Bt * D * N;
  double *u = vec(CT), *dl = vec(CT), *z = vec(CT), *dout = vec(CT);
  double *A = vec(DN), *Bm = vec(BNL), *C = vec(BNL), *Dp = vec(D), *bias = vec(D);
  double *h0 = vec(BDN);
  for (int64_t i = 0; i < DN; ++i) A[i] = -0.5 - fabs(A[i]);
  if (!softplus) for (int64_t i = 0; i < CT; ++i) dl[i] = 0.01 + 0.1 * fabs(dl[i]);
  unsigned char* rst = (unsigned char*)malloc((size_t)(Bt * L));
  for (int64_t i = 0; i < Bt * L; ++i) rst[i] = (i % 7) == 3;
  double *out = vec(CT), *last = vec(BDN);
  const double* Do = full ? Dp : NULL;
  const double* zo = full ? z : NULL;
  const double* bo = full ? bias : NULL;
  const double* ho = full ? h0 : NULL;
  const unsigned char* ro = full ? rst : NULL;
  oracle_scan_fwd(u, dl, A, Bm, C, Do, zo, bo, ho, ro, softplus, disc, Bt, D, N, L, 0, Bt * D, out,
                  full ? last : NULL);
  finite(out, CT, "fwd out");
  double *du = vec(CT), *ddl = vec(CT), *dz = vec(CT), *dA = vec(DN), *dB = vec(BNL),
         *dC = vec(BNL), *dD = vec(D), *db = vec(D), *dh0 = vec(BDN);
  oracle_scan_bwd(u, dl, A, Bm, C, Do, zo, bo, ho, dout, ro, softplus, disc, Bt, D, N, L, 0,
                  Bt * D, du, ddl, dA, dB, dC, full ? dD : NULL, full ? dz : NULL,
                  full ? db : NULL, full ? dh0 : NULL);
  finite(du, CT, "bwd du"); finite(dA, DN, "bwd dA"); finite(dB, BNL, "bwd dB");
  /* one decode step from the final state */
  double *st = vec(BDN), *so = vec(Bt * D);
  oracle_state_update(st, u, dl, A, Bm, C, Do, zo, bo, softplus, disc, Bt, D, N, 0, Bt * D, so);
  finite(so, Bt * D, "step out");
  /* convolution stage, widths 1..4 */
  for (int64_t W = 1; W <= 4; ++W) {
    double *w = vec(D * W), *cb = vec(D), *x = vec(CT), *ux = vec(CT), *dx = vec(CT),
           *dw = vec(D * W), *dcb = vec(D);
    oracle_conv1d_silu_fwd(x, w, full ? cb : NULL, ro, Bt, D, W, L, 0, Bt * D, ux);
    oracle_conv1d_silu_bwd(x, w, full ? cb : NULL, ro, dout, Bt, D, W, L, 0, Bt * D, dx, dw,
                           full ? dcb : NULL);
    finite(ux, CT, "conv u"); finite(dx, CT, "conv dx");
    free(w); free(cb); free(x); free(ux); free(dx); free(dw); free(dcb);
  }
  /* complex variant: interleaved (re, im) pairs */
  double *cA = vec(2 * DN), *cB = vec(2 * BNL), *cC = vec(2 * BNL), *ch0 = vec(2 * BDN);
  for (int64_t i = 0; i < DN; ++i) cA[2 * i] = -0.5 - fabs(cA[2 * i]);
  if (full && DN > 1) { cA[2] = 0.0; cA[3] = 0.0; }   /* the A = 0 limit */
  double *cout = vec(CT), *clast = vec(2 * BDN);
  oracle_scan_fwd_complex(u, dl, cA, cB, cC, Do, zo, bo, full ? ch0 : NULL, ro, softplus, disc,
                          Bt, D, N, L, 0, Bt * D, cout, full ? clast : NULL);
  finite(cout, CT, "cfwd out");
  double *cdA = vec(2 * DN), *cdB = vec(2 * BNL), *cdC = vec(2 * BNL), *cdh0 = vec(2 * BDN);
  oracle_scan_bwd_complex(u, dl, cA, cB, cC, Do, zo, bo, full ? ch0 : NULL, dout, ro, softplus,
                          disc, Bt, D, N, L, 0, Bt * D, du, ddl, cdA, cdB, cdC,
                          full ? dD : NULL, full ? dz : NULL, full ? db : NULL,
                          full ? cdh0 : NULL);
  finite(cdA, 2 * DN, "cbwd dA"); finite(du, CT, "cbwd du");
  double* bufs[] = {u, dl, z, dout, A, Bm, C, Dp, bias, h0, out, last, du, ddl, dz, dA, dB, dC,
                    dD, db, dh0, st, so, cA, cB, cC, ch0, cout, clast, cdA, cdB, cdC, cdh0};
  for (size_t i = 0; i < sizeof(bufs) / sizeof(bufs[0]); ++i) free(bufs[i]);
  free(rst);
}

int main(void) {
  const int64_t shapes[][4] = {{1, 1, 1, 1}, {2, 3, 4, 9}, {1, 2, 16, 130}, {2, 1, 5, 1}};
  for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s)
    for (int full = 0; full < 2; ++full)
      for (int disc = 0; disc < 2; ++disc)
        for (int sp = 0; sp < 2; ++sp)
          run(shapes[s][0], shapes[s][1], shapes[s][2], shapes[s][3], full, disc, sp);
  if (g_bad) { fprintf(stderr, "%d non-finite result(s)\n", g_bad); return 1; }
  printf("oracle ok\n");
  return 0;
}
