/*
 * Float64 CPU oracle for the selective scan (S6).  TEST INFRASTRUCTURE ONLY.
 *
 * This file is the plain, slow reference that the GPU library is checked
 * against.  Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load it; the GPU library never calls, links or includes it,
 * and it shares no code, header or constant with the GPU path.
 *
 * Sources (web pages about Gu & Dao, "Mamba: Linear-Time Sequence Modeling
 * with Selective State Spaces", arXiv 2312.00752):
 *   [KNOWL1]  chapterpal.com page of that title, Knowl 1 "Selective State
 *             Space Layer (S6)": ZOH rule (step 3), the time-varying
 *             recurrence (step 4) and the per-(b, d, t) loop printed under it.
 *   [SUM-3.4] paper-graph-ui.vercel.app summary of the paper, section 3.4
 *             "Detailed, Sentence-Based Technical Breakdown": softplus for
 *             tau_Delta, the selective parameter shapes, backward recompute.
 *   [ESSAY]   trishampatil.com engineering essay on the paper, Part II §4
 *             "The same SSM is also a convolution" (h_0 = 0) and Part III §4
 *             (chunk carry, recomputation in the backward).
 *   [KNOWL3]  chapterpal page, Knowl 3 "Mamba Block Architecture" (SiLU gate).
 * Additions beyond the pages (they come from the library's specification):
 * the skip term D*u, the SiLU(z) gate applied to y inside the scan, the
 * additive delta_bias standing for the "Parameter" inside tau_Delta, and an
 * Euler variant of B-bar (B-bar = Delta*B, A-bar unchanged).
 *
 * Layouts (row-major, contiguous):
 *   u, delta, z, out, dout, du, ddelta, dz : (batch, dim, seqlen)
 *   B, C, dB, dC                           : (batch, dstate, seqlen)
 *   A, dA                                  : (dim, dstate)
 *   D, dD, delta_bias, ddelta_bias         : (dim)
 *   h0, last_state, state                  : (batch, dim, dstate)
 * A "channel" is one (b, d) pair, index c = b*dim + d.  Functions take a
 * channel range [c_begin, c_end) so a caller may split work over threads;
 * the backward accumulates dA, dB, dC, dD, ddelta_bias with += so each
 * thread must be given buffers of its own (the caller sums them).
 *
 * Built without fast-math and without FP contraction: every operation is
 * the plain IEEE double operation written here.
 */
#include <complex.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_ZOH = 0, ORACLE_EULER = 1 };

/* softplus(x) = log(1 + e^x) [SUM-3.4, "specific functional forms"], written
 * in the overflow-free form max(x, 0) + log1p(exp(-|x|)). */
static double softplus(double x) { return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x))); }

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* Step size for one (channel, t): tau_Delta(Parameter + s_Delta(x)) with the
 * Parameter given as delta_bias [KNOWL1 step 2]; without the softplus flag the
 * biased value is used as is. */
static double step_size(double raw, const double* bias, int64_t d, int softplus_on) {
  double r = raw + (bias ? bias[d] : 0.0);
  return softplus_on ? softplus(r) : r;
}

/* B-bar / B for one (t, n).  ZOH [KNOWL1 step 3, diagonal A]:
 * (exp(delta*A) - 1) / A, whose limit at A = 0 is delta.  Euler: delta. */
static double bbar_coef(double dt, double a_n, int disc) {
  if (disc == ORACLE_EULER) return dt;
  if (a_n == 0.0) return dt;
  return expm1(dt * a_n) / a_n;
}

/*
 * Forward scan [KNOWL1 step 4 and its loop], for channels [c_begin, c_end):
 *   h_{-1} = h0 (zero when h0 is NULL, as in [ESSAY] Part II §4)
 *   for t: dt = step_size; for n: Abar = exp(dt*A[d,n]);
 *          h[n] = Abar*h[n] + Bbar*u_t;  y = sum_n C[b,n,t]*h[n]
 *   y += D[d]*u_t;  out = y * z*sigmoid(z)  (each when given)
 *   last_state = h after the final step (when given).
 * reset (nullable, (batch, seqlen) bytes): where reset[b,t] != 0 the state
 * is set to zero before step t, so several sequences packed along t run as
 * if each started alone (boundary resetting [SUM-3.4] / [ESSAY] Part II §8,
 * done here by the boundary flag instead of a learned Delta).
 */
void oracle_scan_fwd(const double* u, const double* delta, const double* A, const double* B,
                     const double* C, const double* D, const double* z, const double* bias,
                     const double* h0, const unsigned char* reset, int softplus_on, int disc,
                     int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int64_t c_begin,
                     int64_t c_end, double* out, double* last_state) {
  (void)batch;
  double* h = (double*)malloc(sizeof(double) * (size_t)dstate);
  for (int64_t c = c_begin; c < c_end; ++c) {
    int64_t b = c / dim, d = c % dim;
    const double* u_r = u + c * seqlen;
    const double* dl_r = delta + c * seqlen;
    const double* z_r = z ? z + c * seqlen : NULL;
    const double* B_b = B + b * dstate * seqlen;
    const double* C_b = C + b * dstate * seqlen;
    const double* A_d = A + d * dstate;
    double* out_r = out + c * seqlen;
    for (int64_t n = 0; n < dstate; ++n) h[n] = h0 ? h0[c * dstate + n] : 0.0;
    for (int64_t t = 0; t < seqlen; ++t) {
      double dt = step_size(dl_r[t], bias, d, softplus_on);
      double y = 0.0;
      if (reset && reset[b * seqlen + t])
        for (int64_t n = 0; n < dstate; ++n) h[n] = 0.0;
      for (int64_t n = 0; n < dstate; ++n) {
        double abar = exp(dt * A_d[n]);
        double bbar = bbar_coef(dt, A_d[n], disc) * B_b[n * seqlen + t];
        h[n] = abar * h[n] + bbar * u_r[t];
        y += C_b[n * seqlen + t] * h[n];
      }
      if (D) y += D[d] * u_r[t];
      if (z_r) y = y * (z_r[t] * sigmoid(z_r[t]));
      out_r[t] = y;
    }
    if (last_state)
      for (int64_t n = 0; n < dstate; ++n) last_state[c * dstate + n] = h[n];
  }
  free(h);
}

/*
 * One recurrent (decode) step for channels [c_begin, c_end): the body of the
 * forward loop applied to a stored state, in place.  Recurrent inference with
 * a fixed-size state is described in [SUM-3.4] ("dual form", recurrence for
 * autoregressive inference).  Per-step tensors are (batch, dim) for u, delta,
 * z, out and (batch, dstate) for B, C.
 */
void oracle_state_update(double* state, const double* u, const double* delta, const double* A,
                         const double* B, const double* C, const double* D, const double* z,
                         const double* bias, int softplus_on, int disc, int64_t batch, int64_t dim,
                         int64_t dstate, int64_t c_begin, int64_t c_end, double* out) {
  (void)batch;
  for (int64_t c = c_begin; c < c_end; ++c) {
    int64_t b = c / dim, d = c % dim;
    double dt = step_size(delta[c], bias, d, softplus_on);
    double y = 0.0;
    for (int64_t n = 0; n < dstate; ++n) {
      double a_n = A[d * dstate + n];
      double abar = exp(dt * a_n);
      double bbar = bbar_coef(dt, a_n, disc) * B[b * dstate + n];
      double hn = abar * state[c * dstate + n] + bbar * u[c];
      state[c * dstate + n] = hn;
      y += C[b * dstate + n] * hn;
    }
    if (D) y += D[d] * u[c];
    if (z) y = y * (z[c] * sigmoid(z[c]));
    out[c] = y;
  }
}

/*
 * Backward of the forward above for the loss L = sum(dout * out).  The pages
 * only say that the backward recomputes the states from the inputs
 * ([SUM-3.4] "Recomputation for the backward pass"); the adjoint below is the
 * chain rule applied to the forward definition, step by step:
 *   1. recompute h_t (all t) from the inputs;
 *   2. gy_t = dout_t * z_t*sigmoid(z_t)   (dout_t when z is absent)
 *      dz_t = dout_t * y_t * sigmoid(z_t) * (1 + z_t*(1 - sigmoid(z_t)))
 *      where y_t is the pre-gate output;
 *   3. reverse time: gh_t[n] = C_t[n]*gy_t + Abar_{t+1}[n]*gh_{t+1}[n]
 *      (gh after the last step is zero: no gradient flows into last_state);
 *   4. with gA = gh_t*h_{t-1}, gB = gh_t*u_t for each n:
 *        du_t     = gy_t*D + sum_n gh_t*Bbar_t
 *        gdt_t    = sum_n gA*A*Abar + gB*dBbar/ddt
 *        dA[d,n] += gA*dt*Abar + gB*dBbar/dA
 *        dB_t[n] += gB*Bbar/B ;  dC_t[n] += gy_t*h_t
 *      ZOH:   dBbar/ddt = Abar*B,  dBbar/dA = (dt*Abar*B - Bbar)/A
 *             (limit dt*dt*B/2 at A = 0),  Bbar/B = expm1(dt*A)/A
 *      Euler: dBbar/ddt = B,  dBbar/dA = 0,  Bbar/B = dt;
 *   5. ddelta_t = gdt_t * sigmoid(delta_t + bias) with softplus, else gdt_t;
 *      ddelta_bias[d] += ddelta_t;  dD[d] += gy_t*u_t;
 *   6. dh0 = Abar_0 * gh_0 (when an initial state was given).
 * With reset flags the state entering a reset step is zero: h_{t-1} counts as
 * zero in gA and no adjoint flows from step t to t-1.
 * dA, dB, dC, dD, ddelta_bias, dh0 are accumulated with +=; du, ddelta, dz
 * are written.  Optional outputs may be NULL.
 */
void oracle_scan_bwd(const double* u, const double* delta, const double* A, const double* B,
                     const double* C, const double* D, const double* z, const double* bias,
                     const double* h0, const double* dout, const unsigned char* reset,
                     int softplus_on, int disc, int64_t batch, int64_t dim, int64_t dstate,
                     int64_t seqlen, int64_t c_begin,
                     int64_t c_end, double* du, double* ddelta, double* dA, double* dB, double* dC,
                     double* dD, double* dz, double* ddelta_bias, double* dh0) {
  (void)batch;
  /* hs[(t+1)*N + n] = h_t[n]; hs[n] = h_{-1}[n] */
  double* hs = (double*)malloc(sizeof(double) * (size_t)((seqlen + 1) * dstate));
  double* gh = (double*)malloc(sizeof(double) * (size_t)dstate);
  for (int64_t c = c_begin; c < c_end; ++c) {
    int64_t b = c / dim, d = c % dim;
    const double* u_r = u + c * seqlen;
    const double* dl_r = delta + c * seqlen;
    const double* z_r = z ? z + c * seqlen : NULL;
    const double* do_r = dout + c * seqlen;
    const double* B_b = B + b * dstate * seqlen;
    const double* C_b = C + b * dstate * seqlen;
    const double* A_d = A + d * dstate;
    /* 1. recompute states */
    for (int64_t n = 0; n < dstate; ++n) hs[n] = h0 ? h0[c * dstate + n] : 0.0;
    for (int64_t t = 0; t < seqlen; ++t) {
      double dt = step_size(dl_r[t], bias, d, softplus_on);
      int rs = reset && reset[b * seqlen + t];
      for (int64_t n = 0; n < dstate; ++n) {
        double abar = exp(dt * A_d[n]);
        double bbar = bbar_coef(dt, A_d[n], disc) * B_b[n * seqlen + t];
        double hprev = rs ? 0.0 : hs[t * dstate + n];
        hs[(t + 1) * dstate + n] = abar * hprev + bbar * u_r[t];
      }
    }
    /* 3.-5. reverse sweep */
    for (int64_t n = 0; n < dstate; ++n) gh[n] = 0.0;
    for (int64_t t = seqlen - 1; t >= 0; --t) {
      double r = dl_r[t] + (bias ? bias[d] : 0.0);
      double dt = softplus_on ? softplus(r) : r;
      /* pre-gate output y_t, from the recomputed state */
      double y = 0.0;
      for (int64_t n = 0; n < dstate; ++n) y += C_b[n * seqlen + t] * hs[(t + 1) * dstate + n];
      if (D) y += D[d] * u_r[t];
      double gy = do_r[t];
      if (z_r) {
        double zt = z_r[t], sg = sigmoid(zt);
        gy = do_r[t] * (zt * sg);
        dz[c * seqlen + t] = do_r[t] * y * sg * (1.0 + zt * (1.0 - sg));
      }
      double du_t = D ? gy * D[d] : 0.0;
      double gdt = 0.0;
      int rs = reset && reset[b * seqlen + t];
      if (D) dD[d] += gy * u_r[t];
      for (int64_t n = 0; n < dstate; ++n) {
        double a_n = A_d[n];
        double abar = exp(dt * a_n);
        double Bv = B_b[n * seqlen + t];
        double coef = bbar_coef(dt, a_n, disc);
        double bbar = coef * Bv;
        /* gh_t = C_t*gy_t + (Abar_{t+1}*gh_{t+1}, already folded into gh[n]) */
        gh[n] = C_b[n * seqlen + t] * gy + gh[n];
        dC[b * dstate * seqlen + n * seqlen + t] += gy * hs[(t + 1) * dstate + n];
        double gA = rs ? 0.0 : gh[n] * hs[t * dstate + n];
        double gB = gh[n] * u_r[t];
        du_t += gh[n] * bbar;
        double dbbar_ddt, dbbar_dA;
        if (disc == ORACLE_EULER) {
          dbbar_ddt = Bv;
          dbbar_dA = 0.0;
        } else {
          dbbar_ddt = abar * Bv;
          dbbar_dA = (a_n == 0.0) ? dt * dt * Bv / 2.0 : (dt * abar * Bv - bbar) / a_n;
        }
        gdt += gA * a_n * abar + gB * dbbar_ddt;
        dA[d * dstate + n] += gA * dt * abar + gB * dbbar_dA;
        dB[b * dstate * seqlen + n * seqlen + t] += gB * coef;
        /* carry to t-1: gh_{t-1} gets Abar_t * gh_t (nothing across a reset) */
        gh[n] = rs ? 0.0 : abar * gh[n];
      }
      du[c * seqlen + t] = du_t;
      double gr = softplus_on ? gdt * sigmoid(r) : gdt;
      ddelta[c * seqlen + t] = gr;
      if (ddelta_bias) ddelta_bias[d] += gr;
    }
    /* 6. after the loop gh[n] = Abar_0 * gh_0 = dL/dh_{-1} */
    if (dh0)
      for (int64_t n = 0; n < dstate; ++n) dh0[c * dstate + n] += gh[n];
  }
  free(hs);
  free(gh);
}

/*
 * Short causal depthwise convolution + SiLU, the stage that feeds the SSM in
 * the Mamba block ([KNOWL3]: a 1-D temporal convolution of width
 * d_conv = 4 on the main branch, then SiLU, then the selective SSM; [ESSAY]
 * Part II §8 draws the same block).  Per channel (b, d), with W taps:
 *   pre_t = cb[d] + sum_{k=0}^{W-1} w[d,k] * x_{t-(W-1)+k}
 *   u_t   = pre_t * sigmoid(pre_t)
 * The convolution is causal: x before t = 0 counts as zero, and with reset
 * flags (reset[b,t] != 0, a packed sequence starts at t) so does every x
 * before the start of the current sequence.  cb may be NULL.
 */
static int conv_tap_valid(const unsigned char* reset_b, int64_t s, int64_t t) {
  /* x_s contributes to step t (s <= t) iff s >= 0 and no sequence starts in (s, t] */
  if (s < 0) return 0;
  if (reset_b)
    for (int64_t q = s + 1; q <= t; ++q)
      if (reset_b[q]) return 0;
  return 1;
}

static double conv_pre(const double* x_r, const double* w_d, double cb, int64_t W,
                       const unsigned char* reset_b, int64_t t) {
  double pre = cb;
  for (int64_t k = 0; k < W; ++k) {
    int64_t s = t - (W - 1) + k;
    if (conv_tap_valid(reset_b, s, t)) pre += w_d[k] * x_r[s];
  }
  return pre;
}

void oracle_conv1d_silu_fwd(const double* x, const double* w, const double* cb,
                            const unsigned char* reset, int64_t batch, int64_t dim, int64_t W,
                            int64_t seqlen, int64_t c_begin, int64_t c_end, double* u) {
  (void)batch;
  for (int64_t c = c_begin; c < c_end; ++c) {
    int64_t b = c / dim, d = c % dim;
    const unsigned char* reset_b = reset ? reset + b * seqlen : NULL;
    for (int64_t t = 0; t < seqlen; ++t) {
      double pre = conv_pre(x + c * seqlen, w + d * W, cb ? cb[d] : 0.0, W, reset_b, t);
      u[c * seqlen + t] = pre * sigmoid(pre);
    }
  }
}

/*
 * Backward of the convolution stage for a gradient du at its output:
 *   dpre_t = du_t * sigmoid(pre_t) * (1 + pre_t * (1 - sigmoid(pre_t)))
 *   dx_s  += w[d,k] * dpre_t      for every valid tap (s = t-(W-1)+k)
 *   dw[d,k] += dpre_t * x_s ;  dcb[d] += dpre_t
 * dx is written; dw and dcb (nullable) are accumulated with +=.
 */
void oracle_conv1d_silu_bwd(const double* x, const double* w, const double* cb,
                            const unsigned char* reset, const double* du, int64_t batch,
                            int64_t dim, int64_t W, int64_t seqlen, int64_t c_begin,
                            int64_t c_end, double* dx, double* dw, double* dcb) {
  (void)batch;
  for (int64_t c = c_begin; c < c_end; ++c) {
    int64_t b = c / dim, d = c % dim;
    const unsigned char* reset_b = reset ? reset + b * seqlen : NULL;
    const double* x_r = x + c * seqlen;
    for (int64_t t = 0; t < seqlen; ++t) dx[c * seqlen + t] = 0.0;
    for (int64_t t = 0; t < seqlen; ++t) {
      double pre = conv_pre(x_r, w + d * W, cb ? cb[d] : 0.0, W, reset_b, t);
      double sg = sigmoid(pre);
      double dpre = du[c * seqlen + t] * sg * (1.0 + pre * (1.0 - sg));
      for (int64_t k = 0; k < W; ++k) {
        int64_t s = t - (W - 1) + k;
        if (!conv_tap_valid(reset_b, s, t)) continue;
        dx[c * seqlen + s] += w[d * W + k] * dpre;
        dw[d * W + k] += dpre * x_r[s];
      }
      if (dcb) dcb[d] += dpre;
    }
  }
}

/*
 * Complex-valued variant: diagonal A, B, C and the state h complex (the
 * S4D-Lin parameterization A_n = -1/2 + i*pi*n of [SUM-3.4] "Real vs.
 * Complex", used by the paper for audio [ESSAY] Part III).  The pages fix no
 * output convention for a complex state; the reading taken here is
 *   y_t = Re( sum_n C[b,n,t] * h_t[n] ) + D[d] * u_t,  out = y * SiLU(z)
 * with Abar = exp(dt*A) and Bbar = (Abar - 1)/A * B (ZOH; limit dt*B at A = 0)
 * or dt*B (Euler), all complex.  Complex arrays are interleaved (re, im)
 * pairs: A (dim, dstate), B and C (batch, dstate, seqlen), h0 and last_state
 * (batch, dim, dstate).  u, delta, z, D, bias and out are real.  Reset flags
 * (nullable) act as in the real forward: the state entering a flagged step is
 * zero.
 */
static double complex cload(const double* p, int64_t i) { return p[2 * i] + I * p[2 * i + 1]; }

static double complex cbbar_coef(double dt, double complex a, int disc) {
  if (disc == ORACLE_EULER) return dt;
  if (a == 0.0) return dt;
  return (cexp(dt * a) - 1.0) / a;
}

void oracle_scan_fwd_complex(const double* u, const double* delta, const double* A,
                             const double* B, const double* C, const double* D, const double* z,
                             const double* bias, const double* h0, const unsigned char* reset,
                             int softplus_on, int disc, int64_t batch, int64_t dim,
                             int64_t dstate, int64_t seqlen, int64_t c_begin, int64_t c_end,
                             double* out, double* last_state) {
  (void)batch;
  double complex* h = (double complex*)malloc(sizeof(double complex) * (size_t)dstate);
  for (int64_t c = c_begin; c < c_end; ++c) {
    int64_t b = c / dim, d = c % dim;
    for (int64_t n = 0; n < dstate; ++n) h[n] = h0 ? cload(h0, c * dstate + n) : 0.0;
    for (int64_t t = 0; t < seqlen; ++t) {
      double dt = step_size(delta[c * seqlen + t], bias, d, softplus_on);
      double ut = u[c * seqlen + t];
      double y = 0.0;
      if (reset && reset[b * seqlen + t])
        for (int64_t n = 0; n < dstate; ++n) h[n] = 0.0;
      for (int64_t n = 0; n < dstate; ++n) {
        double complex a = cload(A, d * dstate + n);
        double complex abar = cexp(dt * a);
        double complex bbar = cbbar_coef(dt, a, disc) * cload(B, (b * dstate + n) * seqlen + t);
        h[n] = abar * h[n] + bbar * ut;
        y += creal(cload(C, (b * dstate + n) * seqlen + t) * h[n]);
      }
      if (D) y += D[d] * ut;
      if (z) y = y * (z[c * seqlen + t] * sigmoid(z[c * seqlen + t]));
      out[c * seqlen + t] = y;
    }
    if (last_state)
      for (int64_t n = 0; n < dstate; ++n) {
        last_state[2 * (c * dstate + n)] = creal(h[n]);
        last_state[2 * (c * dstate + n) + 1] = cimag(h[n]);
      }
  }
  free(h);
}

/*
 * Backward of the complex forward above for L = sum(dout * out), by the
 * chain rule with the gradient of a complex variable w written
 * g_w = dL/dRe(w) + i dL/dIm(w):
 *   y = Re(C h)          -> g_h += conj(C) gy,  g_C = gy conj(h)
 *   h_t = Abar h_{t-1} + beta -> g_{h_{t-1}} += conj(Abar) g_h,
 *                               g_Abar = g_h conj(h_{t-1}),  g_beta = g_h
 *   Abar = exp(dt A)     -> d/ddt: A Abar;   d/dA: dt Abar
 *   beta = E B u, E = (Abar - 1)/A (ZOH) or dt (Euler)
 *                        -> dE/ddt = Abar (ZOH) or 1;  dE/dA = (dt Abar - E)/A (ZOH,
 *                           limit dt^2/2 at A = 0) or 0
 * A real variable x gets Re(conj(g_w) dw/dx); a complex one conj(dw/dx) g_w
 * (the maps are holomorphic in A).  dA, dB, dC, dh0 are complex and
 * accumulated with +=, like dD, ddelta_bias; du, ddelta, dz are written.
 * With reset flags the state entering a flagged step is zero: its h_{t-1}
 * counts as 0 and no adjoint passes back across the step.
 */
void oracle_scan_bwd_complex(const double* u, const double* delta, const double* A,
                             const double* B, const double* C, const double* D, const double* z,
                             const double* bias, const double* h0, const double* dout,
                             const unsigned char* reset,
                             int softplus_on, int disc, int64_t batch, int64_t dim, int64_t dstate,
                             int64_t seqlen, int64_t c_begin, int64_t c_end, double* du,
                             double* ddelta, double* dA, double* dB, double* dC, double* dD,
                             double* dz, double* ddelta_bias, double* dh0) {
  (void)batch;
  double complex* hs = (double complex*)malloc(sizeof(double complex) * (size_t)((seqlen + 1) * dstate));
  double complex* gh = (double complex*)malloc(sizeof(double complex) * (size_t)dstate);
  for (int64_t c = c_begin; c < c_end; ++c) {
    int64_t b = c / dim, d = c % dim;
    for (int64_t n = 0; n < dstate; ++n) hs[n] = h0 ? cload(h0, c * dstate + n) : 0.0;
    for (int64_t t = 0; t < seqlen; ++t) {
      double dt = step_size(delta[c * seqlen + t], bias, d, softplus_on);
      int rs = reset && reset[b * seqlen + t];
      for (int64_t n = 0; n < dstate; ++n) {
        double complex a = cload(A, d * dstate + n);
        double complex bbar = cbbar_coef(dt, a, disc) * cload(B, (b * dstate + n) * seqlen + t);
        double complex hprev = rs ? 0.0 : hs[t * dstate + n];
        hs[(t + 1) * dstate + n] = cexp(dt * a) * hprev + bbar * u[c * seqlen + t];
      }
    }
    for (int64_t n = 0; n < dstate; ++n) gh[n] = 0.0;
    for (int64_t t = seqlen - 1; t >= 0; --t) {
      double r = delta[c * seqlen + t] + (bias ? bias[d] : 0.0);
      double dt = softplus_on ? softplus(r) : r;
      double ut = u[c * seqlen + t];
      double y = 0.0;
      for (int64_t n = 0; n < dstate; ++n)
        y += creal(cload(C, (b * dstate + n) * seqlen + t) * hs[(t + 1) * dstate + n]);
      if (D) y += D[d] * ut;
      double gy = dout[c * seqlen + t];
      if (z) {
        double zt = z[c * seqlen + t], sg = sigmoid(zt);
        gy = dout[c * seqlen + t] * (zt * sg);
        dz[c * seqlen + t] = dout[c * seqlen + t] * y * sg * (1.0 + zt * (1.0 - sg));
      }
      double du_t = D ? gy * D[d] : 0.0;
      if (D) dD[d] += gy * ut;
      double gdt = 0.0;
      int rs = reset && reset[b * seqlen + t];
      for (int64_t n = 0; n < dstate; ++n) {
        int64_t k = (b * dstate + n) * seqlen + t;
        double complex a = cload(A, d * dstate + n);
        double complex abar = cexp(dt * a);
        double complex Bv = cload(B, k), Cv = cload(C, k);
        double complex E = cbbar_coef(dt, a, disc);
        double complex hprev = rs ? 0.0 : hs[t * dstate + n], hcur = hs[(t + 1) * dstate + n];
        gh[n] += conj(Cv) * gy;                       /* g_h_t */
        double complex gC = gy * conj(hcur);
        dC[2 * k] += creal(gC);
        dC[2 * k + 1] += cimag(gC);
        double complex gAbar = gh[n] * conj(hprev);
        double complex gbeta = gh[n];
        double complex dE_ddt = (disc == ORACLE_EULER) ? 1.0 : abar;
        double complex dE_dA;
        if (disc == ORACLE_EULER) dE_dA = 0.0;
        else if (a == 0.0) dE_dA = dt * dt / 2.0;
        else dE_dA = (dt * abar - E) / a;
        gdt += creal(conj(gAbar) * a * abar) + creal(conj(gbeta) * dE_ddt * Bv * ut);
        du_t += creal(conj(gbeta) * E * Bv);
        double complex gB = conj(E * ut) * gbeta;
        dB[2 * k] += creal(gB);
        dB[2 * k + 1] += cimag(gB);
        double complex gA = conj(dt * abar) * gAbar + conj(dE_dA * Bv * ut) * gbeta;
        dA[2 * (d * dstate + n)] += creal(gA);
        dA[2 * (d * dstate + n) + 1] += cimag(gA);
        gh[n] = rs ? 0.0 : conj(abar) * gh[n];        /* carry to t-1 (none across a reset) */
      }
      du[c * seqlen + t] = du_t;
      double gr = softplus_on ? gdt * sigmoid(r) : gdt;
      ddelta[c * seqlen + t] = gr;
      if (ddelta_bias) ddelta_bias[d] += gr;
    }
    if (dh0)
      for (int64_t n = 0; n < dstate; ++n) {
        dh0[2 * (c * dstate + n)] += creal(gh[n]);
        dh0[2 * (c * dstate + n) + 1] += cimag(gh[n]);
      }
  }
  free(hs);
  free(gh);
}

int oracle_version(void) { return 6; }
