"""CPU check of the method the complex kernels use for the ZOH coefficient
and its A-derivative (complex_common.hpp: cexp_expm1_scaled, cdcoef_dA), by
emulating their float32 arithmetic in numpy, as
test_zoh_coefficient_method.py does for real A: every fma and multiply
rounds once to float32, the hardware exponential is off by up to 0.78 ulp
either way, the hardware sine (which takes revolutions) by up to 8.9e-7
relative and the cosine by up to 1.3e-7 absolute, the accuracies measured
for v_exp_f32, v_sin_f32 and v_cos_f32 on gfx950.  With x = delta A,
A = ar + i ai, the coefficient's numerator is e^x - 1 (chapterpal.com
page, Knowl 1 "Selective State Space Layer (S6)", step 3), its derivative
delta^2 psi(x), psi(x) = (x e^x - e^x + 1)/x^2; the references are float64
complex expm1 (written without cancellation) and psi.  This pins the
accuracy the kernels' comments state, not the kernels (the GPU parity tests
do that)."""
import numpy as np

from test_zoh_coefficient_method import F, fma, hw_exp2, mul

LOG2E = F(1.4426950408889634)
INV2PI = F(0.15915494309189535)
C2, C3, LN2 = F(0.24022650695910071), F(0.05550410866482158), F(0.6931471805599453)
EXP_BOUND = F(1.0 + 2.0 ** -23)
KCOS2, KCOS4, KCOS6 = F(19.739208802178716), F(64.939394022668291), F(85.456817206693722)
COS_BOUND = F(1.0 + 2.0 ** -22)
SIN_REL, COS_ABS = 8.9e-7, 1.3e-7


def hw_sin(rev, sign):
    s = np.sin(2 * np.pi * np.float64(rev))
    return (s * (1 + sign * SIN_REL)).astype(F)


def hw_cos(rev, sign):
    return np.clip(np.cos(2 * np.pi * np.float64(rev)) + sign * COS_ABS, -1, 1).astype(F)


def grid():
    dts = np.logspace(-6, 0.5, 120)
    ars = np.array([-1e-3, -0.05, -0.5, -2.0, -10.0])
    ais = np.array([0.0, 1e-3, 0.3, np.pi, 2 * np.pi * 3, 40.0])
    d, r, i = np.meshgrid(dts, ars, ais)
    return d.ravel().astype(F), r.ravel().astype(F), i.ravel().astype(F)


def ref_expm1(xr, xi):
    # e^x - 1 = (expm1(xr) cos xi - 2 sin^2(xi/2)) + i e^xr sin xi, no cancellation
    re = np.expm1(xr) * np.cos(xi) - 2 * np.sin(xi / 2) ** 2
    return re + 1j * np.exp(xr) * np.sin(xi)


def emulated_expm1(dt, ar, ai, se, ss, sc):
    ar2, air = mul(ar, LOG2E), mul(ai, INV2PI)
    zr = mul(dt, ar2)
    mag = hw_exp2(zr, se)
    rev = mul(dt, air)
    co, si = hw_cos(rev, sc), hw_sin(rev, ss)
    w = mul(rev, rev)
    cm1 = np.maximum(mul(w, fma(w, fma(w, -KCOS6, KCOS4), -KCOS2)),
                     (np.float64(co) - np.float64(COS_BOUND)).astype(F))
    poly = mul(zr, fma(zr, fma(zr, C3, C2), LN2))
    em1r = np.maximum(poly, (np.float64(mag) - np.float64(EXP_BOUND)).astype(F))
    re = fma(em1r, co, cm1)
    im = mul(mag, si)
    # the float64 x the kernel's rounded arguments stand for
    x = np.float64(zr) * np.log(2) + 1j * np.float64(rev) * 2 * np.pi
    return re, im, x, mag, co, si


def test_cos_minus_one_within_bound():
    rev = np.concatenate([np.logspace(-8, -0.3, 400), -np.logspace(-8, -0.3, 400)]).astype(F)
    worst = 0.0
    for sc in (-1.0, 1.0):
        co = hw_cos(rev, sc)
        w = mul(rev, rev)
        cm1 = np.maximum(mul(w, fma(w, fma(w, -KCOS6, KCOS4), -KCOS2)),
                         (np.float64(co) - np.float64(COS_BOUND)).astype(F))
        ref = -2 * np.sin(np.pi * np.float64(rev)) ** 2
        worst = max(worst, (np.abs(np.float64(cm1) - ref) / np.abs(ref)).max())
    assert worst < 3e-6, worst          # the comment: below about 3e-6


def test_complex_expm1_within_bound():
    dt, ar, ai = grid()
    worst = 0.0
    for se in (-1.0, 1.0):
        for ss in (-1.0, 1.0):
            for sc in (-1.0, 1.0):
                re, im, *_ = emulated_expm1(dt, ar, ai, se, ss, sc)
                x = np.float64(dt) * (np.float64(ar) + 1j * np.float64(ai))   # exact dt A
                ref = ref_expm1(x.real, x.imag)
                got = np.float64(re) + 1j * np.float64(im)
                keep = np.abs(ref) > 0
                worst = max(worst, (np.abs(got - ref)[keep] / np.abs(ref)[keep]).max())
    # each part to its own bound (expm1 5e-6, cos - 1 3e-6, sin 9e-7), with
    # the roundings of the arguments, the products and the fma
    assert worst < 6e-6, worst


def psi_ref(x):
    small = np.abs(x) < 1e-2
    xs = np.where(small, 1.0, x)
    closed = (np.exp(xs) * (xs - 1) + 1) / (xs * xs)
    series = 0.5 + x / 3 + x * x / 8 + x ** 3 / 30 + x ** 4 / 144
    return np.where(small, series, closed)


def test_complex_coef_derivative_within_bound():
    dt, ar, ai = grid()
    keep = np.float64(dt) * np.abs(np.float64(ar)) < 60
    dt, ar, ai = dt[keep], ar[keep], ai[keep]
    worst = 0.0
    for se in (-1.0, 1.0):
        for ss in (-1.0, 1.0):
            for sc in (-1.0, 1.0):
                re, im, _, mag, co, si = emulated_expm1(dt, ar, ai, se, ss, sc)
                abr, abi = mul(mag, co), mul(mag, si)
                ia = 1.0 / (np.float64(ar) + 1j * np.float64(ai))
                iar, iai = ia.real.astype(F), ia.imag.astype(F)
                # the replay's coefficient, coef = (e^x - 1) / A
                cr, ci = fma(re, iar, -mul(im, iai)), fma(re, iai, mul(im, iar))
                # cdcoef_dA, with x = dt A formed in float32
                xr, xi = mul(ar, dt), mul(ai, dt)
                wr = fma(xr, F(1.0 / 30.0), F(0.125))
                wi = mul(xi, F(1.0 / 30.0))
                wr, wi = fma(xr, wr, -mul(xi, wi)), fma(xr, wi, mul(xi, wr))
                wr = (np.float64(wr) + np.float64(F(1.0 / 3.0))).astype(F)
                wr, wi = fma(xr, wr, -mul(xi, wi)), fma(xr, wi, mul(xi, wr))
                wr = (np.float64(wr) + 0.5).astype(F)
                d2 = mul(dt, dt)
                sr, si_ = mul(wr, d2), mul(wi, d2)
                # above the threshold: (dt Abar - coef) / A
                tr, ti = fma(dt, abr, -cr), fma(dt, abi, -ci)
                kr, ki = fma(tr, iar, -mul(ti, iai)), fma(tr, iai, mul(ti, iar))
                small = fma(xr, xr, mul(xi, xi)) < F(0.0289)
                zr = np.where(small, sr, kr)
                zi = np.where(small, si_, ki)
                x = np.float64(dt) * (np.float64(ar) + 1j * np.float64(ai))   # exact dt A
                ref = np.float64(dt) ** 2 * psi_ref(x)
                got = np.float64(zr) + 1j * np.float64(zi)
                worst = max(worst, (np.abs(got - ref) / np.abs(ref)).max())
    # cdcoef_dA's comment: about 1.5e-5 (the series' truncation, at most
    # 1.2e-5 of psi below |x| = 0.17; above, the coefficient's error grown
    # by at most about 2/|x|)
    assert worst < 1.6e-5, worst
