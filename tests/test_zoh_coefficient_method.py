"""CPU check of the method the kernels use for the ZOH coefficient and its
A-derivative (device_common.hpp: expm1_zoh, zoh_coef_neg, dcoef_dA), by
emulating their float32 arithmetic in numpy: each fma rounds once to
float32, and the hardware exponential's result is perturbed by up to 0.78
ulp either way (the accuracy measured for v_exp_f32 on gfx950).  The
coefficient is (e^x - 1)/A with x = delta A (chapterpal.com page, Knowl 1
"Selective State Space Layer (S6)", step 3); the references are float64
expm1 and the float64 closed form / series of psi.  This pins the error
bounds the kernels' comments state, not the kernels themselves (the GPU
parity tests do that)."""
import numpy as np

F = np.float32
LOG2E = F(1.4426950408889634)
LN2 = F(0.6931471805599453)
C2, C3 = F(0.24022650695910071), F(0.05550410866482158)       # ln2^2/2, ln2^3/6
K2, K3 = F(0.34657359027997264), F(0.08007550231970023)       # ln2/2, ln2^2/6
P1, P2, P3 = F(0.23104906018664844), F(0.06005662673977518), F(0.01110082173296432)
EXP_BOUND = F(1.0 + 2.0 ** -23)
COEF_BOUND = F(1.0 + 2.0 ** -22)
PSI_Z = F(0.11 / 0.6931471805599453)


def fma(a, b, c):
    # the product of two float32 is exact in float64; one rounding to float32
    return (np.float64(a) * np.float64(b) + np.float64(c)).astype(F)


def mul(a, b):
    return (np.float64(a) * np.float64(b)).astype(F)


def hw_exp2(z, sign):
    """The float32 farthest from 2^z, above (sign +1) or below (-1), that is
    still within 0.78 ulp of it: the worst results the hardware may return."""
    e = np.exp2(np.float64(z))
    ulp = np.spacing(e.astype(F)).astype(np.float64)
    v = e + sign * 0.78 * ulp
    f = v.astype(F)
    if sign > 0:   # round v down
        f = np.where(np.float64(f) > v, np.nextafter(f, F(-np.inf)), f)
    else:          # round v up
        f = np.where(np.float64(f) < v, np.nextafter(f, F(np.inf)), f)
    return f


def grid():
    dts = np.logspace(-8, 2, 400)
    As = np.array([-1e-3, -0.05, -0.5, -1.0, -3.0, -16.0, -250.0])
    d, a = np.meshgrid(dts, As)
    return d.ravel().astype(F), a.ravel().astype(F)


def test_coef_for_negative_A_within_bound():
    dt, A = grid()
    x = np.float64(dt) * np.float64(A)
    keep = x > -80.0                       # e^x representable above the float32 subnormals
    dt, A, x = dt[keep], A[keep], x[keep]
    ref = np.expm1(x) / np.float64(A)
    worst = 0.0
    for sign in (-1.0, 1.0):
        z = mul(dt, A * LOG2E)             # the kernels multiply by a2 = A log2(e)
        abar = hw_exp2(z, sign)
        ia = (1.0 / np.float64(A)).astype(F)
        mb = mul(ia, -COEF_BOUND)
        poly = mul(dt, fma(z, fma(z, K3, K2), F(1.0)))
        coef = np.minimum(poly, fma(abar, ia, mb))
        rel = np.abs(np.float64(coef) - ref) / np.abs(ref)
        worst = max(worst, rel.max())
    assert worst < 8e-6, worst          # zoh_coef_neg's comment: below about 8e-6


def test_expm1_any_sign_within_bound():
    xs = np.concatenate([-np.logspace(-8, 1.5, 500), np.logspace(-8, 1.5, 500)])
    worst = 0.0
    for sign in (-1.0, 1.0):
        z = (xs * 1.4426950408889634).astype(F)
        abar = hw_exp2(z, sign)
        poly = mul(z, fma(z, fma(z, C3, C2), LN2))
        em1 = np.maximum(poly, (np.float64(abar) - np.float64(EXP_BOUND)).astype(F))
        ref = np.expm1(np.float64(z) * 0.6931471805599453)
        rel = np.abs(np.float64(em1) - ref) / np.abs(ref)
        worst = max(worst, rel.max())
    assert worst < 5e-6, worst          # expm1_zoh's comment: within about 5e-6


def test_coef_derivative_within_bound():
    dt, A = grid()
    x64 = np.float64(dt) * np.float64(A)
    keep = x64 > -80.0
    dt, A = dt[keep], A[keep]
    worst = 0.0
    for sign in (-1.0, 1.0):
        z = mul(dt, A * LOG2E)
        x = np.float64(z) * 0.6931471805599453    # the x the kernel's z stands for
        abar = hw_exp2(z, sign)
        dt2 = mul(dt, dt)
        iA2 = (1.0 / (np.float64(A) * np.float64(A))).astype(F)
        series = mul(dt2, fma(z, fma(z, fma(z, P3, P2), P1), F(0.5)))
        closed = mul(fma(abar, fma(z, LN2, F(-1.0)), F(1.0)), iA2)
        zeta = np.where(np.abs(z) < PSI_Z, series, closed)
        # reference: dt^2 psi(x) at the same x, psi from its series where it
        # converges fast and from the closed form (in float64) elsewhere
        small = np.abs(x) < 1e-2
        psi = np.where(small, 0.5 + x / 3 + x * x / 8 + x ** 3 / 30 + x ** 4 / 144,
                       (np.exp(x) * (x - 1) + 1) / np.where(small, 1.0, x * x))
        ref = np.float64(dt) ** 2 * psi
        rel = np.abs(np.float64(zeta) - ref) / np.abs(ref)
        worst = max(worst, rel.max())
    # dcoef_dA's comment: the series within about 2e-6 below |x| = 0.11, the
    # closed form within about 2e-7/x^2 above (1.65e-5 at 0.11)
    assert worst < 1.7e-5, worst
