"""Pins of the float64 oracle's complex-valued forward (diagonal complex A,
B, C and state, as in the S4D-Lin parameterization that the paper-graph-ui
summary prints as A_n = -1/2 + n i (section 5, Table 8 discussion) and
names for audio in section 3.4 "Real vs. Complex"; the pins below draw
imaginary parts of several scales), with the reading
y = Re(sum_n C h) + D u.

Pinned against: the real oracle when every imaginary part is zero; an
independent numpy brute-force convolution with the complex kernel
Re(C Abar^k Bbar) when delta, B, C are constant along t; and the
conjugate-pair identity (a pair (a, conj a) gives twice the real part of one).
The complex backward is pinned to central differences of the forward, in
the real and the imaginary direction of every complex input.  Reset flags
(packed sequences) are pinned by splitting: a packed run equals independent
runs of its pieces, forward and backward.
"""
import numpy as np
import pytest

import oracle


def _inputs(seed, batch=2, dim=3, N=4, L=40):
    g = np.random.default_rng(seed)
    A = -0.5 * np.ones((dim, N)) + 1j * np.pi * np.arange(N)[None, :] * (1 + 0.1 * g.random((dim, 1)))
    cplx = lambda *s: g.standard_normal(s) + 1j * g.standard_normal(s)
    return dict(u=g.standard_normal((batch, dim, L)), delta=g.standard_normal((batch, dim, L)),
                A=A, B=cplx(batch, N, L), C=cplx(batch, N, L), D=g.standard_normal(dim),
                z=g.standard_normal((batch, dim, L)), delta_bias=g.standard_normal(dim) - 1.0,
                h0=cplx(batch, dim, N))


@pytest.mark.parametrize("disc", [oracle.ZOH, oracle.EULER])
def test_real_parts_only_equal_the_real_oracle(disc):
    p = _inputs(1)
    p["A"] = -np.exp(np.random.default_rng(2).standard_normal(p["A"].shape)) + 0j
    for k in ("B", "C", "h0"):
        p[k] = p[k].real + 0j
    out, last = oracle.scan_fwd_complex(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"],
                                        p["z"], p["delta_bias"], p["h0"], disc=disc)
    ro, rl = oracle.scan_fwd(p["u"], p["delta"], p["A"].real, p["B"].real, p["C"].real, p["D"],
                             p["z"], p["delta_bias"], p["h0"].real, disc=disc)
    np.testing.assert_allclose(out, ro, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(last.real, rl, rtol=1e-13, atol=1e-13)
    assert np.all(last.imag == 0.0)


@pytest.mark.parametrize("disc", [oracle.ZOH, oracle.EULER])
@pytest.mark.parametrize("softplus", [True, False])
def test_constant_parameters_equal_complex_kernel_convolution(disc, softplus):
    g = np.random.default_rng(3)
    batch, dim, N, L = 1, 2, 3, 30
    p = _inputs(4, batch, dim, N, L)
    dt_raw = g.random((batch, dim, 1)) + 0.1 if not softplus else g.standard_normal((batch, dim, 1))
    delta = np.repeat(dt_raw, L, axis=2)
    Bc = np.repeat(p["B"][:, :, :1], L, axis=2)
    Cc = np.repeat(p["C"][:, :, :1], L, axis=2)
    out, _ = oracle.scan_fwd_complex(p["u"], delta, p["A"], Bc, Cc, p["D"], None, None, None,
                                     delta_softplus=softplus, disc=disc)
    for d in range(dim):
        dt = np.log1p(np.exp(dt_raw[0, d, 0])) if softplus else dt_raw[0, d, 0]
        a = p["A"][d]
        abar = np.exp(dt * a)
        bbar = ((abar - 1) / a if disc == oracle.ZOH else dt) * Bc[0, :, 0]
        K = np.array([np.real(np.sum(Cc[0, :, 0] * abar ** k * bbar)) for k in range(L)])
        x = p["u"][0, d]
        y = np.array([np.sum(K[:t + 1][::-1] * x[:t + 1]) for t in range(L)]) + p["D"][d] * x
        np.testing.assert_allclose(out[0, d], y, rtol=1e-11, atol=1e-11)


def test_conjugate_pair_gives_twice_the_real_part():
    p = _inputs(5, N=1)
    pair = {k: p[k] for k in ("u", "delta", "delta_bias")}
    pair["A"] = np.concatenate([p["A"], np.conj(p["A"])], axis=1)
    pair["B"] = np.concatenate([p["B"], np.conj(p["B"])], axis=1)
    pair["C"] = np.concatenate([p["C"], np.conj(p["C"])], axis=1)
    pair["h0"] = np.concatenate([p["h0"], np.conj(p["h0"])], axis=2)
    one, l1 = oracle.scan_fwd_complex(p["u"], p["delta"], p["A"], p["B"], p["C"], None, None,
                                      p["delta_bias"], p["h0"])
    two, l2 = oracle.scan_fwd_complex(pair["u"], pair["delta"], pair["A"], pair["B"], pair["C"],
                                      None, None, pair["delta_bias"], pair["h0"])
    np.testing.assert_allclose(two, 2 * one, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l2[..., 1], np.conj(l1[..., 0]), rtol=1e-12, atol=1e-12)


def _loss(p, dout, disc, softplus):
    out, _ = oracle.scan_fwd_complex(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"],
                                     p["delta_bias"], p["h0"], delta_softplus=softplus,
                                     disc=disc, threads=1)
    return float(np.sum(out * dout))


def _fd(p, name, dout, disc, softplus, eps=1e-6):
    x = p[name]
    is_c = np.iscomplexobj(x)
    g = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        parts = [1.0, 1j] if is_c else [1.0]
        for unit in parts:
            old = x[idx]
            h = eps * max(1.0, abs(old))
            x[idx] = old + unit * h
            lp = _loss(p, dout, disc, softplus)
            x[idx] = old - unit * h
            lm = _loss(p, dout, disc, softplus)
            x[idx] = old
            g[idx] += unit * (lp - lm) / (2 * h)
    return g


GRADS = dict(u="du", delta="ddelta", A="dA", B="dB", C="dC", D="dD", z="dz",
             delta_bias="ddelta_bias", h0="dh0")


@pytest.mark.parametrize("disc,softplus", [(oracle.ZOH, True), (oracle.EULER, True),
                                           (oracle.ZOH, False)])
def test_complex_backward_matches_central_differences(disc, softplus):
    p = _inputs(6, batch=2, dim=2, N=3, L=9)
    if not softplus:
        p["delta"] = np.abs(p["delta"]) + 0.05
        p["delta_bias"] = np.abs(p["delta_bias"]) * 0.1
    dout = np.random.default_rng(7).standard_normal(p["u"].shape)
    g = oracle.scan_bwd_complex(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"],
                                p["delta_bias"], dout, p["h0"], delta_softplus=softplus,
                                disc=disc)
    for name, gname in GRADS.items():
        ref = _fd(p, name, dout, disc, softplus)
        scale = max(1.0, np.abs(ref).max())
        np.testing.assert_allclose(g[gname], ref, rtol=1e-6, atol=1e-6 * scale, err_msg=name)


def test_complex_backward_zero_A_limit():
    p = _inputs(8, batch=1, dim=2, N=2, L=6)
    p["A"][0, 0] = 0.0
    dout = np.random.default_rng(9).standard_normal(p["u"].shape)
    g = oracle.scan_bwd_complex(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"],
                                p["delta_bias"], dout, p["h0"])
    # (Abar - 1)/A near A = 0 has no complex expm1 in the forward: a wider
    # difference step keeps the rounding of the differences small
    ref = _fd(p, "A", dout, oracle.ZOH, True, eps=1e-4)
    np.testing.assert_allclose(g["dA"], ref, rtol=1e-5, atol=1e-6 * max(1, np.abs(ref).max()))


# ---------------------------------------------------------------------------
# Reset flags: the state entering a flagged step is zero, so a packed run is
# independent runs of its pieces (the first piece keeps the initial state
# unless it is itself reset).  Outputs and per-step gradients must match piece
# by piece; dA, dD, ddelta_bias are sums over the pieces.
# ---------------------------------------------------------------------------
def _pieces(row):
    starts = [0] + [t for t in range(1, row.size) if row[t]]
    return list(zip(starts, starts[1:] + [row.size]))


def _packed(seed):
    p = _inputs(seed)
    batch, _, L = p["u"].shape
    reset = np.zeros((batch, L), np.uint8)
    reset[0, [0, 7, 8, 30]] = 1          # a reset at t = 0 and two adjacent flags
    reset[1, [13, L - 1]] = 1            # a one-step final piece
    dout = np.random.default_rng(seed + 100).standard_normal(p["u"].shape)
    return p, reset, dout


def _piece(p, b, s, e):
    q = {}
    for k, v in p.items():
        if k in ("u", "delta", "z", "B", "C"):
            q[k] = v[b:b + 1, :, s:e]
        elif k == "h0":
            q[k] = v[b:b + 1]
        else:
            q[k] = v
    return q


@pytest.mark.parametrize("disc", [oracle.ZOH, oracle.EULER])
def test_complex_reset_forward_equals_independent_pieces(disc):
    p, reset, _ = _packed(31)
    out, last = oracle.scan_fwd_complex(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"],
                                        p["z"], p["delta_bias"], p["h0"], disc=disc, reset=reset)
    for b in range(reset.shape[0]):
        for i, (s, e) in enumerate(_pieces(reset[b])):
            q = _piece(p, b, s, e)
            h0 = q["h0"] if (i == 0 and not reset[b, 0]) else None
            o, l = oracle.scan_fwd_complex(q["u"], q["delta"], q["A"], q["B"], q["C"], q["D"],
                                           q["z"], q["delta_bias"], h0, disc=disc)
            np.testing.assert_array_equal(out[b, :, s:e], o[0])
        np.testing.assert_array_equal(last[b], l[0])


@pytest.mark.parametrize("disc", [oracle.ZOH, oracle.EULER])
def test_complex_reset_backward_equals_independent_pieces(disc):
    p, reset, dout = _packed(32)
    g = oracle.scan_bwd_complex(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"],
                                p["delta_bias"], dout, p["h0"], disc=disc, reset=reset)
    sums = dict(dA=0.0, dD=0.0, ddelta_bias=0.0)
    for b in range(reset.shape[0]):
        for i, (s, e) in enumerate(_pieces(reset[b])):
            q = _piece(p, b, s, e)
            first = i == 0 and not reset[b, 0]
            gs = oracle.scan_bwd_complex(q["u"], q["delta"], q["A"], q["B"], q["C"], q["D"],
                                         q["z"], q["delta_bias"], dout[b:b + 1, :, s:e],
                                         q["h0"] if first else None, disc=disc)
            for k in ("du", "ddelta", "dz"):
                np.testing.assert_array_equal(g[k][b, :, s:e], gs[k][0], err_msg=k)
            for k in ("dB", "dC"):
                np.testing.assert_allclose(g[k][b, :, s:e], gs[k][0], rtol=1e-12, atol=1e-13)
            for k in sums:
                sums[k] = sums[k] + gs[k]
            if i == 0:
                want = gs["dh0"][0] if first else np.zeros_like(g["dh0"][b])
                np.testing.assert_array_equal(g["dh0"][b], want)
    for k, v in sums.items():
        np.testing.assert_allclose(g[k], v, rtol=1e-12, atol=1e-12, err_msg=k)
