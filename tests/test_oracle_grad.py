"""Pins of the float64 oracle's backward against central finite differences
of its forward (a different computation: only forward evaluations).

The pages give no gradient formulas; they only say the backward recomputes
the states from the inputs (paper-graph-ui.vercel.app summary, section 3.4
"Recomputation for the backward pass"; chapterpal.com page, Knowl 2 item 2).
The oracle's adjoint is the chain rule of its forward, and these tests check
every gradient it returns, on tiny shapes, for both discretizations, with the
softplus on and off, with and without the optional D, z, delta_bias and
initial state, and at A = 0 (the ZOH limit).
"""
import numpy as np
import pytest

import oracle

NAMES = ["u", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0"]
GRAD = dict(u="du", delta="ddelta", A="dA", B="dB", C="dC", D="dD", z="dz",
            delta_bias="ddelta_bias", h0="dh0")


def make(seed, batch=2, dim=3, N=3, L=10, with_D=True, with_z=True, with_bias=True, with_h0=False,
         zero_A=False):
    g = np.random.default_rng(seed)
    p = dict(u=g.standard_normal((batch, dim, L)), delta=g.standard_normal((batch, dim, L)),
             A=-np.exp(g.standard_normal((dim, N))), B=g.standard_normal((batch, N, L)),
             C=g.standard_normal((batch, N, L)),
             D=g.standard_normal(dim) if with_D else None,
             z=g.standard_normal((batch, dim, L)) if with_z else None,
             delta_bias=g.standard_normal(dim) * 0.5 - 1.0 if with_bias else None,
             h0=g.standard_normal((batch, dim, N)) if with_h0 else None)
    if zero_A:
        p["A"][0, 0] = 0.0
    return p, g.standard_normal((batch, dim, L))


def loss(p, dout, softplus_on, disc):
    out, _ = oracle.scan_fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"],
                             p["delta_bias"], p["h0"], delta_softplus=softplus_on, disc=disc,
                             threads=1, return_last_state=False, reset=p.get("reset"))
    return float(np.sum(out * dout))


def fd_grad(p, dout, name, softplus_on, disc):
    x = p[name]
    g = np.zeros_like(x)
    flat = x.reshape(-1)
    gf = g.reshape(-1)
    for i in range(flat.size):
        old = flat[i]
        h = 1e-6 * max(1.0, abs(old))
        flat[i] = old + h
        lp = loss(p, dout, softplus_on, disc)
        flat[i] = old - h
        lm = loss(p, dout, softplus_on, disc)
        flat[i] = old
        gf[i] = (lp - lm) / (2 * h)
    return g


CASES = [
    # (disc, softplus, D, z, bias, h0, zero_A)
    (oracle.ZOH, True, True, True, True, False, False),
    (oracle.ZOH, False, True, True, True, False, False),
    (oracle.EULER, True, True, True, True, False, False),
    (oracle.EULER, False, False, False, False, False, False),
    (oracle.ZOH, True, False, False, False, True, False),
    (oracle.ZOH, True, True, True, True, True, True),
]


@pytest.mark.parametrize("case", CASES)
def test_backward_matches_central_differences(case):
    disc, sp, wD, wz, wb, wh, zA = case
    p, dout = make(hash(case) % 1000, with_D=wD, with_z=wz, with_bias=wb, with_h0=wh, zero_A=zA)
    if not sp:
        p["delta"] = np.abs(p["delta"]) + 0.05   # keep the step positive without softplus
        if p["delta_bias"] is not None:
            p["delta_bias"] = np.abs(p["delta_bias"]) * 0.1
    g = oracle.scan_bwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"],
                        p["delta_bias"], dout, p["h0"], delta_softplus=sp, disc=disc, threads=2)
    for name in NAMES:
        if p[name] is None:
            assert GRAD[name] not in g
            continue
        ref = fd_grad(p, dout, name, sp, disc)
        got = g[GRAD[name]]
        scale = max(1.0, np.abs(ref).max())
        np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-6 * scale, err_msg=name)


def test_backward_thread_split_is_consistent():
    p, dout = make(77, batch=3, dim=4, N=2, L=12, with_h0=True)
    g1 = oracle.scan_bwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"],
                         p["delta_bias"], dout, p["h0"], threads=1)
    g5 = oracle.scan_bwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"],
                         p["delta_bias"], dout, p["h0"], threads=5)
    for k in g1:
        np.testing.assert_allclose(g1[k], g5[k], rtol=1e-13, atol=1e-14, err_msg=k)


@pytest.mark.parametrize("disc", [oracle.ZOH, oracle.EULER])
def test_backward_with_resets_matches_central_differences(disc):
    # packed sequences: flags at t = 0 (the initial state is discarded) for the
    # first batch row, and mid-sequence (including two adjacent steps) in both
    p, dout = make(91 + disc, L=12, with_h0=True)
    reset = np.zeros((2, 12), np.uint8)
    reset[0, [0, 5]] = 1
    reset[1, [3, 4, 9]] = 1
    p["reset"] = reset
    g = oracle.scan_bwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"],
                        p["delta_bias"], dout, p["h0"], disc=disc, threads=2, reset=reset)
    assert np.all(g["dh0"][0] == 0.0)       # row 0 resets before its first step
    for name in NAMES:
        ref = fd_grad(p, dout, name, True, disc)
        got = g[GRAD[name]]
        scale = max(1.0, np.abs(ref).max())
        np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-6 * scale, err_msg=name)
