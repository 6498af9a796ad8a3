"""Pins of the float64 oracle's short causal convolution + SiLU (the stage
that feeds the selective SSM in the Mamba block: chapterpal.com page,
Knowl 3 "Mamba Block Architecture", a width-4 temporal convolution then
SiLU; trishampatil essay, Part II §8, the same block as a diagram).

The forward is checked against numpy's own convolution and against the
identity kernel (u = SiLU(x)); packed sequences against per-segment runs;
the backward against central finite differences of the forward.
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle


def _inputs(seed, batch=2, dim=3, L=30, W=4):
    g = np.random.default_rng(seed)
    return (g.standard_normal((batch, dim, L)), g.standard_normal((dim, W)),
            g.standard_normal(dim))


@pytest.mark.parametrize("W", [1, 2, 3, 4])
def test_forward_equals_numpy_causal_convolution(W):
    x, w, cb = _inputs(1, W=W)
    u = oracle.conv1d_silu_fwd(x, w, cb)
    for b in range(x.shape[0]):
        for d in range(x.shape[1]):
            # full convolution with the reversed taps, cut to the first L
            # outputs: step t sees x[t-W+1 .. t], zeros before t = 0
            pre = np.convolve(x[b, d], w[d, ::-1])[: x.shape[2]] + cb[d]
            np.testing.assert_allclose(u[b, d], pre * expit(pre), rtol=1e-13, atol=1e-14)


def test_identity_kernel_is_plain_silu():
    x, _, _ = _inputs(2)
    w = np.zeros((3, 4))
    w[:, 3] = 1.0
    u = oracle.conv1d_silu_fwd(x, w, None)
    np.testing.assert_allclose(u, x * expit(x), rtol=1e-15, atol=0)


def test_resets_restart_the_convolution():
    x, w, cb = _inputs(3, L=40)
    reset = np.zeros((2, 40), np.uint8)
    reset[0, [0, 5, 6, 20]] = 1
    reset[1, [1, 39]] = 1
    u = oracle.conv1d_silu_fwd(x, w, cb, reset=reset)
    for b in range(2):
        starts = [0] + [t for t in range(1, 40) if reset[b, t]]
        for s, e in zip(starts, starts[1:] + [40]):
            seg = oracle.conv1d_silu_fwd(x[b:b + 1, :, s:e], w, cb)
            np.testing.assert_array_equal(u[b, :, s:e], seg[0])


def _fd(f, x, eps=1e-6):
    g = np.zeros_like(x)
    flat, gf = x.reshape(-1), g.reshape(-1)
    for i in range(flat.size):
        old = flat[i]
        h = eps * max(1.0, abs(old))
        flat[i] = old + h
        lp = f()
        flat[i] = old - h
        lm = f()
        flat[i] = old
        gf[i] = (lp - lm) / (2 * h)
    return g


@pytest.mark.parametrize("W,with_reset", [(4, False), (4, True), (3, True), (1, False)])
def test_backward_matches_central_differences(W, with_reset):
    x, w, cb = _inputs(4 + W, L=14, W=W)
    du = np.random.default_rng(9).standard_normal(x.shape)
    reset = None
    if with_reset:
        reset = np.zeros((2, 14), np.uint8)
        reset[0, [0, 4, 5]] = 1
        reset[1, [9]] = 1

    def loss():
        return float(np.sum(du * oracle.conv1d_silu_fwd(x, w, cb, reset=reset)))

    g = oracle.conv1d_silu_bwd(x, w, cb, du, reset=reset)
    for name, arr in (("dx", x), ("dw", w), ("dcb", cb)):
        ref = _fd(loss, arr)
        scale = max(1.0, np.abs(ref).max())
        np.testing.assert_allclose(g[name], ref, rtol=1e-6, atol=1e-6 * scale, err_msg=name)
    assert "dcb" not in oracle.conv1d_silu_bwd(x, w, None, du, reset=reset)
