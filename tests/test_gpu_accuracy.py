"""GPU parity where float32 is fragile: small steps under ZOH.

With x = delta * A small, Abar = exp(x) rounds to within one float32 ulp of 1,
so a ZOH coefficient formed as (Abar - 1)/A keeps only a few significant
bits, and the dA term u dBbar/dA = u (delta Abar B - Bbar)/A is a difference
of two nearly equal quantities.  At a constant step such errors do not
average out: they add up along the whole recurrence.  These cases hold the
kernels to the float32 bound per row at delta = 1e-4 and 1e-3 (softplus off,
no bias, no D, no gate, so that nothing else dominates the outputs), forward
and backward, in one pass and in segments, real and complex.  The ZOH rule
is the chapterpal.com page's Knowl 1 "Selective State Space Layer (S6)",
step 3.
"""
import numpy as np
import pytest
import torch

import oracle
import scan_selective_fwd_amd as ms
import workloads as W
from parity_utils import RTOL_F32, announce, assert_match, to_device, to_f64

pytestmark = pytest.mark.gpu

SMALL = (1e-4, 1e-3)
SHAPE = (2, 20, 16, 2048)     # two channel groups (one partial), 16 chunks


def _const_step_inputs(wid, delta, batch, dim, N, L, with_dout=False):
    inp = W.make_inputs(wid, batch, dim, N, L, dtype="f32", with_D=False, with_z=False,
                        with_bias=False, with_dout=with_dout)
    inp["delta"] = np.full((batch, dim, L), delta, np.float32)
    return inp


@pytest.mark.parametrize("segments", [1, 4])
@pytest.mark.parametrize("delta", SMALL)
def test_small_step_fwd(delta, segments):
    batch, dim, N, L = SHAPE
    announce(f"small step fwd delta={delta} segments={segments} shape={SHAPE}")
    inp = _const_step_inputs(101, delta, batch, dim, N, L)
    f = W.inputs_f64(inp, "f32")
    g = to_device(inp, "f32")
    out, last = ms.scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], delta_softplus=False,
                            return_last_state=True, segments=segments)
    torch.cuda.synchronize()
    ref, ref_last = oracle.scan_fwd(f["u"], f["delta"], f["A"], f["B"], f["C"],
                                    delta_softplus=False)
    e = assert_match(to_f64(out), ref, RTOL_F32, "out")
    e2 = assert_match(to_f64(last), ref_last, RTOL_F32, "last_state")
    print(f"small step fwd delta={delta} segments={segments}: out {e} state {e2}", flush=True)


@pytest.mark.parametrize("segments", [1, 4])
@pytest.mark.parametrize("delta", SMALL)
def test_small_step_bwd(delta, segments):
    batch, dim, N, L = SHAPE
    announce(f"small step bwd delta={delta} segments={segments} shape={SHAPE}")
    inp = _const_step_inputs(102, delta, batch, dim, N, L, with_dout=True)
    f = W.inputs_f64(inp, "f32")
    g = to_device(inp, "f32")
    res = ms.scan_bwd(g["u"], g["delta"], g["A"], g["B"], g["C"], None, None, None, g["dout"],
                      delta_softplus=False, segments=segments)
    torch.cuda.synchronize()
    ref = oracle.scan_bwd(f["u"], f["delta"], f["A"], f["B"], f["C"], None, None, None,
                          f["dout"], delta_softplus=False)
    assert set(res) == set(ref)
    errs = {k: assert_match(to_f64(res[k]), ref[k], RTOL_F32, k) for k in ref}
    # dA element by element as well: each (d, n) entry sums the once-
    # cancelling term over every (b, t).  An entry far below the largest of
    # its row is itself a cancelling sum of 4096 terms, whose float32
    # rounding is set by the terms, not by the sum: entries below a tenth of
    # their row's largest are held to that tenth instead of their own size.
    got, rd = to_f64(res["dA"]), ref["dA"]
    scale = np.maximum(np.abs(rd), 0.1 * np.abs(rd).max(axis=1, keepdims=True))
    el = np.abs(got - rd) / scale
    i = np.unravel_index(el.argmax(), el.shape)
    print(f"small step bwd delta={delta} segments={segments}: {errs}; dA elementwise worst "
          f"{el.max():.2e} at {i}, |dA| {abs(rd[i]):.3e}, row max {np.abs(rd[i[0]]).max():.3e}",
          flush=True)
    assert el.max() <= RTOL_F32, f"dA elementwise rel err {el.max():.3e}"


@pytest.mark.parametrize("delta", SMALL)
def test_small_step_bwd_from_checkpoints(delta):
    batch, dim, N, L = SHAPE
    announce(f"small step fwd checkpoints + bwd delta={delta} shape={SHAPE}")
    inp = _const_step_inputs(103, delta, batch, dim, N, L, with_dout=True)
    f = W.inputs_f64(inp, "f32")
    g = to_device(inp, "f32")
    ck = torch.full(ms.checkpoint_shape(batch, dim, N, L), float("nan"), device="cuda")
    ms.scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], delta_softplus=False,
                checkpoints=ck, segments=1)
    res = ms.scan_bwd(g["u"], g["delta"], g["A"], g["B"], g["C"], None, None, None, g["dout"],
                      delta_softplus=False, checkpoints=ck, segments=1)
    torch.cuda.synchronize()
    ref = oracle.scan_bwd(f["u"], f["delta"], f["A"], f["B"], f["C"], None, None, None,
                          f["dout"], delta_softplus=False)
    for k in ref:
        assert_match(to_f64(res[k]), ref[k], RTOL_F32, k)


def _as_pairs(x):
    x = np.asarray(x)
    return np.stack([x.real, x.imag], -1).astype(np.float64)


@pytest.mark.parametrize("segments", [1, 4])
@pytest.mark.parametrize("delta", SMALL)
def test_small_step_complex(delta, segments):
    batch, dim, N, L = 1, 20, 16, 2048
    announce(f"small step complex fwd + bwd delta={delta} segments={segments}")
    inp = W.make_complex_inputs(104, batch, dim, N, L, dtype="f32", with_D=False, with_z=False,
                                with_bias=False, with_dout=True)
    inp["delta"] = np.full((batch, dim, L), delta, np.float32)
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in inp.items()}
    out, last = ms.scan_fwd_complex(t["u"], t["delta"], t["A"], t["B"], t["C"],
                                    delta_softplus=False, segments=segments)
    res = ms.scan_bwd_complex(t["u"], t["delta"], t["A"], t["B"], t["C"], None, None, None,
                              t["dout"], delta_softplus=False, segments=segments)
    torch.cuda.synchronize()
    f = {k: (v.astype(np.complex128) if np.iscomplexobj(v) else v.astype(np.float64))
         for k, v in inp.items()}
    ref, ref_last = oracle.scan_fwd_complex(f["u"], f["delta"], f["A"], f["B"], f["C"],
                                            delta_softplus=False)
    assert_match(to_f64(out), ref, RTOL_F32, "out")
    assert_match(_as_pairs(last.cpu().numpy()), _as_pairs(ref_last), RTOL_F32, "last_state",
                 row_ndim=2)
    gref = oracle.scan_bwd_complex(f["u"], f["delta"], f["A"], f["B"], f["C"], None, None, None,
                                   f["dout"], delta_softplus=False)
    for k in gref:
        got = res[k].cpu().numpy()
        if np.iscomplexobj(gref[k]):
            assert_match(_as_pairs(got), _as_pairs(gref[k]), RTOL_F32, k, row_ndim=2)
        else:
            assert_match(got.astype(np.float64), gref[k], RTOL_F32, k)
