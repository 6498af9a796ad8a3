"""GPU parity of the complex-valued forward, backward and decode step
(diagonal complex A, B, C and state; y = Re(sum_n C h) + D u, gated) against
the float64 oracle on the same seeded inputs: float32 and bfloat16
sequences, ZOH and Euler, several state sizes, ragged lengths, an initial
state, optional inputs absent, the softplus off, checkpoints, and sequences
split into segments."""
import numpy as np
import pytest
import torch

import oracle
import scan_selective_fwd_amd as ms
import workloads as W
from parity_utils import RTOL, RTOL_F32, announce, assert_match, to_f64

pytestmark = pytest.mark.gpu


def _dev(x, dtype):
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _case(wid, batch, dim, N, L, dtype, disc, h0=False, softplus=True, opts=None,
          zero_A=False, segments=0, reset=None):
    opts = opts or {}
    announce(f"complex fwd wid={wid} shape=({batch},{dim},{N},{L}) {dtype} {disc} h0={h0} "
             f"softplus={softplus} opts={opts} segments={segments} "
             f"resets={None if reset is None else int(reset.sum())}")
    inp = W.make_complex_inputs(wid, batch, dim, N, L, dtype=dtype, **opts)
    if not softplus:   # a positive raw step without the softplus
        raw = np.abs(W.as_f64(inp["delta"], dtype)) * 0.05 + 0.01
        inp["delta"] = W.bf16_round_bits(raw) if dtype == "bf16" else raw.astype(np.float32)
        if "delta_bias" in inp:
            inp["delta_bias"] = (np.abs(inp["delta_bias"]) * 0.01).astype(np.float32)
    if zero_A:
        inp["A"][::3, 0] = 0.0          # the ZOH limit delta*B for these channels
    h0v = None
    if h0:
        g = np.random.default_rng([wid, 13])
        h0v = (g.standard_normal((batch, dim, N)) + 1j * g.standard_normal((batch, dim, N))
               ).astype(np.complex64)
    t = {k: _dev(v, dtype) for k, v in inp.items()}
    out, last = ms.scan_fwd_complex(t["u"], t["delta"], t["A"], t["B"], t["C"], t.get("D"),
                                    t.get("z"), t.get("delta_bias"),
                                    None if h0v is None else torch.from_numpy(h0v).cuda(),
                                    delta_softplus=softplus, disc=disc, segments=segments,
                                    reset=None if reset is None else torch.from_numpy(reset).cuda())
    torch.cuda.synchronize()
    f = {k: (W.as_f64(v, dtype) if v.dtype == np.uint16 else v) for k, v in inp.items()}
    ref, ref_last = oracle.scan_fwd_complex(
        f["u"], f["delta"], f["A"], f["B"], f["C"], f.get("D"), f.get("z"), f.get("delta_bias"),
        h0v, delta_softplus=softplus, disc=oracle.ZOH if disc == "zoh" else oracle.EULER,
        reset=reset)
    assert_match(to_f64(out), ref, RTOL[dtype], "out")
    got_last = last.cpu().numpy().astype(np.complex128)
    assert_match(np.stack([got_last.real, got_last.imag], -1),
                 np.stack([ref_last.real, ref_last.imag], -1), RTOL_F32, "last_state",
                 row_ndim=2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("disc", ["zoh", "euler"])
def test_complex_fwd_dtypes_discs(dtype, disc):
    # 700 steps: five 128-step chunks and a ragged tail; 37 channels: a
    # partial block
    _case(70, 2, 37, 16, 700, dtype, disc, h0=True)


@pytest.mark.parametrize("N", [1, 5, 16])
@pytest.mark.parametrize("L", [1, 129, 1000])
def test_complex_fwd_sizes(N, L):
    _case(71, 1, 9, N, L, "f32", "zoh")


def test_complex_fwd_optional_inputs_and_softplus_off():
    _case(72, 2, 20, 8, 300, "f32", "zoh", softplus=False,
          opts=dict(with_D=False, with_z=False, with_bias=False))
    _case(73, 2, 20, 8, 300, "f32", "euler", softplus=False, h0=True)


def test_complex_fwd_zero_A_limit():
    _case(79, 1, 12, 4, 260, "f32", "zoh", h0=True, zero_A=True)


def test_complex_fwd_rejects_large_state():
    inp = W.make_complex_inputs(74, 1, 4, 17, 64)
    t = {k: _dev(v, "f32") for k, v in inp.items()}
    with pytest.raises(ms.MambaScanError):
        ms.scan_fwd_complex(t["u"], t["delta"], t["A"], t["B"], t["C"])


def _as_pairs(x):
    x = np.asarray(x).astype(np.complex128)
    return np.stack([x.real, x.imag], -1)


def _bwd_case(wid, batch, dim, N, L, dtype, disc, h0=False, softplus=True, opts=None,
              zero_A=False, segments=0, reset=None):
    opts = opts or {}
    announce(f"complex bwd wid={wid} shape=({batch},{dim},{N},{L}) {dtype} {disc} h0={h0} "
             f"softplus={softplus} opts={opts} zero_A={zero_A} segments={segments} "
             f"resets={None if reset is None else int(reset.sum())}")
    inp = W.make_complex_inputs(wid, batch, dim, N, L, dtype=dtype, with_dout=True, **opts)
    if not softplus:
        raw = np.abs(W.as_f64(inp["delta"], dtype)) * 0.05 + 0.01
        inp["delta"] = W.bf16_round_bits(raw) if dtype == "bf16" else raw.astype(np.float32)
        if "delta_bias" in inp:
            inp["delta_bias"] = (np.abs(inp["delta_bias"]) * 0.01).astype(np.float32)
    if zero_A:
        inp["A"][::3, 0] = 0.0
    h0v = None
    if h0:
        g = np.random.default_rng([wid, 13])
        h0v = (g.standard_normal((batch, dim, N)) + 1j * g.standard_normal((batch, dim, N))
               ).astype(np.complex64)
    t = {k: _dev(v, dtype) for k, v in inp.items()}
    res = ms.scan_bwd_complex(t["u"], t["delta"], t["A"], t["B"], t["C"], t.get("D"), t.get("z"),
                              t.get("delta_bias"), t["dout"],
                              None if h0v is None else torch.from_numpy(h0v).cuda(),
                              delta_softplus=softplus, disc=disc, segments=segments,
                              reset=None if reset is None else torch.from_numpy(reset).cuda())
    torch.cuda.synchronize()
    f = {k: (W.as_f64(v, dtype) if v.dtype == np.uint16 else v) for k, v in inp.items()}
    ref = oracle.scan_bwd_complex(f["u"], f["delta"], f["A"], f["B"], f["C"], f.get("D"),
                                  f.get("z"), f.get("delta_bias"), f["dout"], h0v,
                                  delta_softplus=softplus,
                                  disc=oracle.ZOH if disc == "zoh" else oracle.EULER,
                                  reset=reset)
    assert set(res) == set(ref), (set(res), set(ref))
    for k in ref:
        got = res[k].cpu().numpy()
        if np.iscomplexobj(ref[k]):
            assert_match(_as_pairs(got), _as_pairs(ref[k]), RTOL_F32, k, row_ndim=2)
        else:
            assert_match(got.astype(np.float64), ref[k], RTOL_F32, k)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("disc", ["zoh", "euler"])
def test_complex_bwd_dtypes_discs(dtype, disc):
    # few blocks: the automatic choice splits these 4 chunks into 4 segments;
    # the same case in one pass
    _bwd_case(75, 2, 19, 16, 400, dtype, disc, h0=True)
    _bwd_case(75, 2, 19, 16, 400, dtype, disc, h0=True, segments=1)


# Segmented complex calls: the summary pass writes each segment's end state
# from zero and its product of Abar, the carry composes them, and every
# segment runs from its entering state; the backward carries the adjoint
# from the last segment to the first the same way.  1189 steps are 9 full
# chunks and a ragged one (3 segments: 4 + 4 + 2 chunks; 10: one each).
@pytest.mark.parametrize("segments", [2, 3, 10])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_complex_segmented(segments, dtype):
    _case(84, 1, 20, 16, 1189, dtype, "zoh", h0=True, segments=segments)
    _bwd_case(84, 1, 20, 16, 1189, dtype, "euler", h0=True, segments=segments)


def test_complex_segmented_sizes_zero_A_slow_decay():
    _case(85, 2, 9, 5, 1300, "f32", "euler", segments=4)
    _bwd_case(85, 2, 9, 5, 1300, "f32", "zoh", h0=True, segments=4)
    _case(86, 1, 12, 4, 1024, "f32", "zoh", h0=True, zero_A=True, segments=8)
    _bwd_case(86, 1, 12, 4, 1024, "f32", "zoh", h0=True, zero_A=True, segments=8)
    # small steps: the states keep their phase across many segments, so the
    # carried product of Abar must hold it (A.im up to pi (N - 1))
    _case(87, 1, 16, 16, 4096, "f32", "zoh", h0=True, softplus=False, segments=32)
    _bwd_case(87, 1, 16, 16, 4096, "f32", "zoh", h0=True, softplus=False, segments=32)


# Packed sequences: the state entering each flagged step is zero.  Flags at
# t = 0 (the initial state is dropped), inside a lane's steps, on chunk
# borders, and at the last step.
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("disc", ["zoh", "euler"])
def test_complex_varlen(dtype, disc):
    L = 700
    rs = W.make_resets(89, 2, L, 1, 200, force=(0, 8, 128, 129, L - 1))
    rs[1, 0] = 0
    _case(89, 2, 19, 16, L, dtype, disc, h0=True, reset=rs, segments=1)
    _bwd_case(89, 2, 19, 16, L, dtype, disc, h0=True, reset=rs, segments=1)


def test_complex_varlen_segments_sizes_zero_A():
    # resets with segments: one in a segment's first chunk, a segment free of
    # them between two that have them
    L = 2048
    rs = W.make_resets(90, 2, L, 1, 700, force=(0, 1, 255, 256, 511, 1024, 1025, L - 1))
    rs[1, 512:1024] = 0
    _case(90, 2, 9, 16, L, "f32", "zoh", h0=True, reset=rs, segments=8)
    _bwd_case(90, 2, 9, 16, L, "f32", "zoh", h0=True, reset=rs, segments=8)
    _case(91, 2, 9, 5, L, "bf16", "euler", reset=rs, segments=3)
    _bwd_case(91, 2, 9, 5, L, "bf16", "euler", reset=rs, segments=3)
    rs2 = W.make_resets(92, 1, 1000, 20, 300, force=(0, 384))
    _case(92, 1, 12, 4, 1000, "f32", "zoh", h0=True, zero_A=True, reset=rs2)
    _bwd_case(92, 1, 12, 4, 1000, "f32", "zoh", h0=True, zero_A=True, reset=rs2)


def test_complex_automatic_segmentation_long_sequence():
    # 16 channels over 8192 steps: one channel group, so the forward splits
    # into 64 segments and the backward too
    assert ms.fwd_complex_workspace_bytes(1, 16, 16, 8192) > 0
    assert ms.bwd_complex_workspace_bytes(1, 16, 16, 8192) > \
        ms.bwd_complex_workspace_bytes(1, 16, 16, 8192, segments=1)
    _case(88, 1, 16, 16, 8192, "bf16", "zoh", h0=True)
    _bwd_case(88, 1, 16, 16, 8192, "bf16", "zoh", h0=True)


@pytest.mark.parametrize("N", [1, 5])
@pytest.mark.parametrize("L", [1, 129])
def test_complex_bwd_sizes(N, L):
    _bwd_case(76, 2, 7, N, L, "f32", "zoh")


def test_complex_bwd_optional_inputs_softplus_off_zero_A():
    _bwd_case(77, 2, 9, 6, 300, "f32", "zoh", softplus=False,
              opts=dict(with_D=False, with_z=False, with_bias=False))
    _bwd_case(78, 1, 12, 4, 260, "f32", "zoh", h0=True, zero_A=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("segments", [1, 3])
def test_complex_checkpoints_forward_states_and_backward(dtype, segments):
    """The forward's checkpoints equal the oracle's state after each 128-step
    prefix, and the backward that uses them matches the oracle's gradients
    (in one pass and in 3 segments)."""
    wid, batch, dim, N, L = 80, 2, 19, 16, 400
    announce(f"complex checkpoints wid={wid} shape=({batch},{dim},{N},{L}) {dtype} "
             f"segments={segments}")
    inp = W.make_complex_inputs(wid, batch, dim, N, L, dtype=dtype, with_dout=True)
    g = np.random.default_rng([wid, 13])
    h0v = (g.standard_normal((batch, dim, N)) + 1j * g.standard_normal((batch, dim, N))
           ).astype(np.complex64)
    t = {k: _dev(v, dtype) for k, v in inp.items()}
    h0t = torch.from_numpy(h0v).cuda()
    ckpt = torch.empty(ms.complex_checkpoint_shape(batch, dim, N, L), dtype=torch.complex64,
                       device="cuda")
    ms.scan_fwd_complex(t["u"], t["delta"], t["A"], t["B"], t["C"], t.get("D"), t.get("z"),
                        t.get("delta_bias"), h0t, checkpoints=ckpt, segments=segments)
    res = ms.scan_bwd_complex(t["u"], t["delta"], t["A"], t["B"], t["C"], t.get("D"), t.get("z"),
                              t.get("delta_bias"), t["dout"], h0t, checkpoints=ckpt,
                              segments=segments)
    torch.cuda.synchronize()
    f = {k: (W.as_f64(v, dtype) if v.dtype == np.uint16 else v) for k, v in inp.items()}
    got = ckpt.cpu().numpy()
    for k in range(got.shape[2]):
        if k == 0:
            ref_k = h0v.astype(np.complex128)
        else:
            T = 128 * k
            _, ref_k = oracle.scan_fwd_complex(
                f["u"][..., :T], f["delta"][..., :T], f["A"], f["B"][..., :T], f["C"][..., :T],
                f.get("D"), None, f.get("delta_bias"), h0v)
        assert_match(_as_pairs(got[:, :, k]), _as_pairs(ref_k), RTOL_F32, f"checkpoint {k}",
                     row_ndim=2)
    ref = oracle.scan_bwd_complex(f["u"], f["delta"], f["A"], f["B"], f["C"], f.get("D"),
                                  f.get("z"), f.get("delta_bias"), f["dout"], h0v)
    assert set(res) == set(ref), (set(res), set(ref))
    for k in ref:
        r = res[k].cpu().numpy()
        if np.iscomplexobj(ref[k]):
            assert_match(_as_pairs(r), _as_pairs(ref[k]), RTOL_F32, k, row_ndim=2)
        else:
            assert_match(r.astype(np.float64), ref[k], RTOL_F32, k)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("disc", ["zoh", "euler"])
def test_complex_state_update_continues_forward(dtype, disc):
    """A forward over L steps, then k decode steps from its final state,
    gives the outputs and final state of the oracle's forward over L + k
    steps (one decode step is the forward's step on a stored state)."""
    wid, batch, dim, N, L, k = 83, 2, 21, 16, 300, 3
    announce(f"complex state update wid={wid} shape=({batch},{dim},{N},{L}+{k}) {dtype} {disc}")
    inp = W.make_complex_inputs(wid, batch, dim, N, L + k, dtype=dtype)
    inp["A"][::4, 0] = 0.0                      # the ZOH limit delta B for these channels
    t = {kk: _dev(v, dtype) for kk, v in inp.items()}
    head = lambda name: t[name][..., :L].contiguous()
    _, state = ms.scan_fwd_complex(head("u"), head("delta"), t["A"], head("B"), head("C"),
                                   t.get("D"), head("z"), t.get("delta_bias"), disc=disc)
    outs = []
    for s in range(L, L + k):
        col = lambda name: t[name][..., s].contiguous()
        outs.append(ms.state_update_complex(state, col("u"), col("delta"), t["A"], col("B"),
                                            col("C"), t.get("D"), col("z"), t.get("delta_bias"),
                                            disc=disc))
    torch.cuda.synchronize()
    f = {kk: (W.as_f64(v, dtype) if v.dtype == np.uint16 else v) for kk, v in inp.items()}
    ref, ref_last = oracle.scan_fwd_complex(
        f["u"], f["delta"], f["A"], f["B"], f["C"], f.get("D"), f.get("z"), f.get("delta_bias"),
        None, disc=oracle.ZOH if disc == "zoh" else oracle.EULER)
    got = np.stack([to_f64(o) for o in outs], -1)
    assert_match(got, ref[..., L:], RTOL[dtype], "decode outputs")
    assert_match(_as_pairs(state.cpu().numpy()), _as_pairs(ref_last), RTOL_F32, "state",
                 row_ndim=2)


def test_complex_state_update_rejects_large_state():
    st = torch.zeros((1, 4, 17), dtype=torch.complex64, device="cuda")
    v = torch.zeros((1, 4), device="cuda")
    A = torch.zeros((4, 17), dtype=torch.complex64, device="cuda")
    BC = torch.zeros((1, 17), dtype=torch.complex64, device="cuda")
    with pytest.raises(ms.MambaScanError):
        ms.state_update_complex(st, v, v, A, BC, BC)
