"""GPU parity: the HIP library (through its C ABI) against the float64 oracle
on identical seeded inputs.  Small shapes span several chunks and a ragged
tail in every launch variant (lanes per channel 16/32/64, vector and scalar
loads, N <= 16 and N > 16, ZOH and Euler, float32 and bfloat16, optional
inputs present or absent, initial state, A = 0)."""
import numpy as np
import pytest
import torch

import oracle
import scan_selective_fwd_amd as ms
import workloads as W
from parity_utils import RTOL, RTOL_F32, announce, assert_match, to_device, to_f64

pytestmark = pytest.mark.gpu


def _oracle_fwd(f, disc, softplus=True, h0=None, reset=None):
    return oracle.scan_fwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f.get("D"), f.get("z"),
                           f.get("delta_bias"), h0, delta_softplus=softplus,
                           disc=oracle.ZOH if disc == "zoh" else oracle.EULER, reset=reset)


def _make(wid, batch, dim, N, L, dtype, bias="uniform", **kw):
    inp = W.make_inputs(wid, batch, dim, N, L, dtype=dtype, bias=bias, **kw)
    return inp, W.inputs_f64(inp, dtype)


def _positive_steps(inp, dtype):
    """Without the softplus the raw step is used as is: make it positive
    (0.01 + 0.05|raw| plus a small positive bias) so the recurrence decays."""
    raw = np.abs(W.bf16_bits_to_f32(inp["delta"]) if dtype == "bf16" else inp["delta"])
    raw = raw * 0.05 + 0.01
    inp["delta"] = W.bf16_round_bits(raw) if dtype == "bf16" else raw.astype(np.float32)
    if "delta_bias" in inp:
        inp["delta_bias"] = (np.abs(inp["delta_bias"]) * 0.01).astype(np.float32)
    return inp, W.inputs_f64(inp, dtype)


def _positive_A(inp):
    """Some A > 0 (a state that grows): +0.05 in every fifth channel's state 2
    and +1e-3 in the next channel's state 5 (small x = delta A > 0)."""
    inp["A"][1::5, 2] = 0.05
    inp["A"][2::5, min(5, inp["A"].shape[1] - 1)] = 1e-3
    return inp["A"].astype(np.float64)


def run_fwd_case(wid, batch, dim, N, L, dtype, disc, lanes=0, softplus=True, h0=False, opts=None,
                 zero_A=False, A_mode="s4d_real", rtol=None, segments=0, reset=None,
                 h0_scale=1.0, pos_A=False):
    opts = opts or {}
    announce(f"fwd wid={wid} shape=({batch},{dim},{N},{L}) {dtype} {disc} lanes={lanes} "
             f"softplus={softplus} h0={h0}x{h0_scale} opts={opts} zero_A={zero_A} "
             f"segments={segments} resets={None if reset is None else int(reset.sum())}")
    inp, f = _make(wid, batch, dim, N, L, dtype, A_mode=A_mode, **opts)
    if not softplus:
        inp, f = _positive_steps(inp, dtype)
    if zero_A:
        inp["A"][::3, 0] = 0.0
        f["A"] = inp["A"].astype(np.float64)
    if pos_A:
        f["A"] = _positive_A(inp)
    h0v = None
    if h0:
        h0v = (np.random.default_rng(wid).standard_normal((batch, dim, N))
               * h0_scale).astype(np.float32)
    g = to_device(inp, dtype)
    h0t = torch.from_numpy(h0v).cuda() if h0v is not None else None
    out, last = ms.scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g.get("D"), g.get("z"),
                            g.get("delta_bias"), h0t, delta_softplus=softplus, disc=disc,
                            return_last_state=True, lanes=lanes, segments=segments,
                            reset=None if reset is None else torch.from_numpy(reset).cuda())
    torch.cuda.synchronize()
    ref, ref_last = _oracle_fwd(f, disc, softplus, None if h0v is None else h0v.astype(np.float64),
                                reset)
    rt = rtol or RTOL[dtype]
    assert_match(to_f64(out), ref, rt, "out")
    # the state is float32 in both dtypes: the float32 bound applies
    assert_match(to_f64(last), ref_last, rtol or RTOL_F32, "last_state")
    return out, last


# --------------------------------------------------------------------------
# forward
# --------------------------------------------------------------------------
def test_fwd_workload1_exact_config():
    run_fwd_case(1, 1, 16, 4, 128, "f32", "zoh", opts=dict(bias="const"))


@pytest.mark.parametrize("lanes", [16, 32, 64])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("disc", ["zoh", "euler"])
def test_fwd_lanes_dtypes_discs(lanes, dtype, disc):
    # 1000 steps: several chunks of 16*16/32*16/64*16 and a ragged tail;
    # 37 channels: partial last block and partial last wave.
    run_fwd_case(11, 2, 37, 16, 1000, dtype, disc, lanes=lanes)


@pytest.mark.parametrize("L", [1, 3, 999, 1001])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fwd_ragged_and_unaligned_lengths(L, dtype):
    for lanes in (16, 64):
        run_fwd_case(12, 1, 5, 16, L, dtype, "zoh", lanes=lanes)


@pytest.mark.parametrize("N", [1, 5, 16, 17, 33, 64])
def test_fwd_state_sizes(N):
    run_fwd_case(13, 2, 9, N, 700, "f32", "zoh", lanes=32, A_mode="random_neg")


@pytest.mark.parametrize("disc", ["zoh", "euler"])
def test_fwd_without_optional_inputs_and_softplus_off(disc):
    run_fwd_case(14, 2, 21, 16, 513, "f32", disc, softplus=False,
                 opts=dict(with_D=False, with_z=False, with_bias=False))
    run_fwd_case(15, 2, 21, 16, 513, "f32", disc, softplus=False)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fwd_initial_state(dtype):
    run_fwd_case(16, 3, 10, 16, 600, dtype, "zoh", h0=True)
    run_fwd_case(16, 3, 10, 7, 600, dtype, "euler", h0=True, lanes=64)


def test_fwd_zero_A_limit():
    run_fwd_case(17, 2, 12, 16, 400, "f32", "zoh", zero_A=True)
    run_fwd_case(17, 2, 12, 16, 400, "f32", "zoh", zero_A=True, lanes=64)


def test_fwd_positive_A():
    # A > 0 takes the kernels' general copy (the sign-agnostic expm1); the
    # state grows, and the segment carry multiplies by exp(A sum(delta)) > 1
    run_fwd_case(18, 2, 12, 16, 700, "f32", "zoh", pos_A=True, h0=True)
    run_fwd_case(18, 2, 12, 16, 700, "f32", "zoh", pos_A=True, segments=3)
    run_fwd_case(18, 2, 12, 16, 700, "f32", "zoh", pos_A=True, lanes=32)
    run_fwd_case(18, 2, 12, 16, 700, "bf16", "euler", pos_A=True)


@pytest.mark.parametrize("segments", [2, 3, 10])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("disc", ["zoh", "euler"])
def test_fwd_segmented(segments, dtype, disc):
    # the sequence split into segments joined by the carry kernel: 1189 steps
    # are 9 full 128-step chunks and a ragged one (10 segments = one chunk
    # each); 20 channels leave the second channel group partial
    run_fwd_case(19, 1, 20, 16, 1189, dtype, disc, segments=segments)


def test_fwd_segmented_state_sizes_initial_state_zero_A():
    run_fwd_case(20, 2, 9, 5, 1300, "f32", "zoh", segments=4, h0=True)
    run_fwd_case(20, 2, 9, 33, 1300, "f32", "zoh", segments=4, A_mode="random_neg")
    run_fwd_case(21, 1, 12, 16, 1024, "f32", "zoh", segments=8, zero_A=True, h0=True)
    run_fwd_case(21, 1, 12, 16, 1024, "f32", "euler", segments=5, softplus=False, h0=True)


# Long segments (at least 16 chunks) run from a zero state first; after the
# carry a second launch redoes each segment's first chunks from its entering
# state, until what is left of that state is below float32 resolution.
# 4173 steps are 33 chunks (ragged): 2 segments of 17 and 16 chunks.
LONG_L = 4173


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("disc", ["zoh", "euler"])
def test_fwd_long_segments(dtype, disc):
    run_fwd_case(58, 1, 20, 16, LONG_L, dtype, disc, segments=2, h0=True)


def test_fwd_long_segments_edge_cases():
    run_fwd_case(59, 2, 9, 5, LONG_L, "f32", "zoh", segments=2, h0=True)
    run_fwd_case(59, 2, 9, 33, LONG_L, "f32", "zoh", segments=2, A_mode="random_neg")
    # A = 0 channels never forget the entering state: the second launch
    # redoes the whole segment
    run_fwd_case(60, 1, 12, 16, LONG_L, "f32", "zoh", segments=2, zero_A=True, h0=True)
    # a huge initial state takes longer to fall below resolution
    run_fwd_case(61, 1, 12, 16, LONG_L, "f32", "zoh", segments=2, h0=True, h0_scale=1e20)
    # small steps decay slowly
    run_fwd_case(62, 1, 12, 16, LONG_L, "f32", "euler", segments=2, softplus=False, h0=True)
    # resets, one in the second segment's first chunk
    rs = W.make_resets(63, 2, LONG_L, 100, 1500, force=(0, 17 * 128 + 5))
    rs[1, :] = 0
    rs[1, 3000] = 1
    run_fwd_case(63, 2, 9, 16, LONG_L, "f32", "zoh", segments=2, h0=True, reset=rs)
    run_fwd_case(63, 2, 9, 16, LONG_L, "bf16", "euler", segments=2, reset=rs)


def test_fwd_automatic_segmentation():
    # few channels over a long sequence: the automatic choice splits it
    assert ms.fwd_workspace_bytes(1, 16, 16, 8192, torch.bfloat16) > 0
    run_fwd_case(22, 1, 16, 16, 8192, "bf16", "zoh")
    run_fwd_case(22, 1, 16, 16, 8192, "bf16", "zoh", segments=1)


# steps flagged in every row: the first step (the initial state is dropped),
# a lane border (8), a 128-step chunk border and the step after it, the last
EDGE_RESETS = (0, 8, 128, 129)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("disc", ["zoh", "euler"])
def test_fwd_varlen(dtype, disc):
    L = 1189
    rs = W.make_resets(40, 2, L, 1, 300, force=EDGE_RESETS + (L - 1,))
    rs[1, 0] = 0          # the second row keeps its initial state
    run_fwd_case(40, 2, 20, 16, L, dtype, disc, h0=True, reset=rs)


def test_fwd_varlen_state_sizes_and_segments():
    L = 1300
    rs = W.make_resets(41, 2, L, 1, 200, force=(128, 640))
    run_fwd_case(41, 2, 9, 5, L, "f32", "zoh", h0=True, reset=rs)
    run_fwd_case(41, 2, 9, 33, L, "f32", "zoh", A_mode="random_neg", reset=rs)
    run_fwd_case(41, 2, 9, 16, L, "f32", "zoh", h0=True, reset=rs, segments=4)
    run_fwd_case(42, 1, 12, 16, 1024, "f32", "zoh", zero_A=True, segments=8,
                 reset=W.make_resets(42, 1, 1024, 50, 400))
    # a segment boundary that is also a reset, and a segment without any
    rs = np.zeros((1, 2048), np.uint8)
    rs[0, [256, 1000]] = 1
    run_fwd_case(43, 1, 16, 16, 2048, "bf16", "euler", h0=True, reset=rs, segments=8)


def test_fwd_is_deterministic_and_lane_choice_independent():
    inp, f = _make(18, 2, 40, 16, 2048, "f32")
    g = to_device(inp, "f32")
    outs = []
    for lanes in (16, 16, 32, 64):
        outs.append(ms.scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"],
                                g["delta_bias"], lanes=lanes))
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    for o in outs[2:]:
        assert_match(to_f64(o), to_f64(outs[0]), 1e-5, "lanes")


def test_fwd_reset_by_large_step():
    # a large raw step resets the state: outputs after it do not depend on
    # the prefix (Knowl 4 of the chapterpal page: large step resets).
    inp, _ = _make(19, 1, 8, 16, 512, "f32")
    inp2 = {k: v.copy() for k, v in inp.items()}
    rng = np.random.default_rng(5)
    inp2["u"][..., :200] = rng.standard_normal((1, 8, 200)).astype(np.float32)
    for x in (inp, inp2):
        x["delta"][..., 200] = 60.0
    o = []
    for x in (inp, inp2):
        g = to_device(x, "f32")
        o.append(to_f64(ms.scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"],
                                    g["delta_bias"])))
    assert not np.allclose(o[0][..., :200], o[1][..., :200])
    np.testing.assert_allclose(o[0][..., 200:], o[1][..., 200:], rtol=1e-6, atol=1e-6)


# --------------------------------------------------------------------------
# state update (decode step)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("disc", ["zoh", "euler"])
@pytest.mark.parametrize("N", [16, 40])
def test_state_update_matches_oracle_and_continues_forward(dtype, disc, N):
    announce(f"state_update {dtype} {disc} N={N}")
    batch, dim, L, k = 3, 50, 300, 6
    inp, f = _make(21, batch, dim, N, L + k, dtype, A_mode="random_neg")
    g = to_device(inp, dtype)
    sl = lambda t, a, b: t[..., a:b].contiguous()
    # GPU prefill of the first L steps, then k decode steps
    _, state = ms.scan_fwd(sl(g["u"], 0, L), sl(g["delta"], 0, L), g["A"], sl(g["B"], 0, L),
                           sl(g["C"], 0, L), g["D"], sl(g["z"], 0, L), g["delta_bias"],
                           disc=disc, return_last_state=True)
    ref_full, ref_last = _oracle_fwd(f, disc)
    outs = []
    for t in range(L, L + k):
        outs.append(to_f64(ms.state_update(state, g["u"][..., t].contiguous(),
                                           g["delta"][..., t].contiguous(), g["A"],
                                           g["B"][..., t].contiguous(), g["C"][..., t].contiguous(),
                                           g["D"], g["z"][..., t].contiguous(), g["delta_bias"],
                                           disc=disc)))
    torch.cuda.synchronize()
    rt = RTOL[dtype]
    assert_match(np.stack(outs, -1), ref_full[..., L:], rt, "decode out")
    assert_match(to_f64(state), ref_last, RTOL_F32, "decode state")
    # one step from an arbitrary state against the oracle's step
    st0 = np.random.default_rng(3).standard_normal((batch, dim, N)).astype(np.float32)
    stt = torch.from_numpy(st0).cuda()
    t = 17
    y = ms.state_update(stt, g["u"][..., t].contiguous(), g["delta"][..., t].contiguous(), g["A"],
                        g["B"][..., t].contiguous(), g["C"][..., t].contiguous(), g["D"],
                        g["z"][..., t].contiguous(), g["delta_bias"], disc=disc)
    yr, sr = oracle.state_update(st0.astype(np.float64), f["u"][..., t], f["delta"][..., t], f["A"],
                                 f["B"][..., t], f["C"][..., t], f["D"], f["z"][..., t],
                                 f["delta_bias"],
                                 disc=oracle.ZOH if disc == "zoh" else oracle.EULER)
    assert_match(to_f64(y), yr, rt, "step out")
    assert_match(to_f64(stt), sr, RTOL_F32, "step state")


def test_state_update_without_optionals():
    batch, dim, N = 2, 33, 16
    inp, f = _make(22, batch, dim, N, 4, "f32", with_D=False, with_z=False, with_bias=False)
    g = to_device(inp, "f32")
    st0 = np.random.default_rng(4).standard_normal((batch, dim, N)).astype(np.float32)
    stt = torch.from_numpy(st0).cuda()
    y = ms.state_update(stt, g["u"][..., 1].contiguous(), g["delta"][..., 1].contiguous(), g["A"],
                        g["B"][..., 1].contiguous(), g["C"][..., 1].contiguous())
    yr, sr = oracle.state_update(st0.astype(np.float64), f["u"][..., 1], f["delta"][..., 1],
                                 f["A"], f["B"][..., 1], f["C"][..., 1])
    assert_match(to_f64(y), yr, 1e-4, "out")
    assert_match(to_f64(stt), sr, 1e-4, "state")


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------
def run_bwd_case(wid, batch, dim, N, L, dtype, disc, lanes=0, softplus=True, h0=False,
                 opts=None, zero_A=False, A_mode="s4d_real", rtol=None, reset=None, segments=0,
                 pos_A=False):
    opts = opts or {}
    announce(f"bwd wid={wid} shape=({batch},{dim},{N},{L}) {dtype} {disc} lanes={lanes} "
             f"h0={h0} opts={opts} zero_A={zero_A} segments={segments} "
             f"resets={None if reset is None else int(reset.sum())}")
    inp, f = _make(wid, batch, dim, N, L, dtype, with_dout=True, A_mode=A_mode, **opts)
    if not softplus:
        inp, f = _positive_steps(inp, dtype)
    if zero_A:
        inp["A"][::4, 1] = 0.0
        f["A"] = inp["A"].astype(np.float64)
    if pos_A:
        f["A"] = _positive_A(inp)
    h0v = np.random.default_rng(wid).standard_normal((batch, dim, N)).astype(np.float32) \
        if h0 else None
    g = to_device(inp, dtype)
    h0t = torch.from_numpy(h0v).cuda() if h0v is not None else None
    res = ms.scan_bwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g.get("D"), g.get("z"),
                      g.get("delta_bias"), g["dout"], h0t, delta_softplus=softplus, disc=disc,
                      lanes=lanes, segments=segments,
                      reset=None if reset is None else torch.from_numpy(reset).cuda())
    torch.cuda.synchronize()
    ref = oracle.scan_bwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f.get("D"), f.get("z"),
                          f.get("delta_bias"), f["dout"],
                          None if h0v is None else h0v.astype(np.float64),
                          delta_softplus=softplus,
                          disc=oracle.ZOH if disc == "zoh" else oracle.EULER, reset=reset)
    # every gradient is float32, computed from the same input bits on both
    # sides: the float32 bound applies in both dtypes
    rt = rtol or RTOL_F32
    assert set(res) == set(ref), (set(res), set(ref))
    for k in ref:
        assert_match(to_f64(res[k]), ref[k], rt, k)
    return res


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("disc", ["zoh", "euler"])
def test_bwd_dtypes_discs(dtype, disc):
    # 700 steps: five 128-step chunks and a ragged tail; 19 channels: a
    # partial block and a partial wave.
    run_bwd_case(31, 2, 19, 16, 700, dtype, disc, h0=True)


@pytest.mark.parametrize("L", [1, 77, 128, 1000])
def test_bwd_ragged_lengths(L):
    run_bwd_case(32, 2, 7, 16, L, "f32", "zoh")
    run_bwd_case(32, 2, 7, 16, L, "bf16", "zoh")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("disc", ["zoh", "euler"])
def test_bwd_varlen(dtype, disc):
    L = 700
    rs = W.make_resets(44, 2, L, 1, 200, force=EDGE_RESETS + (L - 1,))
    rs[1, 0] = 0
    run_bwd_case(44, 2, 19, 16, L, dtype, disc, h0=True, reset=rs)


def test_bwd_varlen_state_sizes_and_zero_A():
    L = 1000
    rs = W.make_resets(45, 2, L, 20, 300, force=(0, 384))
    run_bwd_case(45, 2, 7, 5, L, "f32", "zoh", reset=rs)
    run_bwd_case(45, 2, 7, 33, L, "f32", "zoh", A_mode="random_neg", h0=True, reset=rs)
    run_bwd_case(46, 2, 8, 16, 500, "f32", "zoh", zero_A=True, h0=True,
                 reset=W.make_resets(46, 2, 500, 10, 100))


def _ckpt_case(wid, batch, dim, N, L, dtype, disc, h0=False, segments=0, reset=None,
               bwd_segments=0):
    # the forward saves the state entering every 128-step chunk; the backward
    # given them must match the oracle (and the run that recomputes them)
    announce(f"checkpoints wid={wid} shape=({batch},{dim},{N},{L}) {dtype} {disc} h0={h0} "
             f"segments={segments} bwd_segments={bwd_segments} "
             f"resets={None if reset is None else int(reset.sum())}")
    inp, f = _make(wid, batch, dim, N, L, dtype, with_dout=True)
    h0v = np.random.default_rng(wid).standard_normal((batch, dim, N)).astype(np.float32) \
        if h0 else None
    g = to_device(inp, dtype)
    h0t = torch.from_numpy(h0v).cuda() if h0v is not None else None
    rt = torch.from_numpy(reset).cuda() if reset is not None else None
    ck = torch.full(ms.checkpoint_shape(batch, dim, N, L), float("nan"), device="cuda")
    ms.scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"], g["delta_bias"], h0t,
                disc=disc, segments=segments, reset=rt, checkpoints=ck)
    res = ms.scan_bwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"],
                      g["delta_bias"], g["dout"], h0t, disc=disc, reset=rt, checkpoints=ck,
                      segments=bwd_segments)
    res2 = ms.scan_bwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"],
                       g["delta_bias"], g["dout"], h0t, disc=disc, reset=rt,
                       segments=bwd_segments)
    torch.cuda.synchronize()
    assert not torch.isnan(ck).any()
    ref = oracle.scan_bwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                          f["delta_bias"], f["dout"],
                          None if h0v is None else h0v.astype(np.float64),
                          disc=oracle.ZOH if disc == "zoh" else oracle.EULER, reset=reset)
    for k in ref:
        assert_match(to_f64(res[k]), ref[k], RTOL_F32, k)
        assert_match(to_f64(res[k]), to_f64(res2[k]), RTOL_F32, k + " vs recompute")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("disc", ["zoh", "euler"])
def test_bwd_from_forward_checkpoints(dtype, disc):
    _ckpt_case(47, 2, 19, 16, 700, dtype, disc, h0=True)


def test_bwd_from_forward_checkpoints_segmented_varlen_sizes():
    _ckpt_case(48, 1, 16, 16, 2048, "f32", "zoh", h0=True, segments=4)
    _ckpt_case(48, 2, 9, 5, 1000, "f32", "zoh",
               reset=W.make_resets(48, 2, 1000, 20, 300, force=(0, 128)))
    _ckpt_case(49, 2, 9, 33, 513, "bf16", "euler", h0=True)


@pytest.mark.parametrize("segments", [2, 3, 10])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("disc", ["zoh", "euler"])
def test_bwd_segmented(segments, dtype, disc):
    # the backward split into segments: states from a segmented forward pass,
    # the adjoint entering each segment from the reverse carry.  1189 steps
    # are 9 full chunks and a ragged one (3 segments: 4 + 4 + 2 chunks, 10:
    # one chunk each); dh0 comes from the first segment only.
    run_bwd_case(51, 1, 20, 16, 1189, dtype, disc, h0=True, segments=segments)


# Wide backward blocks (12 waves, 48 channels) run when batch * ceil(D/48)
# reaches 171 in a one-pass backward (N <= 16, no reset flags).  These shapes
# reach it with a partial last channel group (2050 = 42 * 48 + 34) and
# ragged sequences.
WIDE_MIN_BLOCKS = 171


def _wide_blocks(batch, dim):
    return batch * -(-dim // 48)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("disc", ["zoh", "euler"])
def test_bwd_wide_blocks(dtype, disc):
    assert _wide_blocks(4, 2050) >= WIDE_MIN_BLOCKS
    run_bwd_case(54, 4, 2050, 16, 300, dtype, disc, h0=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_wide_blocks_small_state_unaligned(dtype):
    # wide blocks with N < 16 (state rows past N are neither read nor
    # flushed) and a length whose rows are not 16-byte aligned (the guarded
    # loads and stores, a ragged last chunk)
    assert _wide_blocks(4, 2050) >= WIDE_MIN_BLOCKS
    run_bwd_case(59, 4, 2050, 5, 301, dtype, "zoh", h0=True)


def test_bwd_positive_A():
    # A > 0: the blocks holding one are deferred to the general launch; one
    # pass, segmented, and in wide blocks
    run_bwd_case(58, 2, 19, 16, 700, "f32", "zoh", pos_A=True, h0=True)
    run_bwd_case(58, 1, 20, 16, 1189, "f32", "zoh", pos_A=True, segments=3)
    run_bwd_case(58, 4, 2050, 16, 300, "f32", "zoh", pos_A=True)


def test_bwd_wide_blocks_zero_A_and_checkpoints():
    # A = 0 in every fourth channel: the wide blocks holding one are deferred
    # to the launch with the A = 0 limit
    assert _wide_blocks(4, 2050) >= WIDE_MIN_BLOCKS
    run_bwd_case(55, 4, 2050, 16, 300, "f32", "zoh", zero_A=True, h0=True)
    _ckpt_case(56, 4, 2050, 16, 300, "f32", "zoh", h0=True)
    # one channel group fewer: narrow blocks (4 * 42 = 168 wide ones)
    assert _wide_blocks(4, 2016) < WIDE_MIN_BLOCKS
    run_bwd_case(57, 4, 2016, 16, 300, "f32", "zoh", h0=True)


def test_bwd_segmented_state_sizes_optionals_zero_A():
    run_bwd_case(52, 2, 9, 5, 1300, "f32", "zoh", segments=4, h0=True)
    run_bwd_case(52, 2, 9, 33, 1300, "f32", "zoh", segments=4, A_mode="random_neg")
    run_bwd_case(53, 1, 12, 16, 1024, "f32", "zoh", segments=8, zero_A=True, h0=True)
    run_bwd_case(53, 1, 12, 16, 1024, "f32", "euler", segments=5, softplus=False,
                 opts=dict(with_D=False, with_z=False, with_bias=False))


def test_bwd_segmented_varlen():
    # resets on segment and chunk boundaries, in a segment's first and last
    # step, and a segment free of resets between two that have them
    L = 2048
    rs = W.make_resets(54, 2, L, 1, 700, force=(0, 1, 255, 256, 511, 1024, 1025, L - 1))
    rs[1, 512:1024] = 0
    run_bwd_case(54, 2, 9, 16, L, "f32", "zoh", h0=True, reset=rs, segments=8)
    run_bwd_case(55, 2, 9, 5, L, "bf16", "euler", reset=rs, segments=3)


def test_bwd_automatic_segmentation():
    # 16 channels over 8192 steps: one channel group, 64 chunks, so the
    # automatic choice splits the sequence (64 segments of one chunk); it must
    # agree with the oracle and with the one-pass backward
    res = run_bwd_case(56, 1, 16, 16, 8192, "bf16", "zoh", h0=True)
    one = run_bwd_case(56, 1, 16, 16, 8192, "bf16", "zoh", h0=True, segments=1)
    for k in res:
        assert_match(to_f64(res[k]), to_f64(one[k]), RTOL["f32"], k + " auto vs one pass")


def test_bwd_long_segments():
    # the state pass in the long-segment scheme (zero start, carry, correction)
    run_bwd_case(64, 1, 20, 16, LONG_L, "f32", "zoh", h0=True, segments=2)
    run_bwd_case(64, 1, 20, 16, LONG_L, "bf16", "euler", h0=True, segments=2)
    run_bwd_case(65, 1, 12, 16, LONG_L, "f32", "zoh", zero_A=True, h0=True, segments=2)
    rs = W.make_resets(66, 2, LONG_L, 100, 1500, force=(0, 17 * 128 + 5))
    run_bwd_case(66, 2, 9, 5, LONG_L, "f32", "zoh", h0=True, reset=rs, segments=2)


def test_bwd_segmented_from_checkpoints():
    _ckpt_case(57, 1, 16, 16, 2048, "f32", "zoh", h0=True, segments=4, bwd_segments=4)
    _ckpt_case(57, 2, 9, 5, 1000, "bf16", "euler", bwd_segments=3,
               reset=W.make_resets(57, 2, 1000, 20, 300, force=(0, 384)))
    # checkpoints from a forward in the long-segment scheme
    _ckpt_case(67, 1, 16, 16, LONG_L, "f32", "zoh", h0=True, segments=2, bwd_segments=2)


def test_bwd_rejects_other_lane_counts():
    inp, _ = _make(38, 1, 4, 16, 64, "f32", with_dout=True)
    g = to_device(inp, "f32")
    with pytest.raises(ms.MambaScanError):
        ms.scan_bwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"],
                    g["delta_bias"], g["dout"], lanes=32)


@pytest.mark.parametrize("N", [1, 5, 17, 64])
def test_bwd_state_sizes(N):
    run_bwd_case(33, 2, 9, N, 300, "f32", "zoh", A_mode="random_neg")


def test_bwd_optionals_absent_softplus_off_zero_A():
    run_bwd_case(34, 2, 13, 16, 400, "f32", "zoh",
                 opts=dict(with_D=False, with_z=False, with_bias=False))
    run_bwd_case(35, 2, 13, 16, 400, "f32", "euler", softplus=False, opts=dict(bias="normal"))
    run_bwd_case(36, 2, 13, 16, 400, "f32", "zoh", zero_A=True)


def test_autograd_function_matches_bwd():
    inp, f = _make(37, 2, 8, 16, 256, "f32", with_dout=True)
    g = to_device(inp, "f32")
    leaves = {k: g[k].clone().requires_grad_(True)
              for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")}
    out = ms.selective_scan(leaves["u"], leaves["delta"], leaves["A"], leaves["B"], leaves["C"],
                            leaves["D"], leaves["z"], leaves["delta_bias"])
    out.backward(g["dout"])
    ref = oracle.scan_bwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                          f["delta_bias"], f["dout"])
    names = dict(u="du", delta="ddelta", A="dA", B="dB", C="dC", D="dD", z="dz",
                 delta_bias="ddelta_bias")
    for k, gk in names.items():
        assert_match(to_f64(leaves[k].grad), ref[gk], 1e-4, gk)


@pytest.mark.parametrize("split", [128, 333])
def test_fwd_split_sequence_resumes_exactly(split):
    """Splitting the sequence and carrying the final state as the initial
    state of the rest gives the outputs of one pass (the chunk-boundary carry
    is exact), and both match the oracle."""
    wid, batch, dim, N, L = 81, 2, 20, 16, 900
    announce(f"split-L wid={wid} shape=({batch},{dim},{N},{L}) split={split}")
    inp, f = _make(wid, batch, dim, N, L, "f32")
    t = to_device(inp, "f32")
    full, last = ms.scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                             t["delta_bias"], return_last_state=True)
    part = lambda k, a, b: t[k][..., a:b].contiguous()
    o1, l1 = ms.scan_fwd(part("u", 0, split), part("delta", 0, split), t["A"],
                         part("B", 0, split), part("C", 0, split), t["D"], part("z", 0, split),
                         t["delta_bias"], return_last_state=True)
    o2, l2 = ms.scan_fwd(part("u", split, L), part("delta", split, L), t["A"],
                         part("B", split, L), part("C", split, L), t["D"], part("z", split, L),
                         t["delta_bias"], l1, return_last_state=True)
    torch.cuda.synchronize()
    ref, ref_last = _oracle_fwd(f, "zoh")
    joined = torch.cat([o1, o2], dim=-1)
    assert_match(to_f64(joined), ref, RTOL["f32"], "split out")
    assert_match(to_f64(l2), ref_last, RTOL["f32"], "split last_state")
    assert_match(to_f64(full), ref, RTOL["f32"], "full out")
    # the two GPU runs agree more closely with each other than with the oracle
    assert_match(to_f64(joined), to_f64(full), 1e-5, "split vs full")


@pytest.mark.parametrize("shape", [(0, 4, 8, 64), (2, 0, 8, 64), (2, 4, 0, 64), (2, 4, 8, 0)])
def test_empty_inputs_are_refused_without_launching(shape):
    """Empty tensors reach the library, which refuses them with
    MAMBA_ERR_SHAPE before enqueuing anything (the forward and backward
    through their workspace queries, the decode step through its entry point);
    caller buffers are left as they were."""
    batch, dim, N, L = shape
    announce(f"empty inputs {shape}")
    dev = "cuda"
    u = torch.zeros((batch, dim, L), device=dev)
    A = -torch.ones((dim, N), device=dev)
    B = torch.zeros((batch, N, L), device=dev)
    out = torch.full((batch, dim, L), 7.0, device=dev)
    with pytest.raises(ms.MambaScanError) as e:
        ms.scan_fwd(u, u, A, B, B, out=out)
    assert e.value.status == 2
    with pytest.raises(ms.MambaScanError) as e:
        ms.scan_bwd(u, u, A, B, B, None, None, None, u)
    assert e.value.status == 2
    state = torch.full((batch, dim, N), 3.0, device=dev)
    x = torch.zeros((batch, dim), device=dev)
    Bs = torch.zeros((batch, N), device=dev)
    if batch == 0 or dim == 0 or N == 0:
        with pytest.raises(ms.MambaScanError) as e:
            ms.state_update(state, x, x, A, Bs, Bs)
        assert e.value.status == 2
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((state == 3.0).all())


def test_nan_and_infinite_step_inputs_propagate():
    """Non-finite inputs never stall a call, and they stay where the
    recurrence carries them.  A NaN in u at one step makes that channel's
    outputs NaN from that step on; a step of +inf (delta_raw = +inf) resets
    the state, the limit the pages give for a large step, and the outputs
    stay finite.  Every other channel matches the oracle as usual (rows are
    independent; the shared B and C are finite)."""
    batch, dim, N, L = 2, 20, 16, 700
    announce(f"non-finite inputs shape=({batch},{dim},{N},{L})")
    inp, _ = _make(63, batch, dim, N, L, "f32", with_dout=True)
    inp["u"][0, 3, 100] = np.nan
    inp["delta"][1, 5, 50] = np.inf
    f = W.inputs_f64(inp, "f32")
    g = to_device(inp, "f32")
    out, last = ms.scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"],
                            g["delta_bias"], return_last_state=True)
    res = ms.scan_bwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"],
                      g["delta_bias"], g["dout"])
    torch.cuda.synchronize()
    ref, ref_last = _oracle_fwd(f, "zoh")
    gref = oracle.scan_bwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                           f["delta_bias"], f["dout"])
    o = to_f64(out)
    # the NaN channel: finite and exact before the step, NaN from it on
    assert np.isnan(o[0, 3, 100:]).all() and np.isnan(ref[0, 3, 100:]).all()
    assert_match(o[0, 3, :100], ref[0, 3, :100], RTOL_F32, "out before the NaN")
    # the infinite step's channel: finite everywhere (the state is reset)
    assert np.isfinite(ref[1, 5]).all()
    assert_match(o[1, 5], ref[1, 5], RTOL_F32, "out across the infinite step")
    # every other channel, forward and per-channel gradients
    keep = np.ones((batch, dim), bool)
    keep[0, 3] = keep[1, 5] = False
    assert_match(o[keep], ref[keep], RTOL_F32, "out, other channels")
    assert_match(to_f64(last)[keep], ref_last[keep], RTOL_F32, "last_state, other channels")
    for k in ("du", "ddelta", "dz"):
        assert_match(to_f64(res[k])[keep], gref[k][keep], RTOL_F32, f"{k}, other channels")
