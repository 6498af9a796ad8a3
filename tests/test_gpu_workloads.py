"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (the default lanes-per-channel choice of the C ABI).

Workloads 2, 3 and 5 are compared element by element with the float64 oracle
over every channel (the oracle is threaded over channels).  Workload 4
(L = 1,048,576) is compared on sampled channels, which the oracle
regenerates row by row from the same seeds, including their final states.
The backward over a long sequence with workload 4's channels (segmented) is
compared on sampled channels too, with dout zero elsewhere so that the
gradients summed over channels (dB, dC) come from the sampled ones alone.
"""
import numpy as np
import pytest
import torch

import oracle
import scan_selective_fwd_amd as ms
import workloads as W
from parity_utils import RTOL, RTOL_F32, announce, assert_match, to_device, to_f64

pytestmark = pytest.mark.gpu


def _disc(d):
    return oracle.ZOH if d == "zoh" else oracle.EULER


def test_workload2_fwd_f32_full():
    announce("workload 2: fwd f32 (8,1536,16,2048) full compare")
    inp = W.workload_inputs(2)
    g = to_device(inp, "f32")
    out, last = ms.scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"],
                            g["delta_bias"], return_last_state=True)
    torch.cuda.synchronize()
    out2 = ms.scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"],
                       g["delta_bias"])
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "forward must be bitwise deterministic"
    f = W.inputs_f64(inp, "f32")
    del g
    ref, ref_last = oracle.scan_fwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                                    f["delta_bias"])
    e = assert_match(to_f64(out), ref, RTOL["f32"], "out")
    assert_match(to_f64(last), ref_last, RTOL["f32"], "last_state")
    print(f"workload 2 rel errors (max, l2): {e}", flush=True)


@pytest.mark.parametrize("disc", ["zoh", "euler"])
def test_workload3_fwd_bf16_full(disc):
    announce(f"workload 3: fwd bf16 (4,4096,16,4096) {disc} full compare")
    inp = W.workload_inputs(3)
    g = to_device(inp, "bf16")
    out, last = ms.scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"],
                            g["delta_bias"], disc=disc, return_last_state=True)
    torch.cuda.synchronize()
    f = W.inputs_f64(inp, "bf16")
    del g
    ref, ref_last = oracle.scan_fwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                                    f["delta_bias"], disc=_disc(disc))
    e = assert_match(to_f64(out), ref, RTOL["bf16"], "out")
    # the state never passes through bf16: the float32 bound applies
    e2 = assert_match(to_f64(last), ref_last, RTOL_F32, "last_state")
    print(f"workload 3 {disc} rel errors out {e} state {e2}", flush=True)


def test_workload4_long_sequence_sampled_channels():
    announce("workload 4: fwd bf16 (1,1536,16,1048576) sampled channels")
    w = W.WORKLOADS[4]
    inp = W.workload_inputs(4)
    g = to_device(inp, "bf16")
    del inp
    out, last = ms.scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"],
                            g["delta_bias"], return_last_state=True)
    torch.cuda.synchronize()
    chans = [0, 1, 511, 1024, 1534, 1535]
    got = to_f64(out[0, chans])
    got_last = to_f64(last[0, chans])
    del g, out
    sub = W.inputs_f64(W.make_inputs(4, w.batch, w.dim, w.dstate, w.seqlen, dtype="bf16",
                                     bias=w.bias, per_row=True, dim_subset=chans), "bf16")
    ref, ref_last = oracle.scan_fwd(sub["u"], sub["delta"], sub["A"], sub["B"], sub["C"],
                                    sub["D"], sub["z"], sub["delta_bias"])
    e = assert_match(got, ref[0], RTOL["bf16"], "out")
    e2 = assert_match(got_last, ref_last[0], RTOL_F32, "last_state")
    print(f"workload 4 rel errors out {e} state {e2}", flush=True)


def test_workload5_bwd_full():
    announce("workload 5: bwd bf16 inputs, f32 grads (2,5120,16,2048) full compare")
    inp = W.workload_inputs(5)
    g = to_device(inp, "bf16")
    res = ms.scan_bwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"],
                      g["delta_bias"], g["dout"])
    torch.cuda.synchronize()
    got = {k: to_f64(v) for k, v in res.items()}
    del g, res
    f = W.inputs_f64(inp, "bf16")
    ref = oracle.scan_bwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                          f["delta_bias"], f["dout"])
    assert set(got) == set(ref)
    errs = {}
    for k in ref:
        # float32 gradients from identical input bits: the float32 bound
        errs[k] = assert_match(got[k], ref[k], RTOL_F32, k)
    print(f"workload 5 rel errors {errs}", flush=True)


def test_long_sequence_bwd_segmented_sampled_channels():
    # batch 1, D 1536, 131072 steps: 1024 chunks over 96 channel groups, so
    # the automatic choice runs 32 segments of 32 chunks (the zero-start state
    # pass with its correction, then the reverse adjoint carry)
    wid, batch, dim, N, L = 68, 1, 1536, 16, 1 << 17
    announce(f"long-sequence bwd bf16 ({batch},{dim},{N},{L}) sampled channels")
    assert ms.bwd_workspace_bytes(batch, dim, N, L, torch.bfloat16) > \
        ms.bwd_workspace_bytes(batch, dim, N, L, torch.bfloat16, segments=1)
    inp = W.make_inputs(wid, batch, dim, N, L, dtype="bf16", bias="const", per_row=True,
                        with_dout=True)
    chans = [0, 1, 700, 1535]
    others = np.ones(dim, bool)
    others[chans] = False
    inp["dout"][:, others] = 0          # bf16 +0.0
    g = to_device(inp, "bf16")
    res = ms.scan_bwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"],
                      g["delta_bias"], g["dout"])
    torch.cuda.synchronize()
    for k in ("du", "ddelta", "dz"):
        assert not res[k][:, torch.from_numpy(others).cuda()].any(), k + ": unsampled channel"
    got = {k: to_f64(v[:, chans]) for k, v in res.items() if k in ("du", "ddelta", "dz")}
    got.update({k: to_f64(res[k][chans]) for k in ("dA", "dD", "ddelta_bias")})
    got.update({k: to_f64(res[k]) for k in ("dB", "dC")})
    del g, res
    sub = {k: (v[:, chans] if k in ("u", "delta", "z", "dout") else
               v[chans] if k in ("A", "D", "delta_bias") else v) for k, v in inp.items()}
    del inp
    f = W.inputs_f64(sub, "bf16")
    ref = oracle.scan_bwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                          f["delta_bias"], f["dout"])
    errs = {}
    for k in got:
        # float32 gradients from identical input bits: the float32 bound
        errs[k] = assert_match(got[k], ref[k], RTOL_F32, k)
    print(f"long-sequence bwd rel errors {errs}", flush=True)


def test_over_2e31_elements_sampled_channels():
    # batch 1, D 2064, 2^20 steps: 2.16e9 elements per (B, D, L) tensor, past
    # 2^31, so every element offset needs 64 bits.  129 channel groups split
    # into 16 segments each.  Forward and backward on sampled channels (the
    # last one in the last group); dout is zero elsewhere, so dB and dC come
    # from the sampled channels alone.
    wid, batch, dim, N, L = 93, 1, 2064, 16, 1 << 20
    assert batch * dim * L > 2 ** 31
    announce(f"over 2^31 elements: bf16 ({batch},{dim},{N},{L}) sampled channels")
    inp = W.make_inputs(wid, batch, dim, N, L, dtype="bf16", bias="const", per_row=True,
                        with_dout=True)
    chans = [0, 1031, 2063]
    others = np.ones(dim, bool)
    others[chans] = False
    inp["dout"][:, others] = 0
    g = to_device(inp, "bf16")
    out, last = ms.scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"],
                            g["delta_bias"], return_last_state=True)
    torch.cuda.synchronize()
    got_out = to_f64(out[:, chans])
    got_last = to_f64(last[:, chans])
    del out
    res = ms.scan_bwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"],
                      g["delta_bias"], g["dout"])
    torch.cuda.synchronize()
    got = {k: to_f64(v[:, chans]) for k, v in res.items() if k in ("du", "ddelta", "dz")}
    got.update({k: to_f64(res[k][chans]) for k in ("dA", "dD", "ddelta_bias")})
    got.update({k: to_f64(res[k]) for k in ("dB", "dC")})
    del g, res
    sub = {k: (v[:, chans] if k in ("u", "delta", "z", "dout") else
               v[chans] if k in ("A", "D", "delta_bias") else v) for k, v in inp.items()}
    del inp
    f = W.inputs_f64(sub, "bf16")
    ref_out, ref_last = oracle.scan_fwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"],
                                        f["z"], f["delta_bias"])
    e = assert_match(got_out, ref_out, RTOL["bf16"], "out")
    e2 = assert_match(got_last, ref_last, RTOL_F32, "last_state")
    ref = oracle.scan_bwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                          f["delta_bias"], f["dout"])
    errs = {k: assert_match(got[k], ref[k], RTOL_F32, k) for k in got}
    print(f"over-2^31 rel errors out {e} state {e2} grads {errs}", flush=True)


def test_workload2_step_as_benchmarked_full():
    """The configuration the benchmark times, at full size: workload 2 in
    float32, the forward saving chunk checkpoints and the last state, then
    the backward from those checkpoints, each with the library's automatic
    launch choice (one pass at this shape), every output against the oracle
    per row."""
    announce("workload 2: fwd with checkpoints + bwd from them, f32 (8,1536,16,2048)")
    w = W.WORKLOADS[2]
    assert ms.fwd_workspace_bytes(w.batch, w.dim, w.dstate, w.seqlen, torch.float32) == 0, \
        "the forward runs in one pass at this shape"
    assert ms.bwd_workspace_bytes(w.batch, w.dim, w.dstate, w.seqlen, torch.float32) == \
        ms.bwd_workspace_bytes(w.batch, w.dim, w.dstate, w.seqlen, torch.float32, segments=1), \
        "the backward runs in one pass at this shape"
    inp = W.workload_inputs(2, with_dout=True)
    g = to_device(inp, "f32")
    ck = torch.full(ms.checkpoint_shape(w.batch, w.dim, w.dstate, w.seqlen), float("nan"),
                    device="cuda")
    out, last = ms.scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"],
                            g["delta_bias"], return_last_state=True, checkpoints=ck)
    res = ms.scan_bwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"],
                      g["delta_bias"], g["dout"], checkpoints=ck)
    torch.cuda.synchronize()
    assert not torch.isnan(ck).any()
    got_out, got_last = to_f64(out), to_f64(last)
    got = {k: to_f64(v) for k, v in res.items()}
    del g, res, out, last, ck
    f = W.inputs_f64(inp, "f32")
    del inp
    ref, ref_last = oracle.scan_fwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                                    f["delta_bias"])
    e = assert_match(got_out, ref, RTOL["f32"], "out")
    e2 = assert_match(got_last, ref_last, RTOL_F32, "last_state")
    del ref, ref_last
    gref = oracle.scan_bwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                           f["delta_bias"], f["dout"])
    assert set(got) == set(gref)
    errs = {k: assert_match(got[k], gref[k], RTOL_F32, k) for k in gref}
    print(f"workload 2 step rel errors out {e} state {e2} grads {errs}", flush=True)


def test_workload5_gradients_directional_finite_differences():
    """Workload 5's GPU gradients against central finite differences of the
    float64 oracle's forward: for a random direction v over every input,
    <grad, v> must equal (l(x + eps v) - l(x - eps v)) / (2 eps), with
    l = sum(dout * out) at the inputs' exact (bf16-widened) values; the same
    for a direction in each input alone."""
    announce("workload 5: directional central differences of the GPU gradients")
    inp = W.workload_inputs(5)
    g = to_device(inp, "bf16")
    res = ms.scan_bwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"],
                      g["delta_bias"], g["dout"])
    torch.cuda.synchronize()
    grads = {k: to_f64(v) for k, v in res.items()}
    del g, res
    f = W.inputs_f64(inp, "bf16")
    del inp
    names = dict(u="du", delta="ddelta", A="dA", B="dB", C="dC", D="dD", z="dz",
                 delta_bias="ddelta_bias")
    rng = np.random.default_rng([5, 99])
    v = {k: rng.standard_normal(f[k].shape) for k in names}

    def loss(shift):
        x = {k: (f[k] + shift[k] if k in shift else f[k]) for k in f}
        out, _ = oracle.scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"],
                                 x["delta_bias"])
        return float(np.sum(x["dout"] * out))

    eps = 1e-3
    checks = [("all", list(names))] + [(k, [k]) for k in names]
    for label, keys in checks:
        dot = sum(float(np.sum(grads[names[k]] * v[k])) for k in keys)
        scale = sum(float(np.sum(np.abs(grads[names[k]] * v[k]))) for k in keys)
        lp = loss({k: eps * v[k] for k in keys})
        lm = loss({k: -eps * v[k] for k in keys})
        fd = (lp - lm) / (2 * eps)
        rel = abs(dot - fd) / scale
        print(f"direction {label}: <grad,v> {dot:.9e} central difference {fd:.9e} "
              f"rel {rel:.2e}", flush=True)
        assert rel <= 1e-4, (label, dot, fd, rel)
