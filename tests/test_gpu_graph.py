"""HIP graph capture of the training step.  The library enqueues only kernels
on the caller's stream (no memset, no allocation of its own when the caller
passes the workspaces, no synchronization), so a forward that saves
checkpoints, the backward from them and a decode step can be captured once
with torch.cuda.graph and replayed.  Each replay follows eager work that
overwrites the outputs and a synchronization, and is checked against the
eager run (the forward bit for bit; the backward, whose reductions use float
atomics, to rounding) and against the float64 oracle.  The step is captured in
one pass and in both segmented schemes (short segments with a summary pass,
long ones with the zero-start pass and its correction), the backward from the
forward's checkpoints and recomputing its states."""
import numpy as np
import pytest
import torch

import oracle
import scan_selective_fwd_amd as ms
import workloads as W
from parity_utils import RTOL, announce, assert_match, to_device, to_f64

pytestmark = pytest.mark.gpu


# (wid, batch, dim, N, L, segments, checkpoints): segments = 0 is the
# automatic choice (for these few channels the backward splits the sequence
# by itself; the forward runs in one pass); short segments (a summary pass);
# long segments (zero-start pass and correction), with the backward from the
# forward's checkpoints and recomputing its states
CASES = [(82, 2, 20, 16, 700, 0, True),
         (83, 1, 20, 16, 1189, 4, False),
         (84, 1, 20, 16, 4173, 2, True),
         (85, 1, 20, 16, 4173, 2, False)]


@pytest.mark.parametrize("wid,batch,dim,N,L,segments,use_ckpt", CASES)
def test_captured_step_replays_match_eager_and_oracle(wid, batch, dim, N, L, segments, use_ckpt):
    announce(f"graph capture wid={wid} shape=({batch},{dim},{N},{L}) f32 zoh "
             f"segments={segments} checkpoints={use_ckpt}")
    inp = W.make_inputs(wid, batch, dim, N, L, dtype="f32", bias="uniform", with_dout=True)
    f = W.inputs_f64(inp, "f32")
    t = to_device(inp, "f32")
    f32 = dict(dtype=torch.float32, device="cuda")
    out = torch.empty((batch, dim, L), **f32)
    state = torch.empty((batch, dim, N), **f32)      # final state, then one decode step
    ckpt = torch.empty(ms.checkpoint_shape(batch, dim, N, L), **f32) if use_ckpt else None
    step_out = torch.empty((batch, dim), **f32)
    nf = ms.fwd_workspace_bytes(batch, dim, N, L, torch.float32, segments=segments)
    fws = torch.empty(nf, dtype=torch.uint8, device="cuda") if nf else None
    bws = torch.empty(ms.bwd_workspace_bytes(batch, dim, N, L, torch.float32, segments=segments),
                      dtype=torch.uint8, device="cuda")
    step = {k: t[k][..., 0].contiguous() for k in ("u", "delta", "B", "C", "z")}

    def run():
        ms.scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"],
                    out=out, last_state=state, return_last_state=True, workspace=fws,
                    checkpoints=ckpt, segments=segments)
        grads = ms.scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                            t["delta_bias"], t["dout"], workspace=bws, checkpoints=ckpt,
                            segments=segments)
        ms.state_update(state, step["u"], step["delta"], t["A"], step["B"], step["C"], t["D"],
                        step["z"], t["delta_bias"], out=step_out)
        return grads

    eager_g = run()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in eager_g.items()}
    eager_out, eager_state, eager_step = out.clone(), state.clone(), step_out.clone()

    side = torch.cuda.Stream()            # warm-up on a side stream before capture
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        graph_g = run()
    torch.cuda.synchronize()

    for r in range(3):
        # eager work between replays: every output overwritten
        for buf in (out, state, step_out, *graph_g.values()):
            buf.fill_(float("nan"))
        if ckpt is not None:
            ckpt.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_out), f"replay {r}: forward output differs"
        assert torch.equal(state, eager_state), f"replay {r}: decode state differs"
        assert torch.equal(step_out, eager_step), f"replay {r}: decode output differs"
        assert set(graph_g) == set(eager)
        for k in eager:
            assert_match(to_f64(graph_g[k]), to_f64(eager[k]), 1e-5, f"replay {r} {k}")

    ref_out, ref_last = oracle.scan_fwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"],
                                        f["z"], f["delta_bias"])
    assert_match(to_f64(out), ref_out, RTOL["f32"], "graph out vs oracle")
    # the decode step continued from the forward's last state
    ref_step, ref_state = oracle.state_update(ref_last, f["u"][..., 0], f["delta"][..., 0],
                                              f["A"], f["B"][..., 0], f["C"][..., 0], f["D"],
                                              f["z"][..., 0], f["delta_bias"])
    assert_match(to_f64(state), ref_state, RTOL["f32"], "graph decode state vs oracle")
    assert_match(to_f64(step_out), ref_step, RTOL["f32"], "graph decode out vs oracle")
    ref = oracle.scan_bwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                          f["delta_bias"], f["dout"])
    for k in ref:
        assert_match(to_f64(graph_g[k]), ref[k], RTOL["f32"], f"graph {k} vs oracle")


@pytest.mark.parametrize("segments", [1, 4])
def test_captured_complex_step_replays_match_eager(segments):
    """The complex forward (saving checkpoints) and backward from them,
    captured and replayed three times, in one pass and in 4 segments, with
    packed-sequence flags: each replay matches the eager run and the oracle."""
    wid, batch, dim, N, L = 86, 1, 20, 16, 1100
    announce(f"graph capture complex wid={wid} shape=({batch},{dim},{N},{L}) "
             f"segments={segments}")
    inp = W.make_complex_inputs(wid, batch, dim, N, L, dtype="f32", with_dout=True)
    reset = W.make_resets(wid, batch, L, 100, 500, force=(0, 300))
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in inp.items()}
    rt = torch.from_numpy(reset).cuda()
    ckpt = torch.empty(ms.complex_checkpoint_shape(batch, dim, N, L), dtype=torch.complex64,
                       device="cuda")
    out = torch.empty((batch, dim, L), dtype=torch.float32, device="cuda")
    nf = ms.fwd_complex_workspace_bytes(batch, dim, N, L, segments)
    fws = torch.empty(max(nf, 1), dtype=torch.uint8, device="cuda")
    bws = torch.empty(max(ms.bwd_complex_workspace_bytes(batch, dim, N, L, segments), 1),
                      dtype=torch.uint8, device="cuda")

    def run():
        ms.scan_fwd_complex(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                            t["delta_bias"], out=out, checkpoints=ckpt, segments=segments,
                            workspace=fws, reset=rt)
        return ms.scan_bwd_complex(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                                   t["delta_bias"], t["dout"], checkpoints=ckpt,
                                   segments=segments, workspace=bws, reset=rt)

    eager = {k: v.clone() for k, v in run().items()}
    torch.cuda.synchronize()
    eager_out = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        graph_g = run()
    torch.cuda.synchronize()
    for r in range(3):
        for buf in (out, ckpt, *graph_g.values()):
            buf.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_out), f"replay {r}: forward output differs"
        for k in eager:
            a = torch.view_as_real(graph_g[k]) if graph_g[k].is_complex() else graph_g[k]
            e = torch.view_as_real(eager[k]) if eager[k].is_complex() else eager[k]
            assert_match(to_f64(a), to_f64(e), 1e-5, f"replay {r} {k}")
    ref, _ = oracle.scan_fwd_complex(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"],
                                     inp["D"], inp["z"], inp["delta_bias"], reset=reset)
    assert_match(to_f64(out), ref, RTOL["f32"], "graph complex out vs oracle")
