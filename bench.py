"""Benchmark of the selective-scan hot path on one MI355X.

One step = the whole hot path over one batch of synthetic input at the
Mamba-130M layer shape (batch 8, D = 1536, N = 16, L = 2048, float32, ZOH,
softplus, D skip and SiLU gate): mamba_scan_fwd (with the final state), then
mamba_scan_bwd (states recomputed from the inputs), then one
mamba_state_update decode step continuing from the final state.

Prints ONE JSON line.  `value` is the achieved algorithmic HBM throughput of
the step (bytes every call must move at least once, divided by the step
time), in GB/s; the roofline object is for the dominant call, timed live with
HIP events on the stream the kernels run on; cpu_baseline is the float64 CPU
oracle on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2|3|4|5]
                       [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E peak, GB/s


def algorithmic_bytes(w, call: str) -> float:
    """Bytes a call must move at least once (inputs read, outputs written);
    the expanded (B, L, D, N) tensors never touch memory."""
    es = 4 if w.dtype == "f32" else 2
    ct = w.batch * w.dim * w.seqlen
    bc = 2 * w.batch * w.dstate * w.seqlen * es          # B and C
    params = w.dim * w.dstate * 4 + 2 * w.dim * 4        # A, D, delta_bias
    state = w.batch * w.dim * w.dstate * 4
    if call == "fwd":      # read u, delta, z; write out; write last_state
        return 4 * ct * es + bc + params + state
    if call == "bwd":      # read u, delta, z, dout; write du, ddelta, dz (f32); dB, dC, dA, dD, dbias
        return 4 * ct * es + 3 * ct * 4 + bc + 2 * w.batch * w.dstate * w.seqlen * 4 + 2 * params
    if call == "step":     # state read + write; u, delta, z, out per channel; B, C per batch row
        return 2 * state + 4 * w.batch * w.dim * es + 2 * w.batch * w.dstate * es + params
    raise ValueError(call)


def gpu_inputs(w, torch, with_dout):
    import workloads as W
    inp = W.workload_inputs(w.wid, with_dout=with_dout)
    dev = "cuda"
    out = {}
    for k, v in inp.items():
        if k in ("u", "delta", "B", "C", "z", "dout") and w.dtype == "bf16":
            out[k] = torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(
                torch.bfloat16).to(dev)
        else:
            out[k] = torch.from_numpy(np.ascontiguousarray(v)).to(dev)
    return out


def cpu_baseline(w, calls):
    """The float64 oracle on a bounded sample of the same workload: the first
    `nb` batch rows (all D channels of each), running the same calls."""
    import oracle
    import workloads as W
    nb = 2 if w.batch >= 2 else 1
    L = w.seqlen
    if w.wid == 4:
        L = 65536   # a prefix of the long sequence keeps the sample ~10 s
    inp = W.make_inputs(w.wid, nb, w.dim, w.dstate, L, dtype=w.dtype, bias=w.bias,
                        with_dout=True, per_row=w.per_row)
    f = W.inputs_f64(inp, w.dtype)
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    if "fwd" in calls:
        oracle.scan_fwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                        f["delta_bias"], threads=threads)
    if "bwd" in calls:
        oracle.scan_bwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                        f["delta_bias"], f["dout"], threads=threads)
    if "step" in calls:
        st = np.zeros((nb, w.dim, w.dstate))
        oracle.state_update(st, f["u"][..., 0], f["delta"][..., 0], f["A"], f["B"][..., 0],
                            f["C"][..., 0], f["D"], f["z"][..., 0], f["delta_bias"])
    dt = time.perf_counter() - t0
    import copy
    ws = copy.copy(w)
    ws.batch, ws.seqlen = nb, L
    nbytes = sum(algorithmic_bytes(ws, c) for c in calls)
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{nb} of {w.batch} batch rows x {w.dim} channels x {L} steps "
                      f"({'+'.join(calls)}), {dt:.2f} s wall",
            "channel_tokens_per_s": round(nb * w.dim * L / dt, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2, choices=[2, 3, 4, 5])
    ap.add_argument("--disc", default="zoh", choices=["zoh", "euler"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calls", default=None,
                    help="comma list of calls to time instead of the full step (fwd,bwd,step)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the selective scan shards over channels with no "
              "communication (see DESIGN.md); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import scan_selective_fwd_amd as ms
    import workloads as W

    w = W.WORKLOADS[args.workload]
    calls = {2: ["fwd", "bwd", "step"], 3: ["fwd"], 4: ["fwd"], 5: ["bwd"]}[w.wid]
    if args.calls:
        calls = args.calls.split(",")
    g = gpu_inputs(w, torch, "bwd" in calls)
    ws = None
    if "bwd" in calls:
        ws = torch.empty(ms.bwd_workspace_bytes(w.batch, w.dim, w.dstate, w.seqlen,
                                                g["u"].dtype), dtype=torch.uint8, device="cuda")
    sdt = g["u"].dtype
    t_last = torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device="cuda")
    t_out = torch.empty_like(g["u"])
    step_args = {k: g[k][..., 0].contiguous() for k in ("u", "delta", "B", "C", "z")}
    step_out = torch.empty((w.batch, w.dim), dtype=sdt, device="cuda")

    def run_call(c):
        if c == "fwd":
            ms.scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"],
                        g["delta_bias"], disc=args.disc, out=t_out, last_state=t_last,
                        return_last_state=True)
        elif c == "bwd":
            ms.scan_bwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"],
                        g["delta_bias"], g["dout"], disc=args.disc, workspace=ws)
        else:   # decode step continuing from the forward's final state, in place
            ms.state_update(t_last, step_args["u"], step_args["delta"], g["A"], step_args["B"],
                            step_args["C"], g["D"], step_args["z"], g["delta_bias"],
                            disc=args.disc, out=step_out)

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        for c in calls:
            run_call(c)
    torch.cuda.synchronize()

    ev = {c: [] for c in calls}
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        for c in calls:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run_call(c)
            e1.record(stream)
            ev[c].append((e0, e1))
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    call_ms = {c: float(np.mean([a.elapsed_time(b) for a, b in ev[c]])) for c in calls}

    step_bytes = sum(algorithmic_bytes(w, c) for c in calls)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    ct = w.batch * w.dim * w.seqlen
    dom = max((c for c in calls if c != "step"), key=lambda c: call_ms[c])
    dom_bytes = algorithmic_bytes(w, dom)
    achieved = dom_bytes / (call_ms[dom] * 1e-3) / 1e9
    kernels = {"fwd": "scan_fwd_kernel", "bwd": "scan_fwd_kernel(states) + scan_bwd_kernel + "
               "bwd_reduce kernels", "step": "state_update_kernel"}
    per_call = {c: {"ms": round(call_ms[c], 5),
                    "algorithmic_MB": round(algorithmic_bytes(w, c) / 1e6, 3),
                    "GB/s": round(algorithmic_bytes(w, c) / (call_ms[c] * 1e-3) / 1e9, 1)}
                for c in calls}
    res = {
        "metric": "selective-scan fwd/bwd achieved HBM GB/s (% peak); channel-tokens/s, "
                  "D=1536 L=2048",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.dtype == "f32" else "bf16-in/f32-compute",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {'+'.join(calls)} ({args.disc})", "batch": w.batch,
                   "dim": w.dim, "dstate": w.dstate, "seqlen": w.seqlen, "dtype": w.dtype,
                   "disc": args.disc, "delta_softplus": True, "D": True, "z": True,
                   "delta_bias": w.bias},
        "pct_of_hbm_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "channel_tokens_per_s": round(ct / (ms_per_step * 1e-3), 1),
        "per_call": per_call,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": kernels[dom], "call": f"mamba_scan_{dom}",
                     "algorithmic_bytes_per_launch": int(dom_bytes),
                     "avg_launch_ms": round(call_ms[dom], 5)},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, calls)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
