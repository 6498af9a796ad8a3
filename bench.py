"""Benchmark of the selective-scan hot path on one MI355X.

One step = the whole hot path over one batch of synthetic input at the
Mamba-130M layer shape (batch 8, D = 1536, N = 16, L = 2048, float32, ZOH,
softplus, D skip and SiLU gate), as a training framework runs it: the
forward (with the final state, saving the state entering every 128-step
chunk), then the backward (every state inside the chunks recomputed from
those checkpoints and the inputs), then one decode step continuing from the
final state.  --no-checkpoints makes the backward recompute the chunk
states too.

Prints ONE JSON line.  `value` is the achieved algorithmic HBM throughput of
the step (bytes every call must move at least once, divided by the step
time), in GB/s.  `roofline` is for the kernel that takes most of the step,
timed alone with HIP events that the library records around it on the
stream it runs on; its `traffic` (HBM bytes per launch) and `issue` (vector
instructions per (t, n) and the issue rate against the FMA rate reachable at
3 waves per SIMD) come from the committed counter summaries of that kernel
when the kernel's sources are unchanged since they were taken.
`cpu_baseline` is the float64 CPU oracle on a bounded sample of the same
workload.  `per_call.<call>.cold` times each scan kernel again with the
caches flushed before every launch (a 1 GiB buffer is written first, more
than the L2s and the 256 MB last-level cache hold): median, p10 and p90 of
--cold-iters launches.  `ms_per_step_graph` is the same step captured once
into a HIP graph and replayed (context: the launch gaps between the calls
removed; `value` stays the plain calls).  `per_config` times the other
specified configurations once each (the Mamba-1.4B layer forward in bf16,
ZOH and Euler; the 2^20-step forward; the bf16 backward as a plain call,
whose state-recompute pass is included), with inputs drawn on the device.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2|3|4|5]
                       [--disc zoh|euler] [--calls fwd,bwd,step] [--no-cpu-baseline]
                       [--copy-calibration] [--cold-iters N] [--no-per-config]
       python bench.py --summarize-counters counter_collection.csv [...]
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E peak, GB/s
# float32 vector peak: the chip's published 157.3 TFLOP/s (256 CUs, 2.4 GHz).
# Plain (non-packed) FMAs issue at most one wave64 instruction per SIMD about
# every 2.4 cycles even with many waves per SIMD (measured on an MI355X), so
# the published figure is the honest ceiling for these kernels too, although
# they use no packed FP32.
PEAK_F32_TFLOPS = 157.3
# Algorithmic float32 work per (t, n) (an exp counts as one flop):
#   forward : dA 1, exp 1, ZOH Bbar*u 4, h update 2, y accumulate 2       = 10
#   backward: forward replay incl. y 10, adjoint 3, ddelta 6, dA 5, du 5,
#             dB 2, dC 2                                                  = 33 (+1 exp)
FLOPS_PER_TN = {"fwd": 10, "bwd": 34}
# Euler Bbar u = delta B u: 2 flops instead of the ZOH coefficient's 4 in the
# forward; the backward loses the coefficient's A-derivative (about 5).
FLOPS_PER_TN_EULER = {"fwd": 8, "bwd": 30}


def flops_per_tn(call: str, disc: str) -> int:
    return (FLOPS_PER_TN if disc == "zoh" else FLOPS_PER_TN_EULER)[call]
CSRC = os.path.join(ROOT, "scan_selective_fwd_amd", "csrc")
# Sources each timed kernel is compiled from (its counter summary is void
# once any of them changes).
KERNEL_SOURCES = {
    "scan_fwd_kernel": ["scan_fwd_impl.hpp", "tile_stage.hpp", "device_common.hpp",
                        "kernels.hpp", "scan_fwd_f32.hip", "scan_fwd_bf16.hip"],
    "scan_bwd_kernel": ["scan_bwd_impl.hpp", "tile_stage.hpp", "device_common.hpp",
                        "kernels.hpp", "scan_bwd_f32_n16.hip", "scan_bwd_bf16_n16.hip"],
}
COPY_BYTES = 1 << 30   # calibration copy: reads and writes 1 GiB
FLUSH_BYTES = 1 << 30  # written before each cold launch: evicts L2 and the last-level cache


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
    if call == "cfwd":     # complex forward: u, delta, z read, out written; complex B, C, A, state
        return 4 * ct * es + 2 * w.batch * w.dstate * w.seqlen * 8 + 2 * params + 2 * state
    if call == "cbwd":     # complex backward: as bwd with complex B, C, dB, dC
        return (4 * ct * es + 3 * ct * 4 + 4 * w.batch * w.dstate * w.seqlen * 8 + 2 * params
                + 2 * state)
    if call == "conv_fwd":  # read x, write u; taps and bias
        return 2 * ct * es + 5 * w.dim * 4
    if call == "conv_bwd":  # read x and du (f32), write dx (f32); dw, db
        return ct * (es + 8) + 10 * w.dim * 4
    raise ValueError(call)


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel: str, workload: str):
    """HBM bytes per launch from profiles/traffic_<kernel>_<workload>.txt, or
    None when there is no such summary or the kernel changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != kernel_source_hash(kernel):
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def committed_issue(kernel: str, workload: str):
    """The kernel's vector-issue figures from profiles/valu_scan_kernels_<workload>.txt
    (VALU instructions and transcendentals per (t, n), and the issue rate as a
    fraction of what independent FMAs reach at the kernels' 3 waves per SIMD,
    transcendentals at their issue cost), or None when the kernel changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"valu_scan_kernels_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields, cur = {}, None
    with open(path) as f:
        for line in f:
            if line.startswith("kernel:"):
                cur = line.split()[1]
            elif cur == kernel and ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != kernel_source_hash(kernel):
        return None
    try:
        return {"valu_per_state_step": float(fields["valu_per_state_step"]),
                "trans_per_state_step": float(fields["trans_per_state_step"]),
                "issue_frac_vs_fma_3_waves": float(fields["fma_equivalent_vs_3_waves"]),
                "waves_per_simd": 3}
    except (KeyError, ValueError):
        return None


def summarize_counters(paths):
    """Per-kernel mean of every counter in rocprofv3 counter_collection.csv
    files (one row per dispatch and counter)."""
    acc = {}
    for p in paths:
        with open(p) as f:
            for row in csv.DictReader(f):
                name = row.get("Kernel_Name", "?")
                key = (name.split("(")[0][:120], row["Counter_Name"])
                d = acc.setdefault(key, {})
                d.setdefault(row["Dispatch_Id"], 0.0)
                d[row["Dispatch_Id"]] += float(row["Counter_Value"])
    for (name, counter), per_dispatch in sorted(acc.items()):
        v = list(per_dispatch.values())
        print(f"{counter:14s} dispatches={len(v):4d} mean={np.mean(v):16.1f} "
              f"min={np.min(v):16.1f} max={np.max(v):16.1f}  {name}")


def traffic_summary(kernel, workload, fetch_csv, write_csv):
    """Prints the HBM traffic summary of `kernel` (scan_fwd_kernel or
    scan_bwd_kernel) from two rocprofv3 counter runs of the same bench
    command with --copy-calibration, one with FETCH_SIZE and one with
    WRITE_SIZE.  The 1 GiB device copy the process starts with gives the
    scale from counter KiB to bytes; the kernel's figures are the mean per
    dispatch of its most expensive template instance (the TINY copy of the
    backward exits at once)."""
    def per_dispatch(path, counter):
        acc = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                d = acc.setdefault(row["Kernel_Name"], {})
                d[row["Dispatch_Id"]] = d.get(row["Dispatch_Id"], 0.0) + float(row["Counter_Value"])
        return acc

    fetch, write = per_dispatch(fetch_csv, "FETCH_SIZE"), per_dispatch(write_csv, "WRITE_SIZE")

    def pick(acc):
        mine = {n: v for n, v in acc.items() if f"mscan::{kernel}<" in n}
        name = max(mine, key=lambda n: np.mean(list(mine[n].values())))
        return name, list(mine[name].values())

    def copy_kib(acc):
        return max(max(v.values()) for n, v in acc.items() if "copyBuffer" in n)

    name, fv = pick(fetch)
    _, wv = pick(write)
    cf, cw = copy_kib(fetch), copy_kib(write)
    fscale, wscale = COPY_BYTES / (cf * 1024), COPY_BYTES / (cw * 1024)
    rd = float(np.mean(fv)) * 1024 * fscale
    wr = float(np.mean(wv)) * 1024 * wscale
    import workloads as W
    wid = int(workload[1:].split("_")[0])
    call = {"scan_fwd_kernel": "fwd", "scan_bwd_kernel": "bwd"}[kernel]
    alg = algorithmic_bytes(W.WORKLOADS[wid], call)
    print(f"kernel: {kernel}\ninstance: {name.split('(')[0]}\nworkload: {workload}\n"
          f"source_sha256: {kernel_source_hash(kernel)}\ndispatches: {len(fv)}\n"
          f"fetch_kib_per_dispatch: {np.mean(fv):.1f}\nwrite_kib_per_dispatch: {np.mean(wv):.1f}\n"
          f"copy_1GiB_fetch_kib: {cf:.1f}\ncopy_1GiB_write_kib: {cw:.1f}\n"
          f"fetch_scale: {fscale:.4f}\nwrite_scale: {wscale:.4f}\n"
          f"read_bytes_per_launch: {rd:.0f}\nwritten_bytes_per_launch: {wr:.0f}\n"
          f"traffic_bytes_per_launch: {rd + wr:.0f}\nalgorithmic_bytes_per_launch: {alg:.0f}\n"
          f"traffic_over_algorithmic: {(rd + wr) / alg:.3f}")


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


def cpu_baseline(w, calls, disc, budget_s=10.0):
    """The float64 oracle on a bounded sample of the same workload, on the
    host cores available to the process.  The sample is the whole batch at
    the full sequence length (a 65536-step prefix of every channel for the
    1M-step workload); passes repeat until `budget_s` seconds have elapsed."""
    import oracle
    import workloads as W
    L = min(w.seqlen, 65536)
    nb = w.batch
    inp = W.make_inputs(w.wid, nb, w.dim, w.dstate, L, dtype=w.dtype, bias=w.bias,
                        with_dout=True, per_row=w.per_row)
    f = W.inputs_f64(inp, w.dtype)
    dcode = oracle.ZOH if disc == "zoh" else oracle.EULER
    threads = oracle.default_threads()
    passes = 0
    t0 = time.perf_counter()
    while True:
        if "fwd" in calls:
            oracle.scan_fwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                            f["delta_bias"], disc=dcode, threads=threads)
        if "bwd" in calls:
            oracle.scan_bwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                            f["delta_bias"], f["dout"], disc=dcode, threads=threads)
        if "step" in calls:
            st = np.zeros((nb, w.dim, w.dstate))
            oracle.state_update(st, f["u"][..., 0], f["delta"][..., 0], f["A"], f["B"][..., 0],
                                f["C"][..., 0], f["D"], f["z"][..., 0], f["delta_bias"],
                                disc=dcode)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s or passes >= 20:
            break
    import copy
    ws = copy.copy(w)
    ws.batch, ws.seqlen = nb, L
    nbytes = passes * sum(algorithmic_bytes(ws, c) for c in calls)
    # one core: the same calls on the first 64 channels of the first batch row
    sub = {k: (v[:1, :64] if k in ("u", "delta", "z", "dout") else
               v[:1] if k in ("B", "C") else v[:64] if k in ("A", "D", "delta_bias") else v)
           for k, v in f.items()}
    t1 = time.perf_counter()
    if "fwd" in calls:
        oracle.scan_fwd(sub["u"], sub["delta"], sub["A"], sub["B"], sub["C"], sub["D"], sub["z"],
                        sub["delta_bias"], disc=dcode, threads=1)
    if "bwd" in calls:
        oracle.scan_bwd(sub["u"], sub["delta"], sub["A"], sub["B"], sub["C"], sub["D"], sub["z"],
                        sub["delta_bias"], sub["dout"], disc=dcode, threads=1)
    dt1 = time.perf_counter() - t1
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{passes} pass(es) over {nb} batch rows x {w.dim} channels x {L} steps "
                      f"({'+'.join(calls)}, float64), {dt:.2f} s wall",
            "channel_tokens_per_s": round(passes * nb * w.dim * L / dt, 1),
            "cpu_model": _cpu_model(),
            "single_core_channel_tokens_per_s": round(64 * L / dt1, 1)}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def copy_bandwidth(torch, nbytes=COPY_BYTES, iters=10):
    """Achieved rate of a plain device-to-device copy (bytes read + written
    per second): the streaming ceiling the scan kernels are compared with."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(iters):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * nbytes * iters / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return gbs


# The pages' scan benchmark shape (batch 1, D 1024, N 16, bf16; sequence
# lengths 2^9 .. 2^19) and the times they read for the fused scan on an A100
# (paper-graph-ui summary, "Speed and Memory Benchmarks", Figure 8 left;
# context only: other hardware, and the page does not say whether forward or
# forward + backward).
SWEEP_COMPLEX_MAX_LOG2 = 17
SWEEP_PAGES_MS = {32768: 2.0, 131072: 10.0}


def sweep(torch, ms_lib, W, steps=10):
    """Forward and backward time over the sequence lengths of the pages'
    scan benchmark, inputs drawn like workload 1; each call with its default
    (automatic) sequence segmentation.  Up to 2^SWEEP_COMPLEX_MAX_LOG2 steps
    the complex-valued forward and backward are timed at the same shape."""
    rows = []
    for e in range(9, 20):
        L = 1 << e
        inp = W.make_inputs(9, 1, 1024, 16, L, dtype="bf16", bias="const", with_dout=True)
        g = {}
        for k, v in inp.items():
            if k in ("u", "delta", "B", "C", "z", "dout"):
                g[k] = torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(
                    torch.bfloat16).cuda()
            else:
                g[k] = torch.from_numpy(np.ascontiguousarray(v)).cuda()
        nfws = ms_lib.fwd_workspace_bytes(1, 1024, 16, L, torch.bfloat16)
        fws = torch.empty(nfws, dtype=torch.uint8, device="cuda") if nfws else None
        out = torch.empty_like(g["u"])

        def fwd():
            ms_lib.scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"],
                            g["delta_bias"], out=out, workspace=fws)

        nbws = ms_lib.bwd_workspace_bytes(1, 1024, 16, L, torch.bfloat16)
        bws = torch.empty(nbws, dtype=torch.uint8, device="cuda")

        def bwd():
            ms_lib.scan_bwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"],
                            g["delta_bias"], g["dout"], workspace=bws)

        row = {"L": L}
        for name, fn in (("fwd", fwd), ("bwd", bwd)):
            fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) / steps
            row[f"{name}_ms"] = round(t, 4)
            row[f"{name}_channel_tokens_per_s"] = round(1024 * L / (t * 1e-3), 1)
        del g, out, fws, bws
        if e <= SWEEP_COMPLEX_MAX_LOG2:
            # the complex-valued calls (S4D-Lin A, complex64 B and C), same shape
            ci = W.make_complex_inputs(9, 1, 1024, 16, L, dtype="bf16", with_dout=True)
            cg = {}
            for k, v in ci.items():
                if v.dtype == np.uint16:
                    cg[k] = torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(
                        torch.bfloat16).cuda()
                else:
                    cg[k] = torch.from_numpy(np.ascontiguousarray(v)).cuda()
            del ci

            def cfwd():
                ms_lib.scan_fwd_complex(cg["u"], cg["delta"], cg["A"], cg["B"], cg["C"], cg["D"],
                                        cg["z"], cg["delta_bias"])

            def cbwd():
                ms_lib.scan_bwd_complex(cg["u"], cg["delta"], cg["A"], cg["B"], cg["C"], cg["D"],
                                        cg["z"], cg["delta_bias"], cg["dout"])

            for name, fn in (("complex_fwd", cfwd), ("complex_bwd", cbwd)):
                fn()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(steps):
                    fn()
                e1.record()
                torch.cuda.synchronize()
                row[f"{name}_ms"] = round(e0.elapsed_time(e1) / steps, 4)
            del cg
        if L in SWEEP_PAGES_MS:
            row["pages_a100_ms"] = SWEEP_PAGES_MS[L]
        rows.append(row)
    return rows


# The other specified configurations, timed after the headline step with
# inputs drawn on the device: (tag, workload id, discretization, call).
PER_CONFIG = [("w3_zoh", 3, "zoh", "fwd"), ("w3_euler", 3, "euler", "fwd"),
              ("w4_zoh", 4, "zoh", "fwd"), ("w5_zoh", 5, "zoh", "bwd")]


def per_config(torch, ms_lib, W, iters=10):
    """Each of PER_CONFIG on its own: `iters` timed calls after two untimed
    ones, events around every call and around its main kernel (the output
    kernel of the forward, the reverse-scan kernel of the backward).  The
    backward is the plain call: no checkpoints, so it includes the pass that
    recomputes the chunk-start states.  Returns {tag: {...}}."""
    res = {}
    for tag, wid, disc, call in PER_CONFIG:
        w = W.WORKLOADS[wid]
        g = W.device_inputs(w, torch, with_dout=call == "bwd")
        sdt = g["u"].dtype
        if call == "fwd":
            nws = ms_lib.fwd_workspace_bytes(w.batch, w.dim, w.dstate, w.seqlen, sdt)
            ws = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws else None
            out = torch.empty_like(g["u"])
            last = torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device="cuda")

            def fn(timing=None):
                ms_lib.scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"],
                                g["delta_bias"], disc=disc, out=out, last_state=last,
                                return_last_state=True, workspace=ws, timing=timing)
        else:
            ws = torch.empty(ms_lib.bwd_workspace_bytes(w.batch, w.dim, w.dstate, w.seqlen, sdt),
                             dtype=torch.uint8, device="cuda")

            def fn(timing=None):
                ms_lib.scan_bwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"],
                                g["delta_bias"], g["dout"], disc=disc, workspace=ws,
                                timing=timing)
        n = max(3, iters if w.seqlen <= 65536 else iters // 2)
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for i in range(n):
            ev[i][0].record()
            fn(kev[i])
            ev[i][1].record()
        torch.cuda.synchronize()
        call_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        kern_ms = float(np.mean([a.elapsed_time(b) for a, b in kev]))
        nbytes = algorithmic_bytes(w, call)
        flops = flops_per_tn(call, disc) * w.batch * w.dim * w.seqlen * w.dstate
        res[tag] = {"workload": w.name, "call": f"mamba_scan_{call}", "disc": disc,
                    "batch": w.batch, "dim": w.dim, "dstate": w.dstate, "seqlen": w.seqlen,
                    "dtype": w.dtype, "iters": n,
                    "ms": round(call_ms, 5), "kernel_ms": round(kern_ms, 5),
                    "algorithmic_MB": round(nbytes / 1e6, 3),
                    "GB/s": round(nbytes / (call_ms * 1e-3) / 1e9, 1),
                    "hbm_frac": round(nbytes / (call_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                    "alu_frac": round(flops / (call_ms * 1e-3) / 1e12 / PEAK_F32_TFLOPS, 4),
                    "channel_tokens_per_s": round(w.batch * w.dim * w.seqlen / (call_ms * 1e-3),
                                                  1)}
        del g, ws, fn
        if call == "fwd":
            del out, last
        torch.cuda.empty_cache()
    return res


def copy_calibration(torch):
    """A plain device copy of known size, so that counter runs over this
    process can scale FETCH_SIZE / WRITE_SIZE to bytes."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2, choices=[2, 3, 4, 5])
    ap.add_argument("--disc", default="zoh", choices=["zoh", "euler"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--varlen", action="store_true",
                    help="pack variable-length sequences (lengths uniform in 64..1024) into each "
                         "row, with reset flags at their starts")
    ap.add_argument("--no-checkpoints", action="store_true",
                    help="the forward saves no chunk states; the backward recomputes them")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a 1 GiB device copy first (for counter calibration)")
    ap.add_argument("--calls", default=None,
                    help="comma list of calls to time instead of the full step (fwd,bwd,step)")
    ap.add_argument("--cold-iters", type=int, default=50,
                    help="launches of each scan kernel timed with the caches flushed before "
                         "each (0: skip)")
    ap.add_argument("--sweep", action="store_true",
                    help="time the forward and backward over sequence lengths 2^9..2^19 "
                         "at the pages' scan benchmark shape; one JSON line")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip timing the step replayed from a captured HIP graph")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip timing the other specified configurations (per_config)")
    ap.add_argument("--summarize-counters", nargs="+", default=None, metavar="CSV")
    ap.add_argument("--traffic-summary", nargs=4, default=None,
                    metavar=("KERNEL", "WORKLOAD", "FETCH_CSV", "WRITE_CSV"),
                    help="print the HBM traffic summary of a kernel from FETCH_SIZE and "
                         "WRITE_SIZE counter runs (workload tag as w2_zoh)")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: every (batch, channel) recurrence is "
              "independent, so the scan shards over channels or batch rows with no exchange "
              "in the forward; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import scan_selective_fwd_amd as ms
    import workloads as W

    if args.sweep:
        print(json.dumps({"sweep": "the pages' scan benchmark shape: batch 1, D 1024, N 16, "
                                   "bf16 inputs, ZOH, softplus, D and z",
                          "rows": sweep(torch, ms, W)}), flush=True)
        return
    w = W.WORKLOADS[args.workload]
    calls = {2: ["fwd", "bwd", "step"], 3: ["fwd"], 4: ["fwd"], 5: ["bwd"]}[w.wid]
    if args.calls:
        calls = args.calls.split(",")
    if args.copy_calibration:
        copy_calibration(torch)
    g = gpu_inputs(w, torch, "bwd" in calls or "cbwd" in calls)
    ws = None
    if "bwd" in calls:
        ws = torch.empty(ms.bwd_workspace_bytes(w.batch, w.dim, w.dstate, w.seqlen,
                                                g["u"].dtype), dtype=torch.uint8, device="cuda")
    sdt = g["u"].dtype
    rst = None
    if args.varlen:
        rst = torch.from_numpy(W.make_resets(w.wid, w.batch, w.seqlen, 64, 1024)).cuda()
    fws = None
    nfws = ms.fwd_workspace_bytes(w.batch, w.dim, w.dstate, w.seqlen, sdt)
    if nfws:
        fws = torch.empty(nfws, dtype=torch.uint8, device="cuda")
    t_last = torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device="cuda")
    ckpt = None
    if "fwd" in calls and "bwd" in calls and not args.no_checkpoints:
        ckpt = torch.empty(ms.checkpoint_shape(w.batch, w.dim, w.dstate, w.seqlen),
                           dtype=torch.float32, device="cuda")
    t_out = torch.empty_like(g["u"])
    step_args = {k: g[k][..., 0].contiguous() for k in ("u", "delta", "B", "C", "z")}
    cplx = None
    if "cfwd" in calls or "cbwd" in calls:
        ci = W.make_complex_inputs(w.wid, w.batch, w.dim, w.dstate, w.seqlen, dtype=w.dtype,
                                   bias=w.bias, per_row=w.per_row)
        cplx = {k: torch.from_numpy(ci[k]).cuda() for k in ("A", "B", "C")}
        if "cfwd" in calls and "cbwd" in calls and not args.no_checkpoints:
            cplx["ckpt"] = torch.empty(ms.complex_checkpoint_shape(w.batch, w.dim, w.dstate,
                                                                   w.seqlen),
                                       dtype=torch.complex64, device="cuda")
    conv_w = conv_b = conv_du = None
    if any(c.startswith("conv") for c in calls):
        cg = np.random.default_rng([w.wid, 10])
        conv_w = torch.from_numpy((cg.standard_normal((w.dim, 4)) * 0.5).astype(np.float32)).cuda()
        conv_b = torch.from_numpy((cg.standard_normal(w.dim) * 0.5).astype(np.float32)).cuda()
        conv_du = g["u"].float()
    step_out = torch.empty((w.batch, w.dim), dtype=sdt, device="cuda")

    def run_call(c, timing=None):
        if c == "fwd":
            ms.scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"],
                        g["delta_bias"], disc=args.disc, out=t_out, last_state=t_last,
                        return_last_state=True, workspace=fws, timing=timing, reset=rst,
                        checkpoints=ckpt)
        elif c == "bwd":
            ms.scan_bwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["D"], g["z"],
                        g["delta_bias"], g["dout"], disc=args.disc, workspace=ws, timing=timing,
                        reset=rst, checkpoints=ckpt)
        elif c == "cfwd":       # complex A, B, C with the workload's real sequences
            ms.scan_fwd_complex(g["u"], g["delta"], cplx["A"], cplx["B"], cplx["C"], g["D"],
                                g["z"], g["delta_bias"], disc=args.disc, out=t_out,
                                checkpoints=cplx.get("ckpt"))
        elif c == "cbwd":
            ms.scan_bwd_complex(g["u"], g["delta"], cplx["A"], cplx["B"], cplx["C"], g["D"],
                                g["z"], g["delta_bias"], g["dout"], disc=args.disc,
                                checkpoints=cplx.get("ckpt"))
        elif c == "conv_fwd":   # x = the workload's u sequence
            ms.conv1d_silu_fwd(g["u"], conv_w, conv_b, reset=rst, out=t_out)
        elif c == "conv_bwd":
            ms.conv1d_silu_bwd(g["u"], conv_w, conv_b, conv_du, reset=rst)
        else:   # decode step continuing from the forward's final state, in place
            ms.state_update(t_last, step_args["u"], step_args["delta"], g["A"], step_args["B"],
                            step_args["C"], g["D"], step_args["z"], g["delta_bias"],
                            disc=args.disc, out=step_out)

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        for c in calls:
            run_call(c)
    torch.cuda.synchronize()

    def new_event():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)      # creates the underlying event
        return e

    # events: per call (whole call) and per timed kernel (fwd / bwd scan kernel)
    ev = {c: [(new_event(), new_event()) for _ in range(args.steps)] for c in calls}
    kev = {c: [(new_event(), new_event()) for _ in range(args.steps)]
           for c in calls if c in ("fwd", "bwd")}
    start, end = new_event(), new_event()
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        for c in calls:
            e0, e1 = ev[c][i]
            e0.record(stream)
            run_call(c, kev[c][i] if c in kev else None)
            e1.record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    call_ms = {c: float(np.mean([a.elapsed_time(b) for a, b in ev[c]])) for c in calls}
    kern_ms = {c: float(np.mean([a.elapsed_time(b) for a, b in kev[c]])) for c in kev}

    copy_gbs = copy_bandwidth(torch)

    # the same step captured once into a HIP graph and replayed K times (the
    # launch gaps of K separate library calls removed); context beside `value`
    graph_ms = None
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for c in calls:
                run_call(c)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for c in calls:
                run_call(c)
        graph.replay()
        torch.cuda.synchronize()
        g0, g1 = new_event(), new_event()
        torch.cuda.synchronize()
        g0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / args.steps
        del graph

    # cold-cache protocol: each scan kernel alone, a 1 GiB write before every
    # launch; the other calls' outputs stay as the timed steps left them
    cold = {}
    if args.cold_iters > 0 and kev:
        flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        for c in kev:
            pairs = [(new_event(), new_event()) for _ in range(args.cold_iters)]
            torch.cuda.synchronize()
            for i in range(args.cold_iters):
                flush.fill_(float(i))
                run_call(c, pairs[i])
            torch.cuda.synchronize()
            t = np.array([a.elapsed_time(b) for a, b in pairs])
            med = float(np.median(t))
            cold[c] = {"iters": args.cold_iters, "median_ms": round(med, 5),
                       "p10_ms": round(float(np.percentile(t, 10)), 5),
                       "p90_ms": round(float(np.percentile(t, 90)), 5),
                       "GB/s_median": round(algorithmic_bytes(w, c) / (med * 1e-3) / 1e9, 1)}
        del flush

    step_bytes = sum(algorithmic_bytes(w, c) for c in calls)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    ct = w.batch * w.dim * w.seqlen
    kernel_names = {"fwd": "scan_fwd_kernel", "bwd": "scan_bwd_kernel"}
    per_call = {c: {"ms": round(call_ms[c], 5),
                    "algorithmic_MB": round(algorithmic_bytes(w, c) / 1e6, 3),
                    "GB/s": round(algorithmic_bytes(w, c) / (call_ms[c] * 1e-3) / 1e9, 1)}
                for c in calls}
    for c in kern_ms:
        per_call[c]["kernel"] = kernel_names[c]
        per_call[c]["kernel_ms"] = round(kern_ms[c], 5)
        if c in cold:
            per_call[c]["cold"] = cold[c]
    res = {
        "metric": "selective-scan fwd/bwd achieved HBM GB/s (% peak); channel-tokens/s, "
                  "D=1536 L=2048",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "ms_per_step_graph": None if graph_ms is None else round(graph_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.dtype == "f32" else "bf16-in/f32-compute",
        "data": "synthetic",
        "config": {"workload": f"{w.name}{' packed varlen' if args.varlen else ''}: "
                               f"{'+'.join(calls)} ({args.disc})"
                               f"{', chunk checkpoints' if ckpt is not None else ''}",
                   "batch": w.batch,
                   "dim": w.dim, "dstate": w.dstate, "seqlen": w.seqlen, "dtype": w.dtype,
                   "disc": args.disc, "delta_softplus": True, "D": True, "z": True,
                   "delta_bias": w.bias},
        "pct_of_hbm_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "stream_copy_GBs": round(copy_gbs, 1),
        "pct_of_stream_copy": round(100.0 * value / copy_gbs, 2),
        "channel_tokens_per_s": round(ct / (ms_per_step * 1e-3), 1),
        "per_call": per_call,
    }
    if kern_ms:
        # The scan kernels are bound by float32 vector arithmetic, not by HBM
        # (which runs far below its peak): the roofline is the ALU one, and the
        # HBM view of the same launch is reported beside it.
        dom = max(kern_ms, key=lambda c: kern_ms[c])
        kname = kernel_names[dom]
        dom_bytes = algorithmic_bytes(w, dom)
        dom_flops = flops_per_tn(dom, args.disc) * w.batch * w.dim * w.seqlen * w.dstate
        secs = kern_ms[dom] * 1e-3
        tflops = dom_flops / secs / 1e12
        gbs = dom_bytes / secs / 1e9
        wl_tag = f"w{w.wid}_{args.disc}"
        res["roofline"] = {"bound": "alu", "achieved": round(tflops, 3), "peak": PEAK_F32_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(tflops / PEAK_F32_TFLOPS, 4),
                           "traffic": committed_traffic(kname, wl_tag),
                           "issue": committed_issue(kname, wl_tag),
                           "kernel": kname, "call": f"mamba_scan_{dom}",
                           "algorithmic_flops_per_launch": int(dom_flops),
                           "flops_per_state_step": flops_per_tn(dom, args.disc),
                           "hbm": {"achieved_GBs": round(gbs, 1), "peak_GBs": PEAK_HBM_GBS,
                                   "frac": round(gbs / PEAK_HBM_GBS, 4),
                                   "algorithmic_bytes_per_launch": int(dom_bytes)},
                           "avg_launch_ms": round(kern_ms[dom], 5),
                           "kernel_source_sha256": kernel_source_hash(kname)}
    if not args.no_per_config and args.workload == 2 and not args.calls and not args.varlen:
        res["per_config"] = per_config(torch, ms, W)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, calls, args.disc)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
