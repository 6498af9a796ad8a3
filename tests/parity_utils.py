"""Helpers for the GPU-vs-oracle parity tests: moving the seeded inputs to the
device with identical bits, running the float64 oracle on the same values,
and the error metric.

Metric (the tolerance of a tensor is "relative"): a GPU tensor g matches the
oracle tensor o at tolerance rtol when both
    max|g - o| <= rtol * max|o|     and     ||g - o||_2 <= rtol * ||o||_2.
Elementwise relative error is meaningless where o is near zero, so the
max-norm is taken over the whole tensor.
"""
from __future__ import annotations

import numpy as np
import torch

import workloads as W

SEQ = ("u", "delta", "B", "C", "z", "dout")
RTOL = {"f32": 1e-4, "bf16": 2e-2}


def to_device(inp: dict, dtype: str, device="cuda") -> dict:
    out = {}
    for k, v in inp.items():
        if k in SEQ and dtype == "bf16":
            t = torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(v))
        out[k] = t.to(device)
    return out


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def rel_errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    e = got - ref
    mx = np.abs(ref).max()
    l2 = np.linalg.norm(ref)
    return (np.abs(e).max() / mx if mx > 0 else np.abs(e).max(),
            np.linalg.norm(e) / l2 if l2 > 0 else np.linalg.norm(e))


def assert_match(got, ref, rtol, name=""):
    emax, el2 = rel_errors(got, ref)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert emax <= rtol and el2 <= rtol, f"{name}: rel max err {emax:.3e}, rel L2 err {el2:.3e} > {rtol}"
    return emax, el2


def announce(msg: str):
    print(f"\n[case] {msg}", flush=True)
