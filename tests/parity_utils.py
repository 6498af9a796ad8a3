"""Helpers for the GPU-vs-oracle parity tests: moving the seeded inputs to the
device with identical bits, running the float64 oracle on the same values,
and the error metric.

Metric (the tolerance of a tensor is "relative", measured per row): the
trailing `row_ndim` axes of a tensor form its rows (one (b, d) channel's
sequence for out, du, ddelta, dz; one (b, d) state vector for last_state and
dh0; one (b, n) row over time for dB, dC; one channel's states for dA); a
1-D tensor (dD, ddelta_bias) is a single row.  A GPU tensor g matches the
oracle tensor o at tolerance rtol when, in EVERY row r,
    max_r|g - o| <= rtol * max_r|o|     and     ||g - o||_r,2 <= rtol * ||o||_r,2.
Elementwise relative error is meaningless where o is near zero, so the norms
are taken over a row; taking them per row (not over the whole tensor) keeps
a channel of small magnitude from hiding behind the large ones.  A row whose
reference is below 1e-9 of the tensor's largest value is held to that floor.

Tolerances: RTOL[dtype] applies to results stored in the input dtype (out);
every float32 result (states, all gradients) is held to the float32 bound
RTOL_F32 whatever the input dtype, since both sides compute it from the same
input bits.
"""
from __future__ import annotations

import numpy as np
import torch

import workloads as W

SEQ = ("u", "delta", "B", "C", "z", "dout")
RTOL = {"f32": 1e-4, "bf16": 2e-2}
RTOL_F32 = 1e-4
FLOOR = 1e-9


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


def _rows(a: np.ndarray, row_ndim: int) -> np.ndarray:
    if a.ndim <= row_ndim:
        return a.reshape(1, -1)
    return a.reshape(-1, int(np.prod(a.shape[a.ndim - row_ndim:])))


def rel_errors(got, ref, row_ndim: int = 1):
    """Worst row's (max-norm, 2-norm) relative errors, and that row's index
    for each."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    g, r = _rows(got, row_ndim), _rows(ref, row_ndim)
    e = g - r
    top = np.abs(r).max() if r.size else 0.0
    scale_max = np.maximum(np.abs(r).max(axis=1), FLOOR * top)
    scale_l2 = np.maximum(np.linalg.norm(r, axis=1), FLOOR * top)
    tiny = np.finfo(np.float64).tiny
    emax = np.abs(e).max(axis=1) / np.maximum(scale_max, tiny)
    el2 = np.linalg.norm(e, axis=1) / np.maximum(scale_l2, tiny)
    return float(emax.max()), float(el2.max()), int(emax.argmax()), int(el2.argmax())


def assert_match(got, ref, rtol, name="", row_ndim: int = 1):
    """Per-row parity (see the module docstring).  Returns the worst row's
    (max-norm, 2-norm) relative errors."""
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    emax, el2, rmax, rl2 = rel_errors(got, ref, row_ndim)
    assert emax <= rtol and el2 <= rtol, (
        f"{name}: worst row rel max err {emax:.3e} (row {rmax}), rel L2 err {el2:.3e} "
        f"(row {rl2}) > {rtol}")
    return emax, el2


def announce(msg: str):
    print(f"\n[case] {msg}", flush=True)
