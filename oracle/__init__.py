"""Float64 CPU oracle for the selective scan (S6) -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library (``scan_selective_fwd_amd``) never
imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, IEEE double, no fast-math, no
FP contraction); this module only marshals numpy arrays into it and splits
channel ranges over threads (ctypes releases the GIL during the C call).

Sources are the web pages about Gu & Dao, "Mamba: Linear-Time Sequence
Modeling with Selective State Spaces":
  * chapterpal.com page, Knowl 1 "Selective State Space Layer (S6)" -- the ZOH
    rule (step 3), the recurrence (step 4) and the per-(b, d, t) loop;
  * paper-graph-ui.vercel.app summary, section 3.4 -- softplus for tau_Delta,
    recurrent (decode) mode, recomputation in the backward.
The backward is the chain rule applied to that forward (the pages give no
gradient formulas); it is pinned by central finite differences in the tests.

Parity pins (see tests/test_oracle_pins.py and tests/test_oracle_grad.py):
forward -- Theorem 1 gated-RNN closed form, LTI convolution brute force with a
matrix-exponential ZOH, reset / preserve limits, an associative tree scan,
chunk resume, linearity and state separability; backward -- central finite
differences of the forward on every input; state update -- equality with the
forward continued one step.  Nothing here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ZOH = 0
EULER = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lib_lock = threading.Lock()

_dp = ctypes.POINTER(ctypes.c_double)
_u8p = ctypes.POINTER(ctypes.c_ubyte)
_i64 = ctypes.c_int64
_int = ctypes.c_int


def _load():
    global _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            from . import build as _build

            _build.build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_scan_fwd.argtypes = [_dp] * 9 + [_u8p, _int, _int] + [_i64] * 6 + [_dp, _dp]
        lib.oracle_scan_fwd.restype = None
        lib.oracle_state_update.argtypes = [_dp] * 9 + [_int, _int] + [_i64] * 5 + [_dp]
        lib.oracle_state_update.restype = None
        lib.oracle_scan_bwd.argtypes = [_dp] * 10 + [_u8p, _int, _int] + [_i64] * 6 + [_dp] * 9
        lib.oracle_scan_bwd.restype = None
        lib.oracle_conv1d_silu_fwd.argtypes = [_dp, _dp, _dp, _u8p] + [_i64] * 6 + [_dp]
        lib.oracle_conv1d_silu_fwd.restype = None
        lib.oracle_conv1d_silu_bwd.argtypes = [_dp, _dp, _dp, _u8p, _dp] + [_i64] * 6 + [_dp] * 3
        lib.oracle_conv1d_silu_bwd.restype = None
        lib.oracle_scan_fwd_complex.argtypes = [_dp] * 9 + [_u8p, _int, _int] + [_i64] * 6 + [_dp, _dp]
        lib.oracle_scan_fwd_complex.restype = None
        lib.oracle_scan_bwd_complex.argtypes = [_dp] * 10 + [_u8p, _int, _int] + [_i64] * 6 + [_dp] * 9
        lib.oracle_scan_bwd_complex.restype = None
        lib.oracle_version.restype = _int
        _lib = lib
        return lib


def _f64(x):
    """Contiguous float64 copy/view (None stays None)."""
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(_dp)


def _reset(reset, batch, L):
    """Contiguous uint8 (batch, L) copy of the reset flags (None stays None)."""
    if reset is None:
        return None
    r = np.ascontiguousarray(np.asarray(reset).astype(np.uint8))
    assert r.shape == (batch, L)
    return r


def _ptr8(a):
    return None if a is None else a.ctypes.data_as(_u8p)


def _split(n_items: int, threads: int):
    threads = max(1, min(threads, n_items))
    step = (n_items + threads - 1) // threads
    return [(i, min(i + step, n_items)) for i in range(0, n_items, step)]


def _check_shapes(batch, dim, N, L, **arrays):
    """Raises ValueError unless every given array has its documented shape
    (the C code reads through the pointers with these sizes).  A required
    array is passed as (array, True); None is allowed only for optional ones."""
    shapes = dict(u=(batch, dim, L), delta=(batch, dim, L), z=(batch, dim, L),
                  dout=(batch, dim, L), A=(dim, N), B=(batch, N, L), C=(batch, N, L),
                  D=(dim,), delta_bias=(dim,), h0=(batch, dim, N))
    for name, (arr, required) in arrays.items():
        if arr is None:
            if required:
                raise ValueError(f"{name} is required")
            continue
        if tuple(arr.shape) != shapes[name]:
            raise ValueError(f"{name} has shape {tuple(arr.shape)}, expected {shapes[name]}")


def default_threads() -> int:
    """Host cores available to this process, capped by OMP_NUM_THREADS when
    the environment sets it (a machine's share of cores may be smaller than
    what the affinity mask shows)."""
    try:
        n = max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return n


def scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, h0=None, *,
             delta_softplus=True, disc=ZOH, threads=None, return_last_state=True, reset=None):
    """Forward selective scan in float64.

    Shapes: u, delta, z (batch, dim, L); A (dim, N); B, C (batch, N, L);
    D, delta_bias (dim,); h0 (batch, dim, N); reset (batch, L) flags (the
    state is zeroed before each flagged step).  Returns (out, last_state).
    """
    lib = _load()
    u, delta, A, B, C = (_f64(t) for t in (u, delta, A, B, C))
    D, z, delta_bias, h0 = (_f64(t) for t in (D, z, delta_bias, h0))
    batch, dim, L = u.shape
    N = A.shape[1]
    _check_shapes(batch, dim, N, L, delta=(delta, True), A=(A, True), B=(B, True),
                  C=(C, True), D=(D, False), z=(z, False), delta_bias=(delta_bias, False),
                  h0=(h0, False))
    out = np.zeros((batch, dim, L), np.float64)
    last = np.zeros((batch, dim, N), np.float64) if return_last_state else None
    nthreads = threads or default_threads()
    args = [_ptr(t) for t in (u, delta, A, B, C, D, z, delta_bias, h0)]
    rs = _reset(reset, batch, L)

    def work(rng):
        lib.oracle_scan_fwd(*args, _ptr8(rs), int(bool(delta_softplus)), int(disc), batch, dim,
                            N, L,
                            rng[0], rng[1], _ptr(out), _ptr(last))

    ranges = _split(batch * dim, nthreads)
    if len(ranges) == 1:
        work(ranges[0])
    else:
        with ThreadPoolExecutor(len(ranges)) as ex:
            list(ex.map(work, ranges))
    return out, last


def state_update(state, u, delta, A, B, C, D=None, z=None, delta_bias=None, *,
                 delta_softplus=True, disc=ZOH):
    """One recurrent step.  state (batch, dim, N) float64 is NOT modified; the
    new state is returned with the output: (out (batch, dim), new_state)."""
    lib = _load()
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    u, delta, A, B, C = (_f64(t) for t in (u, delta, A, B, C))
    D, z, delta_bias = (_f64(t) for t in (D, z, delta_bias))
    batch, dim = u.shape
    N = A.shape[1]
    assert st.shape == (batch, dim, N) and B.shape == (batch, N) and C.shape == (batch, N)
    out = np.zeros((batch, dim), np.float64)
    lib.oracle_state_update(_ptr(st), *[_ptr(t) for t in (u, delta, A, B, C, D, z, delta_bias)],
                            int(bool(delta_softplus)), int(disc), batch, dim, N, 0, batch * dim,
                            _ptr(out))
    return out, st


def scan_bwd(u, delta, A, B, C, D, z, delta_bias, dout, h0=None, *, delta_softplus=True,
             disc=ZOH, threads=None, reset=None):
    """Gradients of sum(dout * out) w.r.t. every input, in float64.

    Returns a dict with du, ddelta, dA, dB, dC and, when the matching input is
    given, dD, dz, ddelta_bias, dh0.
    """
    lib = _load()
    u, delta, A, B, C, dout = (_f64(t) for t in (u, delta, A, B, C, dout))
    D, z, delta_bias, h0 = (_f64(t) for t in (D, z, delta_bias, h0))
    batch, dim, L = u.shape
    N = A.shape[1]
    _check_shapes(batch, dim, N, L, delta=(delta, True), A=(A, True), B=(B, True),
                  C=(C, True), dout=(dout, True), D=(D, False), z=(z, False),
                  delta_bias=(delta_bias, False), h0=(h0, False))
    du = np.zeros_like(u)
    ddelta = np.zeros_like(u)
    dz = np.zeros_like(u) if z is not None else None
    nthreads = threads or default_threads()
    ranges = _split(batch * dim, nthreads)
    # per-thread accumulators for the reduced gradients
    acc = []
    for _ in ranges:
        acc.append(dict(
            dA=np.zeros((dim, N)), dB=np.zeros((batch, N, L)), dC=np.zeros((batch, N, L)),
            dD=np.zeros(dim) if D is not None else None,
            ddb=np.zeros(dim) if delta_bias is not None else None,
            dh0=np.zeros((batch, dim, N)) if h0 is not None else None))
    args = [_ptr(t) for t in (u, delta, A, B, C, D, z, delta_bias, h0, dout)]
    rs = _reset(reset, batch, L)

    def work(i):
        a = acc[i]
        lib.oracle_scan_bwd(*args, _ptr8(rs), int(bool(delta_softplus)), int(disc), batch, dim,
                            N, L,
                            ranges[i][0], ranges[i][1], _ptr(du), _ptr(ddelta), _ptr(a["dA"]),
                            _ptr(a["dB"]), _ptr(a["dC"]), _ptr(a["dD"]), _ptr(dz), _ptr(a["ddb"]),
                            _ptr(a["dh0"]))

    if len(ranges) == 1:
        work(0)
    else:
        with ThreadPoolExecutor(len(ranges)) as ex:
            list(ex.map(work, range(len(ranges))))
    res = dict(du=du, ddelta=ddelta,
               dA=sum(a["dA"] for a in acc), dB=sum(a["dB"] for a in acc),
               dC=sum(a["dC"] for a in acc))
    if D is not None:
        res["dD"] = sum(a["dD"] for a in acc)
    if z is not None:
        res["dz"] = dz
    if delta_bias is not None:
        res["ddelta_bias"] = sum(a["ddb"] for a in acc)
    if h0 is not None:
        res["dh0"] = sum(a["dh0"] for a in acc)
    return res


def conv1d_silu_fwd(x, w, cb=None, *, reset=None):
    """Causal depthwise convolution (W taps, x before t = 0 and before each
    flagged sequence start counts as zero) followed by SiLU, in float64.
    x (batch, dim, L); w (dim, W); cb (dim,).  Returns u (batch, dim, L)."""
    lib = _load()
    x, w, cb = _f64(x), _f64(w), _f64(cb)
    batch, dim, L = x.shape
    W = w.shape[1]
    u = np.zeros_like(x)
    rs = _reset(reset, batch, L)
    lib.oracle_conv1d_silu_fwd(_ptr(x), _ptr(w), _ptr(cb), _ptr8(rs), batch, dim, W, L, 0,
                               batch * dim, _ptr(u))
    return u


def conv1d_silu_bwd(x, w, cb, du, *, reset=None):
    """Gradients of sum(du * u) for u = conv1d_silu_fwd(x, w, cb): returns a
    dict with dx, dw and (when cb is given) dcb."""
    lib = _load()
    x, w, cb, du = _f64(x), _f64(w), _f64(cb), _f64(du)
    batch, dim, L = x.shape
    W = w.shape[1]
    dx = np.zeros_like(x)
    dw = np.zeros_like(w)
    dcb = np.zeros(dim) if cb is not None else None
    rs = _reset(reset, batch, L)
    lib.oracle_conv1d_silu_bwd(_ptr(x), _ptr(w), _ptr(cb), _ptr8(rs), _ptr(du), batch, dim, W, L,
                               0, batch * dim, _ptr(dx), _ptr(dw), _ptr(dcb))
    res = dict(dx=dx, dw=dw)
    if cb is not None:
        res["dcb"] = dcb
    return res


def _c128(x):
    """Complex array as contiguous interleaved float64 (re, im) pairs."""
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.complex128)).view(np.float64)


def scan_fwd_complex(u, delta, A, B, C, D=None, z=None, delta_bias=None, h0=None, *,
                     delta_softplus=True, disc=ZOH, threads=None, reset=None):
    """Complex-valued forward in float64: A (dim, N), B, C (batch, N, L) and
    h0 (batch, dim, N) complex; u, delta, z, D, delta_bias real.  Returns
    (out real (batch, dim, L), last_state complex (batch, dim, N)) with
    y_t = Re(sum_n C_t[n] h_t[n]) + D u_t gated by SiLU(z).  reset (batch,
    L) flags as in scan_fwd."""
    lib = _load()
    _b, _d, _l = np.shape(u)
    _check_shapes(_b, _d, np.shape(A)[1], _l, delta=(delta, True), A=(A, True), B=(B, True),
                  C=(C, True), D=(D, False), z=(z, False), delta_bias=(delta_bias, False),
                  h0=(h0, False))
    u, delta, D, z, delta_bias = (_f64(t) for t in (u, delta, D, z, delta_bias))
    A, B, C, h0 = (_c128(t) for t in (A, B, C, h0))
    batch, dim, L = u.shape
    N = A.shape[1] // 2
    out = np.zeros((batch, dim, L), np.float64)
    last = np.zeros((batch, dim, N), np.complex128)
    lastv = last.view(np.float64)
    rs = _reset(reset, batch, L)
    args = [_ptr(t) for t in (u, delta, A, B, C, D, z, delta_bias, h0)] + [_ptr8(rs)]

    def work(rng):
        lib.oracle_scan_fwd_complex(*args, int(bool(delta_softplus)), int(disc), batch, dim, N,
                                    L, rng[0], rng[1], _ptr(out), _ptr(lastv))

    ranges = _split(batch * dim, threads or default_threads())
    if len(ranges) == 1:
        work(ranges[0])
    else:
        with ThreadPoolExecutor(len(ranges)) as ex:
            list(ex.map(work, ranges))
    return out, last


def scan_bwd_complex(u, delta, A, B, C, D, z, delta_bias, dout, h0=None, *,
                     delta_softplus=True, disc=ZOH, reset=None):
    """Gradients of sum(dout * out) for scan_fwd_complex, in float64 (one
    thread).  dA, dB, dC, dh0 are complex (the gradient of a complex w is
    dL/dRe(w) + i dL/dIm(w)); the others real.  Returns a dict like scan_bwd.
    reset (batch, L) flags as in scan_bwd."""
    lib = _load()
    _b, _d, _l = np.shape(u)
    _check_shapes(_b, _d, np.shape(A)[1], _l, delta=(delta, True), A=(A, True), B=(B, True),
                  C=(C, True), dout=(dout, True), D=(D, False), z=(z, False),
                  delta_bias=(delta_bias, False), h0=(h0, False))
    u, delta, D, z, delta_bias, dout = (_f64(t) for t in (u, delta, D, z, delta_bias, dout))
    A, B, C, h0 = (_c128(t) for t in (A, B, C, h0))
    batch, dim, L = u.shape
    N = A.shape[1] // 2
    du, ddelta = np.zeros_like(u), np.zeros_like(u)
    dz = np.zeros_like(u) if z is not None else None
    dA = np.zeros((dim, N), np.complex128)
    dB = np.zeros((batch, N, L), np.complex128)
    dC = np.zeros((batch, N, L), np.complex128)
    dD = np.zeros(dim) if D is not None else None
    ddb = np.zeros(dim) if delta_bias is not None else None
    dh0 = np.zeros((batch, dim, N), np.complex128) if h0 is not None else None
    v = lambda a: None if a is None else a.view(np.float64)
    rs = _reset(reset, batch, L)
    lib.oracle_scan_bwd_complex(*[_ptr(t) for t in (u, delta, A, B, C, D, z, delta_bias, h0, dout)],
                                _ptr8(rs),
                                int(bool(delta_softplus)), int(disc), batch, dim, N, L, 0,
                                batch * dim, _ptr(du), _ptr(ddelta), _ptr(v(dA)), _ptr(v(dB)),
                                _ptr(v(dC)), _ptr(dD), _ptr(dz), _ptr(ddb), _ptr(v(dh0)))
    res = dict(du=du, ddelta=ddelta, dA=dA, dB=dB, dC=dC)
    if D is not None:
        res["dD"] = dD
    if z is not None:
        res["dz"] = dz
    if delta_bias is not None:
        res["ddelta_bias"] = ddb
    if h0 is not None:
        res["dh0"] = dh0
    return res


def version() -> int:
    return int(_load().oracle_version())
