"""Selective scan (Mamba S6) for MI355X: thin PyTorch binding of libmamba_scan.

Every computation runs in the HIP kernels behind the C ABI of
include/mamba_scan.h; this module only checks tensor metadata, passes device
pointers and the current HIP stream, and allocates outputs and workspace
with PyTorch.  Names and argument order follow the C ABI:

    scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, h0=None, ...)
    scan_bwd(u, delta, A, B, C, D, z, delta_bias, dout, h0=None, ...)
    state_update(state, u, delta, A, B, C, D=None, z=None, delta_bias=None, ...)

Layouts: u, delta, z, out (batch, dim, L); B, C (batch, N, L); A (dim, N);
D, delta_bias (dim,); h0 / states (batch, dim, N).  Sequence tensors are
float32 or bfloat16 (all the same); A, D, delta_bias and states are float32.
"""
from __future__ import annotations

import torch

from . import _lib
from ._lib import BF16, EULER, F32, ZOH, MambaScanError

__all__ = ["scan_fwd", "scan_bwd", "state_update", "SelectiveScanFn", "selective_scan",
           "MambaScanError", "lib", "abi_version"]


def lib():
    return _lib.load()


def abi_version() -> int:
    return int(lib().mamba_abi_version())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"sequence tensors must be float32 or bfloat16, got {t.dtype}")


def _disc_code(disc) -> int:
    if disc in ("zoh", ZOH):
        return ZOH
    if disc in ("euler", EULER):
        return EULER
    raise ValueError(f"disc must be 'zoh' or 'euler', got {disc!r}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _req(t, name, dtype, shape, device):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _flags(reset, shape, device):
    """Reset flags as a contiguous uint8 device tensor (None stays None)."""
    if reset is None:
        return None
    if reset.dtype == torch.bool:
        reset = reset.to(torch.uint8)
    _req(reset, "reset", torch.uint8, shape, device)
    return reset


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _events(timing):
    """Raw hipEvent_t handles of a (begin, end) pair of torch.cuda.Event
    created with enable_timing=True, or (None, None)."""
    if timing is None:
        return None, None
    handles = []
    for ev in timing:
        if not ev.cuda_event:       # torch creates the event on its first record
            ev.record()
        handles.append(ev.cuda_event)
    return handles[0], handles[1]


def scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, h0=None, *,
             delta_softplus=True, disc="zoh", return_last_state=False, out=None, last_state=None,
             lanes=0, segments=0, workspace=None, timing=None, reset=None, checkpoints=None):
    """Fused selective-scan forward.  Returns out, or (out, last_state).
    `reset`: optional (batch, L) uint8/bool device tensor; the state is zeroed
    before every flagged step (packed variable-length sequences).
    `checkpoints`: optional float32 tensor of checkpoint_shape(...) that
    receives the state entering every 128-step chunk, for scan_bwd.
    `segments`: 0 automatic, 1 one pass, k >= 2 that many sequence segments.
    `workspace`: optional uint8 device tensor reused across calls.
    `timing`: optional (begin, end) torch.cuda.Event pair recorded around the
    output kernel on the current stream."""
    L_ = lib()
    if not u.is_cuda:
        raise ValueError("u must be a GPU tensor (no CPU path exists)")
    dev = u.device
    batch, dim, L = u.shape
    N = A.shape[1]
    sdt = u.dtype
    dt = _dtype_code(u)
    _req(u, "u", sdt, (batch, dim, L), dev)
    _req(delta, "delta", sdt, (batch, dim, L), dev)
    _req(A, "A", torch.float32, (dim, N), dev)
    _req(B, "B", sdt, (batch, N, L), dev)
    _req(C, "C", sdt, (batch, N, L), dev)
    _req(D, "D", torch.float32, (dim,), dev)
    _req(z, "z", sdt, (batch, dim, L), dev)
    _req(delta_bias, "delta_bias", torch.float32, (dim,), dev)
    _req(h0, "h0", torch.float32, (batch, dim, N), dev)
    reset = _flags(reset, (batch, L), dev)
    _req(checkpoints, "checkpoints", torch.float32, checkpoint_shape(batch, dim, N, L), dev)
    if out is None:
        out = torch.empty((batch, dim, L), dtype=sdt, device=dev)
    _req(out, "out", sdt, (batch, dim, L), dev)
    if return_last_state and last_state is None:
        last_state = torch.empty((batch, dim, N), dtype=torch.float32, device=dev)
    _req(last_state, "last_state", torch.float32, (batch, dim, N), dev)
    nbytes = fwd_workspace_bytes(batch, dim, N, L, sdt, lanes, segments)
    if nbytes and (workspace is None or workspace.numel() < nbytes):
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    ws_ptr = workspace.data_ptr() if nbytes else None
    st = L_.mamba_scan_fwd_ex(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                              _ptr(delta_bias), _ptr(h0), _ptr(reset), int(bool(delta_softplus)),
                              _disc_code(disc), dt, batch, dim, N, L, _ptr(out),
                              _ptr(last_state), ws_ptr, nbytes, _stream(dev), int(lanes),
                              int(segments), _ptr(checkpoints), *_events(timing))
    _lib.check(st, "mamba_scan_fwd")
    return (out, last_state) if return_last_state else out


def checkpoint_shape(batch, dim, N, L):
    """Shape of the forward's checkpoint buffer: the state entering every
    128-step chunk."""
    return (batch, dim, (L + 127) // 128, N)


def _size_status(*sizes) -> int:
    """The status the library gives sizes its workspace query refuses (the
    query itself returns SIZE_MAX): MAMBA_ERR_SHAPE for an empty or negative
    size, else MAMBA_ERR_UNSUPPORTED."""
    return 2 if min(int(x) for x in sizes) <= 0 else 6


def fwd_workspace_bytes(batch, dim, N, L, dtype=torch.float32, lanes=0, segments=0) -> int:
    code = F32 if dtype == torch.float32 else BF16
    n = lib().mamba_scan_fwd_workspace_size_ex(batch, dim, N, L, code, int(lanes), int(segments))
    if n >= 2 ** 63:
        raise MambaScanError(_size_status(batch, dim, N, L), "mamba_scan_fwd_workspace_size")
    return int(n)


def bwd_workspace_bytes(batch, dim, N, L, dtype=torch.float32, lanes=0, segments=0) -> int:
    code = F32 if dtype == torch.float32 else BF16
    n = lib().mamba_scan_bwd_workspace_size_ex(batch, dim, N, L, code, int(lanes), int(segments))
    if n >= 2 ** 63:
        raise MambaScanError(_size_status(batch, dim, N, L), "mamba_scan_bwd_workspace_size")
    return int(n)


def scan_bwd(u, delta, A, B, C, D, z, delta_bias, dout, h0=None, *, delta_softplus=True,
             disc="zoh", lanes=0, workspace=None, want_dh0=True, timing=None, reset=None,
             checkpoints=None, segments=0):
    """Backward with state recomputation.  Returns a dict of float32 gradients:
    du, ddelta, dA, dB, dC and, when the input is given, dD, dz, ddelta_bias, dh0.
    `timing`: optional (begin, end) torch.cuda.Event pair recorded around the
    reverse-scan kernel on the current stream.  `segments`: 0 = automatic, 1 =
    one pass, k = k sequence segments run in parallel."""
    L_ = lib()
    dev = u.device
    batch, dim, L = u.shape
    N = A.shape[1]
    sdt = u.dtype
    dt = _dtype_code(u)
    for t, name, shp, ty in ((u, "u", (batch, dim, L), sdt), (delta, "delta", (batch, dim, L), sdt),
                             (A, "A", (dim, N), torch.float32), (B, "B", (batch, N, L), sdt),
                             (C, "C", (batch, N, L), sdt), (D, "D", (dim,), torch.float32),
                             (z, "z", (batch, dim, L), sdt),
                             (delta_bias, "delta_bias", (dim,), torch.float32),
                             (h0, "h0", (batch, dim, N), torch.float32),
                             (dout, "dout", (batch, dim, L), sdt)):
        _req(t, name, ty, shp, dev)
    reset = _flags(reset, (batch, L), dev)
    _req(checkpoints, "checkpoints", torch.float32, checkpoint_shape(batch, dim, N, L), dev)
    f32 = dict(dtype=torch.float32, device=dev)
    g = dict(du=torch.empty((batch, dim, L), **f32), ddelta=torch.empty((batch, dim, L), **f32),
             dA=torch.empty((dim, N), **f32), dB=torch.empty((batch, N, L), **f32),
             dC=torch.empty((batch, N, L), **f32))
    if D is not None:
        g["dD"] = torch.empty((dim,), **f32)
    if z is not None:
        g["dz"] = torch.empty((batch, dim, L), **f32)
    if delta_bias is not None:
        g["ddelta_bias"] = torch.empty((dim,), **f32)
    if h0 is not None and want_dh0:
        g["dh0"] = torch.empty((batch, dim, N), **f32)
    nbytes = bwd_workspace_bytes(batch, dim, N, L, sdt, lanes, segments)
    if checkpoints is not None:
        # the chunk-start states come from the checkpoints: the workspace
        # starts at the block flags
        states = checkpoints.numel() * 4
        nbytes -= (states + 255) // 256 * 256
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    st = L_.mamba_scan_bwd_ex(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                              _ptr(delta_bias), _ptr(h0), _ptr(dout), _ptr(reset),
                              int(bool(delta_softplus)),
                              _disc_code(disc), dt, batch, dim, N, L, _ptr(g["du"]),
                              _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]),
                              _ptr(g.get("dD")), _ptr(g.get("dz")), _ptr(g.get("ddelta_bias")),
                              _ptr(g.get("dh0")), workspace.data_ptr(), workspace.numel(),
                              _stream(dev), int(lanes), int(segments), _ptr(checkpoints),
                              *_events(timing))
    _lib.check(st, "mamba_scan_bwd")
    return g


def scan_bwd_noalloc(u, delta, A, B, C, D, z, delta_bias, dout, h0=None, *,
                     delta_softplus=True, disc="zoh", grads=None):
    """scan_bwd through mamba_scan_bwd_noalloc: no workspace, the library's
    fixed per-GPU scratch array instead (calls that overlap on one GPU race).
    `grads`: optional dict of preallocated float32 outputs with the keys and
    shapes scan_bwd returns (allocated here when absent).  Returns them."""
    L_ = lib()
    dev = u.device
    batch, dim, L = u.shape
    N = A.shape[1]
    sdt = u.dtype
    dt = _dtype_code(u)
    for t, name, shp, ty in ((u, "u", (batch, dim, L), sdt), (delta, "delta", (batch, dim, L), sdt),
                             (A, "A", (dim, N), torch.float32), (B, "B", (batch, N, L), sdt),
                             (C, "C", (batch, N, L), sdt), (D, "D", (dim,), torch.float32),
                             (z, "z", (batch, dim, L), sdt),
                             (delta_bias, "delta_bias", (dim,), torch.float32),
                             (h0, "h0", (batch, dim, N), torch.float32),
                             (dout, "dout", (batch, dim, L), sdt)):
        _req(t, name, ty, shp, dev)
    shapes = dict(du=(batch, dim, L), ddelta=(batch, dim, L), dA=(dim, N), dB=(batch, N, L),
                  dC=(batch, N, L))
    if D is not None:
        shapes["dD"] = (dim,)
    if z is not None:
        shapes["dz"] = (batch, dim, L)
    if delta_bias is not None:
        shapes["ddelta_bias"] = (dim,)
    if h0 is not None:
        shapes["dh0"] = (batch, dim, N)
    g = dict(grads or {})
    for k, shp in shapes.items():
        if k not in g:
            g[k] = torch.empty(shp, dtype=torch.float32, device=dev)
        _req(g[k], k, torch.float32, shp, dev)
    st = L_.mamba_scan_bwd_noalloc(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                   _ptr(z), _ptr(delta_bias), _ptr(h0), _ptr(dout),
                                   int(bool(delta_softplus)), _disc_code(disc), dt, batch, dim,
                                   N, L, _ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dA"]),
                                   _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g.get("dD")),
                                   _ptr(g.get("dz")), _ptr(g.get("ddelta_bias")),
                                   _ptr(g.get("dh0")), _stream(dev))
    _lib.check(st, "mamba_scan_bwd_noalloc")
    return {k: g[k] for k in shapes}


def state_update(state, u, delta, A, B, C, D=None, z=None, delta_bias=None, *,
                 delta_softplus=True, disc="zoh", out=None):
    """One recurrent step; `state` (batch, dim, N) float32 is updated in place.
    Per-step tensors: u, delta, z (batch, dim); B, C (batch, N).  Returns out."""
    L_ = lib()
    dev = state.device
    batch, dim, N = state.shape
    sdt = u.dtype
    dt = _dtype_code(u)
    _req(state, "state", torch.float32, (batch, dim, N), dev)
    for t, name, shp, ty in ((u, "u", (batch, dim), sdt), (delta, "delta", (batch, dim), sdt),
                             (A, "A", (dim, N), torch.float32), (B, "B", (batch, N), sdt),
                             (C, "C", (batch, N), sdt), (D, "D", (dim,), torch.float32),
                             (z, "z", (batch, dim), sdt),
                             (delta_bias, "delta_bias", (dim,), torch.float32)):
        _req(t, name, ty, shp, dev)
    if out is None:
        out = torch.empty((batch, dim), dtype=sdt, device=dev)
    _req(out, "out", sdt, (batch, dim), dev)
    st = L_.mamba_state_update(_ptr(state), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                               _ptr(D), _ptr(z), _ptr(delta_bias), int(bool(delta_softplus)),
                               _disc_code(disc), dt, batch, dim, N, _ptr(out), _stream(dev))
    _lib.check(st, "mamba_state_update")
    return out


def state_update_complex(state, u, delta, A, B, C, D=None, z=None, delta_bias=None, *,
                         delta_softplus=True, disc="zoh", out=None):
    """One recurrent step of the complex-valued model; `state` (batch, dim, N)
    complex64 is updated in place.  Per-step tensors: u, delta, z (batch,
    dim) real; B, C (batch, N) complex64; A (dim, N) complex64.  Returns out."""
    L_ = lib()
    dev = state.device
    batch, dim, N = state.shape
    sdt = u.dtype
    _req(state, "state", torch.complex64, (batch, dim, N), dev)
    _req(u, "u", sdt, (batch, dim), dev)
    _req(delta, "delta", sdt, (batch, dim), dev)
    _req(A, "A", torch.complex64, (dim, N), dev)
    _req(B, "B", torch.complex64, (batch, N), dev)
    _req(C, "C", torch.complex64, (batch, N), dev)
    _req(D, "D", torch.float32, (dim,), dev)
    _req(z, "z", sdt, (batch, dim), dev)
    _req(delta_bias, "delta_bias", torch.float32, (dim,), dev)
    if out is None:
        out = torch.empty((batch, dim), dtype=sdt, device=dev)
    _req(out, "out", sdt, (batch, dim), dev)
    st = L_.mamba_state_update_complex(_ptr(state), _ptr(u), _ptr(delta), _ptr(A), _ptr(B),
                                       _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                                       int(bool(delta_softplus)), _disc_code(disc),
                                       _dtype_code(u), batch, dim, N, _ptr(out), _stream(dev))
    _lib.check(st, "mamba_state_update_complex")
    return out


def complex_checkpoint_shape(batch, dim, N, L):
    """Shape of the complex forward's checkpoint buffer (complex64): the state
    entering every 128-step chunk."""
    return (batch, dim, (L + 127) // 128, N)


def fwd_complex_workspace_bytes(batch, dim, N, L, segments=0) -> int:
    n = lib().mamba_scan_fwd_complex_workspace_size_ex(batch, dim, N, L, int(segments))
    if n >= 2 ** 63:
        raise MambaScanError(_size_status(batch, dim, N, L),
                             "mamba_scan_fwd_complex_workspace_size")
    return int(n)


def bwd_complex_workspace_bytes(batch, dim, N, L, segments=0) -> int:
    n = lib().mamba_scan_bwd_complex_workspace_size_ex(batch, dim, N, L, int(segments))
    if n >= 2 ** 63:
        raise MambaScanError(_size_status(batch, dim, N, L),
                             "mamba_scan_bwd_complex_workspace_size")
    return int(n)


def scan_fwd_complex(u, delta, A, B, C, D=None, z=None, delta_bias=None, h0=None, *,
                     delta_softplus=True, disc="zoh", out=None, checkpoints=None, segments=0,
                     workspace=None, reset=None):
    """Complex-valued forward: A (dim, N), B, C (batch, N, L), h0 (batch, dim,
    N) complex64; u, delta, z real.  Returns (out, last_state complex64) with
    y = Re(sum_n C h) + D u gated by SiLU(z).  `checkpoints`: optional
    complex64 tensor of complex_checkpoint_shape, filled with the state
    entering every chunk (for scan_bwd_complex).  `segments`: 0 = automatic,
    1 = one pass, k = k sequence segments run in parallel.  `reset`: optional
    (batch, L) flags of packed sequences, as for scan_fwd."""
    L_ = lib()
    if not u.is_cuda:
        raise ValueError("u must be a GPU tensor (no CPU path exists)")
    dev = u.device
    batch, dim, L = u.shape
    N = A.shape[1]
    sdt = u.dtype
    _req(u, "u", sdt, (batch, dim, L), dev)
    _req(delta, "delta", sdt, (batch, dim, L), dev)
    _req(A, "A", torch.complex64, (dim, N), dev)
    _req(B, "B", torch.complex64, (batch, N, L), dev)
    _req(C, "C", torch.complex64, (batch, N, L), dev)
    _req(D, "D", torch.float32, (dim,), dev)
    _req(z, "z", sdt, (batch, dim, L), dev)
    _req(delta_bias, "delta_bias", torch.float32, (dim,), dev)
    _req(h0, "h0", torch.complex64, (batch, dim, N), dev)
    _req(checkpoints, "checkpoints", torch.complex64, complex_checkpoint_shape(batch, dim, N, L),
         dev)
    reset = _flags(reset, (batch, L), dev)
    if out is None:
        out = torch.empty((batch, dim, L), dtype=sdt, device=dev)
    last = torch.empty((batch, dim, N), dtype=torch.complex64, device=dev)
    nbytes = fwd_complex_workspace_bytes(batch, dim, N, L, segments)
    if nbytes and (workspace is None or workspace.numel() < nbytes):
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    ws_ptr = workspace.data_ptr() if nbytes else None
    st = L_.mamba_scan_fwd_complex_ex(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                      _ptr(z), _ptr(delta_bias), _ptr(h0), _ptr(reset),
                                      int(bool(delta_softplus)), _disc_code(disc),
                                      _dtype_code(u), batch, dim, N, L, _ptr(out), _ptr(last),
                                      _ptr(checkpoints), ws_ptr, nbytes, _stream(dev),
                                      int(segments))
    _lib.check(st, "mamba_scan_fwd_complex_ex")
    return out, last


def scan_bwd_complex(u, delta, A, B, C, D, z, delta_bias, dout, h0=None, *,
                     delta_softplus=True, disc="zoh", checkpoints=None, segments=0,
                     workspace=None, reset=None):
    """Backward of scan_fwd_complex.  Returns a dict: du, ddelta (and dD, dz,
    ddelta_bias when given) float32; dA, dB, dC (and dh0) complex64, the
    gradient of a complex input w being dL/dRe(w) + i dL/dIm(w).
    `checkpoints`: the buffer a scan_fwd_complex over the same inputs filled;
    the chunk states are then not recomputed.  `segments` and `reset` as for
    scan_fwd_complex."""
    L_ = lib()
    dev = u.device
    batch, dim, L = u.shape
    N = A.shape[1]
    sdt = u.dtype
    for t, name, shp, ty in ((u, "u", (batch, dim, L), sdt), (delta, "delta", (batch, dim, L), sdt),
                             (A, "A", (dim, N), torch.complex64),
                             (B, "B", (batch, N, L), torch.complex64),
                             (C, "C", (batch, N, L), torch.complex64),
                             (D, "D", (dim,), torch.float32), (z, "z", (batch, dim, L), sdt),
                             (delta_bias, "delta_bias", (dim,), torch.float32),
                             (h0, "h0", (batch, dim, N), torch.complex64),
                             (dout, "dout", (batch, dim, L), sdt)):
        _req(t, name, ty, shp, dev)
    _req(checkpoints, "checkpoints", torch.complex64, complex_checkpoint_shape(batch, dim, N, L),
         dev)
    reset = _flags(reset, (batch, L), dev)
    f32 = dict(dtype=torch.float32, device=dev)
    c64 = dict(dtype=torch.complex64, device=dev)
    g = dict(du=torch.empty((batch, dim, L), **f32), ddelta=torch.empty((batch, dim, L), **f32),
             dA=torch.empty((dim, N), **c64), dB=torch.empty((batch, N, L), **c64),
             dC=torch.empty((batch, N, L), **c64))
    if D is not None:
        g["dD"] = torch.empty((dim,), **f32)
    if z is not None:
        g["dz"] = torch.empty((batch, dim, L), **f32)
    if delta_bias is not None:
        g["ddelta_bias"] = torch.empty((dim,), **f32)
    if h0 is not None:
        g["dh0"] = torch.empty((batch, dim, N), **c64)
    nbytes = bwd_complex_workspace_bytes(batch, dim, N, L, segments)
    if checkpoints is not None:
        # the chunk states (the workspace's first part, 256-byte rounded) come
        # from the checkpoints instead
        states = 8 * batch * dim * N * ((L + 127) // 128)
        nbytes -= (states + 255) // 256 * 256
    ws_ptr, ws_bytes = None, 0
    if nbytes > 0:
        if workspace is None or workspace.numel() < nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    st = L_.mamba_scan_bwd_complex_ex(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                      _ptr(z), _ptr(delta_bias), _ptr(h0), _ptr(dout),
                                      _ptr(reset), int(bool(delta_softplus)), _disc_code(disc),
                                      _dtype_code(u), batch, dim, N, L, _ptr(g["du"]),
                                      _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]),
                                      _ptr(g["dC"]), _ptr(g.get("dD")), _ptr(g.get("dz")),
                                      _ptr(g.get("ddelta_bias")), _ptr(g.get("dh0")),
                                      _ptr(checkpoints), ws_ptr, ws_bytes, _stream(dev),
                                      int(segments))
    _lib.check(st, "mamba_scan_bwd_complex_ex")
    return g


def conv1d_silu_fwd(x, w, b=None, *, reset=None, out=None):
    """Short causal depthwise convolution (w: (dim, W), W <= 4) followed by
    SiLU.  x (batch, dim, L) float32 or bfloat16; returns u like x."""
    L_ = lib()
    if not x.is_cuda:
        raise ValueError("x must be a GPU tensor (no CPU path exists)")
    dev = x.device
    batch, dim, L = x.shape
    W = w.shape[1]
    _req(x, "x", x.dtype, (batch, dim, L), dev)
    _req(w, "w", torch.float32, (dim, W), dev)
    _req(b, "b", torch.float32, (dim,), dev)
    reset = _flags(reset, (batch, L), dev)
    if out is None:
        out = torch.empty_like(x)
    _req(out, "out", x.dtype, (batch, dim, L), dev)
    st = L_.mamba_conv1d_silu_fwd(_ptr(x), _ptr(w), _ptr(b), _ptr(reset), W, _dtype_code(x),
                                  batch, dim, L, _ptr(out), _stream(dev))
    _lib.check(st, "mamba_conv1d_silu_fwd")
    return out


def conv1d_silu_bwd(x, w, b, du, *, reset=None):
    """Backward of conv1d_silu_fwd for the gradient du (float32) at its
    output: returns a dict with dx, dw and (when b is given) db, float32."""
    L_ = lib()
    dev = x.device
    batch, dim, L = x.shape
    W = w.shape[1]
    _req(x, "x", x.dtype, (batch, dim, L), dev)
    _req(w, "w", torch.float32, (dim, W), dev)
    _req(b, "b", torch.float32, (dim,), dev)
    _req(du, "du", torch.float32, (batch, dim, L), dev)
    reset = _flags(reset, (batch, L), dev)
    f32 = dict(dtype=torch.float32, device=dev)
    g = dict(dx=torch.empty((batch, dim, L), **f32), dw=torch.empty((dim, W), **f32))
    if b is not None:
        g["db"] = torch.empty((dim,), **f32)
    st = L_.mamba_conv1d_silu_bwd(_ptr(x), _ptr(w), _ptr(b), _ptr(reset), _ptr(du), W,
                                  _dtype_code(x), batch, dim, L, _ptr(g["dx"]), _ptr(g["dw"]),
                                  _ptr(g.get("db")), _stream(dev))
    _lib.check(st, "mamba_conv1d_silu_bwd")
    return g


class SelectiveScanFn(torch.autograd.Function):
    """Autograd wrapper: forward = scan_fwd, backward = scan_bwd.  Besides the
    inputs, the forward saves only the state entering every 128-step chunk;
    the backward recomputes every other state from them."""

    @staticmethod
    def forward(ctx, u, delta, A, B, C, D, z, delta_bias, delta_softplus, disc):
        batch, dim, L = u.shape
        ckpt = torch.empty(checkpoint_shape(batch, dim, A.shape[1], L), dtype=torch.float32,
                           device=u.device)
        out = scan_fwd(u, delta, A, B, C, D, z, delta_bias, delta_softplus=delta_softplus,
                       disc=disc, checkpoints=ckpt)
        ctx.save_for_backward(u, delta, A, B, C, D, z, delta_bias, ckpt)
        ctx.flags = (delta_softplus, disc)
        return out

    @staticmethod
    def backward(ctx, dout):
        u, delta, A, B, C, D, z, delta_bias, ckpt = ctx.saved_tensors
        sp, disc = ctx.flags
        g = scan_bwd(u, delta, A, B, C, D, z, delta_bias, dout.contiguous().to(u.dtype),
                     delta_softplus=sp, disc=disc, checkpoints=ckpt)
        cast = lambda t, like: None if t is None else t.to(like.dtype)
        return (cast(g["du"], u), cast(g["ddelta"], delta), g["dA"], cast(g["dB"], B),
                cast(g["dC"], C), g.get("dD"), cast(g.get("dz"), z) if z is not None else None,
                g.get("ddelta_bias"), None, None)


def selective_scan(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                   disc="zoh"):
    return SelectiveScanFn.apply(u, delta, A, B, C, D, z, delta_bias, delta_softplus, disc)
