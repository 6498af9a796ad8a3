"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

The library must load, export every function include/mamba_scan.h declares,
and reject bad arguments with the documented status before enqueuing any
work (so these calls never reach the device).
"""
import ctypes
import os
import re

import pytest

from scan_selective_fwd_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mamba_scan.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(mamba_[a-z0-9_]+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for required in ("mamba_scan_fwd", "mamba_scan_bwd", "mamba_state_update",
                     "mamba_scan_fwd_workspace_size", "mamba_scan_bwd_workspace_size",
                     "mamba_status_string", "mamba_abi_version"):
        assert required in names
    assert set(names) == set(_lib.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_version_and_status_strings(lib):
    assert lib.mamba_abi_version() == 2
    for code in range(0, 10):
        s = lib.mamba_status_string(code)
        assert s and isinstance(s, bytes)
    assert lib.mamba_status_string(0) == b"ok"
    assert b"unknown" in lib.mamba_status_string(99)


def test_workspace_queries(lib):
    assert lib.mamba_scan_fwd_workspace_size(8, 1536, 16, 2048, 0) == 0
    n = lib.mamba_scan_bwd_workspace_size(2, 5120, 16, 2048, 1)
    assert 0 < n < 2 ** 31
    assert n % 256 == 0
    assert lib.mamba_scan_bwd_workspace_size(2, 5120, 65, 2048, 1) == 2 ** 64 - 1
    assert lib.mamba_scan_bwd_workspace_size(0, 5120, 16, 2048, 1) == 2 ** 64 - 1
    # the backward spreads a channel over 16 lanes: 0 (default) and 16 only
    n16 = lib.mamba_scan_bwd_workspace_size_ex(2, 64, 16, 512, 0, 16, 1)
    assert n16 > 0 and n16 == lib.mamba_scan_bwd_workspace_size_ex(2, 64, 16, 512, 0, 0, 1)
    # one pass: the workspace holds the state at each 128-step chunk start,
    # (2*64) * 4 * 16 floats, then one flag per block of 16 channels (8
    # blocks), 256-byte rounded
    assert n16 == 2 * 64 * 4 * 16 * 4 + 256
    # (the automatic choice splits these 8 blocks' 4 chunks into 4 segments)
    assert (lib.mamba_scan_bwd_workspace_size(2, 64, 16, 512, 0)
            == lib.mamba_scan_bwd_workspace_size_ex(2, 64, 16, 512, 0, 0, 4) > n16)
    for lanes in (8, 32, 64):
        assert lib.mamba_scan_bwd_workspace_size_ex(2, 64, 16, 512, 0, lanes, 1) == 2 ** 64 - 1


def test_backward_segment_workspace(lib):
    # 1536 channels are 96 blocks: 2048 / 96 rounded up to a power of two, 32
    # segments of 256 chunks.  The chunk-start states, one flag per (block,
    # segment), then per channel and segment four state-sized buffers (forward
    # end and entering states, adjoint summary and entering adjoint) and four
    # scalars
    states = 1536 * 8192 * 16 * 4
    n = lib.mamba_scan_bwd_workspace_size(1, 1536, 16, 1 << 20, 1)
    assert n == states + 96 * 32 * 4 + 4 * (1536 * 32 * 16 * 4) + 4 * (1536 * 32 * 4)
    assert n == lib.mamba_scan_bwd_workspace_size_ex(1, 1536, 16, 1 << 20, 1, 0, 32)
    # short sequences split down to one chunk per segment: 8 chunks, 8 segments
    assert (lib.mamba_scan_bwd_workspace_size(1, 1024, 16, 1024, 1)
            == lib.mamba_scan_bwd_workspace_size_ex(1, 1024, 16, 1024, 1, 0, 8)
            > lib.mamba_scan_bwd_workspace_size_ex(1, 1024, 16, 1024, 1, 0, 1))
    # 512 blocks still split (4 segments), 640 do not
    assert (lib.mamba_scan_bwd_workspace_size(1, 8192, 16, 4096, 1)
            == lib.mamba_scan_bwd_workspace_size_ex(1, 8192, 16, 4096, 1, 0, 4))
    assert (lib.mamba_scan_bwd_workspace_size(2, 5120, 16, 2048, 1)
            == lib.mamba_scan_bwd_workspace_size_ex(2, 5120, 16, 2048, 1, 0, 1))
    assert lib.mamba_scan_bwd_workspace_size_ex(1, 1536, 16, 1 << 20, 1, 0, 0) == n
    # one pass: states and one flag per block (96 ints, 256-byte rounded)
    assert lib.mamba_scan_bwd_workspace_size_ex(1, 1536, 16, 1 << 20, 1, 0, 1) == states + 512
    # more segments than chunks are capped; negative counts are rejected
    assert (lib.mamba_scan_bwd_workspace_size_ex(1, 16, 4, 1024, 0, 0, 100)
            == lib.mamba_scan_bwd_workspace_size_ex(1, 16, 4, 1024, 0, 0, 8))
    assert lib.mamba_scan_bwd_workspace_size_ex(1, 16, 4, 1024, 0, 0, -1) == 2 ** 64 - 1
    # shapes that fill the chip are not split
    assert (lib.mamba_scan_bwd_workspace_size_ex(8, 1536, 16, 2048, 1, 0, 0)
            == lib.mamba_scan_bwd_workspace_size_ex(8, 1536, 16, 2048, 1, 0, 1))


def bwd_ex(lib, segments, ws=None, wsb=0, ckpt=None):
    return lib.mamba_scan_bwd_ex(P, P, P, P, P, None, None, None, None, P, None, 1, 0, 0, 1, 16,
                                 4, 1024, P, P, P, P, P, None, None, None, None, ws, wsb, None, 0,
                                 segments, ckpt, None, None)


def test_backward_segment_arguments(lib):
    need = lib.mamba_scan_bwd_workspace_size_ex(1, 16, 4, 1024, 0, 0, 3)
    one = lib.mamba_scan_bwd_workspace_size_ex(1, 16, 4, 1024, 0, 0, 1)
    assert need > one > 0
    assert bwd_ex(lib, 3) == 5                          # explicit segments, no workspace
    assert bwd_ex(lib, 3, ws=P, wsb=need - 1) == 5
    assert bwd_ex(lib, 3, ws=P + 8, wsb=need) == 4      # misaligned workspace
    assert bwd_ex(lib, -1, ws=P, wsb=need) == 6
    # with checkpoints the states are not in the workspace, the rest is
    ckpt = lib.mamba_scan_checkpoint_size(1, 16, 4, 1024)
    assert bwd_ex(lib, 3, ws=P, wsb=need - ckpt - 1, ckpt=P) == 5


def test_forward_segment_workspace(lib):
    # a long sequence over few channels is split into segments: 1536 channels
    # are 96 blocks, so 32 segments of 256 chunks; per channel and segment two
    # states of 16 floats, the delta sum and the reset-free factor
    n = lib.mamba_scan_fwd_workspace_size(1, 1536, 16, 1 << 20, 1)
    assert n == 2 * (1536 * 32 * 16 * 4) + 2 * (1536 * 32 * 4)
    assert lib.mamba_scan_fwd_workspace_size_ex(1, 1536, 16, 1 << 20, 1, 0, 0) == n
    assert lib.mamba_scan_fwd_workspace_size_ex(1, 1536, 16, 1 << 20, 1, 16, 0) == n
    # 256 blocks split (2048 / 256: 8 segments), 512 do not; at least 8
    # segments of one chunk or more
    assert (lib.mamba_scan_fwd_workspace_size(1, 4096, 16, 4096, 1)
            == lib.mamba_scan_fwd_workspace_size_ex(1, 4096, 16, 4096, 1, 0, 8) > 0)
    assert lib.mamba_scan_fwd_workspace_size(1, 8192, 16, 4096, 1) == 0
    assert (lib.mamba_scan_fwd_workspace_size(1, 1024, 16, 1024, 1)
            == lib.mamba_scan_fwd_workspace_size_ex(1, 1024, 16, 1024, 1, 0, 8) > 0)
    assert lib.mamba_scan_fwd_workspace_size(1, 1024, 16, 896, 1) == 0      # 7 chunks
    # one pass: no workspace; explicit wider lanes run in one pass as well
    assert lib.mamba_scan_fwd_workspace_size_ex(1, 1536, 16, 1 << 20, 1, 0, 1) == 0
    assert lib.mamba_scan_fwd_workspace_size_ex(1, 1536, 16, 1 << 20, 1, 64, 0) == 0
    # explicit segments need 16 lanes; more segments than chunks are capped
    assert lib.mamba_scan_fwd_workspace_size_ex(1, 16, 4, 1024, 0, 32, 2) == 2 ** 64 - 1
    assert (lib.mamba_scan_fwd_workspace_size_ex(1, 16, 4, 1024, 0, 0, 100)
            == lib.mamba_scan_fwd_workspace_size_ex(1, 16, 4, 1024, 0, 0, 8))
    assert lib.mamba_scan_fwd_workspace_size_ex(1, 16, 4, 1024, 0, 0, -1) == 2 ** 64 - 1


def fwd_ex(lib, segments, ws=None, wsb=0, lanes=0, reset=None, ckpt=None):
    return lib.mamba_scan_fwd_ex(P, P, P, P, P, None, None, None, None, reset, 1, 0, 0, 1, 16, 4,
                                 1024, P, None, ws, wsb, None, lanes, segments, ckpt, None, None)


def test_forward_segment_arguments(lib):
    need = lib.mamba_scan_fwd_workspace_size_ex(1, 16, 4, 1024, 0, 0, 3)
    assert need > 0
    assert fwd_ex(lib, 3) == 5                          # explicit segments, no workspace
    assert fwd_ex(lib, 3, ws=P, wsb=need - 1) == 5
    assert fwd_ex(lib, 3, ws=P + 8, wsb=need) == 4      # misaligned workspace
    assert fwd_ex(lib, 3, lanes=64) == 6                # segments need 16 lanes
    assert fwd_ex(lib, -2) == 6
    assert fwd_ex(lib, 1, lanes=32, reset=P) == 6       # reset flags need 16 lanes
    assert fwd_ex(lib, 1, lanes=64, ckpt=P) == 6        # checkpoints need 16 lanes
    assert fwd_ex(lib, 1, ckpt=P + 4) == 4


def test_checkpoint_size_and_backward_workspace(lib):
    # one state of 16 floats per channel and 128-step chunk (ragged: 17 chunks)
    assert lib.mamba_scan_checkpoint_size(2, 64, 16, 2049) == 2 * 64 * 17 * 16 * 4
    assert lib.mamba_scan_checkpoint_size(0, 64, 16, 2049) == 2 ** 64 - 1
    full = lib.mamba_scan_bwd_workspace_size_ex(2, 64, 16, 2048, 0, 0, 1)   # one pass
    flags = full - 2 * 64 * 16 * 16 * 4          # with checkpoints: the block flags only

    def bwd_ex(ws, wsb, ckpt):
        return lib.mamba_scan_bwd_ex(P, P, P, P, P, None, None, None, None, P, None, 1, 0, 0, 2,
                                     64, 16, 2048, P, P, P, P, P, None, None, None, None, ws, wsb,
                                     None, 0, 1, ckpt, None, None)
    assert bwd_ex(P, flags - 1, P) == 5
    assert bwd_ex(P, flags, None) == 5               # without them the states need room
    assert bwd_ex(P, full, P + 8) == 4


def test_complex_checkpoints_size_and_workspace(lib):
    # one complex state (2 floats) per channel, 128-step chunk and state index
    assert lib.mamba_scan_complex_checkpoint_size(2, 64, 16, 2049) == 2 * 64 * 17 * 16 * 8
    assert lib.mamba_scan_complex_checkpoint_size(2, 64, 17, 2049) == 2 ** 64 - 1   # N <= 16
    # one pass: the workspace holds the complex chunk states only
    need = lib.mamba_scan_bwd_complex_workspace_size_ex(2, 64, 16, 2048, 1)
    assert need == 2 * 64 * 16 * 16 * 8

    def bwd_ex(ws, wsb, ckpt):
        return lib.mamba_scan_bwd_complex_ex(P, P, P, P, P, None, None, None, None, P, None, 1, 0, 0,
                                             2, 64, 16, 2048, P, P, P, P, P, None, None, None,
                                             None, ckpt, ws, wsb, None, 1)
    assert bwd_ex(None, 0, None) == 5                # no checkpoints: the states need room
    assert bwd_ex(P, need - 1, None) == 5
    assert bwd_ex(P, need, P + 8) == 4               # misaligned checkpoints
    assert lib.mamba_scan_fwd_complex_ex(P, P, P, P, P, None, None, None, None, None, 1, 0, 0, 2, 64,
                                         16, 2048, P, None, P + 4, None, 0, None, 1) == 4
    assert lib.mamba_scan_fwd_complex_ex(P, P, P, P, P, None, None, None, None, None, 1, 0, 0, 2, 64,
                                         17, 2048, P, None, P, None, 0, None, 1) == 6


def test_complex_segment_workspace(lib):
    # 1536 channels over 2^20 steps: 96 blocks, 32 segments of 256 chunks (as
    # the real calls); per channel, segment and state three complex buffers in
    # the forward, six in the backward after the chunk states
    nst = 1536 * 32 * 16 * 8
    assert lib.mamba_scan_fwd_complex_workspace_size(1, 1536, 16, 1 << 20) == 3 * nst
    assert lib.mamba_scan_fwd_complex_workspace_size_ex(1, 1536, 16, 1 << 20, 32) == 3 * nst
    assert lib.mamba_scan_fwd_complex_workspace_size_ex(1, 1536, 16, 1 << 20, 1) == 0
    states = 1536 * 8192 * 16 * 8
    assert lib.mamba_scan_bwd_complex_workspace_size(1, 1536, 16, 1 << 20) == states + 6 * nst
    assert lib.mamba_scan_bwd_complex_workspace_size_ex(1, 1536, 16, 1 << 20, 1) == states
    # shapes that fill the chip run in one pass; bad counts are rejected
    assert lib.mamba_scan_fwd_complex_workspace_size(8, 1536, 16, 2048) == 0
    assert lib.mamba_scan_fwd_complex_workspace_size_ex(1, 16, 16, 1024, -1) == 2 ** 64 - 1
    assert lib.mamba_scan_bwd_complex_workspace_size_ex(1, 16, 17, 1024, 2) == 2 ** 64 - 1
    fw = lib.mamba_scan_fwd_complex_workspace_size_ex(1, 16, 16, 1024, 4)
    assert fw > 0
    assert lib.mamba_scan_fwd_complex_ex(P, P, P, P, P, None, None, None, None, None, 1, 0, 0, 1, 16,
                                         16, 1024, P, None, None, P, fw - 1, None, 4) == 5
    assert lib.mamba_scan_fwd_complex_ex(P, P, P, P, P, None, None, None, None, None, 1, 0, 0, 1, 16,
                                         16, 1024, P, None, None, P, fw, None, -1) == 6


def test_varlen_requires_flags(lib):
    assert lib.mamba_scan_fwd_varlen(P, P, P, P, P, None, None, None, None, None, 1, 0, 0, 1, 16,
                                     4, 128, P, None, None, 0, None) == 1
    assert lib.mamba_scan_bwd_varlen(P, P, P, P, P, None, None, None, None, P, None, 1, 0, 0, 1,
                                     16, 4, 128, P, P, P, P, P, None, None, None, None, P, 0,
                                     None) == 1


P = 4096  # a 16-byte aligned fake address; never dereferenced (calls fail first)


def fwd(lib, **kw):
    a = dict(u=P, delta=P, A=P, B=P, C=P, D=None, z=None, bias=None, h0=None, sp=1, disc=0, dt=0,
             batch=1, dim=16, N=4, L=128, out=P, last=None, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.mamba_scan_fwd(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"],
                              a["bias"], a["h0"], a["sp"], a["disc"], a["dt"], a["batch"],
                              a["dim"], a["N"], a["L"], a["out"], a["last"], a["ws"], a["wsb"],
                              a["stream"])


def bwd(lib, **kw):
    a = dict(u=P, delta=P, A=P, B=P, C=P, D=None, z=None, bias=None, h0=None, dout=P, sp=1,
             disc=0, dt=0, batch=1, dim=16, N=4, L=128, du=P, ddelta=P, dA=P, dB=P, dC=P,
             dD=None, dz=None, dbias=None, dh0=None, ws=P, wsb=0, stream=None)
    a.update(kw)
    return lib.mamba_scan_bwd(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"],
                              a["bias"], a["h0"], a["dout"], a["sp"], a["disc"], a["dt"],
                              a["batch"], a["dim"], a["N"], a["L"], a["du"], a["ddelta"], a["dA"],
                              a["dB"], a["dC"], a["dD"], a["dz"], a["dbias"], a["dh0"], a["ws"],
                              a["wsb"], a["stream"])


def step(lib, **kw):
    a = dict(state=P, u=P, delta=P, A=P, B=P, C=P, D=None, z=None, bias=None, sp=1, disc=0, dt=0,
             batch=1, dim=16, N=4, out=P, stream=None)
    a.update(kw)
    return lib.mamba_state_update(a["state"], a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"],
                                  a["z"], a["bias"], a["sp"], a["disc"], a["dt"], a["batch"],
                                  a["dim"], a["N"], a["out"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(u=None), 1), (dict(delta=None), 1), (dict(A=None), 1), (dict(B=None), 1),
    (dict(C=None), 1), (dict(out=None), 1),
    (dict(batch=0), 2), (dict(dim=-1), 2), (dict(N=0), 2), (dict(L=0), 2),
    (dict(dt=2), 3), (dict(disc=7), 3),
    (dict(u=P + 4), 4), (dict(z=P + 8), 4), (dict(last=P + 2), 4), (dict(h0=P + 12), 4),
    (dict(N=65), 6), (dict(batch=2 ** 40, dim=2 ** 30), 6),
])
def test_fwd_rejects_bad_arguments(lib, kw, code):
    assert fwd(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dout=None), 1), (dict(du=None), 1), (dict(dC=None), 1),
    (dict(D=P), 8), (dict(dz=P), 8), (dict(bias=P), 8), (dict(dh0=P), 8),
    (dict(ws=None), 5), (dict(wsb=16), 5),
    (dict(ws=P + 4, wsb=1 << 30), 4), (dict(dt=9), 3), (dict(N=100), 6),
])
def test_bwd_rejects_bad_arguments(lib, kw, code):
    assert bwd(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(state=None), 1), (dict(out=None), 1), (dict(N=0), 2), (dict(N=65), 6),
    (dict(state=P + 4), 4), (dict(disc=3), 3),
])
def test_state_update_rejects_bad_arguments(lib, kw, code):
    assert step(lib, **kw) == code


def test_binding_has_no_cpu_path():
    import torch
    import scan_selective_fwd_amd as ms
    x = torch.zeros(1, 2, 8)
    with pytest.raises(ValueError):
        ms.scan_fwd(x, x, torch.zeros(2, 4), torch.zeros(1, 4, 8), torch.zeros(1, 4, 8))


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ImportError):
        _lib._lib_saved = _lib._lib
        try:
            _lib._lib = None
            _lib.load(str(tmp_path / "nope.so"))
        finally:
            _lib._lib = _lib._lib_saved


def conv_fwd(lib, **kw):
    a = dict(x=P, w=P, b=None, reset=None, width=4, dt=0, batch=1, dim=8, L=64, u=P, stream=None)
    a.update(kw)
    return lib.mamba_conv1d_silu_fwd(a["x"], a["w"], a["b"], a["reset"], a["width"], a["dt"],
                                     a["batch"], a["dim"], a["L"], a["u"], a["stream"])


def conv_bwd(lib, **kw):
    a = dict(x=P, w=P, b=None, reset=None, du=P, width=4, dt=0, batch=1, dim=8, L=64, dx=P, dw=P,
             db=None, stream=None)
    a.update(kw)
    return lib.mamba_conv1d_silu_bwd(a["x"], a["w"], a["b"], a["reset"], a["du"], a["width"],
                                     a["dt"], a["batch"], a["dim"], a["L"], a["dx"], a["dw"],
                                     a["db"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), 1), (dict(w=None), 1), (dict(u=None), 1), (dict(L=0), 2), (dict(dt=3), 3),
    (dict(x=P + 2), 4), (dict(b=P + 4), 4), (dict(width=0), 6), (dict(width=5), 6),
])
def test_conv_fwd_rejects_bad_arguments(lib, kw, code):
    assert conv_fwd(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(du=None), 1), (dict(dx=None), 1), (dict(dw=None), 1), (dict(b=P), 8), (dict(db=P), 8),
    (dict(dx=P + 4), 4), (dict(width=7), 6), (dict(batch=-1), 2),
])
def test_conv_bwd_rejects_bad_arguments(lib, kw, code):
    assert conv_bwd(lib, **kw) == code


def test_noalloc_refuses_problems_beyond_its_scratch(lib):
    """The allocation-free backward checks its fixed scratch size before any
    device call: a problem whose one-pass workspace exceeds it is refused
    (no GPU needed for the check; the pointers are never used)."""
    assert lib.mamba_scan_bwd_workspace_size_ex(64, 5120, 16, 2048, 0, 0, 1) > 32 << 20
    fake = 1 << 20   # 16-byte aligned, never dereferenced
    args = [fake] * 10 + [1, 0, 0, 64, 5120, 16, 2048] + [fake] * 9 + [None]
    assert lib.mamba_scan_bwd_noalloc(*args) == 9   # MAMBA_ERR_SCRATCH_LIMIT
    assert b"scratch" in lib.mamba_status_string(9)
    # invalid sizes are named by the regular checks
    bad = [fake] * 10 + [1, 0, 0, 0, 5120, 16, 2048] + [fake] * 9 + [None]
    assert lib.mamba_scan_bwd_noalloc(*bad) == 2    # MAMBA_ERR_SHAPE


@pytest.mark.parametrize("sizes,status", [
    ((0, 4, 16, 64), 2), ((1, 0, 16, 64), 2), ((1, 4, 0, 64), 2), ((1, 4, 16, 0), 2),
    ((1, 4, 16, -1), 2), ((1, 4, 65, 64), 6)])
def test_binding_size_errors_match_the_abi(lib, sizes, status):
    # the workspace queries answer SIZE_MAX for every refused size; the binding
    # reports the status the entry points themselves give: MAMBA_ERR_SHAPE for
    # an empty or negative size, MAMBA_ERR_UNSUPPORTED beyond the limits
    import scan_selective_fwd_amd as ms
    for query in (ms.fwd_workspace_bytes, ms.bwd_workspace_bytes,
                  ms.fwd_complex_workspace_bytes, ms.bwd_complex_workspace_bytes):
        with pytest.raises(ms.MambaScanError) as e:
            query(*sizes)
        assert e.value.status == status, (query.__name__, sizes)
    batch, dim, N, L = sizes
    assert fwd(lib, batch=batch, dim=dim, N=N, L=L) == status
    assert bwd(lib, batch=batch, dim=dim, N=N, L=L) == status
