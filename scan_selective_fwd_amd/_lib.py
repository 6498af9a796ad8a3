"""ctypes view of libmamba_scan.so (the C ABI in include/mamba_scan.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation of any kind.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmamba_scan.so")

STATUS = {
    0: "MAMBA_OK", 1: "MAMBA_ERR_NULL_PTR", 2: "MAMBA_ERR_SHAPE", 3: "MAMBA_ERR_DTYPE",
    4: "MAMBA_ERR_ALIGNMENT", 5: "MAMBA_ERR_WORKSPACE", 6: "MAMBA_ERR_UNSUPPORTED",
    7: "MAMBA_ERR_HIP", 8: "MAMBA_ERR_INVALID", 9: "MAMBA_ERR_SCRATCH_LIMIT",
}
F32, BF16 = 0, 1
ZOH, EULER = 0, 1
# MAMBA_SCAN_ABI_VERSION of the header these signatures follow
ABI_VERSION = 2

# Every symbol the header declares.
EXPORTS = (
    "mamba_abi_version", "mamba_status_string", "mamba_scan_fwd_workspace_size",
    "mamba_scan_bwd_workspace_size", "mamba_scan_fwd", "mamba_scan_bwd", "mamba_state_update",
    "mamba_scan_fwd_varlen", "mamba_scan_bwd_varlen", "mamba_conv1d_silu_fwd",
    "mamba_conv1d_silu_bwd",
    "mamba_scan_fwd_ex", "mamba_scan_fwd_workspace_size_ex", "mamba_scan_bwd_workspace_size_ex",
    "mamba_scan_bwd_ex", "mamba_scan_checkpoint_size", "mamba_scan_fwd_complex",
    "mamba_scan_bwd_complex", "mamba_scan_bwd_complex_workspace_size",
    "mamba_scan_complex_checkpoint_size", "mamba_scan_fwd_complex_ex",
    "mamba_scan_bwd_complex_ex", "mamba_state_update_complex",
    "mamba_scan_fwd_complex_workspace_size", "mamba_scan_fwd_complex_workspace_size_ex",
    "mamba_scan_bwd_complex_workspace_size_ex", "mamba_scan_bwd_noalloc",
)


class MambaScanError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_sz = ctypes.c_size_t

_lib = None


def load(path: str = LIB_PATH):
    """Loads the library (once) and declares the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build the HIP library first (python -c "
            f"'import __graft_entry__ as g; g.build()' or python {HERE}/build.py)")
    lib = ctypes.CDLL(path)
    lib.mamba_abi_version.restype = _int
    lib.mamba_abi_version.argtypes = []
    found = lib.mamba_abi_version()
    if found != ABI_VERSION:
        raise ImportError(f"{path} has ABI version {found}, these bindings need {ABI_VERSION}: "
                          f"rebuild it")
    lib.mamba_abi_version.argtypes = []
    lib.mamba_status_string.restype = ctypes.c_char_p
    lib.mamba_status_string.argtypes = [_int]
    for name in ("mamba_scan_fwd_workspace_size", "mamba_scan_bwd_workspace_size"):
        f = getattr(lib, name)
        f.restype = _sz
        f.argtypes = [_i64, _i64, _i64, _i64, _int]
    lib.mamba_scan_fwd_workspace_size_ex.restype = _sz
    lib.mamba_scan_fwd_workspace_size_ex.argtypes = [_i64, _i64, _i64, _i64, _int, _int, _int]
    lib.mamba_scan_bwd_workspace_size_ex.restype = _sz
    lib.mamba_scan_bwd_workspace_size_ex.argtypes = [_i64, _i64, _i64, _i64, _int, _int, _int]
    fwd_args = [_vp] * 9 + [_int, _int, _int] + [_i64] * 4 + [_vp, _vp, _vp, _sz, _vp]
    lib.mamba_scan_fwd.restype = _int
    lib.mamba_scan_fwd.argtypes = fwd_args
    fwd_rst = [_vp] * 10 + [_int, _int, _int] + [_i64] * 4 + [_vp, _vp, _vp, _sz, _vp]
    lib.mamba_scan_fwd_varlen.restype = _int
    lib.mamba_scan_fwd_varlen.argtypes = fwd_rst
    lib.mamba_scan_fwd_ex.restype = _int
    lib.mamba_scan_fwd_ex.argtypes = fwd_rst + [_int, _int, _vp, _vp, _vp]
    bwd_args = [_vp] * 10 + [_int, _int, _int] + [_i64] * 4 + [_vp] * 10 + [_sz, _vp]
    lib.mamba_scan_bwd.restype = _int
    lib.mamba_scan_bwd.argtypes = bwd_args
    bwd_rst = [_vp] * 11 + [_int, _int, _int] + [_i64] * 4 + [_vp] * 10 + [_sz, _vp]
    lib.mamba_scan_bwd_varlen.restype = _int
    lib.mamba_scan_bwd_varlen.argtypes = bwd_rst
    lib.mamba_scan_bwd_ex.restype = _int
    lib.mamba_scan_bwd_ex.argtypes = bwd_rst + [_int, _int, _vp, _vp, _vp]
    lib.mamba_scan_bwd_noalloc.restype = _int
    lib.mamba_scan_bwd_noalloc.argtypes = [_vp] * 10 + [_int, _int, _int] + [_i64] * 4 + [_vp] * 10
    lib.mamba_scan_checkpoint_size.restype = _sz
    lib.mamba_scan_checkpoint_size.argtypes = [_i64] * 4
    lib.mamba_conv1d_silu_fwd.restype = _int
    lib.mamba_conv1d_silu_fwd.argtypes = [_vp] * 4 + [_i64, _int] + [_i64] * 3 + [_vp, _vp]
    lib.mamba_conv1d_silu_bwd.restype = _int
    lib.mamba_conv1d_silu_bwd.argtypes = [_vp] * 5 + [_i64, _int] + [_i64] * 3 + [_vp] * 4
    lib.mamba_scan_fwd_complex.restype = _int
    lib.mamba_scan_fwd_complex.argtypes = ([_vp] * 9 + [_int, _int, _int] + [_i64] * 4
                                           + [_vp] * 3 + [_sz, _vp])
    lib.mamba_scan_fwd_complex_workspace_size.restype = _sz
    lib.mamba_scan_fwd_complex_workspace_size.argtypes = [_i64] * 4
    lib.mamba_scan_fwd_complex_workspace_size_ex.restype = _sz
    lib.mamba_scan_fwd_complex_workspace_size_ex.argtypes = [_i64] * 4 + [_int]
    lib.mamba_scan_bwd_complex_workspace_size_ex.restype = _sz
    lib.mamba_scan_bwd_complex_workspace_size_ex.argtypes = [_i64] * 4 + [_int]
    lib.mamba_scan_bwd_complex.restype = _int
    lib.mamba_scan_bwd_complex.argtypes = bwd_args
    lib.mamba_scan_bwd_complex_workspace_size.restype = _sz
    lib.mamba_scan_bwd_complex_workspace_size.argtypes = [_i64] * 4
    lib.mamba_scan_complex_checkpoint_size.restype = _sz
    lib.mamba_scan_complex_checkpoint_size.argtypes = [_i64] * 4
    lib.mamba_scan_fwd_complex_ex.restype = _int
    lib.mamba_scan_fwd_complex_ex.argtypes = ([_vp] * 10 + [_int, _int, _int] + [_i64] * 4
                                              + [_vp] * 4 + [_sz, _vp, _int])
    lib.mamba_scan_bwd_complex_ex.restype = _int
    lib.mamba_scan_bwd_complex_ex.argtypes = ([_vp] * 11 + [_int, _int, _int] + [_i64] * 4
                                              + [_vp] * 11 + [_sz, _vp, _int])
    lib.mamba_state_update_complex.restype = _int
    lib.mamba_state_update_complex.argtypes = ([_vp] * 9 + [_int, _int, _int] + [_i64] * 3
                                               + [_vp, _vp])
    lib.mamba_state_update.restype = _int
    lib.mamba_state_update.argtypes = [_vp] * 9 + [_int, _int, _int] + [_i64] * 3 + [_vp, _vp]
    _lib = lib
    return lib


def check(status: int, where: str):
    if status != 0:
        raise MambaScanError(status, where)
