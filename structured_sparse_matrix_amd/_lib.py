"""ctypes loader for libsnm.so (the HIP library built in-tree by build.py).

There is no fallback: if the library is missing the import of the binding fails loudly.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsnm.so")

_i64 = ctypes.c_int64
_int = ctypes.c_int
_vp = ctypes.c_void_p
_f32 = ctypes.c_float
_p64 = ctypes.POINTER(ctypes.c_int64)

# name -> argument types (every entry point returns its snm_status as a C int)
SIGNATURES = {
    "snm_abi_version": [],
    "snm_status_string": [_int],
    "snm_nm_sizes": [_i64, _i64, _int, _int, _p64, _p64],
    "snm_vnm_sizes": [_i64, _i64, _int, _int, _int, _p64, _p64, _p64],
    "snm_prune_encode_nm": [_vp, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp],
    "snm_prune_encode_vnm": [_vp, _i64, _i64, _i64, _int, _int, _int, _vp, _vp, _vp, _vp],
    "snm_prune_encode_vnm_tiled": [_vp, _i64, _i64, _i64, _int, _int, _int, _vp, _vp, _vp, _vp],
    "snm_spmm_nm": [_vp, _vp, _i64, _i64, _int, _int, _vp, _i64, _i64, _int, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _vp],
    "snm_nm_tiled_sizes": [_i64, _i64, _p64, _p64],
    "snm_prune_encode_nm_tiled": [_vp, _i64, _i64, _i64, _vp, _vp, _vp],
    "snm_spmm_nm_tiled": [_vp, _vp, _i64, _i64, _vp, _i64, _i64, _int, _vp, _i64, _vp],
    "snm_spmm_nm_tiled_ws_bytes": [_i64, _i64, _i64, _vp],
    "snm_spmm_nm_tiled_ws": [_vp, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp],
    "snm_spmm_nm_tiled_noalloc": [_vp, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _vp],
    "snm_ceiling_read": [_vp, _i64, _vp, _vp],
    "snm_ceiling_copy": [_vp, _vp, _i64, _vp],
    "snm_ceiling_lds_fill": [_vp, _i64, _i64, _i64, _vp, _vp],
    "snm_ceiling_matrix": [_int, _i64, _i64, _vp, _vp],
    "snm_spmm_vnm": [_vp, _vp, _vp, _i64, _i64, _int, _int, _int, _vp, _i64, _i64, _vp, _i64, _vp],
    "snm_spmm_vnm_tiled": [_vp, _vp, _vp, _i64, _i64, _int, _int, _int, _vp, _i64, _i64, _vp, _i64, _vp],
    "snm_sddmm_prune_nm": [_vp, _vp, _i64, _i64, _i64, _i64, _f32, _int, _int, _vp, _vp, _vp, _vp],
    "snm_softmax_nm_rows": [_vp, _i64, _i64, _i64, _vp],
    "snm_bitmap_sizes": [_i64, _i64, _p64, _p64],
    "snm_bitmap_count": [_vp, _i64, _i64, _i64, _vp, _vp, _vp],
    "snm_bitmap_encode": [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp],
    "snm_spmm_bitmap": [_vp, _vp, _vp, _i64, _i64, _vp, _i64, _i64, _int, _vp, _i64, _vp],
    "snm_sddmm_prune_nm_rowmax": [_vp, _vp, _i64, _i64, _i64, _i64, _f32, _vp, _vp, _vp, _vp],
    "snm_spmm_nm_softmax": [_vp, _vp, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _i64, _i64, _i64,
                            _i64, _i64, _vp],
    "snm_sddmm_prune_nm_bf16": [_vp, _vp, _i64, _i64, _i64, _i64, _f32, _vp, _vp, _vp, _vp, _vp],
    "snm_softmax_nm_rows_bf16": [_vp, _i64, _i64, _i64, _vp],
    "snm_spmm_nm_bf16": [_vp, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _vp],
    "snm_sddmm_prune_1of2_f32": [_vp, _vp, _i64, _i64, _i64, _i64, _f32, _vp, _vp, _vp, _vp, _vp],
    "snm_softmax_nm_rows_f32": [_vp, _i64, _i64, _i64, _vp],
    "snm_spmm_1of2_f32": [_vp, _vp, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _i64, _i64, _i64,
                          _i64, _i64, _vp],
    "snm_spmm_nm_softmax_bf16": [_vp, _vp, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _i64, _i64,
                                 _i64, _i64, _i64, _vp],
}

STATUS = {0: "SNM_OK", 1: "SNM_E_NULL", 2: "SNM_E_SHAPE", 3: "SNM_E_ALIGN",
          4: "SNM_E_UNSUPPORTED", 5: "SNM_E_DEVICE", 6: "SNM_E_LAUNCH"}

_lib = None


class SnmError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({text})")
        self.status = status


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -m structured_sparse_matrix_amd.build or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    for name, argtypes in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = ctypes.c_char_p if name == "snm_status_string" else ctypes.c_int
    _lib = lib
    return lib


def check(fn: str, status: int) -> None:
    if status != 0:
        text = load().snm_status_string(status).decode()
        raise SnmError(fn, status, text)
