"""Structured-sparse (2:4 and V:2:M) matrix products and dynamic 2:4 attention on MI355X.

Thin binding over libsnm (include/snm.h). Each function takes and returns torch tensors on
a ROCm device; torch provides device memory and the current stream, and every step of
the computation runs in the library's HIP kernels. Functions keep the names of the
C entry points without the ``snm_`` prefix.

Layouts (canonical, see include/snm.h):
  2:4     values fp16 [R, K/2], meta uint8 [R, K/8]
  V:2:M   values fp16 [R, 2K/M], midx uint8 [R, K/(2M)], colloc uint8 [R/V, K/M, 4]
  bitmap  bitmaps [R, K/64] (64-bit words, held in int64), tile_offsets [R*K/64 + 1]
          (uint32 values, held in int32), values fp16 [tile_offsets[-1]]
The ``*_bf16`` functions are the same operations on bf16 tensors (same layouts).
  1:2 fp32  values fp32 [R, K/2], meta uint8 [R, K/4] (one code per pair: 0x4 first kept,
            0xe second kept)
"""
from __future__ import annotations

import ctypes
import math

from ._lib import load, check, SnmError, LIB_PATH

__all__ = [
    "prune_encode_nm", "prune_encode_vnm", "spmm_nm", "spmm_vnm", "sddmm_prune_nm",
    "softmax_nm_rows", "attention_nm", "nm_sizes", "vnm_sizes", "abi_version", "SnmError",
    "nm_tiled_sizes", "prune_encode_nm_tiled", "spmm_nm_tiled",
    "spmm_nm_tiled_ws_bytes", "spmm_nm_tiled_ws",
    "prune_encode_vnm_tiled", "spmm_vnm_tiled",
    "sddmm_prune_nm_rowmax", "spmm_nm_softmax", "attention_nm_fused",
    "bitmap_sizes", "bitmap_encode", "spmm_bitmap",
    "sddmm_prune_nm_bf16", "softmax_nm_rows_bf16", "spmm_nm_bf16", "spmm_nm_softmax_bf16",
    "attention_nm_bf16", "attention_nm_fused_bf16",
    "sddmm_prune_1of2_f32", "softmax_nm_rows_f32", "spmm_1of2_f32", "attention_1of2_f32",
    "attention_1of2_fused_f32",
    "LIB_PATH",
]


def _torch():
    import torch
    return torch


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t, name, dtype, dim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on a ROCm device")
    if dim is not None and t.dim() not in (dim if isinstance(dim, tuple) else (dim,)):
        raise ValueError(f"{name} must have {dim} dimensions, got {t.dim()}")


def abi_version() -> int:
    return load().snm_abi_version()


def nm_sizes(R: int, K: int, n: int = 2, m: int = 4):
    v, mb = ctypes.c_int64(), ctypes.c_int64()
    check("snm_nm_sizes", load().snm_nm_sizes(R, K, n, m, ctypes.byref(v), ctypes.byref(mb)))
    return v.value, mb.value


def vnm_sizes(R: int, K: int, V: int, M: int, N: int = 2):
    v, m, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    check("snm_vnm_sizes", load().snm_vnm_sizes(R, K, V, N, M, ctypes.byref(v), ctypes.byref(m), ctypes.byref(c)))
    return v.value, m.value, c.value


def prune_encode_nm(A, values=None, meta=None, n: int = 2, m: int = 4):
    """2:4 magnitude prune of fp16 A [R, K] along K -> (values [R, K/2], meta [R, K/8])."""
    torch = _torch()
    _need(A, "A", torch.float16, 2)
    if A.stride(1) != 1:
        raise ValueError("A must be row-major (unit stride along K)")
    R, K = A.shape
    if values is None:
        values = torch.empty((R, K // 2), dtype=torch.float16, device=A.device)
    if meta is None:
        meta = torch.empty((R, K // 8), dtype=torch.uint8, device=A.device)
    check("snm_prune_encode_nm",
          load().snm_prune_encode_nm(_ptr(A), R, K, A.stride(0), n, m, _ptr(values), _ptr(meta), _stream(A)))
    return values, meta


def nm_tiled_sizes(R: int, K: int):
    v, m = ctypes.c_int64(), ctypes.c_int64()
    check("snm_nm_tiled_sizes", load().snm_nm_tiled_sizes(R, K, ctypes.byref(v), ctypes.byref(m)))
    return v.value, m.value


def prune_encode_nm_tiled(A, values_t=None, meta_t=None):
    """2:4 prune of fp16 A [R, K] into the operand-major layout (see snm.h):
    values_t fp16 [ceil(R/16)*ceil(K/64)*512], meta_t uint8 [.. *128]."""
    torch = _torch()
    _need(A, "A", torch.float16, 2)
    if A.stride(1) != 1:
        raise ValueError("A must be row-major (unit stride along K)")
    R, K = A.shape
    nv, nm = nm_tiled_sizes(R, K)
    if values_t is None:
        values_t = torch.empty((nv,), dtype=torch.float16, device=A.device)
    if meta_t is None:
        meta_t = torch.empty((nm,), dtype=torch.uint8, device=A.device)
    if values_t.numel() < nv or meta_t.numel() < nm:
        raise ValueError("output buffers too small for the operand-major layout")
    check("snm_prune_encode_nm_tiled",
          load().snm_prune_encode_nm_tiled(_ptr(A), R, K, A.stride(0), _ptr(values_t), _ptr(meta_t), _stream(A)))
    return values_t, meta_t


def spmm_nm_tiled(values_t, meta_t, R: int, B, out=None):
    """Y = decode(values_t, meta_t) @ B for an R x K operand-major matrix; B [K, C]
    (row-major, or column-major such as X.t())."""
    torch = _torch()
    _need(values_t, "values_t", torch.float16)
    _need(meta_t, "meta_t", torch.uint8)
    _need(B, "B", torch.float16, 2)
    K, C = B.shape
    nv, nm = nm_tiled_sizes(R, K)
    if values_t.numel() < nv or meta_t.numel() < nm or not values_t.is_contiguous() or not meta_t.is_contiguous():
        raise ValueError("operand-major arrays do not match R x K")
    layout, ldb = _b_layout(B)
    if out is None:
        out = torch.empty((R, C), dtype=torch.float16, device=B.device)
    if out.stride(1) != 1:
        raise ValueError("out must be row-major")
    check("snm_spmm_nm_tiled",
          load().snm_spmm_nm_tiled(_ptr(values_t), _ptr(meta_t), R, K, _ptr(B), C, ldb, layout,
                                   _ptr(out), out.stride(0), _stream(B)))
    return out


def spmm_nm_tiled_ws_bytes(R: int, K: int, C: int) -> int:
    """Workspace bytes of spmm_nm_tiled_ws for an R x K matrix and C <= 32 columns."""
    n = ctypes.c_int64()
    check("snm_spmm_nm_tiled_ws_bytes", load().snm_spmm_nm_tiled_ws_bytes(R, K, C, ctypes.byref(n)))
    return n.value


def spmm_nm_tiled_ws(values_t, meta_t, R: int, X, workspace, out=None):
    """Y = decode(values_t, meta_t) @ X.T for decode activations X [C, K] (C <= 32),
    with the reduction split across workgroups. workspace: a zero-filled uint8 device
    tensor of at least spmm_nm_tiled_ws_bytes(R, K, C) bytes. Every call leaves the whole
    workspace zero again, so one workspace serves calls of any shape in turn; calls that
    may overlap need separate workspaces."""
    torch = _torch()
    _need(values_t, "values_t", torch.float16)
    _need(meta_t, "meta_t", torch.uint8)
    _need(X, "X", torch.float16, 2)
    if X.stride(1) != 1:
        raise ValueError("X must have unit stride along K (rows of X are the columns of B)")
    C, K = X.shape
    nv, nm = nm_tiled_sizes(R, K)
    if values_t.numel() < nv or meta_t.numel() < nm or not values_t.is_contiguous() or not meta_t.is_contiguous():
        raise ValueError("operand-major arrays do not match R x K")
    need = spmm_nm_tiled_ws_bytes(R, K, C)
    if need > 0:
        _need(workspace, "workspace", torch.uint8)
        if workspace.numel() < need or not workspace.is_contiguous():
            raise ValueError(f"workspace needs {need} contiguous bytes")
    if out is None:
        out = torch.empty((R, C), dtype=torch.float16, device=X.device)
    if out.stride(1) != 1:
        raise ValueError("out must be row-major")
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_len = workspace.numel() if workspace is not None else 0
    check("snm_spmm_nm_tiled_ws",
          load().snm_spmm_nm_tiled_ws(_ptr(values_t), _ptr(meta_t), R, K, _ptr(X), C, X.stride(0),
                                      _ptr(out), out.stride(0), ws_ptr, ws_len, _stream(X)))
    return out


def prune_encode_vnm(A, V: int, M: int):
    """V:2:M prune of fp16 A [R, K] -> (values [R, 2K/M], midx [R, K/(2M)], colloc [R/V, K/M, 4])."""
    return _prune_encode_vnm(A, V, M, "snm_prune_encode_vnm")


def prune_encode_vnm_tiled(A, V: int, M: int):
    """V:2:M prune of fp16 A [R, K] into the row-group interleaved storage (V % 32 == 0):
    (values_t [R, 2K/M], midx_t [R, K/(2M)], colloc [R/V, K/M, 4]). values_t and midx_t
    hold the canonical arrays permuted as snm.h describes; they feed spmm_vnm_tiled."""
    return _prune_encode_vnm(A, V, M, "snm_prune_encode_vnm_tiled")


def _prune_encode_vnm(A, V: int, M: int, entry: str):
    torch = _torch()
    _need(A, "A", torch.float16, 2)
    if A.stride(1) != 1:
        raise ValueError("A must be row-major (unit stride along K)")
    R, K = A.shape
    G = K // M if M > 0 else 0
    values = torch.empty((R, 2 * G), dtype=torch.float16, device=A.device)
    midx = torch.empty((R, G // 2), dtype=torch.uint8, device=A.device)
    colloc = torch.empty((R // V if V > 0 else 0, G, 4), dtype=torch.uint8, device=A.device)
    check(entry, getattr(load(), entry)(_ptr(A), R, K, A.stride(0), V, 2, M, _ptr(values), _ptr(midx),
                                        _ptr(colloc), _stream(A)))
    return values, midx, colloc


def _b_layout(B):
    """(layout, ld) of a [..., K, C] tensor: 0 = row-major (unit stride along C),
    1 = column-major (unit stride along K, e.g. X.t() for activations X [C, K])."""
    if B.stride(-1) == 1 and (B.shape[-1] == 1 or B.stride(-2) >= B.shape[-1]):
        return 0, B.stride(-2)
    if B.stride(-2) == 1:
        return 1, B.stride(-1)
    raise ValueError("B must have unit stride along one of its last two axes")


def spmm_nm(values, meta, B, out=None):
    """Y = decode(values, meta) @ B. 2-D: values [R, K/2], meta [R, K/8], B [K, C] -> Y [R, C].
    3-D (batched): values [b, R, K/2], meta [b, R, K/8], B [b, K, C] -> Y [b, R, C].
    B may be row-major or column-major (a transposed view such as X.t() with X [C, K])."""
    torch = _torch()
    _need(values, "values", torch.float16, (2, 3))
    _need(meta, "meta", torch.uint8, values.dim())
    _need(B, "B", torch.float16, values.dim())
    batched = values.dim() == 3
    if not batched:
        values, meta, B = values[None], meta[None], B[None]
    nb, R, half_k = values.shape
    K = 2 * half_k
    if B.shape[0] != nb or B.shape[1] != K or meta.shape != (nb, R, K // 8):
        raise ValueError(f"shape mismatch: values {tuple(values.shape)}, meta {tuple(meta.shape)}, "
                         f"B {tuple(B.shape)}")
    for t, n in ((values, "values"), (meta, "meta")):
        if t.shape[2] and (t.stride(2) != 1 or t.stride(1) != t.shape[2]):
            raise ValueError(f"{n} must be contiguous per batch entry")
    layout, ldb = _b_layout(B)
    C = B.shape[2]
    if out is None:
        out = torch.empty((nb, R, C), dtype=torch.float16, device=B.device)
    elif not batched:
        out = out[None]
    if out.stride(2) != 1:
        raise ValueError("out must be row-major")
    check("snm_spmm_nm",
          load().snm_spmm_nm(_ptr(values), _ptr(meta), R, K, 2, 4, _ptr(B), C, ldb, layout, _ptr(out),
                             out.stride(1), nb, values.stride(0), meta.stride(0), B.stride(0),
                             out.stride(0), _stream(B)))
    return out if batched else out[0]


def spmm_vnm(values, midx, colloc, B, V: int, M: int, out=None):
    """Y = decode_vnm(values, midx, colloc) @ B with B [K, C] -> Y [R, C]."""
    return _spmm_vnm(values, midx, colloc, B, V, M, out, "snm_spmm_vnm")


def spmm_vnm_tiled(values_t, midx_t, colloc, B, V: int, M: int, out=None):
    """spmm_vnm on the row-group interleaved storage of prune_encode_vnm_tiled (wide-tile
    kernel: V % 32 == 0, C % 8 == 0, B rows 16-byte aligned)."""
    return _spmm_vnm(values_t, midx_t, colloc, B, V, M, out, "snm_spmm_vnm_tiled")


def _spmm_vnm(values, midx, colloc, B, V: int, M: int, out, entry: str):
    torch = _torch()
    _need(values, "values", torch.float16, 2)
    _need(midx, "midx", torch.uint8, 2)
    _need(colloc, "colloc", torch.uint8, 3)
    _need(B, "B", torch.float16, 2)
    R = values.shape[0]
    K, C = B.shape
    if not (values.is_contiguous() and midx.is_contiguous() and colloc.is_contiguous()):
        raise ValueError("values, midx and colloc must be contiguous")
    if B.stride(1) != 1:
        raise ValueError("B must be row-major (unit stride along C)")
    if M <= 0 or V <= 0 or values.shape[1] != 2 * (K // M) or tuple(colloc.shape) != (R // V, K // M, 4):
        raise ValueError("shape mismatch between the V:2:M arrays and B")
    if out is None:
        out = torch.empty((R, C), dtype=torch.float16, device=B.device)
    check(entry, getattr(load(), entry)(_ptr(values), _ptr(midx), _ptr(colloc), R, K, V, 2, M, _ptr(B), C,
                                        B.stride(0), _ptr(out), out.stride(0), _stream(B)))
    return out


def sddmm_prune_nm(Q, Kmat, scale=None, return_dense=False):
    """Scores S = fp16((Q @ Kmat^T) * scale) pruned 2:4 along the key axis.
    Q [b, Lq, d], Kmat [b, Lk, d] -> values [b, Lq, Lk/2], meta [b, Lq, Lk/8] (and S if asked)."""
    torch = _torch()
    _need(Q, "Q", torch.float16, 3)
    _need(Kmat, "Kmat", torch.float16, 3)
    if not (Q.is_contiguous() and Kmat.is_contiguous()):
        raise ValueError("Q and Kmat must be contiguous")
    nb, Lq, d = Q.shape
    if Kmat.shape[0] != nb or Kmat.shape[2] != d:
        raise ValueError("Q and Kmat disagree in batch or head_dim")
    Lk = Kmat.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    values = torch.empty((nb, Lq, Lk // 2), dtype=torch.float16, device=Q.device)
    meta = torch.empty((nb, Lq, Lk // 8), dtype=torch.uint8, device=Q.device)
    S = torch.empty((nb, Lq, Lk), dtype=torch.float16, device=Q.device) if return_dense else None
    check("snm_sddmm_prune_nm",
          load().snm_sddmm_prune_nm(_ptr(Q), _ptr(Kmat), nb, Lq, Lk, d, float(scale), 2, 4, _ptr(values),
                                    _ptr(meta), _ptr(S), _stream(Q)))
    return (values, meta, S) if return_dense else (values, meta)


def sddmm_prune_nm_rowmax(Q, Kmat, scale=None):
    """As sddmm_prune_nm, plus row_max fp32 [b, Lq]: the largest kept score of each row."""
    torch = _torch()
    _need(Q, "Q", torch.float16, 3)
    _need(Kmat, "Kmat", torch.float16, 3)
    if not (Q.is_contiguous() and Kmat.is_contiguous()):
        raise ValueError("Q and Kmat must be contiguous")
    nb, Lq, d = Q.shape
    if Kmat.shape[0] != nb or Kmat.shape[2] != d:
        raise ValueError("Q and Kmat disagree in batch or head_dim")
    Lk = Kmat.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    values = torch.empty((nb, Lq, Lk // 2), dtype=torch.float16, device=Q.device)
    meta = torch.empty((nb, Lq, Lk // 8), dtype=torch.uint8, device=Q.device)
    row_max = torch.empty((nb, Lq), dtype=torch.float32, device=Q.device)
    check("snm_sddmm_prune_nm_rowmax",
          load().snm_sddmm_prune_nm_rowmax(_ptr(Q), _ptr(Kmat), nb, Lq, Lk, d, float(scale), _ptr(values),
                                           _ptr(meta), _ptr(row_max), _stream(Q)))
    return values, meta, row_max


def spmm_nm_softmax(values, meta, row_max, B, out=None):
    """Y = softmax_kept(values) decoded through meta, times B: the row softmax over the kept
    scores is applied inside the product. 2-D: values [R, K/2], meta [R, K/8], row_max [R],
    B [K, C] -> Y [R, C]; 3-D: one more leading batch axis on every argument."""
    torch = _torch()
    _need(values, "values", torch.float16, (2, 3))
    _need(meta, "meta", torch.uint8, values.dim())
    _need(row_max, "row_max", torch.float32, values.dim() - 1)
    _need(B, "B", torch.float16, values.dim())
    batched = values.dim() == 3
    if not batched:
        values, meta, row_max, B = values[None], meta[None], row_max[None], B[None]
    nb, R, half_k = values.shape
    K = 2 * half_k
    if B.shape[0] != nb or B.shape[1] != K or meta.shape != (nb, R, K // 8) or row_max.shape != (nb, R):
        raise ValueError(f"shape mismatch: values {tuple(values.shape)}, meta {tuple(meta.shape)}, "
                         f"row_max {tuple(row_max.shape)}, B {tuple(B.shape)}")
    for t, n in ((values, "values"), (meta, "meta")):
        if t.shape[2] and (t.stride(2) != 1 or t.stride(1) != t.shape[2]):
            raise ValueError(f"{n} must be contiguous per batch entry")
    if row_max.stride(1) != 1:
        raise ValueError("row_max must be contiguous per batch entry")
    if B.stride(2) != 1:
        raise ValueError("B must be row-major (unit stride along C)")
    C = B.shape[2]
    if out is None:
        out = torch.empty((nb, R, C), dtype=torch.float16, device=B.device)
    elif not batched:
        out = out[None]
    if out.stride(2) != 1:
        raise ValueError("out must be row-major")
    check("snm_spmm_nm_softmax",
          load().snm_spmm_nm_softmax(_ptr(values), _ptr(meta), _ptr(row_max), R, K, _ptr(B), C, B.stride(1),
                                     _ptr(out), out.stride(1), nb, values.stride(0), meta.stride(0),
                                     row_max.stride(0), B.stride(0), out.stride(0), _stream(B)))
    return out if batched else out[0]


def bitmap_sizes(R: int, K: int):
    n, m = ctypes.c_int64(), ctypes.c_int64()
    check("snm_bitmap_sizes", load().snm_bitmap_sizes(R, K, ctypes.byref(n), ctypes.byref(m)))
    return n.value, m.value


def bitmap_encode(A):
    """Bitmap format of fp16 A [R, K] (K % 64 == 0) -> (bitmaps int64 [R, K/64],
    tile_offsets int32 [R*K/64 + 1], values fp16 [n]). Two passes; the value count is read
    back between them (one synchronisation)."""
    torch = _torch()
    _need(A, "A", torch.float16, 2)
    if A.stride(1) != 1:
        raise ValueError("A must be row-major (unit stride along K)")
    R, K = A.shape
    nt, no = bitmap_sizes(R, K)
    bitmaps = torch.empty((R, K // 64), dtype=torch.int64, device=A.device)
    offsets = torch.empty((no,), dtype=torch.int32, device=A.device)
    lib = load()
    check("snm_bitmap_count", lib.snm_bitmap_count(_ptr(A), R, K, A.stride(0), _ptr(bitmaps), _ptr(offsets),
                                                   _stream(A)))
    n = int(offsets[-1].item())
    values = torch.empty((n,), dtype=torch.float16, device=A.device)
    check("snm_bitmap_encode", lib.snm_bitmap_encode(_ptr(A), R, K, A.stride(0), _ptr(bitmaps), _ptr(offsets),
                                                     _ptr(values), _stream(A)))
    return bitmaps, offsets, values


def spmm_bitmap(bitmaps, tile_offsets, values, B, out=None):
    """Y = decode(bitmap format) @ B with B [K, C], C <= 32 (row-major, or column-major
    such as X.t() for activations X [C, K])."""
    torch = _torch()
    _need(bitmaps, "bitmaps", torch.int64, 2)
    _need(tile_offsets, "tile_offsets", torch.int32, 1)
    _need(values, "values", torch.float16, 1)
    _need(B, "B", torch.float16, 2)
    R, T = bitmaps.shape
    K, C = B.shape
    if 64 * T != K or tile_offsets.numel() != R * T + 1:
        raise ValueError("bitmap arrays do not match B's K")
    for t, n in ((bitmaps, "bitmaps"), (tile_offsets, "tile_offsets"), (values, "values")):
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    layout, ldb = _b_layout(B)
    if out is None:
        out = torch.empty((R, C), dtype=torch.float16, device=B.device)
    if out.stride(1) != 1:
        raise ValueError("out must be row-major")
    check("snm_spmm_bitmap", load().snm_spmm_bitmap(_ptr(bitmaps), _ptr(tile_offsets), _ptr(values), R, K,
                                                    _ptr(B), C,
                                                    ldb, layout, _ptr(out), out.stride(0), _stream(B)))
    return out


def softmax_nm_rows(values):
    """In-place softmax over the last axis of compressed rows (kept entries only)."""
    torch = _torch()
    _need(values, "values", torch.float16)
    if values.stride(-1) != 1:
        raise ValueError("values must have unit stride along the last axis")
    kept = values.shape[-1]
    rows = values.numel() // kept if kept else 0
    ld = values.stride(-2) if values.dim() >= 2 else kept
    if values.dim() > 2 and not values.is_contiguous():
        raise ValueError("batched values must be contiguous")
    check("snm_softmax_nm_rows", load().snm_softmax_nm_rows(_ptr(values), rows, kept, ld, _stream(values)))
    return values


def attention_nm(Q, Kmat, Vmat, scale=None):
    """Dynamic 2:4 attention: SDDMM-prune, softmax over kept entries, 2:4 SpMM with V.
    Q [b, Lq, d], Kmat [b, Lk, d], Vmat [b, Lk, dv] -> O [b, Lq, dv]."""
    values, meta = sddmm_prune_nm(Q, Kmat, scale)
    softmax_nm_rows(values)
    return spmm_nm(values, meta, Vmat)


def attention_nm_fused(Q, Kmat, Vmat, scale=None):
    """Dynamic 2:4 attention with the softmax folded into the two kernels: the SDDMM also
    writes each row's largest kept score, and the SpMM exponentiates and normalises.
    Same arguments and result as attention_nm."""
    values, meta, row_max = sddmm_prune_nm_rowmax(Q, Kmat, scale)
    return spmm_nm_softmax(values, meta, row_max, Vmat)


# ---------------------------------------------------------------------------------------
# bf16 variants (same layouts; every element buffer holds bf16)

def _qk(Q, Kmat, dtype, scale):
    _need(Q, "Q", dtype, 3)
    _need(Kmat, "Kmat", dtype, 3)
    if not (Q.is_contiguous() and Kmat.is_contiguous()):
        raise ValueError("Q and Kmat must be contiguous")
    nb, Lq, d = Q.shape
    if Kmat.shape[0] != nb or Kmat.shape[2] != d:
        raise ValueError("Q and Kmat disagree in batch or head_dim")
    return nb, Lq, Kmat.shape[1], d, (1.0 / math.sqrt(d) if scale is None else float(scale))


def sddmm_prune_nm_bf16(Q, Kmat, scale=None, return_dense=False, return_rowmax=False):
    """bf16 scores S = bf16((Q @ Kmat^T) * scale) pruned 2:4 along the key axis.
    Returns (values, meta), plus S [b, Lq, Lk] if return_dense and row_max fp32 [b, Lq]
    (largest kept score per row) if return_rowmax, in that order."""
    torch = _torch()
    nb, Lq, Lk, d, scale = _qk(Q, Kmat, torch.bfloat16, scale)
    values = torch.empty((nb, Lq, Lk // 2), dtype=torch.bfloat16, device=Q.device)
    meta = torch.empty((nb, Lq, Lk // 8), dtype=torch.uint8, device=Q.device)
    S = torch.empty((nb, Lq, Lk), dtype=torch.bfloat16, device=Q.device) if return_dense else None
    rmax = torch.empty((nb, Lq), dtype=torch.float32, device=Q.device) if return_rowmax else None
    check("snm_sddmm_prune_nm_bf16",
          load().snm_sddmm_prune_nm_bf16(_ptr(Q), _ptr(Kmat), nb, Lq, Lk, d, scale, _ptr(values), _ptr(meta),
                                         _ptr(S), _ptr(rmax), _stream(Q)))
    return (values, meta) + ((S,) if return_dense else ()) + ((rmax,) if return_rowmax else ())


def softmax_nm_rows_bf16(values):
    """In-place softmax over the last axis of compressed bf16 rows (kept entries only)."""
    torch = _torch()
    _need(values, "values", torch.bfloat16)
    if values.stride(-1) != 1:
        raise ValueError("values must have unit stride along the last axis")
    kept = values.shape[-1]
    rows = values.numel() // kept if kept else 0
    ld = values.stride(-2) if values.dim() >= 2 else kept
    if values.dim() > 2 and not values.is_contiguous():
        raise ValueError("batched values must be contiguous")
    check("snm_softmax_nm_rows_bf16", load().snm_softmax_nm_rows_bf16(_ptr(values), rows, kept, ld,
                                                                      _stream(values)))
    return values


def _rowmajor_spmm_args(values, meta, B, out, dtype, row_max=None):
    """Shapes of a batched 2:4 product with row-major B; adds the batch axis to 2-D input."""
    torch = _torch()
    _need(values, "values", dtype, (2, 3))
    _need(meta, "meta", torch.uint8, values.dim())
    _need(B, "B", dtype, values.dim())
    if row_max is not None:
        _need(row_max, "row_max", torch.float32, values.dim() - 1)
    batched = values.dim() == 3
    if not batched:
        values, meta, B = values[None], meta[None], B[None]
        row_max = row_max[None] if row_max is not None else None
        out = out[None] if out is not None else None
    nb, R, half_k = values.shape
    K = 2 * half_k
    if B.shape[0] != nb or B.shape[1] != K or meta.shape != (nb, R, K // 8) or \
            (row_max is not None and row_max.shape != (nb, R)):
        raise ValueError(f"shape mismatch: values {tuple(values.shape)}, meta {tuple(meta.shape)}, "
                         f"B {tuple(B.shape)}")
    for t, n in ((values, "values"), (meta, "meta")):
        if t.shape[2] and (t.stride(2) != 1 or t.stride(1) != t.shape[2]):
            raise ValueError(f"{n} must be contiguous per batch entry")
    if row_max is not None and row_max.stride(1) != 1:
        raise ValueError("row_max must be contiguous per batch entry")
    if B.stride(2) != 1:
        raise ValueError("B must be row-major (unit stride along C)")
    C = B.shape[2]
    if out is None:
        out = torch.empty((nb, R, C), dtype=dtype, device=B.device)
    if out.stride(2) != 1:
        raise ValueError("out must be row-major")
    return batched, values, meta, B, out, row_max, nb, R, K, C


def spmm_nm_bf16(values, meta, B, out=None):
    """Y = decode(values, meta) @ B on bf16 (row-major B). 2-D: values [R, K/2], meta [R, K/8],
    B [K, C] -> Y [R, C]; 3-D: one more leading batch axis."""
    torch = _torch()
    batched, values, meta, B, out, _, nb, R, K, C = _rowmajor_spmm_args(values, meta, B, out, torch.bfloat16)
    check("snm_spmm_nm_bf16",
          load().snm_spmm_nm_bf16(_ptr(values), _ptr(meta), R, K, _ptr(B), C, B.stride(1), _ptr(out),
                                  out.stride(1), nb, values.stride(0), meta.stride(0), B.stride(0),
                                  out.stride(0), _stream(B)))
    return out if batched else out[0]


def spmm_nm_softmax_bf16(values, meta, row_max, B, out=None):
    """spmm_nm_softmax on bf16 scores, B and Y."""
    torch = _torch()
    batched, values, meta, B, out, row_max, nb, R, K, C = _rowmajor_spmm_args(values, meta, B, out,
                                                                             torch.bfloat16, row_max)
    check("snm_spmm_nm_softmax_bf16",
          load().snm_spmm_nm_softmax_bf16(_ptr(values), _ptr(meta), _ptr(row_max), R, K, _ptr(B), C,
                                          B.stride(1), _ptr(out), out.stride(1), nb, values.stride(0),
                                          meta.stride(0), row_max.stride(0), B.stride(0), out.stride(0),
                                          _stream(B)))
    return out if batched else out[0]


def attention_nm_bf16(Q, Kmat, Vmat, scale=None):
    """attention_nm on bf16 Q, Kmat, Vmat: SDDMM-prune, softmax over kept entries, 2:4 SpMM."""
    values, meta = sddmm_prune_nm_bf16(Q, Kmat, scale)
    softmax_nm_rows_bf16(values)
    return spmm_nm_bf16(values, meta, Vmat)


def attention_nm_fused_bf16(Q, Kmat, Vmat, scale=None):
    """attention_nm_fused on bf16: the SDDMM writes row maxima, the SpMM applies the softmax."""
    values, meta, row_max = sddmm_prune_nm_bf16(Q, Kmat, scale, return_rowmax=True)
    return spmm_nm_softmax_bf16(values, meta, row_max, Vmat)


# ---------------------------------------------------------------------------------------
# 1:2 on fp32 scores

def sddmm_prune_1of2_f32(Q, Kmat, scale=None, return_dense=False, return_rowmax=False):
    """fp32 scores S = (Q @ Kmat^T) * scale pruned 1:2 along the key axis.
    Q [b, Lq, d], Kmat [b, Lk, d] fp32 -> values fp32 [b, Lq, Lk/2], meta uint8 [b, Lq, Lk/4],
    plus S [b, Lq, Lk] if return_dense and row_max [b, Lq] if return_rowmax, in that order."""
    torch = _torch()
    nb, Lq, Lk, d, scale = _qk(Q, Kmat, torch.float32, scale)
    values = torch.empty((nb, Lq, Lk // 2), dtype=torch.float32, device=Q.device)
    meta = torch.empty((nb, Lq, Lk // 4), dtype=torch.uint8, device=Q.device)
    S = torch.empty((nb, Lq, Lk), dtype=torch.float32, device=Q.device) if return_dense else None
    rmax = torch.empty((nb, Lq), dtype=torch.float32, device=Q.device) if return_rowmax else None
    check("snm_sddmm_prune_1of2_f32",
          load().snm_sddmm_prune_1of2_f32(_ptr(Q), _ptr(Kmat), nb, Lq, Lk, d, scale, _ptr(values), _ptr(meta),
                                          _ptr(S), _ptr(rmax), _stream(Q)))
    return (values, meta) + ((S,) if return_dense else ()) + ((rmax,) if return_rowmax else ())


def softmax_nm_rows_f32(values):
    """In-place softmax over the last axis of compressed fp32 rows (kept entries only)."""
    torch = _torch()
    _need(values, "values", torch.float32)
    if values.stride(-1) != 1:
        raise ValueError("values must have unit stride along the last axis")
    kept = values.shape[-1]
    rows = values.numel() // kept if kept else 0
    ld = values.stride(-2) if values.dim() >= 2 else kept
    if values.dim() > 2 and not values.is_contiguous():
        raise ValueError("batched values must be contiguous")
    check("snm_softmax_nm_rows_f32", load().snm_softmax_nm_rows_f32(_ptr(values), rows, kept, ld,
                                                                    _stream(values)))
    return values


def spmm_1of2_f32(values, meta, B, row_max=None, out=None):
    """Y = decode(values, meta) @ B for 1:2 fp32 operands (row-major B). With row_max, the
    row softmax over the kept scores is applied inside the product. 2-D: values [R, K/2],
    meta [R, K/4], B [K, C] (row_max [R]) -> Y [R, C]; 3-D: one more leading batch axis."""
    torch = _torch()
    _need(values, "values", torch.float32, (2, 3))
    _need(meta, "meta", torch.uint8, values.dim())
    _need(B, "B", torch.float32, values.dim())
    if row_max is not None:
        _need(row_max, "row_max", torch.float32, values.dim() - 1)
    batched = values.dim() == 3
    if not batched:
        values, meta, B = values[None], meta[None], B[None]
        row_max = row_max[None] if row_max is not None else None
        out = out[None] if out is not None else None
    nb, R, half_k = values.shape
    K = 2 * half_k
    if B.shape[0] != nb or B.shape[1] != K or meta.shape != (nb, R, K // 4) or \
            (row_max is not None and row_max.shape != (nb, R)):
        raise ValueError(f"shape mismatch: values {tuple(values.shape)}, meta {tuple(meta.shape)}, "
                         f"B {tuple(B.shape)}")
    for t, n in ((values, "values"), (meta, "meta")):
        if t.shape[2] and (t.stride(2) != 1 or t.stride(1) != t.shape[2]):
            raise ValueError(f"{n} must be contiguous per batch entry")
    if row_max is not None and row_max.stride(1) != 1:
        raise ValueError("row_max must be contiguous per batch entry")
    if B.stride(2) != 1:
        raise ValueError("B must be row-major (unit stride along C)")
    C = B.shape[2]
    if out is None:
        out = torch.empty((nb, R, C), dtype=torch.float32, device=B.device)
    if out.stride(2) != 1:
        raise ValueError("out must be row-major")
    check("snm_spmm_1of2_f32",
          load().snm_spmm_1of2_f32(_ptr(values), _ptr(meta), _ptr(row_max), R, K, _ptr(B), C, B.stride(1),
                                   _ptr(out), out.stride(1), nb, values.stride(0), meta.stride(0),
                                   row_max.stride(0) if row_max is not None else 0, B.stride(0),
                                   out.stride(0), _stream(B)))
    return out if batched else out[0]


def attention_1of2_f32(Q, Kmat, Vmat, scale=None):
    """1:2 dynamic attention on fp32: SDDMM-prune, softmax over kept entries, 1:2 product."""
    values, meta = sddmm_prune_1of2_f32(Q, Kmat, scale)
    softmax_nm_rows_f32(values)
    return spmm_1of2_f32(values, meta, Vmat)


def attention_1of2_fused_f32(Q, Kmat, Vmat, scale=None):
    """1:2 fp32 attention with the softmax folded into the two kernels."""
    values, meta, row_max = sddmm_prune_1of2_f32(Q, Kmat, scale, return_rowmax=True)
    return spmm_1of2_f32(values, meta, Vmat, row_max=row_max)
