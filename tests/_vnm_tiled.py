"""Host-side model of the row-group interleaved V:2:M storage, written from its definition
in include/snm.h (snm_prune_encode_vnm_tiled): with W = K/(4M) chunks per row, value chunk c
(8 fp16 values) of row r sits at element ((r/32)*W + c)*256 + (r%32)*8, and the 16-bit
m-index word c of row r at word ((r/32)*W + c)*32 + (r%32)."""
import numpy as np


def tile(values, midx, M):
    """Canonical (values [R, 2K/M] fp16, midx [R, K/(2M)] uint8) -> interleaved arrays of
    the same shapes."""
    values = np.ascontiguousarray(values)
    R, nv = values.shape
    W = nv // 8
    vt = values.reshape(R // 32, 32, W, 8).transpose(0, 2, 1, 3).reshape(R, nv)
    words = np.ascontiguousarray(midx).view(np.uint16).reshape(R // 32, 32, W)
    mt = words.transpose(0, 2, 1).reshape(R, W)
    return np.ascontiguousarray(vt), np.ascontiguousarray(mt).view(np.uint8)


def untile(values_t, midx_t, M):
    """Interleaved -> canonical."""
    values_t = np.ascontiguousarray(values_t)
    R, nv = values_t.shape
    W = nv // 8
    vals = values_t.reshape(R // 32, W, 32, 8).transpose(0, 2, 1, 3).reshape(R, nv)
    words = np.ascontiguousarray(midx_t).view(np.uint16).reshape(R // 32, W, 32)
    mi = words.transpose(0, 2, 1).reshape(R, W)
    return np.ascontiguousarray(vals), np.ascontiguousarray(mi).view(np.uint8)
