"""GPU check of the entry point that allocates nothing (snm_spmm_nm_tiled_noalloc): called
through the C ABI, it must give the bits of snm_spmm_nm_tiled_ws (the same kernels with a
caller's workspace) on calls in a row that share the library's per-device scratch: a split
shape, then a smaller split shape with a different plan (counters and partial tiles at
other offsets), then an unsplit shape, then the first shape again."""
import ctypes

import numpy as np
import pytest

import workloads
from _parity import to_dev, to_host

pytestmark = pytest.mark.gpu


def _c_noalloc(vt, mt, R, K, X, Y):
    import torch
    from structured_sparse_matrix_amd._lib import load
    C = X.shape[0]
    return load().snm_spmm_nm_tiled_noalloc(vt.data_ptr(), mt.data_ptr(), R, K, X.data_ptr(), C,
                                            X.stride(0), Y.data_ptr(), Y.stride(0),
                                            torch.cuda.current_stream().cuda_stream)


def test_noalloc_matches_workspace_entry_point():
    import torch
    import structured_sparse_matrix_amd as snm
    shapes = ((4096, 14336, 32), (3072, 4096, 8), (256, 1024, 16), (4096, 14336, 32))
    assert snm.spmm_nm_tiled_ws_bytes(4096, 14336, 32) > 0 and snm.spmm_nm_tiled_ws_bytes(3072, 4096, 8) > 0
    assert snm.spmm_nm_tiled_ws_bytes(256, 1024, 16) == 0
    for i, (R, K, C) in enumerate(shapes):
        print(f"noalloc call {i}: R={R} K={K} C={C}", flush=True)
        A = workloads.small_matrix(600 + i, (R, K), 0.02)
        X = to_dev(workloads.small_matrix(700 + i, (C, K)))
        vt, mt = snm.prune_encode_nm_tiled(to_dev(A))
        Y = torch.full((R, C), 7.0, dtype=torch.float16, device="cuda")
        assert _c_noalloc(vt, mt, R, K, X, Y) == 0
        nb = snm.spmm_nm_tiled_ws_bytes(R, K, C)
        ws = torch.zeros((max(nb, 16),), dtype=torch.uint8, device="cuda")
        Yref = torch.full((R, C), -3.0, dtype=torch.float16, device="cuda")
        snm.spmm_nm_tiled_ws(vt, mt, R, X, ws, out=Yref)
        got, ref = to_host(Y).view(np.uint16), to_host(Yref).view(np.uint16)
        assert np.array_equal(got, ref), f"call {i} ({R}x{K}x{C}): {np.count_nonzero(got != ref)} outputs differ"


def test_noalloc_rejects_before_launch():
    # host-side checks return their status with nothing enqueued
    import torch
    from structured_sparse_matrix_amd._lib import load
    lib = load()
    X = torch.zeros((40, 64), dtype=torch.float16, device="cuda")
    v = torch.zeros((512,), dtype=torch.float16, device="cuda")
    m = torch.zeros((128,), dtype=torch.uint8, device="cuda")
    Y = torch.zeros((16, 40), dtype=torch.float16, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert lib.snm_spmm_nm_tiled_noalloc(v.data_ptr(), m.data_ptr(), 16, 64, X.data_ptr(), 40, 64,
                                         Y.data_ptr(), 40, s) == 4      # C > 32
    assert lib.snm_spmm_nm_tiled_noalloc(v.data_ptr(), m.data_ptr(), 16, 72, X.data_ptr(), 8, 72,
                                         Y.data_ptr(), 8, s) == 2       # K % 16
