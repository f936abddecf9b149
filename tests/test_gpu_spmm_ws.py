"""GPU parity of the split-reduction decode product (snm_spmm_nm_tiled_ws) against the
float64 oracle: shapes with and without a split, ragged rows and columns, unaligned B
columns, the empty reduction, the full 4096 x 4096 decode workload, and reuse of one
workspace across calls of different shapes (every call must leave the whole workspace
zero, the result must not depend on which split arrives last).""" 
import ctypes

import numpy as np
import pytest

import oracle
import workloads
from _parity import to_dev, to_host, assert_fp16_close

pytestmark = pytest.mark.gpu


def _snm():
    import structured_sparse_matrix_amd as snm
    return snm


def _ws(R, K, C):
    import torch
    n = _snm().spmm_nm_tiled_ws_bytes(R, K, C)
    return torch.zeros((max(n, 16),), dtype=torch.uint8, device="cuda"), n


def _run(A, X, ws=None, ldb_pad=0):
    """X: host [C, K]; ldb_pad > 0 stores it with leading dimension K + ldb_pad."""
    import torch
    snm = _snm()
    R, K = A.shape
    C = X.shape[0]
    vt, mt = snm.prune_encode_nm_tiled(to_dev(A))
    if ldb_pad:
        big = torch.zeros((C, K + ldb_pad), dtype=torch.float16, device="cuda")
        big[:, :K] = to_dev(X)
        Xd = big[:, :K]
    else:
        Xd = to_dev(np.ascontiguousarray(X))
    if ws is None:
        ws, _ = _ws(R, K, C)
    return snm.spmm_nm_tiled_ws(vt, mt, R, Xd, ws)


@pytest.mark.parametrize("R,K,C", [
    (16, 64, 16),      # unsplit kernel
    (33, 1040, 5),     # unsplit kernel, ragged rows and columns
    (100, 4096, 8),    # 4 groups of 2 row tiles (the last partial), 4 splits, ragged rows
    (64, 2048, 32),    # 2 groups of 2 row tiles, 2 splits
    (4100, 8192, 24),  # 65 groups of 4 row tiles (the last partial), 4 splits
    (200, 4096, 24),   # 2 row tiles, 4 splits, 24 of 32 columns
    (1000, 8192, 32),  # 32 groups of 2 row tiles; 8 splits would fill the grid, the plan caps them at 4
    (17, 3072, 12),    # one partial row group
])
def test_spmm_ws_matches_oracle(R, K, C):
    A = workloads.small_matrix(R * 5 + K + C, (R, K), 0.02)
    X = workloads.small_matrix(R + 3 * K + C, (C, K))
    Y = _run(A, X)
    ov, om = oracle.prune_encode_nm(A)
    assert_fp16_close(to_host(Y), oracle.spmm_nm(ov, om, np.ascontiguousarray(X.T)), f"ws {R}x{K}x{C}")


@pytest.mark.parametrize("R,K,C,pad", [(100, 4096, 8, 3), (64, 2048, 32, 5), (40, 512, 16, 1)])
def test_spmm_ws_unaligned_b_columns(R, K, C, pad):
    A = workloads.small_matrix(R + 2 * K + C, (R, K), 0.02)
    X = workloads.small_matrix(R + K + 7 * C, (C, K))
    Y = _run(A, X, ldb_pad=pad)
    ov, om = oracle.prune_encode_nm(A)
    assert_fp16_close(to_host(Y), oracle.spmm_nm(ov, om, np.ascontiguousarray(X.T)), f"ws ldb=K+{pad}")


def test_spmm_ws_empty_reduction_writes_zeros():
    import torch
    from structured_sparse_matrix_amd._lib import load, check
    Y = torch.full((20, 8), 7.0, dtype=torch.float16, device="cuda")
    X = torch.zeros((8, 8), dtype=torch.float16, device="cuda")
    check("ws", load().snm_spmm_nm_tiled_ws(None, None, 20, 0, X.data_ptr(), 8, 8, Y.data_ptr(), 8,
                                            None, 0, torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert not to_host(Y).any()


@pytest.mark.parametrize("R,K", [(4096, 4096), (4096, 14336)])
def test_spmm_ws_decode_workload_full(R, K):
    # decode shapes, N in {8, 16, 32}, X[N][K]: 4096 x 4096 runs the unsplit kernel; at
    # 4096 x 14336 (a feed-forward down projection) N = 16 and 32 run the split reduction.
    # One zero-filled workspace per N, each used twice.
    snm = _snm()
    wl = workloads.WORKLOADS["nm_decode" if K == 4096 else "nm_decode_long_k"]
    assert (wl.R, wl.K) == (R, K)
    A, Bs = workloads.weight_and_activations(wl)
    vt, mt = snm.prune_encode_nm_tiled(to_dev(A))
    ov, om = oracle.prune_encode_nm(A)
    for B in Bs:
        N = B.shape[1]
        ws, n = _ws(R, K, N)
        assert (n > 0) == (K * N >= 163840), (K, N, n)
        X = to_dev(np.ascontiguousarray(B.T))
        Y1 = snm.spmm_nm_tiled_ws(vt, mt, 4096, X, ws)
        assert_fp16_close(to_host(Y1), oracle.spmm_nm(ov, om, B), f"ws decode N={N}")
        Y2 = snm.spmm_nm_tiled_ws(vt, mt, 4096, X, ws)
        assert np.array_equal(to_host(Y1).view(np.uint16), to_host(Y2).view(np.uint16)), f"N={N} rerun"


def test_spmm_ws_reuse_with_smaller_input():
    # the workspace sized for the larger call serves a smaller one next; Y starts filled
    # with a marker so that a call whose last split never fires would be caught
    import torch
    snm = _snm()
    ws, _ = _ws(512, 4096, 32)
    for R, K, seed in ((512, 4096, 1), (136, 2048, 2), (512, 4096, 3)):
        A = workloads.small_matrix(seed, (R, K), 0.02)
        X = workloads.small_matrix(seed + 50, (32, K))
        vt, mt = snm.prune_encode_nm_tiled(to_dev(A))
        out = torch.full((R, 32), 7.0, dtype=torch.float16, device="cuda")
        Y = snm.spmm_nm_tiled_ws(vt, mt, R, to_dev(X), ws, out=out)
        ov, om = oracle.prune_encode_nm(A)
        assert_fp16_close(to_host(Y), oracle.spmm_nm(ov, om, np.ascontiguousarray(X.T)), f"reuse R={R} K={K}")


def test_spmm_ws_two_streams_separate_workspaces():
    # calls that overlap on two streams, each with its own workspace, both give the
    # single-stream result bit for bit
    import torch
    snm = _snm()
    R, K = 1024, 8192
    A = workloads.small_matrix(91, (R, K), 0.02)
    vt, mt = snm.prune_encode_nm_tiled(to_dev(A))
    Xs = [to_dev(workloads.small_matrix(92 + i, (32, K))) for i in range(2)]
    wss = [_ws(R, K, 32)[0] for _ in range(2)]
    assert _snm().spmm_nm_tiled_ws_bytes(R, K, 32) > 0
    ref = [to_host(snm.spmm_nm_tiled_ws(vt, mt, R, X, wss[0])).view(np.uint16).copy() for X in Xs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty((R, 32), dtype=torch.float16, device="cuda") for _ in range(2)]
    for rep in range(8):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                snm.spmm_nm_tiled_ws(vt, mt, R, Xs[i], wss[i], out=outs[i])
        torch.cuda.synchronize()
        for i in range(2):
            assert np.array_equal(to_host(outs[i]).view(np.uint16), ref[i]), f"rep {rep}, stream {i}"


def test_spmm_ws_reuse_across_plans_leaves_workspace_zero():
    # Regression: where the counters end and the partial tiles begin depends on the plan
    # (4096 x 14336, N = 32: counters in bytes [0, 256), partials from 256; 3072 x 4096,
    # N = 8: counters in [0, 512)). One workspace serves both shapes in turn; Y starts
    # filled with a marker, and after every call the whole workspace must be zero again.
    import torch
    snm = _snm()
    shapes = ((4096, 14336, 32), (3072, 4096, 8), (4096, 14336, 32), (1000, 8192, 32))
    nbytes = max(snm.spmm_nm_tiled_ws_bytes(r, k, c) for r, k, c in shapes)
    assert snm.spmm_nm_tiled_ws_bytes(3072, 4096, 8) > 0 and snm.spmm_nm_tiled_ws_bytes(4096, 14336, 32) > 0
    ws = torch.zeros((nbytes,), dtype=torch.uint8, device="cuda")
    for i, (R, K, C) in enumerate(shapes):
        A = workloads.small_matrix(300 + i, (R, K), 0.02)
        X = workloads.small_matrix(400 + i, (C, K))
        vt, mt = snm.prune_encode_nm_tiled(to_dev(A))
        out = torch.full((R, C), 7.0, dtype=torch.float16, device="cuda")
        Y = snm.spmm_nm_tiled_ws(vt, mt, R, to_dev(X), ws, out=out)
        ov, om = oracle.prune_encode_nm(A)
        assert_fp16_close(to_host(Y), oracle.spmm_nm(ov, om, np.ascontiguousarray(X.T)), f"call {i}: {R}x{K}x{C}")
        assert not to_host(ws).any(), f"call {i} ({R}x{K}x{C}) left non-zero bytes in the workspace"
