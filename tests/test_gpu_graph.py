"""The decode step (2:4 encode in the operand-major layout + the three SpMMs) captured into a
HIP graph, as the benchmark replays it: every replay, with eager work and synchronizations
between replays, must reproduce the eager results bit for bit (the kernels record no memset
or allocation, and each launch reads only its arguments)."""
import numpy as np
import pytest

import workloads
from _parity import to_dev, to_host

pytestmark = pytest.mark.gpu


def test_decode_step_graph_replays_match_eager():
    import torch
    import structured_sparse_matrix_amd as snm
    from structured_sparse_matrix_amd._lib import load, check
    lib = load()
    R = K = 1024
    NS = (8, 16, 32)
    A = to_dev(workloads.small_matrix(7, (R, K), 0.02))
    Bs = [to_dev(np.ascontiguousarray(workloads.small_matrix(8 + n, (n, K)))) for n in NS]   # X[N][K]
    nv, nm = snm.nm_tiled_sizes(R, K)

    def buffers():
        return (torch.empty((nv,), dtype=torch.float16, device="cuda"),
                torch.empty((nm,), dtype=torch.uint8, device="cuda"),
                [torch.empty((R, n), dtype=torch.float16, device="cuda") for n in NS])

    def step(vals, meta, Ys, stream):
        h = stream.cuda_stream
        check("encode", lib.snm_prune_encode_nm_tiled(A.data_ptr(), R, K, K, vals.data_ptr(), meta.data_ptr(), h))
        for n, X, Y in zip(NS, Bs, Ys):
            check("spmm", lib.snm_spmm_nm_tiled(vals.data_ptr(), meta.data_ptr(), R, K, X.data_ptr(), n, K, 1,
                                               Y.data_ptr(), n, h))

    ev, em, eY = buffers()
    step(ev, em, eY, torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = [to_host(y).view(np.uint16).copy() for y in eY]

    gv, gm, gY = buffers()
    cap = torch.cuda.Stream()
    step(gv, gm, gY, cap)   # first use outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        step(gv, gm, gY, cap)
    for rep in range(4):
        for y in gY:
            y.fill_(7.0)                                      # eager work between replays
        step(ev, em, eY, torch.cuda.current_stream())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, y in enumerate(gY):
            assert np.array_equal(to_host(y).view(np.uint16), ref[i]), f"replay {rep}, N={NS[i]}"


def test_split_decode_product_graph_replays_match_eager():
    # the split reduction in a captured graph: its counters are reset by the kernel itself
    # (no memset node), so every replay must reproduce the eager result bit for bit
    import torch
    import structured_sparse_matrix_amd as snm
    from structured_sparse_matrix_amd._lib import load, check
    lib = load()
    R, K = 1024, 4096                     # 64 row tiles: the split is chosen for every N
    NS = (8, 16, 32)
    A = to_dev(workloads.small_matrix(17, (R, K), 0.02))
    vt, mt = snm.prune_encode_nm_tiled(A)
    Xs = [to_dev(np.ascontiguousarray(workloads.small_matrix(30 + n, (n, K)))) for n in NS]
    need = [snm.spmm_nm_tiled_ws_bytes(R, K, n) for n in NS]
    assert all(b > 0 for b in need)

    def buffers():
        return ([torch.zeros((b,), dtype=torch.uint8, device="cuda") for b in need],
                [torch.empty((R, n), dtype=torch.float16, device="cuda") for n in NS])

    def step(wss, Ys, stream):
        h = stream.cuda_stream
        for n, X, Y, ws, b in zip(NS, Xs, Ys, wss, need):
            check("ws", lib.snm_spmm_nm_tiled_ws(vt.data_ptr(), mt.data_ptr(), R, K, X.data_ptr(), n, K,
                                                 Y.data_ptr(), n, ws.data_ptr(), b, h))

    ews, eY = buffers()
    step(ews, eY, torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = [to_host(y).view(np.uint16).copy() for y in eY]
    gws, gY = buffers()
    cap = torch.cuda.Stream()
    step(gws, gY, cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        step(gws, gY, cap)
    for rep in range(4):
        for y in gY:
            y.fill_(7.0)
        step(ews, eY, torch.cuda.current_stream())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, y in enumerate(gY):
            assert np.array_equal(to_host(y).view(np.uint16), ref[i]), f"replay {rep}, N={NS[i]}"
