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


@pytest.mark.parametrize("R,K,C,V,M", [
    (2048, 1024, 8192, 128, 16),   # 16 x 16 tiles of 128 x 512: the 128-row large-tile product
    (2048, 1024, 1024, 64, 8),     # 32 x 4 tiles of 64 x 256: the 64-row large-tile product
])
def test_vnm_step_graph_replays_match_eager(R, K, C, V, M):
    """The V:N:M step the benchmark times (V:2:M prune/encode into the row-group interleaved
    storage, then the product) captured into a HIP graph: the large-tile products record no
    memset or allocation, so every replay, with eager work between replays, reproduces the
    eager results bit for bit."""
    import torch
    from structured_sparse_matrix_amd import vnm_sizes
    from structured_sparse_matrix_amd._lib import load, check
    lib = load()
    A = to_dev(workloads.small_matrix(31 + M, (R, K), 0.02))
    B = to_dev(workloads.small_matrix(32 + M, (K, C)))
    nv, nm, nc = vnm_sizes(R, K, V, M)

    def buffers():
        return (torch.empty((nv,), dtype=torch.float16, device="cuda"),
                torch.empty((nm,), dtype=torch.uint8, device="cuda"),
                torch.empty((nc,), dtype=torch.uint8, device="cuda"),
                torch.empty((R, C), dtype=torch.float16, device="cuda"))

    def step(bufs, stream):
        v, mi, cl, Y = bufs
        h = stream.cuda_stream
        check("encode", lib.snm_prune_encode_vnm_tiled(A.data_ptr(), R, K, K, V, 2, M, v.data_ptr(), mi.data_ptr(),
                                                       cl.data_ptr(), h))
        check("spmm", lib.snm_spmm_vnm_tiled(v.data_ptr(), mi.data_ptr(), cl.data_ptr(), R, K, V, 2, M, B.data_ptr(),
                                             C, C, Y.data_ptr(), C, h))

    eager = buffers()
    step(eager, torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = [to_host(t).view(np.uint8).copy() for t in eager]

    graph_bufs = buffers()
    cap = torch.cuda.Stream()
    step(graph_bufs, cap)   # first use outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        step(graph_bufs, cap)
    for rep in range(3):
        graph_bufs[3].fill_(7.0)                                # eager work between replays
        step(eager, torch.cuda.current_stream())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, t in enumerate(graph_bufs):
            assert np.array_equal(to_host(t).view(np.uint8), ref[i]), f"replay {rep}, buffer {i}"
