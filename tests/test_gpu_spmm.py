"""GPU parity: 2:4 and V:2:M SpMM against the float64 oracle (fp16 tolerance bars), plus
exact special cases (B = I returns the decoded matrix bit for bit)."""
import numpy as np
import pytest

import oracle
import workloads
from _parity import to_dev, to_host, assert_fp16_close, assert_bits_equal

pytestmark = pytest.mark.gpu


def _snm():
    import structured_sparse_matrix_amd as snm
    return snm


def _nm_case(R, K, C, seed, sigma=1.0):
    A = workloads.small_matrix(seed, (R, K), sigma)
    B = workloads.small_matrix(seed + 1, (K, C))
    ov, om = oracle.prune_encode_nm(A)
    return ov, om, B


@pytest.mark.parametrize("R,K,C", [
    (16, 64, 16), (1, 16, 1), (5, 48, 3), (100, 256, 8), (33, 272, 17), (64, 512, 32),
    (130, 1040, 40), (256, 256, 64), (200, 320, 100), (64, 2048, 260), (16, 16, 512),
])
def test_spmm_nm_shapes(R, K, C):
    snm = _snm()
    ov, om, B = _nm_case(R, K, C, R * 131 + K + C)
    Y = snm.spmm_nm(to_dev(ov), to_dev(om), to_dev(B))
    assert_fp16_close(to_host(Y), oracle.spmm_nm(ov, om, B), f"{R}x{K}x{C}")


@pytest.mark.parametrize("R,K,C", [
    (16, 64, 16), (1, 16, 1), (5, 48, 3), (100, 256, 8), (33, 272, 17), (64, 512, 32),
    (130, 1040, 40), (200, 320, 100), (64, 2048, 260), (300, 4096, 24),
])
def test_spmm_nm_column_major_b(R, K, C):
    # B given as the transpose of a contiguous C x K activation matrix
    snm = _snm()
    ov, om, B = _nm_case(R, K, C, R * 17 + K + C)
    Bcm = to_dev(np.ascontiguousarray(B.T)).t()
    assert Bcm.stride(0) == 1
    Y = snm.spmm_nm(to_dev(ov), to_dev(om), Bcm)
    assert_fp16_close(to_host(Y), oracle.spmm_nm(ov, om, B), f"col-major {R}x{K}x{C}")


@pytest.mark.parametrize("C", [8, 32, 72])
def test_spmm_nm_column_major_padded_ld(C):
    snm = _snm()
    import torch
    R, K = 48, 512
    ov, om, B = _nm_case(R, K, C, 500 + C)
    X = torch.zeros((C, K + 24), dtype=torch.float16, device="cuda")
    X[:, :K] = to_dev(np.ascontiguousarray(B.T))
    Y = snm.spmm_nm(to_dev(ov), to_dev(om), X[:, :K].t())
    assert_fp16_close(to_host(Y), oracle.spmm_nm(ov, om, B), f"col-major ld {K + 24}")
    # odd leading dimension: unaligned columns take the scalar path
    X2 = torch.zeros((C, K + 3), dtype=torch.float16, device="cuda")
    X2[:, :K] = to_dev(np.ascontiguousarray(B.T))
    Y2 = snm.spmm_nm(to_dev(ov), to_dev(om), X2[:, :K].t())
    assert_fp16_close(to_host(Y2), oracle.spmm_nm(ov, om, B), f"col-major ld {K + 3}")


def test_spmm_nm_identity_is_exact_decode():
    snm = _snm()
    A = workloads.small_matrix(21, (48, 128))
    ov, om = oracle.prune_encode_nm(A)
    Y = snm.spmm_nm(to_dev(ov), to_dev(om), to_dev(np.eye(128, dtype=np.float16)))
    dense = oracle.decode_nm(ov, om, 128)
    got = to_host(Y)
    assert np.array_equal(got.astype(np.float64), dense.astype(np.float64))


def test_spmm_nm_batched_column_major():
    snm = _snm()
    nb, R, K, C = 4, 64, 1024, 16
    cases = [_nm_case(R, K, C, 900 + i) for i in range(nb)]
    X = np.stack([np.ascontiguousarray(c[2].T) for c in cases])            # [b, C, K]
    Y = snm.spmm_nm(to_dev(np.stack([c[0] for c in cases])), to_dev(np.stack([c[1] for c in cases])),
                    to_dev(X).transpose(1, 2))
    ref = np.stack([oracle.spmm_nm(*c) for c in cases])
    assert_fp16_close(to_host(Y), ref, "batched column-major")


def test_spmm_nm_batched_and_strided():
    snm = _snm()
    import torch
    nb, R, K, C = 3, 40, 192, 24
    vs, ms, Bs, refs = [], [], [], []
    for i in range(nb):
        ov, om, B = _nm_case(R, K, C, 100 + i)
        vs.append(ov); ms.append(om); Bs.append(B); refs.append(oracle.spmm_nm(ov, om, B))
    Y = snm.spmm_nm(to_dev(np.stack(vs)), to_dev(np.stack(ms)), to_dev(np.stack(Bs)))
    assert_fp16_close(to_host(Y), np.stack(refs), "batched")
    # B and Y with padded leading dimensions
    Bp = torch.zeros((K, 40), dtype=torch.float16, device="cuda")
    Bp[:, :C] = to_dev(Bs[0])
    Yp = torch.full((R, 48), 7.0, dtype=torch.float16, device="cuda")
    snm.spmm_nm(to_dev(vs[0]), to_dev(ms[0]), Bp[:, :C], out=Yp[:, :C])
    got = to_host(Yp)
    assert_fp16_close(got[:, :C], refs[0], "strided")
    assert np.all(got[:, C:] == 7.0), "wrote outside the output view"


def test_spmm_nm_workload_tiny():
    snm = _snm()
    A, (B,) = workloads.weight_and_activations(workloads.WORKLOADS["nm_tiny"])
    ov, om = oracle.prune_encode_nm(A)
    Y = snm.spmm_nm(to_dev(ov), to_dev(om), to_dev(B))
    assert_fp16_close(to_host(Y), oracle.spmm_nm(ov, om, B), "nm_tiny")


def test_spmm_nm_workload_decode_full():
    # the decode-shaped workload at full size, through the same launch path the benchmark times
    snm = _snm()
    A, Bs = workloads.weight_and_activations(workloads.WORKLOADS["nm_decode"])
    v, m = snm.prune_encode_nm(to_dev(A))
    ov, om = oracle.prune_encode_nm(A)
    assert_bits_equal(to_host(v), ov, "decode values")
    for B in Bs:
        ref = oracle.spmm_nm(ov, om, B)
        Y = snm.spmm_nm(v, m, to_dev(B))
        assert_fp16_close(to_host(Y), ref, f"decode N={B.shape[1]}")
        Ycm = snm.spmm_nm(v, m, to_dev(np.ascontiguousarray(B.T)).t())   # activations X[N][K]
        assert_fp16_close(to_host(Ycm), ref, f"decode N={B.shape[1]} column-major B")


def _vnm_case(R, K, C, V, M, seed):
    A = workloads.small_matrix(seed, (R, K), 0.02)
    B = workloads.small_matrix(seed + 1, (K, C))
    return oracle.prune_encode_vnm(A, V, M) + (B,)


@pytest.mark.parametrize("R,K,C,V,M", [
    (64, 512, 64, 64, 8), (128, 1024, 200, 128, 16), (32, 320, 40, 32, 10), (16, 4096, 16, 16, 256),
    (96, 256, 130, 32, 4), (256, 2048, 256, 64, 8), (128, 640, 9, 64, 5),
])
def test_spmm_vnm_shapes(R, K, C, V, M):
    snm = _snm()
    ov, omi, ocl, B = _vnm_case(R, K, C, V, M, R + K + C + V + M)
    Y = snm.spmm_vnm(to_dev(ov), to_dev(omi), to_dev(ocl), to_dev(B), V, M)
    assert_fp16_close(to_host(Y), oracle.spmm_vnm(ov, omi, ocl, V, M, B), f"vnm {R}x{K}x{C} V{V} M{M}")


def test_spmm_vnm_identity_is_exact_decode():
    snm = _snm()
    V, M, K = 32, 8, 256
    A = workloads.small_matrix(31, (64, K))
    ov, omi, ocl = oracle.prune_encode_vnm(A, V, M)
    Y = snm.spmm_vnm(to_dev(ov), to_dev(omi), to_dev(ocl), to_dev(np.eye(K, dtype=np.float16)), V, M)
    dense = oracle.decode_vnm(ov, omi, ocl, V, M, K)
    assert np.array_equal(to_host(Y).astype(np.float64), dense.astype(np.float64))


def test_spmm_vnm_m4_matches_nm():
    snm = _snm()
    A = workloads.small_matrix(41, (64, 256))
    B = workloads.small_matrix(42, (256, 48))
    ov, omi, ocl = oracle.prune_encode_vnm(A, 32, 4)
    Yv = to_host(snm.spmm_vnm(to_dev(ov), to_dev(omi), to_dev(ocl), to_dev(B), 32, 4))
    Yn = to_host(snm.spmm_nm(to_dev(ov), to_dev(omi), to_dev(B)))
    ref = oracle.spmm_nm(ov, omi, B)
    assert_fp16_close(Yv, ref, "vnm M=4")
    assert_fp16_close(Yn, ref, "nm")


def test_spmm_vnm_workload_64_2_8_full():
    snm = _snm()
    A, (B,) = workloads.weight_and_activations(workloads.WORKLOADS["vnm_64_2_8"])
    v, mi, cl = snm.prune_encode_vnm(to_dev(A), 64, 8)
    ov, omi, ocl = oracle.prune_encode_vnm(A, 64, 8)
    assert_bits_equal(to_host(cl), ocl, "colloc")
    Y = snm.spmm_vnm(v, mi, cl, to_dev(B), 64, 8)
    assert_fp16_close(to_host(Y), oracle.spmm_vnm(ov, omi, ocl, 64, 8, B), "vnm_64_2_8")


def test_spmm_vnm_workload_128_2_16_sampled_rows():
    # 8192 x 8192 x 4096: compare 512 sampled rows (every column) with the oracle
    snm = _snm()
    A, (B,) = workloads.weight_and_activations(workloads.WORKLOADS["vnm_128_2_16"])
    v, mi, cl = snm.prune_encode_vnm(to_dev(A), 128, 16)
    Y = snm.spmm_vnm(v, mi, cl, to_dev(B), 128, 16)
    ov, omi, ocl = oracle.prune_encode_vnm(A, 128, 16)
    assert_bits_equal(to_host(v), ov, "values")
    rows = np.sort(np.random.default_rng(0).choice(8192, size=512, replace=False))
    rows = np.unique(np.concatenate([rows, [0, 127, 128, 8191]]))
    Yh = to_host(Y)[rows]
    dense = oracle.decode_vnm(ov, omi, ocl, 128, 16, 8192)[rows]
    ref = dense.astype(np.float64) @ B.astype(np.float64)
    assert_fp16_close(Yh, ref, "vnm_128_2_16 sampled rows")


# ---- wide outputs (C > 32, row-major B, C % 8 == 0): the LDS-ring sparse-MFMA path ------

@pytest.mark.parametrize("R,K,C", [
    (128, 64, 40), (130, 1040, 64), (257, 2080, 136), (96, 528, 256), (384, 4096, 264),
    (33, 16, 512), (1, 48, 48),
])
def test_spmm_nm_wide_shapes(R, K, C):
    snm = _snm()
    ov, om, B = _nm_case(R, K, C, R * 7 + K * 3 + C)
    Y = snm.spmm_nm(to_dev(ov), to_dev(om), to_dev(B))
    assert_fp16_close(to_host(Y), oracle.spmm_nm(ov, om, B), f"wide {R}x{K}x{C}")


@pytest.mark.parametrize("C", [64, 128])
def test_spmm_nm_wide_batched_padded(C):
    snm = _snm()
    import torch
    nb, R, K = 3, 200, 1056
    vs, ms, Bs, refs = [], [], [], []
    for i in range(nb):
        ov, om, B = _nm_case(R, K, C, 900 + i + C)
        vs.append(ov); ms.append(om); Bs.append(B); refs.append(oracle.spmm_nm(ov, om, B))
    Y = snm.spmm_nm(to_dev(np.stack(vs)), to_dev(np.stack(ms)), to_dev(np.stack(Bs)))
    assert_fp16_close(to_host(Y), np.stack(refs), f"wide batched C={C}")
    # B with a padded leading dimension (a multiple of 8) and Y inside a wider buffer
    Bp = torch.zeros((K, C + 16), dtype=torch.float16, device="cuda")
    Bp[:, :C] = to_dev(Bs[1])
    Yp = torch.full((R, C + 8), 7.0, dtype=torch.float16, device="cuda")
    snm.spmm_nm(to_dev(vs[1]), to_dev(ms[1]), Bp[:, :C], out=Yp[:, :C])
    got = to_host(Yp)
    assert_fp16_close(got[:, :C], refs[1], "wide strided")
    assert np.all(got[:, C:] == 7.0), "wrote outside the output view"


def test_spmm_nm_wide_identity_is_exact_decode():
    snm = _snm()
    A = workloads.small_matrix(78, (160, 320))
    ov, om = oracle.prune_encode_nm(A)
    dense = oracle.decode_nm(ov, om, 320).astype(np.float64)
    for C in (64, 128, 320):
        Y = snm.spmm_nm(to_dev(ov), to_dev(om), to_dev(np.eye(320, dtype=np.float16)[:, :C].copy()))
        assert np.array_equal(to_host(Y).astype(np.float64), dense[:, :C]), f"C={C}"


@pytest.mark.parametrize("V,M,K,C", [(128, 16, 1024, 256), (128, 8, 512, 128), (64, 8, 768, 256),
                                     (256, 16, 2048, 72), (64, 12, 960, 48), (64, 8, 96, 64)])
def test_spmm_vnm_wide_identity_is_exact_decode(V, M, K, C):
    snm = _snm()
    A = workloads.small_matrix(V + M + K, (2 * V, K))
    ov, omi, ocl = oracle.prune_encode_vnm(A, V, M)
    dense = oracle.decode_vnm(ov, omi, ocl, V, M, K).astype(np.float64)
    B = np.eye(K, dtype=np.float16)[:, :C].copy()
    Y = snm.spmm_vnm(to_dev(ov), to_dev(omi), to_dev(ocl), to_dev(B), V, M)
    assert np.array_equal(to_host(Y).astype(np.float64), dense[:, :C])


@pytest.mark.parametrize("R,K,C,V,M", [(256, 1024, 200, 128, 16), (384, 640, 136, 128, 10),
                                       (192, 2048, 64, 64, 8), (128, 204, 520, 64, 17)])
def test_spmm_vnm_wide_shapes(R, K, C, V, M):
    snm = _snm()
    ov, omi, ocl, B = _vnm_case(R, K, C, V, M, R * 3 + K + C + V + M)
    Y = snm.spmm_vnm(to_dev(ov), to_dev(omi), to_dev(ocl), to_dev(B), V, M)
    assert_fp16_close(to_host(Y), oracle.spmm_vnm(ov, omi, ocl, V, M, B), f"wide vnm {R}x{K}x{C} V{V} M{M}")


@pytest.mark.parametrize("C,colmajor", [(8, False), (8, True), (32, False), (48, False), (48, True)])
def test_spmm_nm_empty_reduction_writes_zeros(C, colmajor):
    # K = 0: every output is an empty sum; each kernel (decode C <= 32, wide row-major,
    # column-major fallback) must write zeros without reading A or B
    import torch
    snm = _snm()
    b, R = 2, 40
    values = torch.empty((b, R, 0), dtype=torch.float16, device="cuda")
    meta = torch.empty((b, R, 0), dtype=torch.uint8, device="cuda")
    B = (torch.empty((b, C, 0), dtype=torch.float16, device="cuda").transpose(1, 2) if colmajor
         else torch.empty((b, 0, C), dtype=torch.float16, device="cuda"))
    out = torch.full((b, R, C), 7.0, dtype=torch.float16, device="cuda")
    snm.spmm_nm(values, meta, B, out=out)
    assert torch.count_nonzero(out).item() == 0
