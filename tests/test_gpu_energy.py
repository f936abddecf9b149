"""Energy (VENOM, Sec. 5, Fig. 11) of the GPU's V:2:M encodings: a 768 x 768 Gaussian weight
(the size of the page's BERT-base query weight), every V and N:M ratio of the figure; the
GPU's kept values must be the oracle's bit for bit, so the energies are identical."""
import numpy as np
import pytest

import oracle
from oracle import energy as E
import workloads
from _parity import to_dev, to_host, assert_bits_equal

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("V", [1, 16, 32, 64, 128])
def test_energy_of_gpu_encodings(V):
    import torch
    import structured_sparse_matrix_amd as snm
    A = workloads.normal_f16(np.random.default_rng(5), (768, 768))
    for M in (4, 5, 8, 10, 20, 40):
        Ap = E.pad_k_for(A, M)
        K = Ap.shape[1]
        lda = -(-K // 8) * 8
        buf = torch.zeros((768, lda), dtype=torch.float16, device="cuda")
        buf[:, :K] = to_dev(Ap)
        v, _, _ = snm.prune_encode_vnm(buf[:, :K], V, M)
        ov, _, _ = oracle.prune_encode_vnm(Ap, V, M)
        got = to_host(v)
        assert_bits_equal(got, ov, f"V{V} M{M} values")
        assert E.energy_of_kept(got, A) == E.energy_vnm(A, V, M)
