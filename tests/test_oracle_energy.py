"""Pins of the energy oracle (VENOM, Sec. 5 and Fig. 11) against closed forms for Gaussian
weights, the page's own figure, brute force and invariants."""
import math

import numpy as np
import pytest
from scipy import integrate, special, stats

import oracle
from oracle import energy as E
import workloads


def _gauss(seed=11, shape=(768, 768)):
    return workloads.normal_f16(np.random.default_rng(seed), shape)


def _halfnormal_order_mean(k: int, n: int) -> float:
    """E[X_(k:n)] for n iid |N(0, 1)|: integral of x times the k-th order-statistic density."""
    c = math.factorial(n) / (math.factorial(k - 1) * math.factorial(n - k))
    F = lambda x: special.erf(x / math.sqrt(2.0))
    f = lambda x: math.sqrt(2.0 / math.pi) * math.exp(-0.5 * x * x)
    val, _ = integrate.quad(lambda x: x * c * F(x) ** (k - 1) * (1 - F(x)) ** (n - k) * f(x), 0, np.inf)
    return val


@pytest.mark.parametrize("s", [0.5, 0.6, 0.75, 0.8, 0.9, 0.95])
def test_unstructured_closed_form_gaussian(s):
    # keeping the fraction q of largest |x| of N(0, 1) keeps exp(-t^2/2) of E|x|, t = the
    # (1 - q/2) quantile
    q = 1.0 - s
    t = stats.norm.ppf(1.0 - q / 2.0)
    assert abs(E.energy_unstructured(_gauss(), s) - math.exp(-0.5 * t * t)) < 0.004


def test_unstructured_loses_a_fifth_at_half_sparsity():
    # VENOM Sec. 5: at 50 % sparsity unstructured magnitude pruning already loses about
    # 20 % of the dense energy (their BERT-base weight; a Gaussian loses 20.3 %)
    assert abs((1.0 - E.energy_unstructured(_gauss(), 0.5)) - 0.20) < 0.01


@pytest.mark.parametrize("M", [4, 8, 10])
def test_top2_of_m_closed_form_gaussian(M):
    # V = 1 (and plain 2:4 for M = 4): each group of M keeps its two largest |x|
    expect = (_halfnormal_order_mean(M - 1, M) + _halfnormal_order_mean(M, M)) / (M * math.sqrt(2 / math.pi))
    A = _gauss(seed=12, shape=(512, 40 * M))
    got = E.energy_vnm(A, 1, M)
    assert abs(got - expect) < 0.005
    if M == 4:
        assert E.energy_nm(A) == got


def test_v1_brute_force_per_group():
    A = _gauss(seed=13, shape=(16, 8 * 10))
    a = np.abs(A.astype(np.float64)).reshape(16, -1, 10)
    top2 = np.sort(a, axis=-1)[..., -2:].sum()
    assert abs(E.energy_vnm(A, 1, 10) - top2 / a.sum()) < 1e-15


def test_vw1_is_unstructured():
    A = _gauss(seed=14, shape=(64, 96))
    for s in (0.5, 0.75, 0.9):
        assert abs(E.energy_vw(A, 1, s) - E.energy_unstructured(A, s)) < 1e-15


@pytest.mark.parametrize("V", [1, 16, 32, 64, 128])
@pytest.mark.parametrize("M", [4, 5, 8, 10, 20, 40])
def test_ideal_bounds_every_structured_policy(V, M):
    A = _gauss(seed=15, shape=(256, 400))
    values, _, _ = oracle.prune_encode_vnm(E.pad_k_for(A, M), V, M)
    e = E.energy_of_kept(values, A)
    assert 0.0 <= e <= E.energy_unstructured_k(A, values.size) + 1e-12
    for l in (4, 8):
        ev = E.energy_vw(A, l, 1.0 - 2.0 / M)
        assert ev <= E.energy_unstructured(A, 1.0 - 2.0 / M) + 1e-12


def test_vnm_m4_keeps_the_2to4_energy_for_every_v():
    A = _gauss(seed=16, shape=(128, 256))
    e24 = E.energy_nm(A)
    for V in (1, 16, 32, 64, 128):
        assert E.energy_vnm(A, V, 4) == e24


def test_padding_adds_nothing():
    # K = 768 with M = 5: padded to 780 columns; the padded zeros never count
    A = _gauss(seed=17, shape=(64, 768))
    Ap = E.pad_k_for(A, 5)
    assert Ap.shape == (64, 780) and np.all(Ap[:, 768:] == 0)
    assert E.energy_of_kept(Ap, A) == 1.0
