"""Energy (magnitude preservation) of a pruning policy.

Test infrastructure (see the package docstring): imported only by tests, the
smoke check and the benchmark.

Source
------
"VENOM: A vectorized N:M format ...", Sec. 5 (Energy evaluation of V:N:M) and
Fig. 11: the energy of a pruned weight tensor is the sum of the magnitudes of
the weights it keeps over the sum of the magnitudes of the dense tensor, a
score in [0, 1]. The section compares unstructured magnitude pruning (the
ideal policy: no constraint on where non-zeros sit), V:N:M for several V
(here V:2:M, sparsity 1 - 2/M), and vector-wise pruning with vector length l
(vw_l), at the sparsity levels of plain N:M ratios 2:4 ... 2:40.

Readings where the pages are silent
-----------------------------------
* Unstructured at sparsity s keeps the round((1 - s) d) weights of largest
  magnitude (d = number of weights).
* vw_l: the vectors are l consecutive rows of one column (the orientation of
  V:N:M's V), ranked by the sum of their magnitudes (the L1 norm, which is the
  quantity the energy counts); the round((1 - s) n) vectors of largest norm are
  kept, n = number of vectors. R must be a multiple of l.
* V:2:M with K not a multiple of 4M: K is zero-padded up to the next multiple,
  as in the sweep; padded zeros add nothing to either sum.
"""
from __future__ import annotations

import numpy as np

from .vnm import prune_encode_vnm
from .nm import prune_encode_nm


def _abs_sum(x) -> float:
    return float(np.abs(np.asarray(x, dtype=np.float64)).sum())


def energy_of_kept(kept_values, A) -> float:
    """sum |kept| / sum |A| (float64)."""
    total = _abs_sum(np.asarray(A, dtype=np.float16))
    return _abs_sum(np.asarray(kept_values, dtype=np.float16)) / total if total > 0 else 1.0


def energy_unstructured(A, sparsity: float) -> float:
    """Keep the round((1 - s) d) largest |a| anywhere in A."""
    a = np.abs(np.asarray(A, dtype=np.float16).astype(np.float64)).ravel()
    k = int(round((1.0 - sparsity) * a.size))
    if k <= 0:
        return 0.0
    top = np.partition(a, a.size - k)[a.size - k:]
    return float(top.sum()) / float(a.sum())


def energy_unstructured_k(A, k: int) -> float:
    """Keep the k largest |a| anywhere in A."""
    a = np.abs(np.asarray(A, dtype=np.float16).astype(np.float64)).ravel()
    if k <= 0:
        return 0.0
    k = min(k, a.size)
    top = np.partition(a, a.size - k)[a.size - k:]
    return float(top.sum()) / float(a.sum())


def pad_k_for(A, M: int):
    """A zero-padded along K to the next multiple of 4M."""
    A = np.asarray(A, dtype=np.float16)
    R, K = A.shape
    q = 4 * M
    Kp = -(-K // q) * q
    if Kp == K:
        return A
    out = np.zeros((R, Kp), dtype=np.float16)
    out[:, :K] = A
    return out


def energy_nm(A) -> float:
    """Plain 2:4 (the lecture notes' rule)."""
    values, _ = prune_encode_nm(np.asarray(A, dtype=np.float16))
    return energy_of_kept(values, A)


def energy_vnm(A, V: int, M: int) -> float:
    """V:2:M with the oracle's selection rule (K zero-padded to a multiple of 4M)."""
    values, _, _ = prune_encode_vnm(pad_k_for(A, M), V, M)
    return energy_of_kept(values, A)


def energy_vw(A, l: int, sparsity: float) -> float:
    """Vector-wise: l x 1 column vectors ranked by L1 norm; keep round((1 - s) n)."""
    a = np.abs(np.asarray(A, dtype=np.float16).astype(np.float64))
    R, K = a.shape
    norms = a.reshape(R // l, l, K).sum(axis=1).ravel()
    n = norms.size
    k = int(round((1.0 - sparsity) * n))
    if k <= 0:
        return 0.0
    top = np.partition(norms, n - k)[n - k:]
    return float(top.sum()) / float(a.sum())
