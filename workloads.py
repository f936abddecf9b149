"""Seeded synthetic inputs for the five structured-sparse workloads.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It holds only random-number generation and the workload table
(shapes, value distributions, seeds); none of the pruning, encoding or product
arithmetic lives here.

Every tensor is drawn as float64 ``standard_normal`` from
``numpy.random.default_rng(seed)``, multiplied by the workload's sigma and
rounded once to float16 (round to nearest even). Tensors of one workload are
drawn from one generator in the order listed. The same float16 bits feed the
oracle and the GPU. The bf16 and fp32 variants of the attention workload draw
the same float64 numbers and round them to float32, then (bf16) to bf16.

The pages measure on pruned BERT / GPT / OPT / Llama weights and on SQuAD
attention; none of those is available, so these Gaussian tensors, at the
shapes the pages use, stand in for them.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def normal_f16(rng: np.random.Generator, shape, sigma: float = 1.0) -> np.ndarray:
    """float64 standard normal x sigma, rounded once to float16 (RNE)."""
    return (rng.standard_normal(size=shape) * sigma).astype(np.float16)


def normal_f32(rng: np.random.Generator, shape, sigma: float = 1.0) -> np.ndarray:
    """float64 standard normal x sigma, rounded once to float32 (RNE)."""
    return (rng.standard_normal(size=shape) * sigma).astype(np.float32)


def normal_bf16(rng: np.random.Generator, shape, sigma: float = 1.0) -> np.ndarray:
    """bf16 bit patterns (uint16): float64 standard normal x sigma, rounded to float32 and
    then to bf16, both round to nearest even (the second step adds half an ulp minus one,
    plus the kept lowest bit, and truncates)."""
    b = normal_f32(rng, shape, sigma).view(np.uint32)
    return ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                  # "nm", "vnm" or "attention"
    seed: int
    R: int = 0                 # rows of A (and of Y)
    K: int = 0                 # reduction dimension, along which A is pruned
    Cs: tuple = ()             # columns of B (one entry per B drawn)
    sigma_a: float = 1.0
    V: int = 0
    M: int = 4
    batch: int = 0
    heads: int = 0
    seq: int = 0
    head_dim: int = 0
    extra: dict = field(default_factory=dict)


# The workloads. Seeds of all but the first are this library's choice.
WORKLOADS = {
    "nm_tiny": Workload("nm_tiny", "nm", seed=0, R=256, K=256, Cs=(64,), sigma_a=1.0),
    "nm_decode": Workload("nm_decode", "nm", seed=1, R=4096, K=4096, Cs=(8, 16, 32), sigma_a=0.02),
    "vnm_64_2_8": Workload("vnm_64_2_8", "vnm", seed=2, R=11008, K=4096, Cs=(256,), sigma_a=0.02,
                           V=64, M=8),
    "attention_2_4": Workload("attention_2_4", "attention", seed=3, batch=4, heads=16, seq=4096,
                              head_dim=64),
    "vnm_128_2_16": Workload("vnm_128_2_16", "vnm", seed=4, R=8192, K=8192, Cs=(4096,), sigma_a=0.02,
                             V=128, M=16),
    # decode with a long reduction (a feed-forward down projection, 4096 x 14336): the
    # shape on which the split reduction of the decode product is measured
    "nm_decode_long_k": Workload("nm_decode_long_k", "nm", seed=5, R=4096, K=14336, Cs=(8, 16, 32),
                                 sigma_a=0.02),
}


# ---- the general V:N:M sweep (VENOM, Sec. 4 ablations, Fig. 9 and Fig. 10) ---------------
# Problem sizes are R x K x C (A is R x K, B is K x C). The pages' K values are not all
# multiples of 4M, which the format needs (K/M groups, in sets of 4 for whole metadata
# words); K is padded with zero columns of A and zero rows of B up to the next multiple
# of 4M, which changes neither the pruning nor the product.
SWEEP_V = (32, 64, 128)
SWEEP_M = (5, 7, 8, 10, 20, 40, 100)


def pad_k(K: int, M: int) -> int:
    """Smallest multiple of 4M that is >= K."""
    q = 4 * M
    return -(-K // q) * q


def vnm_sweep():
    """(family, R, K_padded, C, V, M) of every sweep point:
    fig9:  1024 x K x 4096, K = 768, 1536, ..., 12288, V = 128, M in {10, 20, 40, 100};
    fig10: 1024 x 4096 x 4096, V in {32, 64, 128}, M in {5, 7, 8, 10, 20, 40, 100};
    gpt3:  36864 x 12288 x 4096, V = 128, M in {8, 10, 20} (the larger problem the
           pages repeat the study on)."""
    pts = []
    for M in (10, 20, 40, 100):
        for K in range(768, 12288 + 1, 768):
            pts.append(("fig9", 1024, pad_k(K, M), 4096, 128, M))
    for V in SWEEP_V:
        for M in SWEEP_M:
            pts.append(("fig10", 1024, pad_k(4096, M), 4096, V, M))
    for M in (8, 10, 20):
        pts.append(("gpt3", 36864, pad_k(12288, M), 4096, 128, M))
    return pts


# ---- unstructured sparsity in the bitmap format (Coruscant, Sec. 4 and 5.2) ----------------
# The pages measure the kernel on OPT-30B / OPT-66B weight matrices (7168 x 7168 and
# 9216 x 9216) pruned to 30-70 % unstructured sparsity, at N = 8 activations. Stand-in:
# A ~ N(0, 0.02) with every entry below the s-quantile of |A| set to zero (magnitude
# pruning over the whole matrix); B ~ N(0, 1).
BITMAP_SHAPES = (7168, 9216)
BITMAP_SPARSITY = (0.3, 0.5, 0.7)


def pruned_unstructured(seed: int, R: int, K: int, sparsity: float, sigma: float = 0.02) -> np.ndarray:
    """Gaussian fp16 matrix with the smallest-magnitude fraction `sparsity` zeroed."""
    A = normal_f16(np.random.default_rng(seed), (R, K), sigma)
    if sparsity > 0:
        mag = np.abs(A.astype(np.float32))
        t = np.quantile(mag, sparsity)
        A[mag <= t] = 0
    return A


def weight_and_activations(w: Workload):
    """A (R x K) then one B (K x C) per entry of ``w.Cs``, from one generator."""
    rng = np.random.default_rng(w.seed)
    A = normal_f16(rng, (w.R, w.K), w.sigma_a)
    Bs = [normal_f16(rng, (w.K, c), 1.0) for c in w.Cs]
    return A, Bs


def attention_qkv(w: Workload):
    """Q, K, V of shape [batch*heads, seq, head_dim], drawn in that order."""
    rng = np.random.default_rng(w.seed)
    shape = (w.batch * w.heads, w.seq, w.head_dim)
    return tuple(normal_f16(rng, shape, 1.0) for _ in range(3))


def attention_qkv_typed(w: Workload, dtype: str):
    """attention_qkv drawn in another element type: "bf16" (uint16 bit patterns) or "f32"."""
    rng = np.random.default_rng(w.seed)
    shape = (w.batch * w.heads, w.seq, w.head_dim)
    draw = {"bf16": normal_bf16, "f32": normal_f32}[dtype]
    return tuple(draw(rng, shape, 1.0) for _ in range(3))


def small_matrix(seed: int, shape, sigma: float = 1.0) -> np.ndarray:
    """One seeded float16 matrix, for small parity and edge cases."""
    return normal_f16(np.random.default_rng(seed), shape, sigma)


def ties_matrix(seed: int, shape, levels: int = 4) -> np.ndarray:
    """float16 values drawn from a few magnitudes with random signs, so that many
    groups hold exact magnitude ties and signed zeros."""
    rng = np.random.default_rng(seed)
    mags = rng.integers(0, levels, size=shape).astype(np.float64) * 0.5
    sign = np.where(rng.integers(0, 2, size=shape) == 0, -1.0, 1.0)
    return (mags * sign).astype(np.float16)
