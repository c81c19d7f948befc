"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the method: it only draws random numbers
with numpy's PCG64 and stores them as fp32 or as bfloat16 bit patterns.  Both
the HIP path and the CPU oracle receive exactly the arrays produced here.

Distributions follow the workloads the pages describe: LLaMA-style layers with
latent weights drawn N(0, 0.02^2) before ternarisation, activations N(0, 1),
and, for prefill, heavy-tailed Student-t activations (nu = 4).
"""
from __future__ import annotations

import numpy as np

BASE_SEED = 20240227


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), round to nearest even.
    Inputs are finite by construction."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def latent_weights(N: int, K: int, seed: int, std: float = 0.02) -> np.ndarray:
    """Latent fp32 weights W[N x K] ~ N(0, std^2)."""
    return (rng(seed).standard_normal((N, K), dtype=np.float32) * np.float32(std)).astype(np.float32)


def activations_f32(M: int, K: int, seed: int) -> np.ndarray:
    """Activations X[M x K] ~ N(0, 1) in fp32."""
    return rng(seed).standard_normal((M, K), dtype=np.float32)


def activations_bf16(M: int, K: int, seed: int) -> np.ndarray:
    """Activations X[M x K] ~ N(0, 1), returned as bfloat16 bit patterns."""
    return to_bf16_bits(activations_f32(M, K, seed))


def activations_student_t_bf16(M: int, K: int, seed: int, nu: float = 4.0) -> np.ndarray:
    """Heavy-tailed activations X[M x K] ~ Student-t(nu), as bfloat16 bit patterns."""
    x = rng(seed).standard_t(nu, size=(M, K)).astype(np.float32)
    return to_bf16_bits(x)


def ternary_weights(N: int, K: int, seed: int, p_zero: float = 0.31) -> np.ndarray:
    """Random ternary T[N x K] in {-1, 0, +1} (for pack and product tests that
    start from T rather than from latent weights)."""
    r = rng(seed).random((N, K))
    t = np.where(r < p_zero, 0, np.where(r < p_zero + (1 - p_zero) / 2, -1, 1))
    return t.astype(np.int8)


def binary_weights(N: int, K: int, seed: int) -> np.ndarray:
    """Random binary T[N x K] in {-1, +1}, equally likely."""
    return np.where(rng(seed).random((N, K)) < 0.5, -1, 1).astype(np.int8)


def int8_activations(M: int, K: int, seed: int) -> np.ndarray:
    """Random int8 activations in [-127, 127]."""
    return rng(seed).integers(-127, 128, size=(M, K), dtype=np.int16).astype(np.int8)
