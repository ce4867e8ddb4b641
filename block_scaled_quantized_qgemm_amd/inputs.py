"""Seeded synthetic inputs for the quantized linear layer.

This module only draws fp32 matrices. It holds none of the quantization or
GEMM arithmetic, and it is the one piece of code that both the CPU oracle's
tests and the GPU path's tests and benchmark share.

Every workload is an activation matrix ``A`` of shape ``[M, K]`` (row-major,
one row per token) and a weight matrix ``W`` of shape ``[N, K]`` (one row per
output channel, K contiguous, the ``nn.Linear`` orientation). Both are float32
and C-contiguous. Generation uses numpy's ``Generator(PCG64(seed))``.

The five named workloads follow the shapes and value distributions of the
pages' experiments:

* ``c1_tiny`` -- "100 Days of GPU, Day 98: Quantization and sparsity",
  section "The program, and the gate that has to be per column": a weight
  whose columns span a 64x range of gains. Here B[k, j] = N(0,1) * 2^(-6j/63)
  for j = 0..63, passed as W = B^T.
* ``c2_per_token`` -- "Activation Quantization Architecture, in depth",
  section "Why activations are harder than weights": a few hidden channels
  tens of times larger than the rest, and one token with extreme values.
  A ~ N(0,1) with channels {7, 1031, 2055, 3079} x30, then row 0 x50;
  W ~ N(0, 0.02^2) with per-channel gains log-uniform over 64x.
* ``c3_asym_uint8`` -- a one-sided (ReLU-like) activation, A = |N(0,1)|;
  W ~ N(0, 0.02^2).
* ``c4_decode`` -- 8 tokens against a wide weight, A ~ N(0,1),
  W ~ N(0, 0.02^2).
* ``c5_mxfp8`` -- A, W ~ N(0,1) with each element x64 with probability 0.01.

One grouped workload, for the grouped (MoE) MX GEMM of "TileLang tutorial,
chapter 27", section 6.2 (MoE): ``make_moe_inputs`` draws E experts' weights
``W [E, N, K]``, the per-expert row counts of the routed activations (a
multinomial over the experts with uneven routing probabilities, softmax of
N(0, 0.5^2) logits), and ``A [M_total, K]`` with every expert's rows stored
one expert after the other; values as ``c5_mxfp8``.
"""
from __future__ import annotations

import numpy as np

__all__ = ["WORKLOADS", "MOE_WORKLOADS", "make_inputs", "make_moe_inputs", "rng_for"]

# name -> (M, K, N, seed, recipe)
WORKLOADS = {
    "c1_tiny": (64, 256, 64, 101, "gain64"),
    "c2_per_token": (512, 4096, 4096, 102, "outliers"),
    "c3_asym_uint8": (2048, 4096, 11008, 103, "relu"),
    "c4_decode": (8, 4096, 14336, 104, "normal"),
    "c5_mxfp8": (8192, 8192, 8192, 105, "spiky"),
}

# name -> (experts E, routed rows M_total (tokens x top-k), K, N per expert, seed)
MOE_WORKLOADS = {
    "c6_moe_mxfp8": (8, 8192, 4096, 4096, 106),
}

_OUTLIER_CHANNELS = (7, 1031, 2055, 3079)


def rng_for(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _normal(rng, shape, sigma=1.0):
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def make_inputs(name: str, M: int | None = None, K: int | None = None,
                N: int | None = None, seed: int | None = None):
    """Return ``(A, W)`` for workload ``name``; M, K, N and seed may be overridden.

    Overriding the sizes keeps the recipe (distribution and structure) and
    only changes the shape, which is how the parity tests build small and
    ragged cases of each workload.
    """
    dM, dK, dN, dseed, recipe = WORKLOADS[name]
    M = dM if M is None else int(M)
    K = dK if K is None else int(K)
    N = dN if N is None else int(N)
    seed = dseed if seed is None else int(seed)
    rng = rng_for(seed)

    if recipe == "gain64":
        A = _normal(rng, (M, K))
        B = _normal(rng, (K, N))
        j = np.arange(N, dtype=np.float64)
        denom = max(N - 1, 1)
        gain = np.exp2(-6.0 * j / denom).astype(np.float32)
        B *= gain[None, :]
        W = np.ascontiguousarray(B.T)
    elif recipe == "outliers":
        A = _normal(rng, (M, K))
        for c in _OUTLIER_CHANNELS:
            if c < K:
                A[:, c] *= np.float32(30.0)
        if M > 0:
            A[0, :] *= np.float32(50.0)
        W = _normal(rng, (N, K), 0.02)
        u = rng.random(N, dtype=np.float64)
        W *= np.exp2(-6.0 * u).astype(np.float32)[:, None]
    elif recipe == "relu":
        A = np.abs(_normal(rng, (M, K)))
        W = _normal(rng, (N, K), 0.02)
    elif recipe == "normal":
        A = _normal(rng, (M, K))
        W = _normal(rng, (N, K), 0.02)
    elif recipe == "spiky":
        A = _normal(rng, (M, K))
        A[rng.random((M, K), dtype=np.float32) < np.float32(0.01)] *= np.float32(64.0)
        W = _normal(rng, (N, K))
        W[rng.random((N, K), dtype=np.float32) < np.float32(0.01)] *= np.float32(64.0)
    else:  # pragma: no cover
        raise ValueError(recipe)
    return np.ascontiguousarray(A, dtype=np.float32), np.ascontiguousarray(W, dtype=np.float32)


def make_moe_inputs(name: str = "c6_moe_mxfp8", E: int | None = None, M: int | None = None,
                    K: int | None = None, N: int | None = None, seed: int | None = None):
    """Return ``(A, W, sizes)`` for a grouped workload: A [M_total, K] (rows of
    expert e at sizes[:e].sum() ..), W [E, N, K], sizes [E] int64."""
    dE, dM, dK, dN, dseed = MOE_WORKLOADS[name]
    E = dE if E is None else int(E)
    M = dM if M is None else int(M)
    K = dK if K is None else int(K)
    N = dN if N is None else int(N)
    seed = dseed if seed is None else int(seed)
    rng = rng_for(seed)
    logits = rng.normal(0.0, 0.5, size=E)
    p = np.exp(logits - logits.max())
    sizes = rng.multinomial(M, p / p.sum()).astype(np.int64)
    A = _normal(rng, (M, K))
    A[rng.random((M, K), dtype=np.float32) < np.float32(0.01)] *= np.float32(64.0)
    W = _normal(rng, (E, N, K))
    W[rng.random((E, N, K), dtype=np.float32) < np.float32(0.01)] *= np.float32(64.0)
    return np.ascontiguousarray(A), np.ascontiguousarray(W), sizes
