"""Error metrics and derived tolerances -- TEST INFRASTRUCTURE ONLY.

Same import rule as the rest of ``oracle/``: only tests, the smoke check and
the benchmark's CPU-baseline leg use it.

* ``column_gate_atol`` / ``column_stat_atol``: "100 Days of GPU -- Day 98:
  Quantization and sparsity", section "The program, and the gate that has to
  be per column". With a = a_hat + e_a, |e_a| <= s_a/2 and likewise for b, one
  product carries at most amax*bColMax/127 of error; the deterministic gate
  adds K of them, the statistical diagnostic sqrt(K) of them, and both carry
  a slack factor of 4. The gate is per output column because columns differ.
* ``rel_l2``, ``max_abs``, ``mismatch_ratio``: "TileLang tutorial, chapter
  27", section 5.2 -- look at the three together.
* ``sqnr_db``: "Activation Quantization Architecture, in depth", section
  "The integer GEMM, written out".
"""
from __future__ import annotations

import numpy as np

GATE_SLACK = 4.0


def column_gate_atol(amax: float, b_col_max, K: int):
    return GATE_SLACK * K * float(amax) * np.asarray(b_col_max, np.float64) / 127.0


def column_stat_atol(amax: float, b_col_max, K: int):
    return GATE_SLACK * np.sqrt(K) * float(amax) * np.asarray(b_col_max, np.float64) / 127.0


def gate_fractions(got, ref, A, W):
    """Largest |got - ref| / atol over all outputs, for the K gate and the sqrt(K) diagnostic.

    ``ref`` is the float64 product of the ORIGINAL float32 inputs (never of
    dequantized copies), A is [M, K], W is [N, K] (column c of B is row c of W).
    Returns (k_frac, sqrtk_frac, first_offender) where first_offender is the
    first (row, col) that fails the K gate, or None.
    """
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    K = A.shape[1]
    amax = float(np.max(np.abs(A))) if A.size else 0.0
    bcol = np.max(np.abs(W), axis=1) if W.size else np.zeros(W.shape[0])
    err = np.abs(got - ref)
    gate = column_gate_atol(amax, bcol, K)[None, :]
    stat = column_stat_atol(amax, bcol, K)[None, :]
    with np.errstate(divide="ignore", invalid="ignore"):
        kf = np.where(gate > 0, err / gate, np.where(err > 0, np.inf, 0.0))
        sf = np.where(stat > 0, err / stat, np.where(err > 0, np.inf, 0.0))
    bad = np.argwhere(kf > 1.0)
    first = tuple(int(v) for v in bad[0]) if len(bad) else None
    return float(kf.max(initial=0.0)), float(sf.max(initial=0.0)), first


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.sqrt(np.sum(ref * ref))
    return float(np.sqrt(np.sum((got - ref) ** 2)) / den) if den > 0 else float(np.sqrt(np.sum(got * got)))


def max_abs(got, ref):
    d = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    return float(d.max(initial=0.0))


def mismatch_ratio(got, ref, rtol, atol):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    bad = np.abs(got - ref) > (atol + rtol * np.abs(ref))
    return float(np.mean(bad))


def sqnr_db(ref, approx):
    ref = np.asarray(ref, np.float64)
    approx = np.asarray(approx, np.float64)
    noise = np.sum((ref - approx) ** 2)
    return float(10.0 * np.log10(np.sum(ref ** 2) / max(noise, 1e-30)))
