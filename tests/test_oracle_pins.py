"""Pins for the CPU oracle: each test ties one oracle function to something the
pages or the mathematics fix, independently of the oracle's own code.

Pages: [D98] "100 Days of GPU -- Day 98: Quantization and sparsity";
[TL27] "TileLang tutorial, chapter 27: low-precision quantization";
[SK] "Skill: Write an INT8 Quantized Kernel";
[AQ] "Activation Quantization Architecture, in depth".
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from oracle import metrics as MT
from block_scaled_quantized_qgemm_amd.inputs import make_inputs, rng_for
from conftest import GOLDEN


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# Symmetric quantizer: the worked outlier example ([AQ] "Why activations are
# harder than weights")
# --------------------------------------------------------------------------
def test_outlier_row_worked_example():
    g = _golden("aq_outlier_row.json")
    rng = rng_for(1)
    row = rng.uniform(-2.0, 2.0, size=64).astype(np.float32)
    row[5] = np.float32(g["with_outlier"]["x"])
    row[9] = np.float32(g["with_outlier"]["row_max"])
    q, s = O.quantize_sym_int8(row[None, :], per_row=True)
    assert abs(float(s[0]) - g["with_outlier"]["scale_approx"]) < 0.005
    assert int(q[0, 5]) == g["with_outlier"]["code"]
    xhat = float(q[0, 5]) * float(s[0])
    assert abs(xhat - g["with_outlier"]["dequant_approx"]) < 0.005
    assert abs(xhat - 0.3) / 0.3 > g["with_outlier"]["rel_error_greater_than"]

    row2 = row.copy()
    row2[9] = np.float32(1.0)
    row2[10] = np.float32(g["without_outlier"]["row_max"])
    row2 = np.clip(row2, -2.0, 2.0).astype(np.float32)
    q2, s2 = O.quantize_sym_int8(row2[None, :], per_row=True)
    assert abs(float(s2[0]) - g["without_outlier"]["scale_approx"]) < 0.001
    xhat2 = float(q2[0, 5]) * float(s2[0])
    assert abs(xhat2 - 0.3) / 0.3 < g["without_outlier"]["rel_error_within"]
    # the exact value: rint(0.3 / (2/127)) = rint(19.05) = 19
    assert int(q2[0, 5]) == 19


# --------------------------------------------------------------------------
# Per-tensor code starvation ([D98] opening and "What a scale actually promises")
# --------------------------------------------------------------------------
def test_code_starvation_per_tensor_vs_per_channel():
    g = _golden("d98_code_starvation.json")
    A, W = make_inputs("c1_tiny")
    # column j of B is row j of W; row 63 carries gain 2^-6 = 1/64
    qt, st = O.quantize_sym_int8(W, per_row=False)
    mags = sorted(set(np.abs(qt[63].astype(int)).tolist()))
    assert mags == g["per_tensor_code_magnitudes"]
    qc, sc = O.quantize_sym_int8(W, per_row=True)
    assert np.all(np.max(np.abs(qc.astype(int)), axis=1) == g["per_channel_max_code"])
    assert len(set(qc[63].tolist())) > 100          # the quiet column keeps its range
    assert st.shape == (1,) and sc.shape == (64,)


# --------------------------------------------------------------------------
# Rounding: half to even on the float32 quotient; clamp always ([D98] Pitfalls)
# --------------------------------------------------------------------------
def test_round_half_even_ties_and_clamp():
    # amax = 127/8 makes s = 1/8 exactly, so x = (n + 1/2)/8 is an exact tie
    x = np.array([[127 / 8, 2.5 / 8, 3.5 / 8, -2.5 / 8, -3.5 / 8, 0.5 / 8, -0.5 / 8, 0.0]], np.float32)
    q, s = O.quantize_sym_int8(x)
    assert float(s[0]) == 0.125
    assert q[0].tolist() == [127, 2, 4, -2, -4, 0, 0, 0]


def test_scale_floor_all_zero_row():
    q, s = O.quantize_sym_int8(np.zeros((2, 16), np.float32))
    assert np.all(s == np.float32(1e-8)) and np.all(q == 0)
    q, s, z = O.quantize_asym_uint8(np.full((1, 8), 3.0, np.float32))
    assert float(s[0]) == np.float32(1e-8)
    assert int(z[0]) == 0 and np.all(q == 255)  # clamped, reading: z in [0, 255]


# --------------------------------------------------------------------------
# Storage error ([TL27] 2.4: max error s/2, RMS s/sqrt(12), u = 1/254 of absmax;
# [SK] "Correctness requirements": round trip within 0.5 * scale)
# --------------------------------------------------------------------------
def test_storage_error_bounds_symmetric():
    g = _golden("format_constants.json")
    A, _ = make_inputs("c2_per_token", M=64, K=4096, N=8)
    q, s = O.quantize_sym_int8(A)
    err = np.abs(A.astype(np.float64) - q.astype(np.float64) * s[:, None])
    half = s.astype(np.float64)[:, None] / 2
    assert np.all(err <= half * (1 + 1e-6))
    amax = np.max(np.abs(A), axis=1).astype(np.float64)
    assert np.all(err.max(axis=1) / amax <= g["int8_u"] * (1 + 1e-3))
    rms = np.sqrt(np.mean(err[1:] ** 2, axis=1)) / s[1:]
    assert np.all(np.abs(rms - 1 / math.sqrt(12)) < 0.02)


def test_storage_error_bounds_asymmetric():
    A, _ = make_inputs("c2_per_token", M=32, K=2048, N=8)   # rows contain both signs
    q, s, z = O.quantize_asym_uint8(A)
    xhat = (q.astype(np.float64) - z[:, None]) * s[:, None]
    err = np.abs(A - xhat)
    assert np.all(err <= s[:, None].astype(np.float64) / 2 * (1 + 1e-5) + 1e-7)
    assert np.all(z > 0) and np.all(z < 255)


def test_one_sided_rows_get_zero_point_zero():
    # reading: on |N(0,1)| rows -min/s rounds to 0, so z = 0 and x = q*s
    A, _ = make_inputs("c3_asym_uint8", M=16, K=4096, N=8)
    q, s, z = O.quantize_asym_uint8(A)
    assert np.all(z == 0)
    assert np.max(q) == 255


# --------------------------------------------------------------------------
# Accumulator bound ([D98] "What a scale actually promises", [AQ] "The integer
# GEMM, written out", [SK] step 2)
# --------------------------------------------------------------------------
def test_accumulator_bounds_and_limits():
    g = _golden("format_constants.json")
    assert 127 * 127 == g["sym_product_max"]
    ks = O.k_limit(asymmetric=False)
    assert abs(ks - g["sym_terms_about"]) < 1000 and ks * 16129 <= 2**31 - 1 < (ks + 1) * 16129
    ka = O.k_limit(asymmetric=True)
    assert ka * 255 * 127 <= 2**31 - 1 < (ka + 1) * 255 * 127
    K = 4096
    full = np.full((1, K), 127, np.int8)
    assert O.int_gemm(full, 0, full)[0, 0] == K * 16129
    # uint8 code 0 with zero point 128 is -128: the K*127*128 extreme of [D98]
    zero = np.zeros((1, K), np.uint8)
    neg = np.full((1, K), -127, np.int8)
    assert O.int_gemm(zero, 128, neg)[0, 0] == K * 127 * 128
    top = np.full((1, K), 255, np.uint8)
    assert O.int_gemm(top, 0, full)[0, 0] == K * 255 * 127


# --------------------------------------------------------------------------
# Integer GEMM: brute force against pure-Python integers on tiny shapes
# --------------------------------------------------------------------------
def test_int_gemm_every_code_pair():
    a = np.arange(-127, 128, dtype=np.int8)
    for qw in (-127, -1, 0, 1, 5, 127):
        C = O.int_gemm(a[:, None], 0, np.array([[qw]], np.int8))
        assert C[:, 0].tolist() == [int(v) * qw for v in a]
    u = np.arange(0, 256, dtype=np.uint8)
    for z in (0, 1, 128, 255):
        C = O.int_gemm(u[:, None], z, np.array([[-127]], np.int8))
        assert C[:, 0].tolist() == [(int(v) - z) * -127 for v in u]


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (2, 3, 7), (7, 17, 33), (17, 5, 65), (3, 33, 127)])
def test_int_gemm_brute_force(M, N, K):
    rng = rng_for(M * 1000 + N * 10 + K)
    qa = rng.integers(0, 256, (M, K)).astype(np.uint8)
    z = rng.integers(0, 256, M).astype(np.int32)
    qw = rng.integers(-127, 128, (N, K)).astype(np.int8)
    C = O.int_gemm(qa, z, qw)
    for m in range(M):
        for n in range(N):
            ref = 0
            for k in range(K):
                ref += (int(qa[m, k]) - int(z[m])) * int(qw[n, k])
            assert C[m, n] == ref
    rows = np.arange(M).repeat(N)
    cols = np.tile(np.arange(N), M)
    assert np.array_equal(O.int_gemm_entries(qa, z, qw, rows, cols), C.reshape(-1))


# --------------------------------------------------------------------------
# Epilogue: scales once, against dequantize-then-multiply in float64
# ([AQ] "The integer GEMM, written out"; [D98] section on the program)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("act", ["sym_row", "sym_tensor", "asym_row", "asym_tensor"])
@pytest.mark.parametrize("wgt", ["channel", "tensor"])
def test_epilogue_equals_dequantize_then_multiply(act, wgt):
    A, W = make_inputs("c2_per_token", M=24, K=512, N=40, seed=7)
    r = O.quantized_linear(A, W, act=act, wgt=wgt)
    za = np.broadcast_to(r["z_a"].reshape(-1, 1), (24, 1)).astype(np.float64)
    sa = np.broadcast_to(r["s_a"].reshape(-1, 1), (24, 1)).astype(np.float64)
    sw = np.broadcast_to(r["s_w"].reshape(-1, 1), (40, 1)).astype(np.float64)
    xhat = (r["q_a"].astype(np.float64) - za) * sa
    what = r["q_w"].astype(np.float64) * sw
    direct = xhat @ what.T
    S = np.abs(xhat) @ np.abs(what).T
    assert np.all(np.abs(direct - r["y"]) <= 1e-13 * S + 1e-300)
    # integer identity: sum (qa - z) qw == sum qa qw - z * colsum(qw)
    raw = O.int_gemm(r["q_a"], 0, r["q_w"])
    assert np.array_equal(r["C"], raw - r["z_a"].astype(np.int64).reshape(-1, 1) * r["colsum"][None, :])


def test_dropped_zero_point_is_a_per_column_offset():
    # [D98] Pitfalls, [AQ] Failure modes: dropping z*colsum shifts each column by a constant
    A, W = make_inputs("c3_asym_uint8", M=16, K=256, N=12)
    A = A - np.float32(0.5)                      # rows with both signs, z != 0
    qa, sa, za = O.quantize_asym_uint8(A, per_row=False)
    qw, sw, colsum = O.prepare_weights_int8(W)
    good = O.int_gemm(qa, za, qw)
    planted = O.int_gemm(qa, 0, qw)              # the mistake, planted in the oracle
    d = planted - good
    assert int(za[0]) != 0
    assert np.all(d == d[0:1, :])                # constant down every column
    assert np.array_equal(d[0], int(za[0]) * colsum)


# --------------------------------------------------------------------------
# The per-column gate of [D98] against the float64 product of the ORIGINAL inputs
# --------------------------------------------------------------------------
def test_quality_gate_per_column_c1():
    A, W = make_inputs("c1_tiny")
    ref = A.astype(np.float64) @ W.astype(np.float64).T
    pc = O.quantized_linear(A, W, act="sym_tensor", wgt="channel")["y"]
    pt = O.quantized_linear(A, W, act="sym_tensor", wgt="tensor")["y"]
    kf_c, sf_c, first_c = MT.gate_fractions(pc, ref, A, W)
    kf_t, sf_t, first_t = MT.gate_fractions(pt, ref, A, W)
    assert first_c is None and kf_c <= 1.0           # per-column rows pass the K gate
    assert sf_c < 1.0 < sf_t                         # the sqrt(K) diagnostic separates them
    # the per-tensor error concentrates in the quiet columns (an axis-correlated error)
    err_t = np.abs(pt - ref).max(axis=0)
    err_c = np.abs(pc - ref).max(axis=0)
    assert err_t[-8:].mean() > 4 * err_c[-8:].mean()


def test_per_token_scales_recover_bits():
    # [D98] Exercise and [AQ] "Why activations...": one extreme row sets a
    # per-tensor scale and costs every other row several bits
    A, W = make_inputs("c2_per_token", M=32, K=4096, N=64)
    ref = A.astype(np.float64) @ W.astype(np.float64).T
    tok = O.quantized_linear(A, W, act="sym_row")["y"]
    ten = O.quantized_linear(A, W, act="sym_tensor")["y"]
    _, s_row = O.quantize_sym_int8(A, per_row=True)
    _, s_ten = O.quantize_sym_int8(A, per_row=False)
    # the step of every other row is more than 2^4 times finer per token
    assert np.all(np.log2(s_ten[0] / s_row[1:]) > 4.0)
    e_tok = np.sqrt(np.mean((tok[1:] - ref[1:]) ** 2))
    e_ten = np.sqrt(np.mean((ten[1:] - ref[1:]) ** 2))
    assert e_ten / e_tok > 4.0


# --------------------------------------------------------------------------
# E8M0 ([TL27] 2.3(b)) -- pinned to a definition through frexp, not the bit trick
# --------------------------------------------------------------------------
def _ceil_pow2_exponent(t: float) -> int:
    m, e = math.frexp(abs(t))          # t = m * 2^e, m in [0.5, 1)
    k = e - 1 if m == 0.5 else e       # smallest k with 2^k >= t
    return min(max(k + 127, 1), 254)


def test_ceil_to_ue8m0_spot_values_and_sweep():
    g = _golden("format_constants.json")
    spots = {1.0: 127, 1.5: 128, 0.75: 127, 2.0: 128, 0.5: 126, 448.0: 136,
             2.0 ** -126: 1, 2.0 ** -140: 1, 1e-45: 1, 2.0 ** 127: 254, 3e38: 254}
    for t, E in spots.items():
        assert int(O.ceil_to_ue8m0(np.float32(t))) == E, t
    rng = rng_for(5)
    t = np.exp2(rng.uniform(-135, 128, 20000)).astype(np.float32)
    t = t[np.isfinite(t) & (t > 0)]
    E = O.ceil_to_ue8m0(t)
    ref = np.array([_ceil_pow2_exponent(float(v)) for v in t])
    assert np.array_equal(E.astype(int), ref)
    assert E.min() >= 1 and E.max() <= 254 and g["e8m0_nan_code"] == 255
    assert O.e8m0_value(np.array([1]))[0] == 2.0 ** (1 - 127)
    assert O.e8m0_value(np.array([254]))[0] == 2.0 ** g["e8m0_max_exp"]


# --------------------------------------------------------------------------
# e4m3 codec ([TL27] 2.2) -- pinned to the format facts and to torch's cast
# --------------------------------------------------------------------------
def test_e4m3_format_facts():
    g = _golden("format_constants.json")
    v = O.E4M3_VALUES
    assert v[g["e4m3_max_code"]] == g["e4m3_max"] == 1.75 * 2 ** 8
    assert all(np.isnan(v[c]) for c in g["e4m3_nan_codes"])
    assert np.sum(np.isnan(v)) == 2
    assert v[0x38] == 1.0 and v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6
    assert v[g["e4m3_neg_zero_code"]] == 0.0 and math.copysign(1, v[0x80]) == -1
    assert int(O.e4m3_encode_rne(np.float32(448.0))) == 0x7E
    assert int(O.e4m3_encode_rne(np.float32(-0.0))) == 0x80
    assert int(O.e4m3_encode_rne(np.float32(1.0))) == 0x38
    fin = [c for c in range(256) if not np.isnan(v[c])]
    assert np.array_equal(O.e4m3_encode_rne(v[fin].astype(np.float32)), np.array(fin, np.uint8))


def test_e4m3_ties_to_even_and_relative_error():
    g = _golden("format_constants.json")
    pos = O.E4M3_VALUES[:127]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    codes = O.e4m3_encode_rne(mids)
    assert np.all(codes % 2 == 0)
    assert np.all((codes == np.arange(126)) | (codes == np.arange(1, 127)))
    rng = rng_for(9)
    y = rng.uniform(2.0 ** -6, 448.0, 100000).astype(np.float32)
    rel = np.abs(O.e4m3_decode(O.e4m3_encode_rne(y)) - y) / y
    assert rel.max() <= g["e4m3_u"] * (1 + 1e-9)         # u = 2^-p, p = 4
    assert rel.max() > g["e4m3_u"] * 0.9                  # and the bound is tight


def test_e4m3_matches_torch_cast():
    torch = pytest.importorskip("torch")
    rng = rng_for(10)
    y = np.concatenate([
        rng.uniform(-448, 448, 200000),
        np.exp2(rng.uniform(-14, 8.8, 200000)) * rng.choice([-1, 1], 200000),
        ((O.E4M3_VALUES[:126] + O.E4M3_VALUES[1:127]) / 2),
    ]).astype(np.float32)
    y = np.clip(y, -448, 448).astype(np.float32)
    ours = O.e4m3_encode_rne(y)
    theirs = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch turns tiny negatives into +0 or -0 consistently with the sign; compare values
    assert np.array_equal(O.e4m3_decode(ours), O.e4m3_decode(theirs))


# --------------------------------------------------------------------------
# MX quantization ([TL27] 2.2 item 3, 2.3, 7 pitfall 6)
# --------------------------------------------------------------------------
def test_mx_quantize_scales_are_exact_and_never_overflow():
    A, _ = make_inputs("c5_mxfp8", M=64, K=1024, N=8)
    codes, E = O.quantize_mx(A)
    assert codes.shape == A.shape and E.shape == (64, 32)
    sf = O.e8m0_value(E)
    blocks = A.reshape(64, 32, 32).astype(np.float64)
    amax = np.maximum(np.abs(blocks).max(axis=2), 1e-4)
    assert np.all(amax / sf <= 448.0)                         # never past e4m3's max
    assert np.all(sf >= amax / 448.0)
    assert np.all(sf < 2 * amax / 448.0 * (1 + 1e-7))         # the smallest such power
    # x * 2^-k * 2^k == x (exact power-of-two scaling) in float32
    inv = np.ldexp(np.float32(1), 127 - E.astype(np.int32)).astype(np.float32)
    y = (blocks.astype(np.float32) * inv[:, :, None]).astype(np.float32)
    back = (y * sf[:, :, None].astype(np.float32)).astype(np.float32)
    assert np.array_equal(back, blocks.astype(np.float32))
    # dequantized codes * sf are exact in float32 (<= 4 significant bits)
    dq = O.mx_dequantize(codes, E)
    assert np.array_equal(dq.astype(np.float32).astype(np.float64), dq)
    # round trip: relative 2^-4 for normal scaled values, half a subnormal step below
    err = np.abs(dq - A.astype(np.float64)).reshape(64, 32, 32)
    yabs = np.abs(y.astype(np.float64))
    bound = np.where(yabs >= 2.0 ** -6, yabs * 2.0 ** -4, 2.0 ** -10) * sf[:, :, None]
    assert np.all(err <= bound * (1 + 1e-9))


def test_mx_quantize_matches_recipe_with_torch_cast():
    torch = pytest.importorskip("torch")
    A, _ = make_inputs("c5_mxfp8", M=32, K=512, N=8, seed=11)
    codes, E = O.quantize_mx(A)
    amax = np.maximum(np.abs(A.reshape(32, 16, 32)).max(axis=2), np.float32(1e-4)).astype(np.float32)
    t = (amax / np.float32(448.0)).astype(np.float32)
    Eref = np.array([_ceil_pow2_exponent(float(v)) for v in t.reshape(-1)]).reshape(32, 16)
    assert np.array_equal(E.astype(int), Eref)
    inv = torch.from_numpy(np.exp2(127.0 - Eref).astype(np.float32))
    y = torch.from_numpy(A.reshape(32, 16, 32)) * inv[:, :, None]
    ref_codes = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy().reshape(32, 512)
    assert np.array_equal(O.e4m3_decode(codes), O.e4m3_decode(ref_codes))


def test_mx_block_scale_on_every_block():
    # [TL27] 4.3 and 7 pitfall 3: each K block multiplies by its own scale.
    # Two blocks with different scales; the reference must weight each block separately.
    qa = np.full((1, 64), 0x38, np.uint8)      # 1.0
    qw = np.full((1, 64), 0x38, np.uint8)
    Ea = np.array([[127, 130]], np.uint8)      # 1, 8
    Ew = np.array([[126, 127]], np.uint8)      # 0.5, 1
    ref, S = O.mx_gemm_ref(qa, Ea, qw, Ew)
    assert ref[0, 0] == 32 * 1 * 0.5 + 32 * 8 * 1
    hoisted = 64 * 8 * 1                       # last scale applied to the whole K: wrong
    assert ref[0, 0] != hoisted


def test_mx_reference_against_exact_rationals():
    A, W = make_inputs("c5_mxfp8", M=6, K=256, N=5, seed=12)
    qa, Ea = O.quantize_mx(A)
    qw, Ew = O.quantize_mx(W)
    ref, S = O.mx_gemm_ref(qa, Ea, qw, Ew)

    def frac_val(code):
        s = -1 if code & 0x80 else 1
        e, m = (code >> 3) & 0xF, code & 7
        if e == 0:
            return s * Fraction(m, 512)
        return s * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)

    for m in range(6):
        for n in range(5):
            exact = Fraction(0)
            for b in range(256 // 32):
                blk = sum(frac_val(int(qa[m, k])) * frac_val(int(qw[n, k])) for k in range(32 * b, 32 * b + 32))
                exact += Fraction(2) ** (int(Ea[m, b]) + int(Ew[n, b]) - 254) * blk
            assert abs(float(exact) - ref[m, n]) <= 256 * 2.0 ** -53 * S[m, n]
    r2, s2 = O.mx_gemm_ref_entries(qa, Ea, qw, Ew, [1, 5, 0], [4, 0, 2])
    assert np.allclose(r2, [ref[1, 4], ref[5, 0], ref[0, 2]], rtol=1e-15, atol=0)


# --------------------------------------------------------------------------
# Metrics ([TL27] 5.2) sanity on known cases
# --------------------------------------------------------------------------
def test_metrics_known_values():
    ref = np.array([3.0, 4.0])
    assert MT.rel_l2(ref, ref) == 0.0
    assert abs(MT.rel_l2(np.zeros(2), ref) - 1.0) < 1e-15
    assert MT.max_abs([1, 2], [1, 5]) == 3
    assert MT.mismatch_ratio([1, 2], [1, 5], rtol=0, atol=1) == 0.5
    assert abs(MT.sqnr_db(ref, ref * 1.1) - 20.0) < 1e-9
    # gate: 4*K*amax*bcolmax/127
    assert MT.column_gate_atol(2.0, [3.0], 10)[0] == 4 * 10 * 2 * 3 / 127


# --------------------------------------------------------------------------
# x/s is a correctly rounded float32 division (not x * (1/s)), then rint
# ([AQ] numpy reference, [SK] step 1, [TL27] 2.4 all divide by the scale)
# --------------------------------------------------------------------------
def _rint_exact_quotient(x: float, s: float) -> int:
    # float64 holds the exactly rounded quotient well enough that rounding it
    # once more to float32 is the correctly rounded float32 quotient (53 >= 2*24+2)
    qf = np.float32(float(Fraction(float(x)) / Fraction(float(s))))
    return int(np.rint(qf))


def test_quotient_is_correctly_rounded_division():
    rng = rng_for(21)
    x = rng.standard_normal((40, 257), dtype=np.float32)
    x[:, 0] = rng.uniform(0.5, 9.0, 40).astype(np.float32)        # varied row maxima
    q, s = O.quantize_sym_int8(x)
    for m in range(40):
        for k in range(257):
            assert int(q[m, k]) == max(-127, min(127, _rint_exact_quotient(x[m, k], s[m])))
    # near-tie quotients: x = (n + 1/2) * s nudged by one float32 ulp either way
    s0 = np.float32(3.0) / np.float32(127.0)
    n = np.arange(-120, 120, dtype=np.float64)
    base = ((n + 0.5) * np.float64(s0)).astype(np.float32)
    xs = np.concatenate([np.nextafter(base, np.float32(-1e9)), base, np.nextafter(base, np.float32(1e9))])
    row = np.concatenate([[np.float32(3.0)], xs]).astype(np.float32)[None, :]
    q, s = O.quantize_sym_int8(row)
    assert float(s[0]) == float(s0)
    for k in range(1, row.shape[1]):
        assert int(q[0, k]) == max(-127, min(127, _rint_exact_quotient(row[0, k], s0)))


def test_oracle_and_product_share_no_imports():
    import re
    import glob
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for f in glob.glob(os.path.join(root, "oracle", "*.py")):
        src = open(f).read()
        assert not re.search(r"^\s*(from|import)\s+block_scaled_quantized_qgemm_amd", src, re.M), f
    for f in glob.glob(os.path.join(root, "block_scaled_quantized_qgemm_amd", "**", "*.*"), recursive=True):
        if f.endswith((".py", ".hip", ".cpp", ".h", ".hpp")):
            src = open(f).read()
            assert not re.search(r"^\s*(from|import)\s+oracle|#include\s+\S*oracle", src, re.M), f


# --------------------------------------------------------------------------
# Bias after the scales ([AQ] int8_linear: y + bias; [SK] step 5)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("act", ["sym_row", "asym_row"])
def test_bias_is_added_after_dequantize_then_multiply(act):
    """With a bias, the output is the float64 product of the dequantized
    operands plus the bias per output channel: a route through dequantized
    values instead of the integer GEMM."""
    A, W = make_inputs("c2_per_token", M=9, K=70, N=13, seed=41)
    if act == "asym_row":
        A = A - np.float32(0.3)
    b = rng_for(42).normal(0.0, 3.0, size=13).astype(np.float32)
    r = O.quantized_linear(A, W, act=act, wgt="channel", bias=b)
    xa = (r["q_a"].astype(np.float64) - r["z_a"].astype(np.float64)[:, None]) * r["s_a"].astype(np.float64)[:, None]
    xw = r["q_w"].astype(np.float64) * r["s_w"].astype(np.float64)[:, None]
    ref = xa @ xw.T + b.astype(np.float64)[None, :]
    assert np.allclose(r["y"], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    r0 = O.quantized_linear(A, W, act=act, wgt="channel")
    assert np.array_equal(r0["C"], r["C"])          # the bias never enters the integer sum
    d = r["y"] - r0["y"]
    assert np.allclose(d, np.broadcast_to(b.astype(np.float64), d.shape), rtol=0, atol=1e-12 * np.abs(r["y"]).max())


# --------------------------------------------------------------------------
# RMSNorm in front of the per-token quantizer ([AQ] "Fusion: making
# quantization nearly free")
# --------------------------------------------------------------------------
def test_rmsnorm_hand_example():
    """x = [3, 4]: mean(x^2) = 12.5, so y = x / sqrt(12.5 + eps) * gamma."""
    x = np.array([[3.0, 4.0]], np.float32)
    g = np.array([1.0, 2.0], np.float32)
    for eps in (0.0, 1.0):
        y = O.rmsnorm(x, g, eps).astype(np.float64)
        rms = math.sqrt(12.5 + eps)
        want = np.array([3.0 / rms, 2.0 * 4.0 / rms])
        assert np.allclose(y[0], want, rtol=2.0 ** -22, atol=0)


def test_rmsnorm_constant_rows():
    """A constant row c normalizes to sign(c) * gamma (eps = 0); for c a power
    of two every step is exact."""
    g = np.array([1.0, -0.5, 3.0, 0.0], np.float32)
    for c in (1.0, -8.0, 2.0 ** -20, 2.0 ** 30):
        y = O.rmsnorm(np.full((1, 4), c, np.float32), g, 0.0)
        assert np.array_equal(y[0], np.sign(c) * g)
    y = O.rmsnorm(np.full((1, 4), 3.0, np.float32), np.ones(4, np.float32), 0.0)
    assert np.all(y == 1.0)                          # rms = 3 exactly, 3 / 3 = 1


def test_rmsnorm_power_of_two_scale_invariance():
    """RMSNorm(2^j x) == RMSNorm(x) bit for bit with eps = 0: scaling by a
    power of two commutes with every rounding step (in range)."""
    x = make_inputs("c2_per_token", M=6, K=300, N=1, seed=7)[0]
    g = rng_for(8).normal(1.0, 0.3, size=300).astype(np.float32)
    base = O.rmsnorm(x, g, 0.0)
    for j in (-20, -3, 5, 40):
        assert np.array_equal(O.rmsnorm(x * np.float32(2.0 ** j), g, 0.0), base)


def test_rmsnorm_output_has_unit_rms():
    x = make_inputs("c2_per_token", M=8, K=4096, N=1, seed=9)[0]
    y = O.rmsnorm(x, np.ones(4096, np.float32), 0.0).astype(np.float64)
    assert np.allclose(np.sqrt((y * y).mean(axis=1)), 1.0, rtol=0, atol=1e-6)
    # eps > 0 only shrinks the output
    y_eps = O.rmsnorm(x, np.ones(4096, np.float32), 10.0).astype(np.float64)
    assert np.all(np.abs(y_eps) <= np.abs(y))


def test_rmsnorm_quantize_edge_rows():
    """An all-zero row normalizes to zeros (rms = sqrt(eps)) and takes the
    1e-8 scale floor and code 0; a one-hot row puts its spike on code 127."""
    x = np.zeros((2, 64), np.float32)
    x[1, 17] = -5.0
    q, s = O.rmsnorm_quantize(x, np.ones(64, np.float32), 1e-6)
    assert not q[0].any() and s[0] == np.float32(1e-8)
    assert q[1, 17] == -127 and np.count_nonzero(q[1]) == 1
    q, s, z = O.rmsnorm_quantize(x, np.ones(64, np.float32), 1e-6, act="asym_row")
    assert not q[0].any() and z[0] == 0
    assert q[1, 17] == 0 and np.all(q[1, np.arange(64) != 17] == z[1]) and z[1] == 255


# --------------------------------------------------------------------------
# int4 weights per group of 64 and the W4A8 GEMM ([TL27] 2.4, 4.3, 5.1)
# --------------------------------------------------------------------------
def test_int4_group_error_bound_is_the_pages_u():
    """[TL27] 2.4: the int4 error is at most s / 2 = absmax / 14, printed as
    u = 7.143e-2 of the absmax; codes stay in [-7, 7] with scales from the
    same data (the -8 bound of the clip never bites)."""
    W = make_inputs("c4_decode", M=1, K=1000, N=37, seed=5)[1]
    q, s = O.quantize_int4_groups(W)
    assert q.min() >= -7 and q.max() <= 7 and q.dtype == np.int8
    Wp = np.zeros((37, 1024), np.float32)
    Wp[:, :1000] = W
    qp = np.zeros((37, 1024), np.int8)
    qp[:, :1000] = q
    err = np.abs(Wp.reshape(37, 16, 64) - qp.reshape(37, 16, 64) * s[:, :, None].astype(np.float64))
    amax = np.abs(Wp.reshape(37, 16, 64)).max(axis=2)
    ratio = err.max(axis=2) / amax
    assert ratio.max() <= 1.0 / 14 * (1 + 1e-6)
    assert abs(1.0 / 14 - 7.143e-2) < 5e-6 and ratio.max() > 0.06     # the bound is nearly reached


def test_int4_granularity_beats_per_channel():
    """[TL27] 2.4: precision is set by how many elements share a scale; with
    outliers along K, per-group-64 int4 beats one int4 scale per row."""
    W = make_inputs("c4_decode", M=1, K=4096, N=16, seed=6)[1].copy()
    W[:, ::700] *= 50.0
    q, s = O.quantize_int4_groups(W)
    deq_g = (q.reshape(16, 64, 64) * s[:, :, None]).reshape(16, 4096)
    q1, s1 = O.quantize_int4_groups(W, group=4096)
    deq_c = q1 * s1[:, :1]
    e_g = np.linalg.norm(deq_g - W) / np.linalg.norm(W)
    e_c = np.linalg.norm(deq_c - W) / np.linalg.norm(W)
    assert e_g < 0.5 * e_c


def test_w4a8_gemm_equals_dequantize_then_multiply_and_catches_scale_mistakes():
    """The per-group reference equals the float64 product of the dequantized
    operands; [TL27] 5.1's two planted mistakes -- only the last group's
    scale, or no weight scale at all -- are far from it."""
    A, W = make_inputs("c4_decode", M=5, K=700, N=23, seed=11)
    qa, sa = O.quantize_sym_int8(A, per_row=True)
    qw, sw = O.quantize_int4_groups(W)
    out, S = O.w4a8_gemm(qa, sa, qw, sw)
    swk = np.repeat(sw.astype(np.float64), 64, axis=1)[:, :700]
    xhat = qa.astype(np.float64) * sa.astype(np.float64)[:, None]
    what = qw.astype(np.float64) * swk
    ref = xhat @ what.T
    assert np.all(np.abs(out - ref) <= 1e-13 * S)
    last = xhat @ (qw.astype(np.float64) * sw[:, -1:].astype(np.float64)).T
    none = xhat @ qw.astype(np.float64).T
    for bad in (last, none):
        assert np.linalg.norm(bad - ref) / np.linalg.norm(ref) > 0.05


def test_w4a8_gemm_integer_partials_brute_force():
    """Tiny shapes against pure-Python integers and exact rationals."""
    rng = rng_for(12)
    for M, N, K in [(1, 1, 1), (2, 3, 65), (3, 2, 130)]:
        qa = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
        qw = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
        sa = rng.uniform(0.01, 1, size=M).astype(np.float32)
        ng = -(-K // 64)
        sw = rng.uniform(0.01, 1, size=(N, ng)).astype(np.float32)
        out, S = O.w4a8_gemm(qa, sa, qw, sw)
        for m in range(M):
            for n in range(N):
                tot = Fraction(0)
                for g in range(ng):
                    P = sum(int(qa[m, k]) * int(qw[n, k]) for k in range(g * 64, min(K, g * 64 + 64)))
                    tot += Fraction(float(sw[n, g])) * P
                exact = Fraction(float(sa[m])) * tot
                # float64 scaling and group sum: a few ulps of S (sum of |terms|)
                assert abs(Fraction(out[m, n]) - exact) <= Fraction(S[m, n]) * Fraction(4 * ng, 2 ** 53) + Fraction(1, 2 ** 100)


def test_w4a8_reference_table_rows_b_and_d():
    """[TL27] 5.1's table: with int4 per-group-64 weights, a product that takes
    only the last group's scale sits ~0.21 from the quantization-aware
    reference, and the unquantized product ~0.108 (the int4 error)."""
    g = _golden("tl27_w4a8_reference_table.json")
    rng = rng_for(13)
    A = rng.standard_normal((96, 2048)).astype(np.float32)
    W = rng.standard_normal((192, 2048)).astype(np.float32)
    qa, sa = O.quantize_sym_int8(A, per_row=True)
    qw, sw = O.quantize_int4_groups(W, group=g["group"])
    out, _ = O.w4a8_gemm(qa, sa, qw, sw, group=g["group"])
    xhat = qa.astype(np.float64) * sa.astype(np.float64)[:, None]
    row_b = xhat @ (qw.astype(np.float64) * sw[:, -1:].astype(np.float64)).T
    row_d = A.astype(np.float64) @ W.astype(np.float64).T
    rel = lambda x: np.linalg.norm(x - out) / np.linalg.norm(out)
    for got, want in ((rel(row_b), g["row_B_only_last_group_scale_rel_l2"]),
                      (rel(row_d), g["row_D_unquantized_weights_rel_l2"])):
        assert abs(got - want) <= g["tolerance_rel"] * want, (got, want)


def test_int4_pair_packing_bytes_and_sign_restoration():
    """[TL27] 3.3(b)/(c) and pitfall 9: low nibble first, two's complement,
    arithmetic shift on the way back. Every one of the 256 code pairs
    round-trips; -1 packs to 0xF (not 15 on the way back)."""
    codes = np.array([(a, b) for a in range(-8, 8) for b in range(-8, 8)], np.int8).reshape(1, -1)
    packed = O.pack_int4_pairs(codes)
    assert packed.shape == (1, 256)
    for i in range(256):
        a, b = int(codes[0, 2 * i]), int(codes[0, 2 * i + 1])
        assert int(packed[0, i]) == (a % 16) + 16 * (b % 16)
    assert sorted(set(packed[0].tolist())) == list(range(256))
    assert np.array_equal(O.unpack_int4_pairs(packed, 512), codes)
    assert O.pack_int4_pairs(np.array([[-1, 0]], np.int8))[0, 0] == 0x0F
    assert O.unpack_int4_pairs(np.array([[0x0F]], np.uint8), 2).tolist() == [[-1, 0]]
    # odd K pads one zero code
    assert O.pack_int4_pairs(np.array([[3, -2, -8]], np.int8)).tolist() == [[0xE3, 0x08]]
    assert O.unpack_int4_pairs(np.array([[0xE3, 0x08]], np.uint8), 3).tolist() == [[3, -2, -8]]


# --------------------------------------------------------------------------
# fp4 e2m1 and MXFP4 ([TL27] 1.2, 2.3, 8; the e2m1 recipe is a reading)
# --------------------------------------------------------------------------
def test_e2m1_values_from_the_format_fields():
    """Derived independently from the bit fields: exponent bias 1, one
    mantissa bit, field 0 subnormal; largest value 1.5 * 2^2; code 8 is -0."""
    v = O.E2M1_VALUES
    pos = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert v[:8].tolist() == pos and (v[8:] == -np.array(pos)).all()
    assert v[7] == O.E2M1_MAX == 1.5 * 2 ** 2
    assert math.copysign(1, v[8]) == -1
    assert not np.isnan(v).any()


def test_e2m1_rounding_ties_even_and_u():
    """Every midpoint between neighbours goes to the even code; elsewhere the
    nearest value; on the normal range the relative error is within
    u = 2^-2 ([TL27] 1.2 and 8: fp4 e2m1 2.5e-1)."""
    g = _golden("format_constants.json")
    mids = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for a, code in mids.items():
        assert int(O.e2m1_encode_rne(np.float32(a))) == code, a
        assert int(O.e2m1_encode_rne(np.float32(-a))) == code | 8, -a
    assert int(O.e2m1_encode_rne(np.float32(-0.0))) == 8
    rng = rng_for(21)
    y = rng.uniform(-6, 6, 200000).astype(np.float32)
    c = O.e2m1_encode_rne(y)
    d = np.abs(O.e2m1_decode(c) - y.astype(np.float64))
    # nearest: no grid value is closer
    best = np.min(np.abs(O.E2M1_VALUES[None, :] - y.astype(np.float64)[:, None]), axis=1)
    assert np.array_equal(d, best)
    normal = np.abs(y) >= 1.0
    assert (d[normal] / np.abs(y[normal]) <= g["e2m1_u"]).all()
    with pytest.raises(ValueError):
        O.e2m1_encode_rne(np.float32(6.01))


def test_mxfp4_scaling_and_error():
    """sf is the smallest power of two with amax / sf <= 6; scaled values
    stay within e2m1; every block has its own scale; the error per element is
    within u of the value on the normal range and within 0.25 sf below it."""
    A, _ = make_inputs("c5_mxfp8", M=16, K=512, N=1, seed=23)
    q, E = O.quantize_mxfp4(A)
    sf = O.e8m0_value(E)
    amax = np.maximum(np.abs(A.reshape(16, 16, 32)).max(axis=2), 1e-4).astype(np.float64)
    assert (amax / sf <= 6.0).all() and (amax / (sf / 2) > 6.0).all()
    deq = O.mx_dequantize(q, E, "e2m1").reshape(16, 16, 32)
    x = A.astype(np.float64).reshape(16, 16, 32)
    err = np.abs(deq - x)
    scaled = np.abs(x) / sf[:, :, None]
    assert (err[scaled >= 1] <= 0.25 * np.abs(x[scaled >= 1]) + 1e-300).all()
    assert (err[scaled < 1] <= 0.25 * np.broadcast_to(sf[:, :, None], x.shape)[scaled < 1]).all()
    # one block with an outlier spends its own range only
    B = np.ones((1, 64), np.float32)
    B[0, 5] = 600.0
    qb, Eb = O.quantize_mxfp4(B)
    assert Eb[0, 0] > Eb[0, 1] and (O.mx_dequantize(qb, Eb, "e2m1")[0, 32:] == 1.0).all()


def test_mxfp4_gemm_reference_against_exact_rationals():
    """The float64 reference over dequantized e2m1 values against exact
    rational arithmetic, and fp4 packing round trip of the codes."""
    A, W = make_inputs("c5_mxfp8", M=3, K=96, N=4, seed=24)
    qa, Ea = O.quantize_mxfp4(A)
    qw, Ew = O.quantize_mxfp4(W)
    out, S = O.mx_gemm_ref(qa, Ea, qw, Ew, "e2m1", "e2m1")
    for m in range(3):
        for n in range(4):
            tot = Fraction(0)
            for k in range(96):
                b = k // 32
                av = Fraction(O.E2M1_VALUES[qa[m, k]]) * Fraction(2) ** (int(Ea[m, b]) - 127)
                wv = Fraction(O.E2M1_VALUES[qw[n, k]]) * Fraction(2) ** (int(Ew[n, b]) - 127)
                tot += av * wv
            assert abs(Fraction(out[m, n]) - tot) <= Fraction(S[m, n]) * Fraction(1, 2 ** 50)
    packed = O.pack_int4_pairs(qa.astype(np.int8))
    assert np.array_equal(O.unpack_int4_pairs(packed, 96).astype(np.uint8) & 0xF, qa)


# --------------------------------------------------------------------------
# Grouped (MoE) MX GEMM ([TL27] 6.2, MoE point 3)
# --------------------------------------------------------------------------
def _grouped_inputs(sizes, N=6, K=96, seed=31):
    M = int(sum(sizes))
    E = len(sizes)
    A, Wall = make_inputs("c5_mxfp8", M=M, K=K, N=E * N, seed=seed)
    qa, Ea = O.quantize_mx(A)
    qw, Ew = O.quantize_mx(Wall)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    return qa, Ea, qw.reshape(E, N, K), Ew.reshape(E, N, K // 32), offsets


def test_mx_grouped_reference_equals_row_wise_expert_selection():
    # An independent formulation: every row against every expert (no
    # slicing), then each row keeps the product with its own expert, found
    # by searching the offsets.
    sizes = [3, 0, 5, 1, 4]
    qa, Ea, qw, Ew, off = _grouped_inputs(sizes)
    ref, S = O.mx_grouped_gemm_ref(qa, Ea, off, qw, Ew)
    A = O.mx_dequantize(qa, Ea)
    E, N, K = qw.shape
    Wd = O.mx_dequantize(qw.reshape(E * N, K), Ew.reshape(E * N, K // 32)).reshape(E, N, K)
    every = np.einsum("mk,enk->emn", A, Wd)
    expert = np.searchsorted(off, np.arange(qa.shape[0]), side="right") - 1
    direct = every[expert, np.arange(qa.shape[0])]
    assert np.allclose(ref, direct, rtol=1e-13, atol=0)
    assert np.allclose(S, np.einsum("mk,enk->emn", np.abs(A), np.abs(Wd))[expert, np.arange(qa.shape[0])],
                       rtol=1e-13, atol=0)


def test_mx_grouped_reference_catches_routing_and_scale_index_mistakes():
    sizes = [4, 3, 5]
    qa, Ea, qw, Ew, off = _grouped_inputs(sizes, seed=32)
    ref, S = O.mx_grouped_gemm_ref(qa, Ea, off, qw, Ew)
    # a row routed to the neighbouring expert (an off-by-one offset)
    shifted = off.copy()
    shifted[1] += 1
    bad, _ = O.mx_grouped_gemm_ref(qa, Ea, shifted, qw, Ew)
    assert not np.allclose(bad[4], ref[4], rtol=1e-3)
    assert np.array_equal(bad[:4], ref[:4]) and np.array_equal(bad[5:], ref[5:])
    # expert 1's weights scaled with expert 0's scales (a wrong expert index)
    Ew_bad = Ew.copy()
    Ew_bad[1] = Ew[0]
    bad2, _ = O.mx_grouped_gemm_ref(qa, Ea, off, qw, Ew_bad)
    assert np.array_equal(bad2[:4], ref[:4]) and not np.allclose(bad2[4:7], ref[4:7], rtol=1e-3)


def test_mx_grouped_reference_single_and_empty_groups():
    qa, Ea, qw, Ew, off = _grouped_inputs([7], seed=33)
    ref, S = O.mx_grouped_gemm_ref(qa, Ea, off, qw, Ew)
    dense, Sd = O.mx_gemm_ref(qa, Ea, qw[0], Ew[0])
    assert np.array_equal(ref, dense) and np.array_equal(S, Sd)
    qa, Ea, qw, Ew, off = _grouped_inputs([0, 0, 2, 0], seed=34)
    ref, _ = O.mx_grouped_gemm_ref(qa, Ea, off, qw, Ew)
    assert np.array_equal(ref, O.mx_gemm_ref(qa, Ea, qw[2], Ew[2])[0])
