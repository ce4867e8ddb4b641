"""Exact-arithmetic pins for the quantizers' rounding, on the CPU.

Each check recomputes a quantizer's output from the formula on the page with
exact rationals (``fractions.Fraction``) and an independent round-to-nearest-
even to float32, so it shares no arithmetic with the oracle. Every check is
also run against deliberately wrong quantizers (a reciprocal multiply instead
of the division, round-half-away instead of half-to-even, a dropped term),
planted here in oracle-shaped copies on the CPU, and must reject each one.

Pages: [AQ] "Activation Quantization Architecture, in depth";
[SK] "Skill: Write an INT8 Quantized Kernel";
[TL27] "TileLang tutorial, chapter 27: low-precision quantization".
"""
import math
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle as O
from block_scaled_quantized_qgemm_amd.inputs import rng_for

F32 = np.float32


# --------------------------------------------------------------------------
# Exact rounding helpers (independent of numpy's rounding)
# --------------------------------------------------------------------------
def rn32(q) -> np.float32:
    """The float32 nearest to the rational q, ties to the even significand
    (normal and subnormal range; no overflow in these tests)."""
    q = Fr(q)
    if q == 0:
        return F32(0.0)
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fr(2) ** e > a:
        e -= 1
    while Fr(2) ** (e + 1) <= a:
        e += 1
    ulp = Fr(2) ** (max(e, -126) - 23)
    n = a / ulp
    k = n.numerator // n.denominator
    rem = n - k
    if rem > Fr(1, 2) or (rem == Fr(1, 2) and k % 2 == 1):
        k += 1
    v = float(k * ulp)            # exact: an integer of at most 25 bits times a power of two
    return F32(-v if q < 0 else v)


def rn32_sqrt(m) -> np.float32:
    """The float32 nearest to sqrt(m) for a rational m >= 0 (ties to even)."""
    m = Fr(m)
    if m == 0:
        return F32(0.0)
    c = F32(math.sqrt(float(m)))
    cands = [c]
    for _ in range(3):
        cands.insert(0, np.nextafter(cands[0], F32(-np.inf)))
        cands.append(np.nextafter(cands[-1], F32(np.inf)))
    for i in range(1, len(cands) - 1):
        lo = (Fr(float(cands[i - 1])) + Fr(float(cands[i]))) / 2
        hi = (Fr(float(cands[i])) + Fr(float(cands[i + 1]))) / 2
        if lo * lo < m < hi * hi:
            return cands[i]
        if m == hi * hi:           # a tie: the even significand
            even = cands[i] if (cands[i].view(np.uint32) & 1) == 0 else cands[i + 1]
            return even
    raise AssertionError("sqrt candidate not bracketed")


def rint_even(f) -> int:
    """Round an exactly representable value half to even (Python's round)."""
    return int(round(float(f)))


def fr(v) -> Fr:
    return Fr(float(v))


# --------------------------------------------------------------------------
# The formulas, exactly: asymmetric uint8 ([SK] step 1, [AQ] "The quantizer
# itself"), int4 groups ([TL27] 2.4), RMSNorm ([AQ] "Fusion")
# --------------------------------------------------------------------------
def exact_asym_row(x):
    """(codes, s, z) of one row: s = RN32(RN32(max - min) / 255) floored at
    1e-8, z = clamp(rint(RN32(-min / s)), 0, 255), q = clamp(rint(RN32(x / s))
    + z, 0, 255); every quotient the correctly rounded float32 one."""
    mn, mx = min(float(v) for v in x), max(float(v) for v in x)
    s = rn32(fr(rn32(Fr(mx) - Fr(mn))) / 255)
    s = max(s, F32(1e-8))
    z = min(max(rint_even(rn32(-Fr(mn) / fr(s))), 0), 255)
    q = [min(max(rint_even(rn32(fr(v) / fr(s))) + z, 0), 255) for v in x]
    return q, s, z


def exact_int4_group(w):
    """(codes, s) of one group: s = RN32(amax / 7) floored at 1e-8,
    q = clamp(rint(RN32(w / s)), -8, 7)."""
    amax = max(abs(float(v)) for v in w)
    s = max(rn32(Fr(amax) / 7), F32(1e-8))
    return [min(max(rint_even(rn32(fr(v) / fr(s))), -8), 7) for v in w], s


def exact_rms(x, eps):
    """RN32(sqrt(sum x^2 / K + eps)) with the sum and the mean exact."""
    S = sum(fr(v) * fr(v) for v in x)
    return rn32_sqrt(S / len(x) + fr(F32(eps)))


# --------------------------------------------------------------------------
# Checks (raise AssertionError on a mismatch); each takes the implementation
# --------------------------------------------------------------------------
def _asym_rows():
    """Rows with both signs and non-dyadic scales, plus rows whose quotients
    sit within one float32 ulp of a half-integer (where a reciprocal multiply
    or a different tie rule changes the code)."""
    rng = rng_for(61)
    rows = [rng.standard_normal(97).astype(F32) * F32(1.7) + F32(0.4) for _ in range(6)]
    # near ties: min -1, max 2 -> s = RN32(3 / 255); x = RN32((n + 1/2) s) and neighbours
    s0 = rn32(fr(F32(3.0)) / 255)
    near = []
    for n in range(-80, 150, 3):
        t = rn32((n + Fr(1, 2)) * fr(s0))
        near += [np.nextafter(t, F32(-9)), t, np.nextafter(t, F32(9))]
    rows.append(np.array([-1.0, 2.0] + [float(v) for v in near if -1.0 <= v <= 2.0], F32))
    return rows


def check_asym_exact(quant):
    for row in _asym_rows():
        q, s, z = quant(row[None, :], per_row=True)
        qe, se, ze = exact_asym_row(row)
        assert s[0].view(np.uint32) == se.view(np.uint32), (s[0], se)
        assert int(z[0]) == ze, (z[0], ze)
        assert q[0].astype(int).tolist() == qe


def check_asym_ties(quant):
    """s = 1/8 exactly (max - min = 255/8): the quotients (n + 1/2) are exact
    ties and go to the even integer; so do the zero points -min/s = 2.5 and 3.5."""
    half = [(n + 0.5) / 8 for n in range(0, 200, 7)]
    row = np.array([0.0, 255 / 8] + half, F32)
    q, s, z = quant(row[None, :], per_row=True)
    assert float(s[0]) == 0.125 and int(z[0]) == 0
    want = [0, 255] + [n + (n % 2) for n in range(0, 200, 7)]   # n + 1/2 -> the even neighbour
    assert q[0].astype(int).tolist() == want
    for zt, zwant in ((2.5, 2), (3.5, 4)):
        mn = -zt / 8
        row = np.array([mn, mn + 255 / 8, 0.0, 1.5 / 8], F32)
        q, s, z = quant(row[None, :], per_row=True)
        assert float(s[0]) == 0.125
        assert int(z[0]) == zwant, (zt, z[0])
        # min and max land on the ties -zt and 255 - zt; x = 0 is stored as
        # code z; 1.5/8 is the tie 1.5 -> 2, plus z
        ends = [min(max(round(-zt) + zwant, 0), 255), min(max(round(255 - zt) + zwant, 0), 255)]
        assert q[0].astype(int).tolist() == ends + [zwant, 2 + zwant]


def _int4_groups():
    rng = rng_for(62)
    w = rng.standard_normal((5, 64 * 3)).astype(F32) * F32(0.02)
    # near ties: amax 3 -> s = RN32(3 / 7); w = RN32((n + 1/2) s) and neighbours
    s0 = rn32(fr(F32(3.0)) / 7)
    vals = [3.0]
    for n in range(-7, 7):
        t = rn32((n + Fr(1, 2)) * fr(s0))
        vals += [float(np.nextafter(t, F32(-9))), float(t), float(np.nextafter(t, F32(9)))]
    vals = [v for v in vals if abs(v) <= 3.0][:64]
    g = np.array(vals + [0.0] * (64 - len(vals)), F32)
    return np.concatenate([w, np.tile(g, 3)[None, :]], axis=0)


def check_int4_exact(quant):
    W = _int4_groups()
    q, s = quant(W)
    for n in range(W.shape[0]):
        for gi in range(W.shape[1] // 64):
            qe, se = exact_int4_group(W[n, 64 * gi:64 * gi + 64])
            assert s[n, gi].view(np.uint32) == se.view(np.uint32), (n, gi, s[n, gi], se)
            assert q[n, 64 * gi:64 * gi + 64].astype(int).tolist() == qe, (n, gi)


def check_int4_ties(quant):
    """amax = 7/8 makes s = 1/8 exactly; w = (n + 1/2)/8 are ties -> even."""
    ns = list(range(-7, 7))           # (n + 1/2)/8 stays below the amax 7/8
    g = np.array([7 / 8] + [(n + 0.5) / 8 for n in ns] + [0.0] * (64 - 1 - len(ns)), F32)
    q, s = quant(g[None, :])
    assert float(s[0, 0]) == 0.125
    want = [7] + [n + (n % 2) for n in ns] + [0] * (64 - 1 - len(ns))
    assert q[0].astype(int).tolist() == want


# the row found by a search over float32 rows: its normalized element 1
# straddles a code boundary, so x / rms and x * RN32(1 / rms) give codes 41 and 40
RMS_ROW_BITS = [0x42C80000, 0x41FF1E3E, 0xBF400000, 0x3E99999A]   # 100, 31.889767, -0.75, 0.3


def check_rmsnorm_exact(norm):
    """rms and every normalized value from exact rationals: rms =
    RN32(sqrt(sum x^2 / K + eps)), y = RN32(RN32(x / rms) * gamma)."""
    rng = rng_for(63)
    x = rng.standard_normal((4, 37)).astype(F32) * F32(3.0)
    g = rng.normal(1.0, 0.5, size=37).astype(F32)
    for eps in (0.0, 1e-5):
        y = norm(x, g, eps)
        for m in range(x.shape[0]):
            rms = exact_rms(x[m], eps)
            for k in range(x.shape[1]):
                want = rn32(fr(rn32(fr(x[m, k]) / fr(rms))) * fr(g[k]))
                assert y[m, k].view(np.uint32) == want.view(np.uint32), (m, k, y[m, k], want)


def check_rmsnorm_codes_follow_the_division(norm_quant):
    """The hand example: with gamma = 1 and eps = 0 the page's x / rms puts
    element 1 on code 41; the reciprocal form would put it on 40."""
    row = np.array(RMS_ROW_BITS, np.uint32).view(F32)
    rms = exact_rms(row, 0.0)
    y = [rn32(fr(v) / fr(rms)) for v in row]
    s = max(rn32(fr(max(abs(float(v)) for v in y)) / 127), F32(1e-8))
    code = rint_even(rn32(fr(y[1]) / fr(s)))
    recip = rn32(Fr(1) / fr(rms))
    y_r = [rn32(fr(v) * fr(recip)) for v in row]
    s_r = max(rn32(fr(max(abs(float(v)) for v in y_r)) / 127), F32(1e-8))
    assert s_r == s and code == 41 and rint_even(rn32(fr(y_r[1]) / fr(s_r))) == 40
    q, sq = norm_quant(row[None, :], np.ones(4, F32), 0.0)
    assert int(q[0, 1]) == code and sq[0] == s


# --------------------------------------------------------------------------
# The oracle passes every check
# --------------------------------------------------------------------------
def test_asym_quantizer_exact_quotients_scale_and_zero_point():
    check_asym_exact(O.quantize_asym_uint8)


def test_asym_quantizer_ties_round_half_to_even():
    check_asym_ties(O.quantize_asym_uint8)


def test_int4_quantizer_exact_quotients_and_scales():
    check_int4_exact(O.quantize_int4_groups)


def test_int4_quantizer_ties_round_half_to_even():
    check_int4_ties(O.quantize_int4_groups)


def test_rmsnorm_exact_rms_and_division_order():
    check_rmsnorm_exact(O.rmsnorm)


def test_rmsnorm_hand_example_codes_differ_from_the_reciprocal_form():
    check_rmsnorm_codes_follow_the_division(lambda x, g, eps: O.rmsnorm_quantize(x, g, eps)[:2])


# --------------------------------------------------------------------------
# Planted mistakes: oracle-shaped quantizers with one error each
# --------------------------------------------------------------------------
def _asym_variant(recip=False, half_away=False, z_sign=False, z_noround=False):
    def rnd(v):
        v = np.asarray(v, np.float64)
        return np.sign(v) * np.floor(np.abs(v) + 0.5) if half_away else np.rint(v)

    def quant(x, per_row=True):
        x = np.asarray(x, F32)
        mn = np.min(x, axis=1, keepdims=True)
        mx = np.max(x, axis=1, keepdims=True)
        s = np.maximum((mx - mn) / F32(255), F32(1e-8)).astype(F32)
        zq = (mn / s) if z_sign else (-mn / s)
        zq = np.asarray(zq, np.float64) if z_noround else rnd(zq)
        z = np.clip(np.floor(zq) if z_noround else zq, 0, 255).astype(np.int32)
        quot = (x * (F32(1) / s)).astype(F32) if recip else (x / s).astype(F32)
        q = np.clip(rnd(quot) + z, 0, 255).astype(np.uint8)
        return q, s.reshape(-1), z.reshape(-1)
    return quant


def _int4_variant(recip=False, half_away=False, qmax=7):
    def quant(w, group=64):
        w = np.asarray(w, F32)
        N, K = w.shape
        g = w.reshape(N, K // group, group)
        s = np.maximum(np.max(np.abs(g), axis=2) / F32(qmax), F32(1e-8)).astype(F32)
        quot = (g * (F32(1) / s)[:, :, None]).astype(F32) if recip else (g / s[:, :, None]).astype(F32)
        quot = quot.astype(np.float64)
        r = np.sign(quot) * np.floor(np.abs(quot) + 0.5) if half_away else np.rint(quot)
        q = np.clip(r, -8, 7).astype(np.int8)
        return q.reshape(N, K), s
    return quant


def _rmsnorm_recip(x, gamma, eps):
    x = np.asarray(x, F32)
    rms = O.rms_value(x, eps)
    r = (F32(1) / rms).astype(F32)
    return ((x * r[:, None]).astype(F32) * np.asarray(gamma, F32)[None, :]).astype(F32)


def _rmsnorm_recip_quant(x, gamma, eps):
    return O.quantize_sym_int8(_rmsnorm_recip(x, gamma, eps))


def _rmsnorm_no_eps(x, gamma, eps):
    return O.rmsnorm(x, gamma, 0.0)


def _rmsnorm_sum_not_mean(x, gamma, eps):
    x = np.asarray(x, F32)
    rms = O.rms_value(x, eps) * F32(math.sqrt(x.shape[1]))
    return ((x / rms[:, None]).astype(F32) * np.asarray(gamma, F32)[None, :]).astype(F32)


def _fails(check, impl):
    try:
        check(impl)
    except AssertionError:
        return True
    return False


@pytest.mark.parametrize("name,impl", [
    ("reciprocal multiply", _asym_variant(recip=True)),
    ("round half away", _asym_variant(half_away=True)),
    ("zero point sign", _asym_variant(z_sign=True)),
    ("zero point truncated", _asym_variant(z_noround=True)),
])
def test_asym_checks_reject_planted_mistakes(name, impl):
    assert _fails(check_asym_exact, impl) or _fails(check_asym_ties, impl), name


def test_asym_variant_without_mistakes_passes():
    check_asym_exact(_asym_variant())
    check_asym_ties(_asym_variant())


@pytest.mark.parametrize("name,impl", [
    ("reciprocal multiply", _int4_variant(recip=True)),
    ("round half away", _int4_variant(half_away=True)),
    ("qmax 8", _int4_variant(qmax=8)),
])
def test_int4_checks_reject_planted_mistakes(name, impl):
    assert _fails(check_int4_exact, impl) or _fails(check_int4_ties, impl), name


def test_int4_variant_without_mistakes_passes():
    check_int4_exact(_int4_variant())
    check_int4_ties(_int4_variant())


@pytest.mark.parametrize("name,impl", [
    ("reciprocal multiply", _rmsnorm_recip),
    ("eps dropped", _rmsnorm_no_eps),
    ("sum instead of mean", _rmsnorm_sum_not_mean),
])
def test_rmsnorm_checks_reject_planted_mistakes(name, impl):
    assert _fails(check_rmsnorm_exact, impl), name


def test_rmsnorm_hand_example_rejects_the_reciprocal_form():
    assert _fails(check_rmsnorm_codes_follow_the_division, _rmsnorm_recip_quant)
