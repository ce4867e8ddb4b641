"""CPU oracle for the quantized linear layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package. The product path
(the HIP library and its Python binding) never imports it, and this package
imports nothing from the product path: the two share no code. Inputs come
from the seeded generator module, which holds no quantization arithmetic.

Each function is the plain definition of one step, written with numpy and
citing the page passage it follows. Precision:

* quantizers decide integer codes in float32, because the pages compute them
  in float32 (the numpy reference in "Activation Quantization Architecture,
  in depth", section "The integer GEMM, written out", works on float32 arrays;
  the MXFP8 recipe of "TileLang tutorial, chapter 27", section 2.2, works on
  float32 amax values). The GPU takes the same decisions in the same
  precision, so codes, scales and zero points compare bit for bit;
* integer dot products are exact (see ``int_gemm``);
* the dequantization epilogue and the MX reference are float64.

Pages cited (titles as they appear on the pages):

* [D98] "100 Days of GPU -- Day 98: Quantization and sparsity"
* [TL27] "TileLang tutorial, chapter 27: low-precision quantization"
  (Chinese; sections numbered 1-8)
* [SK] "Skill: Write an INT8 Quantized Kernel"
* [AQ] "Activation Quantization Architecture, in depth"

Readings where the pages are silent or disagree are listed in the header of
each function that takes one. Every function has at least one pin in
``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32

INT8_QMAX = 127          # [SK] step 1, [AQ] "The quantizer itself": symmetric range +-127
UINT8_QMAX = 255         # [SK] step 1: asymmetric range [0, 255]
SCALE_FLOOR = F32(1e-8)  # [AQ] "The integer GEMM, written out": floor for all-zero rows
MX_BLOCK = 32            # [TL27] 2.3(a): one shared scale per 32 elements
E4M3_MAX = 448.0         # [TL27] 2.2 item 1: largest finite e4m3 value, 1.75 * 2^8
MX_AMAX_FLOOR = F32(1e-4)  # [TL27] 2.2 item 3: amax.clamp_min(1e-4)
E2M1_MAX = 6.0           # reading: the largest fp4 e2m1 value, 1.5 * 2^2 (1 sign, 2 exponent bits with bias 1, 1 mantissa bit)

INT4_QMAX = 7            # [TL27] 2.4: int4 takes qmax = 7, codes clipped to [-qmax - 1, qmax]
W4_GROUP = 64            # [TL27] 5.1: the W4A8 check uses int8 X and int4 W per group of 64

# Exact-int32 limits on K (see ``k_limit``).
INT32_MAX = 2**31 - 1


# ----------------------------------------------------------------------------
# Symmetric int8 quantizer
# ----------------------------------------------------------------------------
def quantize_sym_int8(x, per_row: bool = True):
    """Symmetric int8 quantization, per row (token / channel) or per tensor.

    [D98] "What a scale actually promises": x = q*s with s = max|x|/127, code 0
    meaning 0. [AQ] "The integer GEMM, written out" (``quantize_per_token``):
    s = max|x|/127 in float32, floored at 1e-8 for all-zero rows,
    q = clip(rint(x/s), -127, 127). [D98] "Pitfalls": always clamp after
    rounding. [TL27] 2.4 gives the same formula with a lower bound of -128;
    the +-127 range of [SK] step 1 and [AQ] is used (with s from the same
    data, rint(x/s) never leaves [-127, 127] anyway).

    Rounding: np.rint, half to even, on the float32 quotient x/s (a correctly
    rounded IEEE division). Returns (q int8 [R, K], s float32 [R] or [1]).
    """
    x = np.asarray(x, dtype=F32)
    assert x.ndim == 2
    if x.shape[0] == 0:
        return np.zeros(x.shape, np.int8), np.zeros((0 if per_row else 1,), F32)
    if per_row:
        amax = np.max(np.abs(x), axis=1, keepdims=True)
    else:
        amax = np.max(np.abs(x)).reshape(1, 1)
    s = amax / F32(INT8_QMAX)
    s = np.maximum(s, SCALE_FLOOR).astype(F32)
    q = np.clip(np.rint(x / s), -INT8_QMAX, INT8_QMAX).astype(np.int8)
    return q, s.reshape(-1)


# ----------------------------------------------------------------------------
# Asymmetric uint8 quantizer
# ----------------------------------------------------------------------------
def quantize_asym_uint8(x, per_row: bool = True):
    """Asymmetric uint8 quantization with a zero point, per row or per tensor.

    [SK] step 1: s = (max(x) - min(x))/255, z = round(-min(x)/s),
    q = clamp(round(x/s) + z, 0, 255). [AQ] "The quantizer itself":
    q = clamp(round(x/s) + z, qmin, qmax), x_hat = s*(q - z).
    [D98] "What a scale actually promises": x = (q - z)*s.

    Readings: (1) s is floored at 1e-8 like the symmetric scale (a constant
    row would otherwise divide by zero, [AQ] "Failure modes"); (2) z is
    clamped to [0, 255] so it is itself a code -- the pages do not clamp it,
    and it only matters for rows that do not contain 0 in [min, max];
    (3) round first, then add the integer z (both pages' order).
    Arithmetic in float32; rint half to even.
    Returns (q uint8, s float32 [R] or [1], z int32 [R] or [1]).
    """
    x = np.asarray(x, dtype=F32)
    assert x.ndim == 2
    if x.shape[0] == 0:
        n = 0 if per_row else 1
        return np.zeros(x.shape, np.uint8), np.zeros((n,), F32), np.zeros((n,), np.int32)
    if per_row:
        mn = np.min(x, axis=1, keepdims=True)
        mx = np.max(x, axis=1, keepdims=True)
    else:
        mn = np.min(x).reshape(1, 1)
        mx = np.max(x).reshape(1, 1)
    s = (mx - mn) / F32(UINT8_QMAX)
    s = np.maximum(s, SCALE_FLOOR).astype(F32)
    z = np.clip(np.rint(-mn / s), 0, UINT8_QMAX).astype(np.int32)
    q = np.clip(np.rint(x / s).astype(np.float64) + z, 0, UINT8_QMAX).astype(np.uint8)
    return q, s.reshape(-1), z.reshape(-1)


# ----------------------------------------------------------------------------
# Weight preparation
# ----------------------------------------------------------------------------
def prepare_weights_int8(w, per_channel: bool = True):
    """Symmetric int8 weights with per-channel scales and column sums.

    W is [N, K] (one row per output channel). [AQ] "The integer GEMM, written
    out" (``quantize_per_channel``): one scale per output channel, the same
    symmetric rule as the activations (the 1e-8 floor is applied here too).
    [D98] "The program, and the gate that has to be per column": the column
    sum sum_k q_w[k][col] depends only on the weights and is computed once,
    when they are quantized. Returns (q_w int8 [N, K], s_w float32 [N] or [1],
    colsum int64 [N]).
    """
    q, s = quantize_sym_int8(w, per_row=per_channel)
    colsum = q.astype(np.int64).sum(axis=1)
    return q, s, colsum


def quantize_int4_groups(w, group: int = W4_GROUP):
    """Symmetric int4 weights with one scale per ``group`` consecutive K of a row.

    [TL27] 2.4: s = absmax / qmax with qmax = 7, q = clip(round(x / s),
    -qmax - 1, qmax), x_hat = q * s; its error is at most s / 2, i.e.
    1 / (2 * 7) = 7.143e-2 of the absmax. [TL27] 2.4 and 5.1: int4 needs a
    fine granularity, per group of 64 along K in the W4A8 measurement.
    Readings: float32 arithmetic and rint (half to even) as for int8; s
    floored at 1e-8 for all-zero groups; a last, partial group takes the
    amax of its own elements. Returns (q int8 [N, K] with values in [-8, 7],
    s float32 [N, ceil(K / group)]).
    """
    w = np.asarray(w, dtype=F32)
    N, K = w.shape
    ng = -(-K // group)
    wp = np.zeros((N, ng * group), F32)
    wp[:, :K] = w
    g = wp.reshape(N, ng, group)
    s = np.maximum(np.max(np.abs(g), axis=2) / F32(INT4_QMAX), SCALE_FLOOR).astype(F32)
    q = np.clip(np.rint(g / s[:, :, None]), -INT4_QMAX - 1, INT4_QMAX).astype(np.int8)
    return q.reshape(N, ng * group)[:, :K], s


def pack_int4_pairs(q):
    """Two int4 codes per byte along the last axis: element 2i in the low
    nibble and 2i + 1 in the high nibble, each as its low four two's-complement
    bits ([TL27] 3.3(b) and pitfall 9: (a & 0x0F) | ((b & 0x0F) << 4)). An odd
    length is padded with a zero code. Returns uint8 [..., ceil(K / 2)]."""
    q = np.asarray(q, np.int16)
    if q.shape[-1] % 2:
        q = np.concatenate([q, np.zeros(q.shape[:-1] + (1,), np.int16)], axis=-1)
    lo = q[..., 0::2] & 0x0F
    hi = q[..., 1::2] & 0x0F
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_int4_pairs(b, K: int):
    """Inverse of pack_int4_pairs: each nibble moved to the top of a signed
    byte, then shifted right arithmetically by four, which restores the sign
    ([TL27] 3.3(c) and pitfall 9: a logical shift would turn -1 into 15).
    Returns int8 [..., K]."""
    b = np.asarray(b, np.uint8)
    lo = ((b << 4).astype(np.uint8).view(np.int8) >> 4).astype(np.int8)
    hi = (b.view(np.int8) >> 4).astype(np.int8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out[..., :K]


def w4a8_gemm(q_a, s_a, q_w, s_w, group: int = W4_GROUP):
    """out[m, n] = s_a[m] * sum_g s_w[n, g] * P_g[m, n] with the exact integer
    partial sums P_g[m, n] = sum_{k in group g} q_a[m, k] * q_w[n, k].

    [TL27] 4.3: a scale that changes along K must multiply its own block's
    partial sum inside the K loop (multiplying once after the integer sum
    only works for scales that do not depend on K). [TL27] 5.1: the
    quantization-aware float64 reference. The partials are exact (int64);
    scaling and the sum over groups are float64. s_a is [M] or [1] (per
    token or per tensor, symmetric int8). Returns (out float64 [M, N],
    S float64 [M, N] = sum_g |s_a s_w P_g|, the basis of the float32 error).
    """
    qa = np.asarray(q_a, np.int64)
    qw = np.asarray(q_w, np.int64)
    M, K = qa.shape
    N = qw.shape[0]
    sa = np.broadcast_to(np.asarray(s_a, F32).astype(np.float64).reshape(-1), (M,))
    sw = np.asarray(s_w, F32).astype(np.float64)
    out = np.zeros((M, N))
    S = np.zeros((M, N))
    for gi in range(sw.shape[1]):
        k0, k1 = gi * group, min(K, (gi + 1) * group)
        P = (qa[:, k0:k1] @ qw[:, k0:k1].T).astype(np.float64)
        term = sa[:, None] * sw[None, :, gi] * P
        out += term
        S += np.abs(term)
    return out, S


def k_limit(asymmetric: bool) -> int:
    """Largest K for which every int32 accumulator value is exact.

    [D98] "What a scale actually promises": |acc| <= K*127*128 when one
    operand may reach 128 in magnitude. [AQ] "The integer GEMM, written out":
    symmetric products are at most 127*127 = 16129, so up to about 133,000
    terms fit in int32. [SK] step 2 asks for this check. For uint8 codes with a
    zero point the corrected sum sum (q_a - z) q_w has terms up to 255*127.
    """
    per_term = 255 * 127 if asymmetric else 127 * 127
    return INT32_MAX // per_term


# ----------------------------------------------------------------------------
# Integer GEMM and epilogue
# ----------------------------------------------------------------------------
def int_gemm(q_a, z_a, q_w):
    """C[m, n] = sum_k (q_a[m, k] - z_a[m]) * q_w[n, k], exactly.

    [AQ] "The integer GEMM, written out": y = s_a*s_w*(sum qa*qw - z_a*sum qw);
    [D98] "What a scale actually promises": integer products accumulated in
    int32 round nothing. z_a is a scalar, a [1] array (per tensor) or an [M]
    array (per token); pass 0 for symmetric codes.

    The sum is evaluated with a float64 matrix product. That is exact here:
    every operand is an integer of magnitude <= 255, every product and every
    partial sum is an integer below K*255*128 < 2^53, and float64 represents
    all such integers, so no addition in any order rounds.
    """
    q_a = np.asarray(q_a)
    q_w = np.asarray(q_w)
    M, K = q_a.shape
    N = q_w.shape[0]
    assert q_w.shape[1] == K
    assert K * 255 * 128 < 2**53
    z = np.broadcast_to(np.asarray(z_a, dtype=np.float64).reshape(-1, 1), (M, 1))
    a = q_a.astype(np.float64) - z
    if M == 0 or N == 0:
        return np.zeros((M, N), np.int64)
    C = a @ q_w.astype(np.float64).T
    return C.astype(np.int64)


def int_gemm_entries(q_a, z_a, q_w, rows, cols):
    """C at the (rows[i], cols[i]) pairs only, exactly (int64 dot products)."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    za = np.asarray(z_a, dtype=np.int64).reshape(-1)
    if za.size == 1:
        za = np.full(q_a.shape[0], za[0], np.int64)
    a = q_a[rows].astype(np.int64) - za[rows][:, None]
    w = q_w[cols].astype(np.int64)
    return np.einsum("ik,ik->i", a, w)


def epilogue(C, s_a, s_w):
    """y[m, n] = s_a[m] * s_w[n] * C[m, n], in float64.

    [D98] "The program, and the gate that has to be per column": the scales
    multiply the corrected integer once per output element, after the loop.
    [SK] step 4 (per-token activations, per-channel weights):
    out[m][n] = int32_result[m][n] * scale_A[m] * scale_B[n]; [SK] "Correctness
    requirements": zero-point correction before scaling (``int_gemm`` already
    returns the corrected integer). s_a and s_w may be [1] (per tensor).
    """
    C = np.asarray(C, dtype=np.float64)
    M, N = C.shape
    sa = np.broadcast_to(np.asarray(s_a, dtype=np.float64).reshape(-1, 1), (M, 1))
    sw = np.broadcast_to(np.asarray(s_w, dtype=np.float64).reshape(1, -1), (1, N))
    return C * sa * sw


def add_bias(y, bias):
    """y[m, n] + bias[n] in float64: the bias after the scales ([AQ] "The
    integer GEMM, written out", int8_linear returns y + bias; [SK] step 5,
    "optionally apply bias (in fp32)" in the epilogue)."""
    if bias is None:
        return y
    return np.asarray(y, np.float64) + np.asarray(bias, np.float32).astype(np.float64)[None, :]


def quantized_linear(x, w, act: str = "sym_row", wgt: str = "channel", bias=None):
    """The whole path on the CPU: quantize A, prepare W, integer GEMM, epilogue.

    act: "sym_row" (per-token int8), "sym_tensor" (one int8 scale),
    "asym_row" (per-token uint8 + zero point). wgt: "channel" or "tensor".
    bias: optional float32 [N] added after the scales (``add_bias``).
    Returns a dict with every intermediate (codes, scales, zero points, column
    sums, the exact integer C and the float64 output).
    """
    if act == "sym_row":
        qa, sa = quantize_sym_int8(x, per_row=True)
        za = np.zeros(qa.shape[0], np.int32)
    elif act == "sym_tensor":
        qa, sa = quantize_sym_int8(x, per_row=False)
        za = np.zeros(1, np.int32)
    elif act == "asym_row":
        qa, sa, za = quantize_asym_uint8(x, per_row=True)
    elif act == "asym_tensor":
        qa, sa, za = quantize_asym_uint8(x, per_row=False)
    else:
        raise ValueError(act)
    qw, sw, colsum = prepare_weights_int8(w, per_channel=(wgt == "channel"))
    C = int_gemm(qa, za, qw)
    y = add_bias(epilogue(C, sa, sw), bias)
    return dict(q_a=qa, s_a=sa, z_a=za, q_w=qw, s_w=sw, colsum=colsum, C=C, y=y)


# ----------------------------------------------------------------------------
# RMSNorm in front of the per-token quantizer
# ----------------------------------------------------------------------------
def rms_value(x, eps):
    """rms[m] = sqrt(mean_k x[m, k]^2 + eps) per row, as float32.

    [AQ] "Fusion: making quantization nearly free" (the fused norm-and-quantize
    pseudocode loads the row as float32 and forms rms = sqrt(mean(x * x) +
    eps)). The page fixes the formula, not the arithmetic. Reading: every
    square is exact in float64 (a float32 significand squared has 48 bits),
    the row's sum of squares is rounded once (math.fsum, the correctly
    rounded float64 sum), the mean, the sum with eps and the square root are
    float64 operations, and rms is rounded once to float32, the precision of
    the row it divides.
    """
    import math
    x = np.asarray(x, np.float32)
    K = x.shape[1]
    r = np.empty(x.shape[0], np.float32)
    for m in range(x.shape[0]):
        row = x[m].astype(np.float64)
        ss = math.fsum((row * row).tolist())
        r[m] = np.float32(math.sqrt(ss / K + float(np.float32(eps))))
    return r


def rmsnorm(x, gamma, eps, rms=None):
    """y[m, k] = x[m, k] / rms[m] * gamma[k] ([AQ] "Fusion: making
    quantization nearly free", the RMSNorm line of the pseudocode).

    Evaluated in the pseudocode's order on float32 values: the correctly
    rounded float32 quotient x / rms (an IEEE division by the float32
    ``rms_value``, not a multiplication by a reciprocal, which rounds twice),
    then its float32 product with gamma. ``rms`` may be passed in (a float32
    value per row) to evaluate the same formula with another rms.
    """
    x = np.asarray(x, np.float32)
    g = np.asarray(gamma, np.float32)
    rms = rms_value(x, eps) if rms is None else np.asarray(rms, np.float32)
    return ((x / rms[:, None]).astype(np.float32) * g[None, :]).astype(np.float32)


def rmsnorm_quantize(x, gamma, eps, act: str = "sym_row", rms=None):
    """The fused norm-and-quantize step: ``rmsnorm`` then the per-token
    quantizer on its float32 output ([AQ] "Fusion: making quantization nearly
    free": amax of the normalized row, s = amax / 127, codes and one scale per
    token). Reading: the quantizer is exactly ``quantize_sym_int8`` /
    ``quantize_asym_uint8`` per row (s floored at 1e-8 after the division, as
    everywhere else), so the fused step equals the two steps composed.
    Returns (q, s) or (q, s, z)."""
    y = rmsnorm(x, gamma, eps, rms)
    if act == "sym_row":
        return quantize_sym_int8(y, per_row=True)
    if act == "asym_row":
        return quantize_asym_uint8(y, per_row=True)
    raise ValueError(act)


# ----------------------------------------------------------------------------
# bf16 output rounding
# ----------------------------------------------------------------------------
def bf16_to_f32(bits_u16):
    """Decode bf16 bit patterns: the upper half of a float32 ([TL27] 2.1)."""
    b = np.asarray(bits_u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


# ----------------------------------------------------------------------------
# MX: E8M0 scales and e4m3 codes
# ----------------------------------------------------------------------------
def ceil_to_ue8m0(t):
    """Biased exponent E of the smallest power of two >= |t|, as E8M0.

    [TL27] 2.3(b): E8M0 is exactly a float32's biased exponent byte, values
    2^-127 .. 2^127, code 255 reserved for NaN; rounding up to a power of two
    adds one to the exponent when the mantissa is non-zero, then the code is
    clamped to [1, 254] (skipping 0 and the NaN code). Returns uint8 codes;
    the scale they stand for is 2^(E - 127).
    """
    t = np.abs(np.asarray(t, dtype=F32))
    bits = t.view(np.uint32)
    e = ((bits >> np.uint32(23)) & np.uint32(0xFF)).astype(np.int32)
    e = e + ((bits & np.uint32(0x7FFFFF)) != 0).astype(np.int32)
    return np.clip(e, 1, 254).astype(np.uint8)


def e8m0_value(E):
    """2^(E - 127) as float64 ([TL27] 2.3(b))."""
    return np.ldexp(1.0, np.asarray(E, dtype=np.int32) - 127)


def _e4m3_table():
    """Values of all 256 OCP e4m3fn codes ([TL27] 2.2).

    Sign bit, 4 exponent bits (bias 7), 3 mantissa bits. Exponent field 0 is
    subnormal: m * 2^-9. No infinities; only 0x7f and 0xff are NaN, so the
    largest finite value is 0x7e = 1.75 * 2^8 = 448. 0x80 is -0.
    """
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = s * m * 2.0**-9
        else:
            vals[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3_VALUES = _e4m3_table()
_E4M3_POS = E4M3_VALUES[:127]  # codes 0x00..0x7e, strictly increasing


def e4m3_decode(codes):
    """float64 value of each e4m3 code (NaN for 0x7f / 0xff)."""
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode_rne(y):
    """Nearest e4m3 code to each float32 y, ties to the even code.

    Round to nearest, ties to even, over the 127 non-negative finite values,
    sign carried separately (so -0.0 and negatives that round to zero give
    0x80). Subnormal codes are used below 2^-6. |y| > 448 is rejected: the
    MX scale guarantees it cannot happen ([TL27] 7, pitfall 6).
    """
    y = np.asarray(y, dtype=F32)
    a = np.abs(y).astype(np.float64)
    if np.any(~np.isfinite(a)) or np.any(a > E4M3_MAX):
        raise ValueError("e4m3 input outside [-448, 448]")
    hi = np.searchsorted(_E4M3_POS, a, side="left")     # first value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(np.signbit(y), code | np.uint8(0x80), code).astype(np.uint8)
    return code


def quantize_mx(x):
    """MXFP8 quantization: e4m3 codes plus one E8M0 scale per 32 K-elements.

    [TL27] 2.2 item 3 (the MXFP8 recipe): per block, amax = max|x| floored at
    1e-4; sf = ceil_to_ue8m0(amax / 448); codes = e4m3(x * (1/sf)).
    [TL27] 2.3(a): the block is 32 contiguous elements along K, in every row.
    1/sf is an exact power of two, so the scaling is exact and only the e4m3
    rounding (``e4m3_encode_rne``) loses information. Because sf >= amax/448,
    every scaled value is <= 448 in magnitude.

    x: float32 [R, K] with K % 32 == 0. Returns (codes uint8 [R, K],
    E uint8 [R, K/32]) -- the public layout: row-major codes and row-major
    scale bytes.
    """
    x = np.asarray(x, dtype=F32)
    R, K = x.shape
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    blocks = x.reshape(R, K // MX_BLOCK, MX_BLOCK)
    amax = np.max(np.abs(blocks), axis=2) if R else np.zeros((0, K // MX_BLOCK), F32)
    amax = np.maximum(amax, MX_AMAX_FLOOR).astype(F32)
    E = ceil_to_ue8m0(amax / F32(E4M3_MAX))
    inv = np.ldexp(F32(1.0), (127 - E.astype(np.int32))).astype(F32)
    y = (blocks * inv[:, :, None]).astype(F32)
    codes = e4m3_encode_rne(y).reshape(R, K)
    return codes, E


def _e2m1_table():
    """Values of the 16 fp4 e2m1 codes ([TL27] 1.2 and 8 name the format and
    its u = 2^-2; the field layout is the format's name): sign bit 3,
    exponent bits 2-1 with bias 1, mantissa bit 0. Exponent field 0 is
    subnormal, m * 0.5. No infinities or NaNs: the largest value is
    1.5 * 2^2 = 6. Code 8 is -0."""
    vals = np.empty(16, dtype=np.float64)
    for c in range(16):
        s = -1.0 if c & 0x8 else 1.0
        e = (c >> 1) & 0x3
        m = c & 0x1
        vals[c] = s * (m * 0.5 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1))
    return vals


E2M1_VALUES = _e2m1_table()
_E2M1_POS = E2M1_VALUES[:8]  # codes 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6


def e2m1_decode(codes):
    """float64 value of each e2m1 code (0..15)."""
    return E2M1_VALUES[np.asarray(codes, dtype=np.uint8) & np.uint8(0xF)]


def e2m1_encode_rne(y):
    """Nearest e2m1 code to each float32 y, ties to the even code (the even
    mantissa bit), sign carried separately (-0.0 and negatives that round to
    zero give code 8). |y| > 6 is rejected: the MX scale keeps every scaled
    value within the format."""
    y = np.asarray(y, dtype=F32)
    a = np.abs(y).astype(np.float64)
    if np.any(~np.isfinite(a)) or np.any(a > E2M1_MAX):
        raise ValueError("e2m1 input outside [-6, 6]")
    hi = np.minimum(np.searchsorted(_E2M1_POS, a, side="left"), 7)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E2M1_POS[lo]
    d_hi = _E2M1_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(y), code | np.uint8(0x8), code).astype(np.uint8)


def quantize_mxfp4(x):
    """MXFP4 quantization: e2m1 codes plus one E8M0 scale per 32 K-elements.

    [TL27] 2.3: the MX block of 32 with an E8M0 power-of-two scale, which
    moves only the exponent. The pages print the recipe for e4m3 (amax
    floored at 1e-4, sf = ceil_to_ue8m0(amax / 448)); reading for e2m1: the
    same recipe with the format's largest value, sf = ceil_to_ue8m0(amax / 6),
    codes = e2m1(x * (1/sf)) rounded to nearest, ties to even. Every scaled
    value is then <= 6 in magnitude.

    x: float32 [R, K] with K % 32 == 0. Returns (codes uint8 [R, K], one
    code 0..15 per element, E uint8 [R, K/32]); ``pack_int4_pairs`` gives the
    stored two-codes-per-byte form.
    """
    x = np.asarray(x, dtype=F32)
    R, K = x.shape
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    blocks = x.reshape(R, K // MX_BLOCK, MX_BLOCK)
    amax = np.max(np.abs(blocks), axis=2) if R else np.zeros((0, K // MX_BLOCK), F32)
    amax = np.maximum(amax, MX_AMAX_FLOOR).astype(F32)
    E = ceil_to_ue8m0(amax / F32(E2M1_MAX))
    inv = np.ldexp(F32(1.0), (127 - E.astype(np.int32))).astype(F32)
    y = (blocks * inv[:, :, None]).astype(F32)
    codes = e2m1_encode_rne(y).reshape(R, K)
    return codes, E


def mx_dequantize(codes, E, fmt: str = "e4m3"):
    """float64 values codes * 2^(E - 127), E broadcast over each 32-block;
    codes are e4m3 bytes or (fmt "e2m1") one e2m1 code per element."""
    codes = np.asarray(codes, dtype=np.uint8)
    R, K = codes.shape
    dec = e2m1_decode if fmt == "e2m1" else e4m3_decode
    v = dec(codes).reshape(R, K // MX_BLOCK, MX_BLOCK)
    v = v * e8m0_value(E)[:, :, None]
    return v.reshape(R, K)


def mx_gemm_ref(qa, Ea, qw, Ew, fmt_a: str = "e4m3", fmt_w: str = "e4m3"):
    """out[m, n] = sum_b 2^(Ea[m,b]-127) 2^(Ew[n,b]-127) sum_{k in b} a[m,k] w[n,k].

    [TL27] 4.1: the block-scaled product is (A * scale_A)(B * scale_B) + D;
    [TL27] 4.3: a per-K-block scale must be applied inside the K loop, to its
    own block. Evaluated as a float64 dot product of the dequantized values.
    Every dequantized value and every product is exact in float64 (at most 4
    significant bits each); the sum over K rounds only at float64 precision.
    Also returns S[m, n] = sum_k |a[m,k] w[n,k]|, the error basis of
    [TL27] 2.5. Both [M, N] float64.
    """
    A = mx_dequantize(qa, Ea, fmt_a)
    W = mx_dequantize(qw, Ew, fmt_w)
    return A @ W.T, np.abs(A) @ np.abs(W).T


def mx_gemm_ref_entries(qa, Ea, qw, Ew, rows, cols, fmt_a: str = "e4m3", fmt_w: str = "e4m3"):
    """``mx_gemm_ref`` at the (rows[i], cols[i]) pairs only."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    A = mx_dequantize(qa[rows], Ea[rows], fmt_a)
    W = mx_dequantize(qw[cols], Ew[cols], fmt_w)
    return np.einsum("ik,ik->i", A, W), np.einsum("ik,ik->i", np.abs(A), np.abs(W))


# ----------------------------------------------------------------------------
# Grouped (MoE) block-scaled GEMM
# ----------------------------------------------------------------------------
def mx_grouped_gemm_ref(qa, Ea, offsets, qw, Ew, fmt_a: str = "e4m3", fmt_w: str = "e4m3"):
    """Grouped MX GEMM: the rows offsets[e] .. offsets[e+1] - 1 of A (the
    tokens routed to expert e, concatenated in expert order) times expert e's
    weights, each product the block-scaled product of ``mx_gemm_ref``.

    [TL27] 6.2, MoE point 3: a grouped MX matmul takes A as the concatenation
    of the experts' rows, with A's scales indexed by the concatenated row,
    and one weight matrix per expert, with W's scales indexed by expert and
    output column. qa [M_total, K] codes with Ea [M_total, K/32]; qw
    [E, N, K] codes with Ew [E, N, K/32]; offsets: E + 1 non-decreasing row
    offsets from 0 to M_total. Returns out and S (``mx_gemm_ref``'s error
    basis), both [M_total, N] float64.
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    E = len(offsets) - 1
    M, N = qa.shape[0], qw.shape[1]
    assert qw.shape[0] == E and Ew.shape[0] == E
    assert offsets[0] == 0 and offsets[-1] == M and np.all(np.diff(offsets) >= 0)
    out = np.zeros((M, N))
    S = np.zeros((M, N))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            out[lo:hi], S[lo:hi] = mx_gemm_ref(qa[lo:hi], Ea[lo:hi], qw[e], Ew[e], fmt_a, fmt_w)
    return out, S
