"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Integer results (codes, zero points, column sums, int32 sums) and float32
scales must be bit-exact; float32 outputs within 1e-6 relative of the
oracle's float64 epilogue; bfloat16 outputs within half a bf16 ulp (plus
float32 slack); MX outputs within 1e-5 * sum_k |a_k w_k| of the float64
reference over the dequantized e4m3 values.
"""
import math

import numpy as np
import pytest

import oracle as O
from block_scaled_quantized_qgemm_amd.inputs import make_inputs, rng_for
from conftest import print_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

F32_RTOL = 1e-6
BF16_RTOL = 2.0 ** -8 + 2.0 ** -20
MX_STOL = 1e-5


@pytest.fixture(scope="module")
def ops():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_scaled_quantized_qgemm_amd import ops as _ops
    _ops.L.load()
    return _ops


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


ACT = {  # name -> (fmt, gran, oracle act)
    "sym_row": (0, 1, "sym_row"), "sym_tensor": (0, 0, "sym_tensor"),
    "asym_row": (1, 1, "asym_row"), "asym_tensor": (1, 0, "asym_tensor"),
}


def _edge_rows(K, rng):
    rows = [np.zeros(K), np.full(K, 3.25), np.full(K, -2.0), np.linspace(-10, -9, K),
            np.linspace(4, 5, K), rng.standard_normal(K) * 1e-30]
    spike = np.zeros(K)
    spike[K // 2] = -7.0
    rows.append(spike)
    big = rng.standard_normal(K)
    big[0] = 6.0e4
    rows.append(big)
    return np.stack(rows).astype(np.float32)


# ---------------------------------------------------------------------------
# Q1-Q3: row quantization, bit-exact
# ---------------------------------------------------------------------------
QSHAPES = [(1, 1), (3, 5), (7, 17), (64, 256), (33, 1000), (5, 4095), (4, 4097), (9, 8192), (2, 9000), (512, 4096)]


@pytest.mark.parametrize("act", list(ACT))
@pytest.mark.parametrize("M,K", QSHAPES)
def test_quantize_rows_bit_exact(ops, act, M, K):
    print_case("quantize_rows", act, M, K)
    fmt, gran, oact = ACT[act]
    A, _ = make_inputs("c3_asym_uint8" if act.startswith("asym") and M % 2 else "c2_per_token", M=M, K=K, N=1,
                       seed=M * 7919 + K)
    r = ops.qgemm_quantize_rows(dev(A), fmt, gran)
    codes = host(r.codes())
    if fmt == 0:
        q, s = O.quantize_sym_int8(A, per_row=(gran == 1))
    else:
        q, s, z = O.quantize_asym_uint8(A, per_row=(gran == 1))
        assert np.array_equal(host(r.zero_points), z)
    assert np.array_equal(codes.view(np.uint8), q.view(np.uint8))
    assert np.array_equal(host(r.scales).view(np.uint32), s.view(np.uint32))


@pytest.mark.parametrize("act", list(ACT))
@pytest.mark.parametrize("K", [7, 256, 4096, 8200])
def test_quantize_rows_edge_rows(ops, act, K):
    print_case("quantize_rows edge rows", act, K)
    fmt, gran, _ = ACT[act]
    A = _edge_rows(K, rng_for(K))
    r = ops.qgemm_quantize_rows(dev(A), fmt, gran)
    if fmt == 0:
        q, s = O.quantize_sym_int8(A, per_row=(gran == 1))
    else:
        q, s, z = O.quantize_asym_uint8(A, per_row=(gran == 1))
        assert np.array_equal(host(r.zero_points), z)
    assert np.array_equal(host(r.codes()).view(np.uint8), q.view(np.uint8))
    assert np.array_equal(host(r.scales).view(np.uint32), s.view(np.uint32))


def test_quantize_rows_empty(ops):
    r = ops.qgemm_quantize_rows(torch.empty((0, 64), device="cuda"), 0, 1)
    assert r.codes().shape == (0, 64)


# ---------------------------------------------------------------------------
# MXQ: MX quantization, bit-exact (the two zero codes 0x00 / 0x80 are one value)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,K", [(1, 32), (3, 64), (17, 96), (64, 1024), (130, 4192), (8, 8192)])
def test_quantize_mx_bit_exact(ops, M, K):
    print_case("quantize_mx", M, K)
    A, _ = make_inputs("c5_mxfp8", M=M, K=K, N=1, seed=M * 31 + K)
    if M >= 8:
        A[-8:] = _edge_rows(K, rng_for(K))
    r = ops.qgemm_quantize_rows(dev(A), 2, 2)
    codes, E = O.quantize_mx(A)
    got = host(r.codes())
    assert np.array_equal(host(r.mx_scales)[:, : K // 32], E)
    same = (got == codes) | (((got | 0x80) == 0x80) & ((codes | 0x80) == 0x80))
    assert same.all()


# ---------------------------------------------------------------------------
# Weight preparation, bit-exact, padding zero
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("per_channel", [True, False])
@pytest.mark.parametrize("N,K", [(1, 1), (5, 7), (64, 256), (300, 1000), (257, 4097)])
def test_prepack_int8_bit_exact(ops, N, K, per_channel):
    print_case("prepack int8", N, K, per_channel)
    _, W = make_inputs("c2_per_token", M=1, K=K, N=N, seed=N * 101 + K)
    pw = ops.qgemm_prepack_weights(dev(W), 0, 1 if per_channel else 0)
    q, s, colsum = O.prepare_weights_int8(W, per_channel=per_channel)
    codes = host(pw.codes())
    assert np.array_equal(codes[:N, :K], q)
    assert not codes[N:].any() and not codes[:, K:].any()
    sc = host(pw.scales())
    assert np.array_equal(sc[: s.size].view(np.uint32), s.view(np.uint32))
    cs = host(pw.colsum())
    assert np.array_equal(cs[:N], colsum) and not cs[N:].any()


@pytest.mark.parametrize("N,K", [(1, 32), (70, 96), (300, 1024)])
def test_prepack_mx_bit_exact(ops, N, K):
    print_case("prepack mx", N, K)
    _, W = make_inputs("c5_mxfp8", M=1, K=K, N=N, seed=N + K)
    pw = ops.qgemm_prepack_weights(dev(W), 2, 2)
    codes, E = O.quantize_mx(W)
    got = host(pw.codes())
    assert np.array_equal(O.e4m3_decode(got[:N, :K]), O.e4m3_decode(codes))
    assert not got[N:].any() and not got[:, K:].any()
    e = host(pw.scales())
    assert np.array_equal(e[:N, : K // 32], E)
    assert (e[N:] == 127).all() and (e[:, K // 32:] == 127).all()


# ---------------------------------------------------------------------------
# G + E: int8 GEMM and epilogue, end to end from float32 inputs
# ---------------------------------------------------------------------------
GSHAPES = [(1, 1, 1), (3, 5, 7), (33, 65, 129), (64, 64, 256), (130, 260, 300), (257, 513, 1000),
           (300, 300, 4112), (17, 1030, 64),
           # decode-shaped (M <= 16): ragged weight-row groups, K tails inside and past a load batch
           (8, 300, 4112), (16, 1030, 1000), (5, 77, 9000), (12, 2000, 600), (1, 16, 8192)]


def _run_int(ops, A, W, act, wgt, out_type):
    fmt, gran, _ = ACT[act]
    a = ops.qgemm_quantize_rows(dev(A), fmt, gran)
    pw = ops.qgemm_prepack_weights(dev(W), 0, 1 if wgt == "channel" else 0)
    return host(ops.qgemm_run(a, pw, out_type))


def _check_out(got, y, out_type, C=None):
    if out_type == 2:
        assert np.array_equal(got, C)
    elif out_type == 0:
        err = np.abs(got.astype(np.float64) - y)
        bad = err > F32_RTOL * np.abs(y)
        assert not bad.any(), (np.argwhere(bad)[:5], err.max())
    else:
        g = O.bf16_to_f32(got.view(np.uint16)).astype(np.float64)
        err = np.abs(g - y)
        bad = err > BF16_RTOL * np.abs(y)
        assert not bad.any(), (np.argwhere(bad)[:5], err.max())


@pytest.mark.parametrize("act", list(ACT))
@pytest.mark.parametrize("wgt", ["channel", "tensor"])
@pytest.mark.parametrize("M,N,K", GSHAPES)
def test_gemm_int32_exact(ops, M, N, K, act, wgt):
    print_case("gemm i32", M, N, K, act, wgt)
    recipe = "c3_asym_uint8" if act.startswith("asym") else "c2_per_token"
    A, W = make_inputs(recipe, M=M, K=K, N=N, seed=M + 3 * N + 7 * K)
    if act.startswith("asym"):
        A = A - np.float32(0.3)     # both signs: zero points strictly inside (0, 255)
    ref = O.quantized_linear(A, W, act=ACT[act][2], wgt=wgt)
    got = _run_int(ops, A, W, act, wgt, 2)
    _check_out(got, None, 2, ref["C"])


@pytest.mark.parametrize("out_type", [0, 1])
@pytest.mark.parametrize("act", list(ACT))
@pytest.mark.parametrize("M,N,K", [(3, 5, 7), (64, 64, 256), (257, 513, 1000), (300, 300, 4112), (8, 700, 4096)])
def test_gemm_epilogue_float(ops, M, N, K, act, out_type):
    print_case("gemm epilogue", M, N, K, act, out_type)
    A, W = make_inputs("c2_per_token", M=M, K=K, N=N, seed=5 * M + N + K)
    ref = O.quantized_linear(A, W, act=ACT[act][2], wgt="channel")
    got = _run_int(ops, A, W, act, "channel", out_type)
    _check_out(got, ref["y"], out_type)


def test_gemm_c1_both_weight_granularities_and_gate(ops):
    print_case("gemm c1 gate")
    A, W = make_inputs("c1_tiny")
    ref64 = A.astype(np.float64) @ W.astype(np.float64).T
    fr = {}
    for wgt in ("tensor", "channel"):
        ref = O.quantized_linear(A, W, act="sym_tensor", wgt=wgt)
        got = _run_int(ops, A, W, "sym_tensor", wgt, 0)
        _check_out(got, ref["y"], 0)
        fr[wgt] = O.metrics.gate_fractions(got, ref64, A, W)
    assert fr["channel"][2] is None and fr["channel"][1] < 1.0 < fr["tensor"][1]


def test_gemm_deterministic(ops):
    A, W = make_inputs("c3_asym_uint8", M=200, K=1000, N=300)
    a = ops.qgemm_quantize_rows(dev(A), 1, 1)
    pw = ops.qgemm_prepack_weights(dev(W), 0, 1)
    o1 = host(ops.qgemm_run(a, pw, 1))
    o2 = host(ops.qgemm_run(a, pw, 1))
    assert np.array_equal(o1.view(np.uint16), o2.view(np.uint16))


@pytest.mark.parametrize("act", ["sym_row", "asym_row"])
@pytest.mark.parametrize("M,N,K", [(1100, 3900, 700), (4100, 4100, 320), (4000, 4090, 300)])
def test_gemm_large_tile_configs(ops, M, N, K, act):
    """Shapes whose tile count selects, on a 256-CU device, the 128x128 tiles
    (1100 x 3900), the 128x256 tiles two per CU (4100 x 4100: 289 tiles of
    256 x 256, a partial round) and the 256x256 tiles (4000 x 4090: exactly
    256 of them), ragged in M, N and K; int32 sums exact, float32 epilogue in
    tolerance."""
    print_case("gemm tile config", M, N, K, act)
    A, W = make_inputs("c2_per_token", M=M, K=K, N=N, seed=3 * M + N + 5 * K)
    if act == "asym_row":
        A = A - np.float32(0.3)
    ref = O.quantized_linear(A, W, act=ACT[act][2], wgt="channel")
    fmt, gran, _ = ACT[act]
    a = ops.qgemm_quantize_rows(dev(A), fmt, gran)
    pw = ops.qgemm_prepack_weights(dev(W), 0, 1)
    _check_out(host(ops.qgemm_run(a, pw, 2)), None, 2, ref["C"])
    _check_out(host(ops.qgemm_run(a, pw, 0)), ref["y"], 0)


WIDE_CASES = [(M, N, K, act) for M, N, K in [(2000, 11000, 320), (4000, 4090, 300)]
              for act in ("sym_row", "asym_row", "sym_tensor")] + [(2048, 11008, 4096, "asym_row")]


@pytest.mark.parametrize("out_type", [0, 1])
@pytest.mark.parametrize("M,N,K,act", WIDE_CASES)
def test_gemm_wide_tiles(ops, M, N, K, act, out_type):
    """Shapes the one-tile-per-CU kernel takes on a 256-CU device: 2000 x 11000
    as 8 row bands x 32 strips of 352 columns (ragged in M and N, and in the
    last strip), 4000 x 4090 as 16 x 16 tiles of 256 x 256, and the full
    2048 x 11008 x 4096 shape; int32 sums exact (every output), float32 /
    bf16 epilogue in tolerance."""
    print_case("gemm wide tiles", M, N, K, act, out_type)
    A, W = make_inputs("c3_asym_uint8" if act == "asym_row" else "c2_per_token", M=M, K=K, N=N,
                       seed=M + 7 * N + K)
    if act == "asym_row":
        A = A - np.float32(0.3)     # both signs: zero points strictly inside (0, 255)
    ref = O.quantized_linear(A, W, act=ACT[act][2], wgt="channel")
    fmt, gran, _ = ACT[act]
    a = ops.qgemm_quantize_rows(dev(A), fmt, gran)
    pw = ops.qgemm_prepack_weights(dev(W), 0, 1)
    _check_out(host(ops.qgemm_run(a, pw, 2)), None, 2, ref["C"])
    _check_out(host(ops.qgemm_run(a, pw, out_type)), ref["y"], out_type)


@pytest.mark.parametrize("out_type", [0, 1, 2])
def test_gemm_wide_tiles_into_a_padded_output(ops, out_type):
    """The one-tile-per-CU kernel writing into a caller's [M, 11004] buffer:
    bf16 rows then start 8 bytes into a 16-byte unit every other row (ldo is
    4 mod 8), float32 / int32 rows 16-byte aligned. Outputs as in
    test_gemm_wide_tiles; the padding columns past N keep their sentinel."""
    M, N, K = 2000, 11000, 320
    print_case("gemm wide padded out", M, N, K, out_type)
    A, W = make_inputs("c3_asym_uint8", M=M, K=K, N=N, seed=11)
    A = A - np.float32(0.3)
    ref = O.quantized_linear(A, W, act="asym_row", wgt="channel")
    a = ops.qgemm_quantize_rows(dev(A), 1, 1)
    pw = ops.qgemm_prepack_weights(dev(W), 0, 1)
    import torch
    dt = {0: torch.float32, 1: torch.bfloat16, 2: torch.int32}[out_type]
    buf = torch.full((M, 11004), 7, dtype=dt, device="cuda")
    ops.qgemm_run(a, pw, out_type, out=buf)
    got = buf.cpu()
    assert (got[:, N:] == 7).all()
    if out_type == 1:
        got = got.view(torch.int16)
    _check_out(got[:, :N].numpy(), ref["y"], out_type, ref["C"])


@pytest.mark.parametrize("asym", [False, True])
@pytest.mark.parametrize("M", [8, 17, 300])
def test_gemm_int32_at_the_k_limit(ops, M, asym):
    """The largest K the boundary accepts for the format (the oracle's k_limit,
    rounded down to a whole 256), with every activation code at its extreme
    (127; uint8: 255 against zero point 0) and weight rows of +127 and -127
    codes, so the sums reach within 0.02% of 2^31; one activation row and one
    weight row are random. The decode kernel (8 rows) and the tiled kernel
    (17 and 300 rows) must return the oracle's exact sums."""
    K = O.k_limit(asym) // 256 * 256
    N = 40
    print_case("gemm i32 k limit", M, N, K, "asym", asym)
    rng = rng_for(7 + M + int(asym))
    A = np.ones((M, K), np.float32)
    if asym:
        A[:, 0] = 0.0   # row min 0, max 1: s = 1/255, z = 0, codes 0 and 255
    A[-1] = rng.standard_normal(K)
    W = np.where(np.arange(N)[:, None] % 2 == 0, 1.0, -1.0) * np.ones((N, K))
    W[-1] = rng.standard_normal(K)
    W = W.astype(np.float32)
    act = "asym_row" if asym else "sym_row"
    ref = O.quantized_linear(A, W, act=act, wgt="channel")
    assert np.abs(ref["C"]).max() > 0.9998 * 2**31
    _check_out(_run_int(ops, A, W, act, "channel", 2), None, 2, ref["C"])


@pytest.mark.parametrize("M,N,asym", [(1100, 3900, False), (4100, 4100, False), (4000, 4090, False),
                                      (4000, 4090, True), (2000, 11000, False), (2000, 11000, True)])
def test_gemm_int32_at_the_k_limit_large_tiles(ops, M, N, asym):
    """The 128x128, 128x256 (two per CU) and one-tile-per-CU (256 x 256 and
    256 x 352) tile configurations at
    the largest K, on inputs whose exact sums have a closed form: every
    activation code at its extreme and weight rows of alternating +127 and
    -127 codes give C[m][n] = +-127 * 127 * K (uint8: +-255 * 127 * (K - 1),
    the first column being code 0)."""
    K = O.k_limit(asym) // 256 * 256
    print_case("gemm i32 k limit tiles", M, N, K, "asym", asym)
    A = torch.ones((M, K), device="cuda")
    if asym:
        A[:, 0] = 0.0
    sign = np.where(np.arange(N) % 2 == 0, 1, -1).astype(np.int64)
    W = torch.from_numpy(sign.astype(np.float32)).cuda()[:, None].expand(N, K).contiguous()
    a = ops.qgemm_quantize_rows(A, 1 if asym else 0, 1)
    pw = ops.qgemm_prepack_weights(W, 0, 1)
    del A, W
    got = host(ops.qgemm_run(a, pw, 2))
    per = 255 * 127 * (K - 1) if asym else 127 * 127 * K
    assert per < 2**31
    assert np.array_equal(got, np.broadcast_to((per * sign)[None, :], (M, N)))


def test_gemm_empty_m(ops):
    pw = ops.qgemm_prepack_weights(dev(np.ones((8, 64), np.float32)), 0, 1)
    a = ops.qgemm_quantize_rows(torch.empty((0, 64), device="cuda"), 0, 1)
    assert ops.qgemm_run(a, pw, 0).shape == (0, 8)


# ---------------------------------------------------------------------------
# MXG: block-scaled GEMM
# ---------------------------------------------------------------------------
MX_SCALED_STOL = 2.0 ** -10   # derived in qgemm.h from the measured 13-binade window per 8-K group


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (33, 65, 96), (130, 260, 320), (64, 64, 1024),
                                   (300, 200, 2080), (257, 300, 4096), (520, 530, 1024)])
def test_gemm_mx_parity(ops, M, N, K, mode):
    print_case("gemm mx", M, N, K, "mode", mode)
    A, W = make_inputs("c5_mxfp8", M=M, K=K, N=N, seed=M * 13 + N + K)
    a = ops.qgemm_quantize_rows(dev(A), 2, 2)
    pw = ops.qgemm_prepack_weights(dev(W), 2, 2)
    got = host(ops.qgemm_run_mx(a, pw, mode=mode)).astype(np.float64)
    qa, Ea = O.quantize_mx(A)
    qw, Ew = O.quantize_mx(W)
    ref, S = O.mx_gemm_ref(qa, Ea, qw, Ew)
    err = np.abs(got - ref)
    tol = MX_STOL if mode == 0 else MX_SCALED_STOL
    assert (err <= tol * S).all(), (err / np.maximum(S, 1e-300)).max()
    if mode == 0:
        assert O.metrics.rel_l2(got, ref) < 1e-6


def _mx_check(got, A, W, tol):
    qa, Ea = O.quantize_mx(A)
    qw, Ew = O.quantize_mx(W)
    ref, S = O.mx_gemm_ref(qa, Ea, qw, Ew)
    err = np.abs(got.astype(np.float64) - ref)
    assert (err <= tol * S).all(), (err / np.maximum(S, 1e-300)).max()


@pytest.mark.parametrize("mode", [0, 1])
def test_gemm_mx_large_tiles_ragged(ops, mode):
    """At least one 256x256 tile per CU, M and N not multiples of the tile:
    the large-tile configuration of both modes, with clamped rows and padded
    weight columns."""
    M, N, K = 4000, 4352 - 40, 256
    print_case("gemm mx large tiles", M, N, K, "mode", mode)
    A, W = make_inputs("c5_mxfp8", M=M, K=K, N=N, seed=4242)
    a = ops.qgemm_quantize_rows(dev(A), 2, 2)
    pw = ops.qgemm_prepack_weights(dev(W), 2, 2)
    _mx_check(host(ops.qgemm_run_mx(a, pw, mode=mode)), A, W, MX_STOL if mode == 0 else MX_SCALED_STOL)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("K", [64, 128, 192])
def test_gemm_mx_large_tiles_fewer_stages_than_the_ring(ops, K, mode):
    """The 256x256 tile configurations (4 waves in the exact mode, 8 in the
    scaled one) with one to three 64-deep stages, fewer than the 4-stage ring
    their prologue fills: the loads of the stages past K take an empty range,
    and every stage's wait must still cover its own loads. Ragged M and N."""
    M, N = 4000, 4312
    print_case("gemm mx large tiles short K", M, N, K, "mode", mode)
    A, W = make_inputs("c5_mxfp8", M=M, K=K, N=N, seed=77 + K)
    a = ops.qgemm_quantize_rows(dev(A), 2, 2)
    pw = ops.qgemm_prepack_weights(dev(W), 2, 2)
    _mx_check(host(ops.qgemm_run_mx(a, pw, mode=mode)), A, W, MX_STOL if mode == 0 else MX_SCALED_STOL)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("M,N,K", [(130, 260, 320), (600, 700, 1088)])
def test_gemm_mx_both_scale_pitches(ops, M, N, K, mode):
    """K % 64 == 0: the LDS-DMA kernel (E8M0 rows padded to a dword) and the
    register-staged kernel (E8M0 rows of exactly K/32 bytes, not a multiple of
    4) both meet the mode's bound. In the scaled mode they also give the same
    bits: the same matrix-core instruction sums the same 64-deep steps in the
    same order (the exact mode's two kernels sum in different orders)."""
    print_case("gemm mx pitches", M, N, K, "mode", mode)
    tol = MX_STOL if mode == 0 else MX_SCALED_STOL
    A, W = make_inputs("c5_mxfp8", M=M, K=K, N=N, seed=M + N + K)
    a = ops.qgemm_quantize_rows(dev(A), 2, 2)
    pw = ops.qgemm_prepack_weights(dev(W), 2, 2)
    assert a.mx_scales.stride(0) % 4 == 0 and (K // 32) % 4 != 0
    tight = torch.empty((M, K // 32), dtype=torch.uint8, device="cuda")
    tight.copy_(a.mx_scales[:, : K // 32])
    b = ops.QuantizedRows(a.q, K, a.fmt, a.gran, None, None, tight)
    got_dma = host(ops.qgemm_run_mx(a, pw, mode=mode))
    got_reg = host(ops.qgemm_run_mx(b, pw, mode=mode))
    _mx_check(got_dma, A, W, tol)
    _mx_check(got_reg, A, W, tol)
    if mode == 1:
        assert np.array_equal(got_dma.view(np.uint32), got_reg.view(np.uint32))


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (1, 300, 128), (2, 3, 192), (33, 17, 64), (129, 1, 448)])
def test_gemm_mx_dma_small_and_ragged(ops, M, N, K, mode):
    """K % 64 == 0 (the LDS-DMA kernel) with one-row, one-column and ragged
    tiles: clamped A rows, padded weight rows, masked output columns."""
    print_case("gemm mx dma small", M, N, K, "mode", mode)
    A, W = make_inputs("c5_mxfp8", M=M, K=K, N=N, seed=3 * M + N + K)
    a = ops.qgemm_quantize_rows(dev(A), 2, 2)
    pw = ops.qgemm_prepack_weights(dev(W), 2, 2)
    _mx_check(host(ops.qgemm_run_mx(a, pw, mode=mode)), A, W, MX_STOL if mode == 0 else MX_SCALED_STOL)


@pytest.mark.parametrize("mode", [0, 1])
def test_gemm_mx_dma_ignores_row_padding(ops, mode):
    """Activation rows wider than K whose padding holds e4m3 NaN codes (0x7f)
    and E8M0 NaN bytes (0xff): the LDS-DMA kernel reads codes [0, K) and the
    scale bytes of blocks [0, K/32) only, so the result is the unpadded one."""
    M, N, K = 70, 90, 192
    print_case("gemm mx dma padded rows", M, N, K, "mode", mode)
    A, W = make_inputs("c5_mxfp8", M=M, K=K, N=N, seed=77)
    a = ops.qgemm_quantize_rows(dev(A), 2, 2)
    pw = ops.qgemm_prepack_weights(dev(W), 2, 2)
    q = torch.full((M, K + 48), 0x7F, dtype=torch.uint8, device="cuda")
    q[:, :K].copy_(a.q[:, :K])
    e = torch.full((M, K // 32 + 6), 0xFF, dtype=torch.uint8, device="cuda")
    e[:, : K // 32].copy_(a.mx_scales[:, : K // 32])
    assert e.stride(0) % 4 == 0 and q.stride(0) % 16 == 0
    b = ops.QuantizedRows(q, K, a.fmt, a.gran, None, None, e)
    got = host(ops.qgemm_run_mx(b, pw, mode=mode))
    assert np.isfinite(got).all()
    _mx_check(got, A, W, MX_STOL if mode == 0 else MX_SCALED_STOL)
    assert np.array_equal(got.view(np.uint32), host(ops.qgemm_run_mx(a, pw, mode=mode)).view(np.uint32))


@pytest.mark.parametrize("fmt,mode", [(2, 0), (2, 1), (4, 1)])
def test_gemm_mx_dma_bias(ops, fmt, mode):
    """The float32 bias after the block-scaled sum on the LDS-DMA kernel
    (e4m3 in both modes, e2m1 on the fp4 matrix cores)."""
    M, N, K = 70, 200, 256
    print_case("gemm mx dma bias", M, N, K, "fmt", fmt, "mode", mode)
    A, W = make_inputs("c5_mxfp8", M=M, K=K, N=N, seed=fmt * 10 + mode)
    b = rng_for(N + fmt).normal(0.0, 10.0, size=N).astype(np.float32)
    a = ops.qgemm_quantize_rows(dev(A), fmt, 2)
    pw = ops.qgemm_prepack_weights(dev(W), fmt, 2)
    got = host(ops.qgemm_run_mx(a, pw, mode=mode, bias=dev(b))).astype(np.float64)
    quant = O.quantize_mxfp4 if fmt == 4 else O.quantize_mx
    f = "e2m1" if fmt == 4 else "e4m3"
    qa, Ea = quant(A)
    qw, Ew = quant(W)
    ref, S = O.mx_gemm_ref(qa, Ea, qw, Ew, f, f)
    ref = ref + b.astype(np.float64)[None, :]
    tol = MX_SCALED_STOL if (mode == 1 and fmt == 2) else MX_STOL
    assert (np.abs(got - ref) <= tol * S + F32_RTOL * np.abs(ref)).all()


def test_gemm_mx_exact_large_tiles_bias_and_padded_output(ops):
    """The exact mode's 256x256 tiles as 4 waves of 128x128 (at least one tile
    per CU): ragged M and N, several stages of K, a float32 bias, and an output
    whose leading dimension is past N (the padding keeps its sentinel)."""
    M, N, K, ldo = 4000, 4312, 512, 4400
    print_case("gemm mx exact large tiles bias", M, N, K, "ldo", ldo)
    A, W = make_inputs("c5_mxfp8", M=M, K=K, N=N, seed=5151)
    b = rng_for(N + 7).normal(0.0, 10.0, size=N).astype(np.float32)
    a = ops.qgemm_quantize_rows(dev(A), 2, 2)
    pw = ops.qgemm_prepack_weights(dev(W), 2, 2)
    out = torch.full((M, ldo), -3.0, dtype=torch.float32, device="cuda")
    ops.qgemm_run_mx(a, pw, mode=0, bias=dev(b), out=out[:, :N])
    o = host(out)
    assert (o[:, N:] == -3.0).all()
    got = o[:, :N].astype(np.float64)
    qa, Ea = O.quantize_mx(A)
    qw, Ew = O.quantize_mx(W)
    ref, S = O.mx_gemm_ref(qa, Ea, qw, Ew)
    ref = ref + b.astype(np.float64)[None, :]
    assert (np.abs(got - ref) <= MX_STOL * S + F32_RTOL * np.abs(ref)).all()


@pytest.mark.parametrize("K", [32, 64])
def test_gemm_mx_modes_on_an_8_group_with_a_wide_exponent_spread(ops, K):
    """448 and 2^-6 in one group of 8 K: exact mode keeps the small product;
    the block-scaled fp8 matrix cores drop it (the behaviour qgemm.h documents).
    K = 32 runs the register-staged kernel, K = 64 the LDS-DMA one."""
    A = np.zeros((1, K), np.float32)
    A[0, 0], A[0, 1] = 448.0, 2.0 ** -6
    W = np.ones((1, K), np.float32)
    a = ops.qgemm_quantize_rows(dev(A), 2, 2)
    pw = ops.qgemm_prepack_weights(dev(W), 2, 2)
    qa, Ea = O.quantize_mx(A)
    qw, Ew = O.quantize_mx(W)
    ref, S = O.mx_gemm_ref(qa, Ea, qw, Ew)
    assert ref[0, 0] == 448.0 + 2.0 ** -6
    exact = host(ops.qgemm_run_mx(a, pw, mode=0))[0, 0]
    mfma = host(ops.qgemm_run_mx(a, pw, mode=1))[0, 0]
    assert exact == ref[0, 0]
    assert mfma == 448.0 and abs(mfma - ref[0, 0]) <= MX_SCALED_STOL * S[0, 0]
    print(f"[measured] wide-exponent group, K={K}: scaled-mode err/S = {abs(mfma - ref[0, 0]) / S[0, 0]:.3e} "
          f"(bound 2^-10 = {2.0 ** -10:.3e}); exact-mode err/S = {abs(exact - ref[0, 0]) / S[0, 0]:.3e}", flush=True)


# ---------------------------------------------------------------------------
# Bias after the scales (int8 and MX) and the fused RMSNorm + quantize step
# ---------------------------------------------------------------------------
def _bias_bar(ref, b, out_type):
    """float32: two roundings (the scaled product, then + bias) on top of the
    epilogue's; bf16 adds half a bf16 ulp of the result."""
    y0 = np.abs(ref - b.astype(np.float64)[None, :])
    bar = F32_RTOL * (y0 + np.abs(ref))
    return bar + (BF16_RTOL * np.abs(ref) if out_type == 1 else 0.0)


@pytest.mark.parametrize("out_type", [0, 1])
@pytest.mark.parametrize("act", ["sym_row", "asym_row", "sym_tensor"])
@pytest.mark.parametrize("M,N,K", [(8, 300, 4112), (64, 64, 256), (257, 513, 1000), (1100, 3900, 700)])
def test_gemm_bias(ops, M, N, K, act, out_type):
    print_case("gemm bias", M, N, K, act, out_type)
    A, W = make_inputs("c2_per_token", M=M, K=K, N=N, seed=2 * M + 3 * N + K)
    if act == "asym_row":
        A = A - np.float32(0.3)
    b = rng_for(N + K).normal(0.0, 2.0, size=N).astype(np.float32)
    ref = O.quantized_linear(A, W, act=ACT[act][2], wgt="channel", bias=b)["y"]
    fmt, gran, _ = ACT[act]
    a = ops.qgemm_quantize_rows(dev(A), fmt, gran)
    pw = ops.qgemm_prepack_weights(dev(W), 0, 1)
    got = host(ops.qgemm_run(a, pw, out_type, bias=dev(b)))
    g = got.astype(np.float64) if out_type == 0 else O.bf16_to_f32(got.view(np.uint16)).astype(np.float64)
    err = np.abs(g - ref)
    bad = err > _bias_bar(ref, b, out_type)
    assert not bad.any(), (np.argwhere(bad)[:5], err.max())


@pytest.mark.parametrize("M,N,K", [(33, 65, 96), (300, 200, 2080)])
def test_gemm_mx_bias(ops, M, N, K):
    print_case("gemm mx bias", M, N, K)
    A, W = make_inputs("c5_mxfp8", M=M, K=K, N=N, seed=M + 5 * N + K)
    b = rng_for(K).normal(0.0, 10.0, size=N).astype(np.float32)
    a = ops.qgemm_quantize_rows(dev(A), 2, 2)
    pw = ops.qgemm_prepack_weights(dev(W), 2, 2)
    got = host(ops.qgemm_run_mx(a, pw, mode=0, bias=dev(b))).astype(np.float64)
    qa, Ea = O.quantize_mx(A)
    qw, Ew = O.quantize_mx(W)
    ref, S = O.mx_gemm_ref(qa, Ea, qw, Ew)
    ref = O.add_bias(ref, b)
    assert (np.abs(got - ref) <= MX_STOL * S + F32_RTOL * np.abs(ref)).all()


@pytest.mark.parametrize("act", ["sym_row", "asym_row"])
def test_rmsnorm_rms_on_a_float32_midpoint(ops, act):
    """Rows whose float64 rms lies exactly on the midpoint between two float32
    values: x = (1 + 2^-23, 1, 1, 1) with eps = 2^-24 gives mean(x^2) + eps =
    (1 + 2^-24)^2 exactly, so rms is the midpoint between 1 and 1 + 2^-23 and
    rounds to the even 1.0; the kernel's float64 sum cannot decide such a row
    by itself and sums it again exactly. Codes and scales equal the oracle's;
    a second row, scaled by 3, is an ordinary one."""
    print_case("rmsnorm rms on a midpoint", act)
    A = np.array([[1 + 2.0 ** -23, 1, 1, 1], [3 * (1 + 2.0 ** -23), 3, 3, 3]], np.float32)
    g = np.array([0.5, -1.0, 2.0, 1.0], np.float32)
    eps = np.float32(2.0 ** -24)
    assert O.rms_value(A[:1], eps)[0] == np.float32(1.0)  # the tie went to even
    fmt = ACT[act][0]
    r = ops.qgemm_rmsnorm_quantize_rows(dev(A), dev(g), float(eps), fmt)
    out = O.rmsnorm_quantize(A, g, eps, act=act)
    assert np.array_equal(host(r.codes()).view(np.uint8), out[0].view(np.uint8))
    assert np.array_equal(host(r.scales).view(np.uint32), out[1].view(np.uint32))


@pytest.mark.parametrize("act", ["sym_row", "asym_row"])
@pytest.mark.parametrize("M,K,misaligned", [(1, 1, False), (3, 5, False), (7, 17, False), (64, 256, False),
                                            (33, 1000, False), (5, 4097, False), (512, 4096, False),
                                            (9, 8192, False), (2, 9000, False), (6, 260, True)])
def test_rmsnorm_quantize_parity(ops, act, M, K, misaligned):
    """Codes, scales and zero points of the fused step equal the oracle's bit
    for bit on every row. The kernel divides by the float32 rms as the page
    writes (x / rms * gamma). Its float64 sum of squares decides the float32
    rms unless the float64 rms is within the sum's error bound of a float32
    rounding midpoint; such rows are summed again as a double-double, which
    rounds to the oracle's exact sum (it could differ only for an exact sum
    within about K * 2^-104 of the midpoint between two doubles)."""
    print_case("rmsnorm quantize", act, M, K, misaligned)
    A, _ = make_inputs("c2_per_token", M=M, K=K, N=1, seed=M * 17 + K)
    if M >= 8:
        A[-8:] = _edge_rows(K, rng_for(K))
    g = rng_for(K + 1).normal(1.0, 0.3, size=K).astype(np.float32)
    g[:: max(K // 7, 1)] = 0.0
    g[1:: max(K // 5, 1)] *= -1.0
    eps = 1e-6
    fmt = ACT[act][0]
    gd = dev(np.concatenate([np.zeros(1, np.float32), g]))[1:] if misaligned else dev(g)
    r = ops.qgemm_rmsnorm_quantize_rows(dev(A), gd, eps, fmt)
    out = O.rmsnorm_quantize(A, g, eps, act=act)
    assert np.array_equal(host(r.codes()).view(np.uint8), out[0].view(np.uint8))
    assert np.array_equal(host(r.scales).view(np.uint32), out[1].view(np.uint32))
    if fmt == 1:
        assert np.array_equal(host(r.zero_points), out[2])
