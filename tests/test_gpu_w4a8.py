"""GPU parity of the W4A8 path (int8 activations x int4 weights, one float32
scale per group of 64 K), through the C ABI, against the CPU oracle.

int4 codes and their float32 scales are bit-exact. GEMM outputs are within
the float32 bound the header states: the kernel sums the groups' scaled
partials in float32 (one FMA each, then an 8-way sum, the activation scale
and the bias), so |out - exact| <= (K_pad / 64 + 16) * 2^-24 * (S + |bias|)
with S = sum_g |s_a s_w P_g| from the oracle; bfloat16 adds half a bf16 ulp.
A wrong scale, group or sign moves outputs by a large fraction of S and
fails by orders of magnitude.
"""
import numpy as np
import pytest

import oracle as O
from block_scaled_quantized_qgemm_amd.inputs import make_inputs, rng_for
from conftest import print_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

BF16_RTOL = 2.0 ** -8 + 2.0 ** -20


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


def _k_pad(K):
    return (K + 255) // 256 * 256


def _edge_weight_rows(K, rng):
    """Rows that hit the rounding and range corners of the int4 rule."""
    rows = [np.zeros(K), np.full(K, 3.25), np.full(K, -2.0), rng.standard_normal(K) * 1e-30,
            rng.standard_normal(K) * 6.0e4]
    # exact ties: a group with amax 7 has s = 1, so 0.5, 1.5, 2.5 ... sit half-way between codes
    ties = np.tile(np.array([7.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5, -3.5, 6.5, -6.5, -7.0]), K // 12 + 1)[:K]
    rows.append(ties)
    spike = np.zeros(K)
    spike[K // 2] = -7.0
    rows.append(spike)
    return np.stack(rows).astype(np.float32)


# ---------------------------------------------------------------------------
# int4 weight preparation, bit-exact, padding zero
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("N,K", [(1, 1), (5, 7), (16, 64), (17, 65), (64, 256), (300, 1000), (257, 4097),
                                 (33, 8200)])
def test_prepack_int4_bit_exact(ops, N, K):
    print_case("prepack int4", N, K)
    _, W = make_inputs("c4_decode", M=1, K=K, N=N, seed=N * 131 + K)
    if N >= 16:
        W[:7] = _edge_weight_rows(K, rng_for(K))
    pw = ops.qgemm_prepack_weights(dev(W), ops.FMT_INT4_SYM, ops.GRAN_GROUP64)
    q, s = O.quantize_int4_groups(W)
    codes = host(pw.codes())
    assert codes.shape == (pw.desc.N_pad, _k_pad(K))
    assert np.array_equal(codes[:N, :K], q)
    assert not codes[N:].any() and not codes[:, K:].any()
    sc = host(pw.scales())
    ng = s.shape[1]
    assert np.array_equal(sc[:N, :ng].view(np.uint32), s.view(np.uint32))
    assert not sc[N:].any() and not sc[:, ng:].any()


def test_prepack_int4_tie_rounding_and_floor(ops):
    """Half-way quotients round to even, an all-zero group takes the 1e-8
    floor, and codes never reach -8 from the weights' own scale."""
    print_case("prepack int4 ties")
    W = _edge_weight_rows(128, rng_for(3))
    pw = ops.qgemm_prepack_weights(dev(W), ops.FMT_INT4_SYM, ops.GRAN_GROUP64)
    codes = host(pw.codes())[:W.shape[0], :128]
    sc = host(pw.scales())
    assert sc[0, 0] == np.float32(1e-8) and not codes[0].any()
    assert codes[5, :12].tolist() == [7, 0, 2, 2, 0, -2, -2, 4, -4, 6, -6, -7]
    assert codes.min() >= -7


# ---------------------------------------------------------------------------
# W4A8 GEMM
# ---------------------------------------------------------------------------
def _w4a8_ref(A, W, per_row=True, bias=None):
    qa, sa = O.quantize_sym_int8(A, per_row=per_row)
    qw, sw = O.quantize_int4_groups(W)
    y, S = O.w4a8_gemm(qa, sa, qw, sw)
    if bias is not None:
        y = y + bias.astype(np.float64)[None, :]
        S = S + np.abs(bias.astype(np.float64))[None, :]
    return y, S


def _check(got, y, S, K, out_type):
    bar = (_k_pad(K) / 64 + 16) * 2.0 ** -24 * S
    if out_type == 0:
        g = got.astype(np.float64)
    else:
        g = O.bf16_to_f32(got.view(np.uint16)).astype(np.float64)
        bar = bar + BF16_RTOL * np.abs(y)
    err = np.abs(g - y)
    bad = err > bar
    assert not bad.any(), (np.argwhere(bad)[:5], err.max(), float((err / np.maximum(S, 1e-300)).max()))


W4SHAPES = [(1, 1, 1), (3, 5, 7), (1, 16, 64), (8, 17, 65), (16, 300, 127), (5, 1030, 1000),
            (8, 77, 4096), (2, 40, 4112), (12, 200, 9000), (1, 16, 8192),
            # several 16-row bands of A
            (17, 33, 300), (40, 130, 1000), (300, 64, 256)]


@pytest.mark.parametrize("out_type", [0, 1])
@pytest.mark.parametrize("M,N,K", W4SHAPES)
def test_w4a8_parity(ops, M, N, K, out_type):
    print_case("w4a8", M, N, K, out_type)
    A, W = make_inputs("c4_decode", M=M, K=K, N=N, seed=M + 11 * N + 3 * K)
    y, S = _w4a8_ref(A, W)
    a = ops.qgemm_quantize_rows(dev(A), ops.FMT_INT8_SYM, ops.GRAN_ROW)
    pw = ops.qgemm_prepack_weights(dev(W), ops.FMT_INT4_SYM, ops.GRAN_GROUP64)
    got = host(ops.qgemm_run_w4a8(a, pw, out_type))
    _check(got, y, S, K, out_type)


@pytest.mark.parametrize("M,N,K", [(8, 300, 4112), (33, 65, 700)])
def test_w4a8_per_tensor_activation_and_bias(ops, M, N, K):
    print_case("w4a8 tensor+bias", M, N, K)
    A, W = make_inputs("c2_per_token", M=M, K=K, N=N, seed=7 * M + N + K)
    b = rng_for(N).normal(0.0, 2.0, size=N).astype(np.float32)
    y, S = _w4a8_ref(A, W, per_row=False, bias=b)
    a = ops.qgemm_quantize_rows(dev(A), ops.FMT_INT8_SYM, ops.GRAN_TENSOR)
    pw = ops.qgemm_prepack_weights(dev(W), ops.FMT_INT4_SYM, ops.GRAN_GROUP64)
    _check(host(ops.qgemm_run_w4a8(a, pw, 0, bias=dev(b))), y, S, K, 0)


def test_w4a8_ignores_activation_bytes_past_k(ops):
    """Bytes of A's rows between K and lda meet zero weight codes."""
    print_case("w4a8 junk past K")
    M, N, K = 9, 50, 130
    A, W = make_inputs("c4_decode", M=M, K=K, N=N, seed=17)
    y, S = _w4a8_ref(A, W)
    a = ops.qgemm_quantize_rows(dev(A), ops.FMT_INT8_SYM, ops.GRAN_ROW)
    a.q[:, K:] = 77
    pw = ops.qgemm_prepack_weights(dev(W), ops.FMT_INT4_SYM, ops.GRAN_GROUP64)
    _check(host(ops.qgemm_run_w4a8(a, pw, 0)), y, S, K, 0)


@pytest.mark.parametrize("out_type", [0, 1])
def test_w4a8_tiled_large_tiles_ragged(ops, out_type):
    """More than 16 rows runs the tiled kernel; at least one 128 x 128 tile
    per CU takes its large-tile configuration. M and N are not multiples of
    the tile, K not of the 128-deep stage."""
    M, N, K = 2000, 2100, 320
    print_case("w4a8 tiled large", M, N, K, out_type)
    A, W = make_inputs("c2_per_token", M=M, K=K, N=N, seed=23 + out_type)
    y, S = _w4a8_ref(A, W)
    a = ops.qgemm_quantize_rows(dev(A), ops.FMT_INT8_SYM, ops.GRAN_ROW)
    pw = ops.qgemm_prepack_weights(dev(W), ops.FMT_INT4_SYM, ops.GRAN_GROUP64)
    _check(host(ops.qgemm_run_w4a8(a, pw, out_type)), y, S, K, out_type)


def test_w4a8_tiled_ignores_activation_bytes_past_k(ops):
    """The tiled kernel (more than 16 rows): bytes of A's rows between K and
    lda meet zero weight codes."""
    M, N, K = 40, 150, 200
    print_case("w4a8 tiled junk past K", M, N, K)
    A, W = make_inputs("c4_decode", M=M, K=K, N=N, seed=19)
    y, S = _w4a8_ref(A, W)
    a = ops.qgemm_quantize_rows(dev(A), ops.FMT_INT8_SYM, ops.GRAN_ROW)
    a.q[:, K:] = -77
    pw = ops.qgemm_prepack_weights(dev(W), ops.FMT_INT4_SYM, ops.GRAN_GROUP64)
    _check(host(ops.qgemm_run_w4a8(a, pw, 0)), y, S, K, 0)


def test_w4a8_prefill_shape_full_size(ops):
    """W4A8 at the per-token workload's full size (512 x 4096 x 4096, the
    tiled kernel's 64 x 128 tiles as the benchmark launches them), checked on
    64 rows spread over all row tiles against the oracle (each output row
    depends only on its own activation row)."""
    print_case("w4a8 prefill full size")
    A, W = make_inputs("c2_per_token")
    M, K = A.shape
    a = ops.qgemm_quantize_rows(dev(A), ops.FMT_INT8_SYM, ops.GRAN_ROW)
    pw = ops.qgemm_prepack_weights(dev(W), ops.FMT_INT4_SYM, ops.GRAN_GROUP64)
    got = host(ops.qgemm_run_w4a8(a, pw, 0))
    rows = np.unique(np.concatenate([[0, 1, 63, 64, M - 1], rng_for(5).choice(M, 59, replace=False)]))
    y, S = _w4a8_ref(A[rows], W)
    _check(got[rows], y, S, K, 0)


def test_w4a8_decode_workload_full_size(ops):
    """The decode-shaped workload at its full size (8 x 4096 x 14336), the
    launch the benchmark times, element by element against the full oracle."""
    print_case("w4a8 full decode workload")
    A, W = make_inputs("c4_decode")
    M, K = A.shape
    y, S = _w4a8_ref(A, W)
    a = ops.qgemm_quantize_rows(dev(A), ops.FMT_INT8_SYM, ops.GRAN_ROW)
    pw = ops.qgemm_prepack_weights(dev(W), ops.FMT_INT4_SYM, ops.GRAN_GROUP64)
    got = host(ops.qgemm_run_w4a8(a, pw, 0))
    _check(got, y, S, K, 0)
    rel = np.linalg.norm(got - y) / np.linalg.norm(y)
    assert rel < 1e-6


def test_w4a8_deterministic_and_empty(ops):
    A, W = make_inputs("c4_decode", M=13, K=1000, N=300)
    a = ops.qgemm_quantize_rows(dev(A), ops.FMT_INT8_SYM, ops.GRAN_ROW)
    pw = ops.qgemm_prepack_weights(dev(W), ops.FMT_INT4_SYM, ops.GRAN_GROUP64)
    o1 = host(ops.qgemm_run_w4a8(a, pw, 0))
    o2 = host(ops.qgemm_run_w4a8(a, pw, 0))
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    e = ops.qgemm_quantize_rows(torch.empty((0, 1000), device="cuda"), ops.FMT_INT8_SYM, ops.GRAN_ROW)
    assert ops.qgemm_run_w4a8(e, pw, 0).shape == (0, 300)
