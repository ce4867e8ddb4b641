"""GPU parity of qgemm_unpack_weights, through the C ABI, against the CPU
oracle: the plain codes, scales, column sums and E8M0 scales read back out of
a prepared weight buffer equal the oracle's weight preparation bit for bit,
for every weight format, on ragged shapes (N not a multiple of 16, K not a
multiple of 64 or 256) and into padded outputs (the padding keeps its
sentinel)."""
import numpy as np
import pytest

import oracle as O
from block_scaled_quantized_qgemm_amd.inputs import make_inputs
from conftest import print_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SHAPES = [(1, 64), (17, 96), (70, 320), (300, 1030)]
MX_SHAPES = [(1, 64), (17, 96), (70, 320), (300, 1056)]  # K % 32 == 0


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
    return t.cpu().numpy()


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


@pytest.mark.parametrize("per_channel", [True, False])
@pytest.mark.parametrize("N,K", SHAPES)
def test_unpack_int8(ops, N, K, per_channel):
    print_case("unpack int8", N, K, per_channel)
    _, W = make_inputs("c2_per_token", M=1, K=K, N=N, seed=5 * N + K)
    pw = ops.qgemm_prepack_weights(dev(W), ops.FMT_INT8_SYM, ops.GRAN_ROW if per_channel else ops.GRAN_TENSOR)
    got = ops.qgemm_unpack_weights(pw)
    q, s, colsum = O.prepare_weights_int8(W, per_channel=per_channel)
    assert np.array_equal(host(got["codes"]), q)
    assert np.array_equal(_bits(host(got["scales"])), _bits(np.asarray(s, np.float32).reshape(-1)))
    assert np.array_equal(host(got["colsums"]), colsum)


@pytest.mark.parametrize("N,K", SHAPES)
def test_unpack_int4(ops, N, K):
    print_case("unpack int4", N, K)
    _, W = make_inputs("c4_decode", M=1, K=K, N=N, seed=7 * N + K)
    pw = ops.qgemm_prepack_weights(dev(W), ops.FMT_INT4_SYM, ops.GRAN_GROUP64)
    got = ops.qgemm_unpack_weights(pw)
    q, s = O.quantize_int4_groups(W)
    assert np.array_equal(host(got["codes"]), q)
    assert np.array_equal(_bits(host(got["scales"])), _bits(np.asarray(s, np.float32)))


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
@pytest.mark.parametrize("N,K", MX_SHAPES)
def test_unpack_mx(ops, N, K, fmt):
    print_case("unpack mx", N, K, fmt)
    _, W = make_inputs("c5_mxfp8", M=1, K=K, N=N, seed=11 * N + K)
    f = ops.FMT_MXFP8_E4M3 if fmt == "e4m3" else ops.FMT_MXFP4_E2M1
    pw = ops.qgemm_prepack_weights(dev(W), f, ops.GRAN_BLOCK32)
    got = ops.qgemm_unpack_weights(pw)
    if fmt == "e4m3":
        codes, E = O.quantize_mx(W)
        assert np.array_equal(O.e4m3_decode(host(got["codes"])), O.e4m3_decode(codes))  # +-0 as one value
    else:
        codes, E = O.quantize_mxfp4(W)
        c = np.asarray(codes, np.uint8)
        assert np.array_equal(host(got["codes"]), c[:, 0::2] | (c[:, 1::2] << 4))  # element 2i in the low nibble
    assert np.array_equal(host(got["mx_scales"]), E)


def test_unpack_into_padded_outputs_and_subsets(ops):
    """Outputs with leading dimensions past their rows, and only some outputs
    requested: each requested output is filled, the padding and every output
    not requested keep their sentinels."""
    L = ops.L
    lib = L.load()
    N, K = 33, 200
    _, W = make_inputs("c4_decode", M=1, K=K, N=N, seed=3)
    pw = ops.qgemm_prepack_weights(dev(W), ops.FMT_INT4_SYM, ops.GRAN_GROUP64)
    q, s = O.quantize_int4_groups(W)
    codes = torch.full((N, K + 13), 77, dtype=torch.int8, device="cuda")
    scales = torch.full((N, 9), -1.0, dtype=torch.float32, device="cuda")
    st = lib.qgemm_unpack_weights(ops.ctypes.byref(pw.desc), ops._ptr(pw.packed), ops._ptr(codes), K + 13,
                                  None, 0, None, None, 0, None)
    assert st == 0
    c = host(codes)
    assert np.array_equal(c[:, :K], q) and (c[:, K:] == 77).all()
    assert (host(scales) == -1.0).all()
    st = lib.qgemm_unpack_weights(ops.ctypes.byref(pw.desc), ops._ptr(pw.packed), None, 0, ops._ptr(scales), 9,
                                  None, None, 0, None)
    assert st == 0
    sc = host(scales)
    g = (K + 63) // 64
    assert np.array_equal(_bits(sc[:, :g]), _bits(np.asarray(s, np.float32))) and (sc[:, g:] == -1.0).all()
