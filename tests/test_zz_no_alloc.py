"""The allocation-free quantize entry point against the workspace one.

qgemm_quantize_rows_noalloc keeps the per-tensor statistics in the library's
static device array instead of a caller workspace. Its codes, scales and zero
points must equal qgemm_quantize_rows' bit for bit (and the oracle's) on two
calls in a row, the second with fewer rows, so nothing left in the array by
the first call leaks into the second; sizes beyond the array are refused
before anything is launched.
"""
import numpy as np
import pytest

import oracle as O
from block_scaled_quantized_qgemm_amd.inputs import make_inputs
from conftest import print_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ops():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_scaled_quantized_qgemm_amd import ops as _ops
    _ops.L.load()
    return _ops


def _host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _same(a, b):
    """Bit-exact equality of two quantize results."""
    assert np.array_equal(_host(a.codes()).view(np.uint8), _host(b.codes()).view(np.uint8))
    for x, y in ((a.scales, b.scales), (a.zero_points, b.zero_points)):
        assert (x is None) == (y is None)
        if x is not None:
            assert np.array_equal(_host(x).view(np.uint8), _host(y).view(np.uint8))
    assert (a.mx_scales is None) == (b.mx_scales is None)
    if a.mx_scales is not None:   # the E8M0 rows are padded to 4 bytes; the padding is never written
        nb = a.K // 32
        assert np.array_equal(_host(a.mx_scales)[:, :nb], _host(b.mx_scales)[:, :nb])


CASES = [(0, 0), (1, 0), (0, 1), (1, 1), (2, 2)]   # (fmt, gran): per tensor, per row, MXFP8


@pytest.mark.parametrize("fmt,gran", CASES)
def test_noalloc_equals_workspace_entry_point_on_two_calls(ops, fmt, gran):
    """Two calls in a row, the second smaller: each equals the workspace
    entry point's result and the oracle's."""
    for M, K, seed in ((3000, 1024, 71), (700, 320, 72)):
        print_case("noalloc quantize", fmt, gran, M, K)
        A, _ = make_inputs("c2_per_token", M=M, K=K, N=1, seed=seed)
        if fmt == 1:
            A = A - np.float32(0.25)         # both signs: a zero point strictly inside (0, 255)
        x = torch.from_numpy(A).cuda()
        ref = ops.qgemm_quantize_rows(x, fmt, gran)
        got = ops.qgemm_quantize_rows_noalloc(x, fmt, gran)
        _same(got, ref)
        if fmt == 2:
            qa, Ea = O.quantize_mx(A)
            assert np.array_equal(O.e4m3_decode(_host(got.codes())), O.e4m3_decode(qa))
            assert np.array_equal(_host(got.mx_scales)[:, : K // 32], Ea)
        elif fmt == 0:
            qa, sa = O.quantize_sym_int8(A, per_row=(gran == 1))
            assert np.array_equal(_host(got.codes()), qa)
            assert np.array_equal(_host(got.scales).view(np.uint32), sa.view(np.uint32))
        else:
            qa, sa, za = O.quantize_asym_uint8(A, per_row=(gran == 1))
            assert np.array_equal(_host(got.codes()), qa)
            assert np.array_equal(_host(got.scales).view(np.uint32), sa.view(np.uint32))
            assert np.array_equal(_host(got.zero_points), za)


def test_noalloc_reuses_caller_buffers(ops):
    """With the output buffers passed in, repeated calls write the same bits."""
    A, _ = make_inputs("c2_per_token", M=513, K=4096, N=1, seed=73)
    x = torch.from_numpy(A).cuda()
    ref = ops.qgemm_quantize_rows(x, 0, 0)
    out = ops.qgemm_quantize_rows_noalloc(x, 0, 0)
    for _ in range(3):
        ops.qgemm_quantize_rows_noalloc(x, 0, 0, out=out)
        _same(out, ref)


def test_noalloc_refuses_rows_beyond_the_static_array(ops):
    """Per-tensor statistics need 4 bytes per row (8 for uint8): beyond the
    1 MiB array the call returns QGEMM_E_WORKSPACE without launching; the
    per-row granularity needs no scratch and takes the same rows."""
    for fmt, rows in ((0, (1 << 18) + 1), (1, (1 << 17) + 1)):
        x = torch.zeros((rows, 1), dtype=torch.float32, device="cuda")
        with pytest.raises(ops.QgemmError) as e:
            ops.qgemm_quantize_rows_noalloc(x, fmt, 0)
        assert e.value.status == -8                      # QGEMM_E_WORKSPACE
        ok = ops.qgemm_quantize_rows_noalloc(x[: rows - 1], fmt, 0)   # the largest accepted size
        assert not _host(ok.codes()).any()                    # zeros quantize to code 0 (z = 0)
        r = ops.qgemm_quantize_rows_noalloc(x, fmt, 1)
        assert _host(r.scales).shape == (rows,)
