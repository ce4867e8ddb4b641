"""Parity at the full workload sizes, in the launch configuration bench.py
times: codes, scales and zero points compared in full (the oracle quantizes a
few hundred rows in well under a second), GEMM outputs on sampled (m, n)
pairs that the oracle evaluates one dot product at a time."""
import numpy as np
import pytest

import oracle as O
from block_scaled_quantized_qgemm_amd.inputs import make_inputs, rng_for
from conftest import print_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

WL = {  # name -> (fmt, gran, out_type)
    "c1_tiny": (0, 0, 0),
    "c2_per_token": (0, 1, 0),
    "c3_asym_uint8": (1, 1, 1),
    "c4_decode": (0, 1, 0),
}


@pytest.fixture(scope="module")
def ops():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_scaled_quantized_qgemm_amd import ops as _ops
    _ops.L.load()
    return _ops


def _host(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _pairs(M, N, n, seed):
    rng = rng_for(seed)
    rows = np.concatenate([rng.integers(0, M, n), [0, M - 1, 0, M - 1]])
    cols = np.concatenate([rng.integers(0, N, n), [0, 0, N - 1, N - 1]])
    return rows, cols


@pytest.mark.parametrize("name", list(WL))
def test_int8_workload_full_size(ops, name):
    fmt, gran, out_type = WL[name]
    A, W = make_inputs(name)
    M, K = A.shape
    N = W.shape[0]
    print_case("workload", name, M, N, K)
    a = ops.qgemm_quantize_rows(torch.from_numpy(A).cuda(), fmt, gran)
    pw = ops.qgemm_prepack_weights(torch.from_numpy(W).cuda(), 0, 1)
    y = _host(ops.qgemm_run(a, pw, out_type))
    c = _host(ops.qgemm_run(a, pw, 2))
    # quantization: full comparison
    if fmt == 0:
        qa, sa = O.quantize_sym_int8(A, per_row=(gran == 1))
        za = np.zeros(1, np.int32)
    else:
        qa, sa, za = O.quantize_asym_uint8(A, per_row=(gran == 1))
        assert np.array_equal(_host(a.zero_points), za)
    assert np.array_equal(_host(a.codes()).view(np.uint8), qa.view(np.uint8))
    assert np.array_equal(_host(a.scales).view(np.uint32), sa.view(np.uint32))
    qw, sw, colsum = O.prepare_weights_int8(W, per_channel=True)
    assert np.array_equal(_host(pw.codes())[:N, :K], qw)
    assert np.array_equal(_host(pw.colsum())[:N], colsum)
    # GEMM and epilogue on sampled outputs
    rows, cols = _pairs(M, N, 4096, M + N)
    Cref = O.int_gemm_entries(qa, za, qw, rows, cols)
    assert np.array_equal(c[rows, cols], Cref)
    sa_r = sa[rows] if sa.size > 1 else np.repeat(sa, rows.size)
    yref = Cref.astype(np.float64) * sa_r.astype(np.float64) * sw[cols].astype(np.float64)
    got = y[rows, cols]
    if out_type == 0:
        assert (np.abs(got.astype(np.float64) - yref) <= 1e-6 * np.abs(yref)).all()
    else:
        g = O.bf16_to_f32(got).astype(np.float64)
        assert (np.abs(g - yref) <= (2.0 ** -8 + 2.0 ** -20) * np.abs(yref)).all()


@pytest.mark.parametrize("mode", [0, 1])
def test_mx_workload_full_size(ops, mode):
    A, W = make_inputs("c5_mxfp8")
    M, K = A.shape
    N = W.shape[0]
    print_case("workload c5_mxfp8", M, N, K, "mode", mode)
    a = ops.qgemm_quantize_rows(torch.from_numpy(A).cuda(), 2, 2)
    pw = ops.qgemm_prepack_weights(torch.from_numpy(W).cuda(), 2, 2)
    y = _host(ops.qgemm_run_mx(a, pw, mode=mode))
    rows, cols = _pairs(M, N, 2048, 5)
    ur, uc = np.unique(rows), np.unique(cols)
    qa, Ea = O.quantize_mx(A[ur])
    qw, Ew = O.quantize_mx(W[uc])
    # quantization of the sampled rows: full comparison
    ga = _host(a.codes())[ur]
    assert np.array_equal(O.e4m3_decode(ga), O.e4m3_decode(qa))
    assert np.array_equal(_host(a.mx_scales)[ur, : K // 32], Ea)
    assert np.array_equal(O.e4m3_decode(_host(pw.codes())[uc, :K]), O.e4m3_decode(qw))
    ri = np.searchsorted(ur, rows)
    ci = np.searchsorted(uc, cols)
    ref, S = O.mx_gemm_ref_entries(qa, Ea, qw, Ew, ri, ci)
    err = np.abs(y[rows, cols].astype(np.float64) - ref)
    tol = 1e-5 if mode == 0 else 2.0 ** -10
    rel = np.abs(ref) > 0
    print(f"[measured] c5_mxfp8 mode {mode} on {rows.size} sampled outputs: max err/S = {(err / S).max():.3e} "
          f"(gate {tol:.3e}), median err/S = {np.median(err / S):.3e}, "
          f"max err/|ref| = {(err[rel] / np.abs(ref[rel])).max():.3e}, "
          f"outputs with err > 1e-5*S: {int((err > 1e-5 * S).sum())}", flush=True)
    assert (err <= tol * S).all(), (err / S).max()
