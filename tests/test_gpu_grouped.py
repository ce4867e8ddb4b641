"""GPU parity of the grouped (MoE) block-scaled GEMM, through the C ABI,
against the CPU oracle ("TileLang tutorial, chapter 27", section 6.2, MoE
point 3: A is the concatenation of the rows routed to each expert, one weight
matrix per expert).

Bars: the exact mode within 1e-5 * S of the float64 reference over the
dequantized values (S = sum_k |a_k w_k|), the block-scaled fp8 matrix cores
within 2^-10 * S, e2m1 on the fp4 matrix cores within 1e-5 * S; and each
expert's rows the same bits as the plain MX GEMM of that expert's slice.
"""
import numpy as np
import pytest

import oracle as O
from block_scaled_quantized_qgemm_amd.inputs import make_inputs, rng_for
from conftest import print_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

MX_STOL = 1e-5
MX_SCALED_STOL = 2.0 ** -10
F32_RTOL = 1e-6
E4M3, E2M1 = 2, 4


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


def _setup(ops, sizes, N, K, fmt=E4M3, seed=0, wfmt=None):
    E = len(sizes)
    M = int(sum(sizes))
    A, Wall = make_inputs("c5_mxfp8", M=max(M, 1), K=K, N=E * N, seed=seed)
    A = A[:M]
    W = Wall.reshape(E, N, K)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    a = ops.qgemm_quantize_rows(dev(A), fmt, ops.GRAN_BLOCK32)
    w = ops.qgemm_prepack_experts(dev(W), fmt if wfmt is None else wfmt)
    return A, W, offsets, a, w


def _quant(x, fmt):
    return (O.quantize_mxfp4(x), "e2m1") if fmt == E2M1 else (O.quantize_mx(x), "e4m3")


def _ref(A, W, offsets, fmt=E4M3, wfmt=None):
    E, N, K = W.shape
    (qa, Ea), fa = _quant(A, fmt)
    (qw, Ew), fw = _quant(W.reshape(E * N, K), fmt if wfmt is None else wfmt)
    return O.mx_grouped_gemm_ref(qa, Ea, offsets, qw.reshape(E, N, K), Ew.reshape(E, N, K // 32), fa, fw)


def _check(got, ref, S, tol):
    err = np.abs(got.astype(np.float64) - ref)
    assert (err <= tol * S).all(), (err / np.maximum(S, 1e-300)).max()


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("sizes,N,K", [([0, 1, 130, 257], 200, 320), ([64, 64], 128, 64), ([5], 33, 128),
                                       ([300, 0, 0, 17, 129], 70, 1088)])
def test_grouped_mx_parity(ops, sizes, N, K, mode):
    print_case("grouped mx", sizes, N, K, "mode", mode)
    A, W, off, a, w = _setup(ops, sizes, N, K, seed=sum(sizes) + N + K)
    got = host(ops.qgemm_run_mx_grouped(a, w, dev(off), mode=mode))
    ref, S = _ref(A, W, off)
    _check(got, ref, S, MX_STOL if mode == 0 else MX_SCALED_STOL)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("K", [64, 256])
@pytest.mark.parametrize("sizes", [[700, 0, 1, 1023, 256, 513, 900, 710], [2100, 2571]])
def test_grouped_mx_large_tiles_uneven_experts(ops, sizes, K, mode):
    """Enough rows for the 256x256 tiles; experts of uneven sizes (one empty,
    several ragged), so tile-rows of one expert never take rows of the next.
    The exact mode takes the 128x128 tiles when the average expert has under
    2048 rows (the first layout) and the 256x256 ones otherwise. K = 64 is a
    single stage, fewer than the 4-stage ring the prologue fills."""
    N = 4352 - 32
    print_case("grouped mx large", sizes, N, K, "mode", mode)
    A, W, off, a, w = _setup(ops, sizes, N, K, seed=11 + mode)
    got = host(ops.qgemm_run_mx_grouped(a, w, dev(off), mode=mode))
    ref, S = _ref(A, W, off)
    _check(got, ref, S, MX_STOL if mode == 0 else MX_SCALED_STOL)


def test_grouped_mxfp4_scaled(ops):
    sizes = [40, 300, 0, 129]
    N, K = 150, 384
    print_case("grouped mxfp4", sizes, N, K)
    A, W, off, a, w = _setup(ops, sizes, N, K, fmt=E2M1, seed=5)
    got = host(ops.qgemm_run_mx_grouped(a, w, dev(off), mode=1))
    ref, S = _ref(A, W, off, fmt=E2M1)
    _check(got, ref, S, MX_STOL)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("fa,fw", [(E4M3, E2M1), (E2M1, E4M3), (E2M1, E2M1)])
@pytest.mark.parametrize("sizes,N,K", [([40, 300, 0, 129], 150, 384), ([700, 0, 1, 1023, 256, 513, 900, 710], 4320, 128)])
def test_grouped_mx_e2m1_pairs(ops, sizes, N, K, fa, fw, mode):
    """Pairs with an e2m1 operand: the exact mode (e2m1 codes converted to
    bf16 after the fragment read) within 1e-5 * S, the block-scaled matrix
    cores (each operand in its own layout and format code) within the scaled
    mode's e4m3 bound, 1e-5 * S for e2m1 x e2m1; the second case on 256 x 256
    tiles."""
    print_case("grouped mx e2m1 pairs", sizes, N, K, fa, fw, "mode", mode)
    A, W, off, a, w = _setup(ops, sizes, N, K, fmt=fa, wfmt=fw, seed=17 + K)
    got = host(ops.qgemm_run_mx_grouped(a, w, dev(off), mode=mode))
    ref, S = _ref(A, W, off, fmt=fa, wfmt=fw)
    _check(got, ref, S, MX_SCALED_STOL if mode == 1 and (fa, fw) != (E2M1, E2M1) else MX_STOL)


@pytest.mark.parametrize("fmt,mode", [(E4M3, 0), (E4M3, 1), (E2M1, 1)])
def test_grouped_mx_bias_per_expert(ops, fmt, mode):
    sizes = [33, 0, 70]
    N, K = 90, 256
    print_case("grouped mx bias", sizes, N, K, "fmt", fmt, "mode", mode)
    A, W, off, a, w = _setup(ops, sizes, N, K, fmt=fmt, seed=21)
    b = rng_for(99).normal(0.0, 10.0, size=(len(sizes), N)).astype(np.float32)
    got = host(ops.qgemm_run_mx_grouped(a, w, dev(off), mode=mode, bias=dev(b))).astype(np.float64)
    ref, S = _ref(A, W, off, fmt)
    expert = np.searchsorted(off, np.arange(len(got)), side="right") - 1
    ref = ref + b.astype(np.float64)[expert]
    tol = MX_SCALED_STOL if (fmt == E4M3 and mode == 1) else MX_STOL
    assert (np.abs(got - ref) <= tol * S + F32_RTOL * np.abs(ref)).all()


@pytest.mark.parametrize("fmt,mode", [(E4M3, 0), (E4M3, 1), (E2M1, 1)])
def test_grouped_rows_are_the_plain_gemm_of_each_expert(ops, fmt, mode):
    """Expert e's rows are the same bits as qgemm_run_mx on that expert's
    slice of A and its own weights: the same kernel body, the same
    matrix-core instructions in the same K order."""
    sizes = [90, 1, 0, 257, 40]
    N, K = 300, 512
    print_case("grouped vs plain", sizes, N, K, "fmt", fmt, "mode", mode)
    A, W, off, a, w = _setup(ops, sizes, N, K, fmt=fmt, seed=31)
    got = host(ops.qgemm_run_mx_grouped(a, w, dev(off), mode=mode))
    for e in range(len(sizes)):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        ae = ops.QuantizedRows(a.q[lo:hi], K, a.fmt, a.gran, None, None, a.mx_scales[lo:hi])
        plain = host(ops.qgemm_run_mx(ae, w.expert(e), mode=mode))
        assert np.array_equal(got[lo:hi].view(np.uint32), plain.view(np.uint32)), e


def test_grouped_single_expert_is_the_plain_gemm(ops):
    sizes = [777]
    N, K = 260, 192
    A, W, off, a, w = _setup(ops, sizes, N, K, seed=41)
    for mode in (0, 1):
        got = host(ops.qgemm_run_mx_grouped(a, w, dev(off), mode=mode))
        plain = host(ops.qgemm_run_mx(a, w.expert(0), mode=mode))
        assert np.array_equal(got.view(np.uint32), plain.view(np.uint32))


def test_grouped_rejects_unsupported_calls(ops):
    A, W, off, a, w = _setup(ops, [8, 8], 32, 96, seed=51)   # K % 64 != 0
    with pytest.raises(ops.QgemmError):
        ops.qgemm_run_mx_grouped(a, w, dev(off), mode=0)
