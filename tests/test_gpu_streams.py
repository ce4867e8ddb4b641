"""Calls on several streams at once.

The library keeps no per-call device state (every buffer is the caller's;
the only library-owned device memory belongs to the allocation-free
quantizer, whose concurrent use is documented as racing), so the same calls
enqueued on two streams without any synchronization between them, their
kernels free to overlap, must give the bits the calls give one after
another. Each kernel family is covered: the row quantizers, the fused
RMSNorm quantizer, the int8 tiled / one-tile-per-CU / decode GEMMs, the MX
GEMM in both modes, the grouped MX GEMM and W4A8.
"""
import numpy as np
import pytest

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


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _bits(t):
    """The tensor's bytes (bf16 viewed as int16 first: numpy has no bfloat16)."""
    x = t.contiguous()
    if x.dtype == torch.bfloat16:
        x = x.view(torch.int16)
    return x.cpu().numpy().view(np.uint8).copy()


def _calls(ops):
    """(name, fn) pairs; fn(stream) enqueues one call on `stream` and returns
    the tensors it writes (allocated before the call, on the caller's side)."""
    calls = []

    A2, W2 = make_inputs("c2_per_token", M=300, K=1024, N=520, seed=1)
    A3, W3 = make_inputs("c3_asym_uint8", M=2048, K=512, N=11008, seed=2)
    A4, W4 = make_inputs("c4_decode", M=8, K=4096, N=1000, seed=3)
    A5, W5 = make_inputs("c5_mxfp8", M=600, K=512, N=700, seed=4)
    x2, x3, x4, x5 = _dev(A2), _dev(A3), _dev(A4), _dev(A5)
    gamma = _dev(np.linspace(0.5, 1.5, 1024).astype(np.float32))
    w2 = ops.qgemm_prepack_weights(_dev(W2), ops.FMT_INT8_SYM, ops.GRAN_ROW)
    w3 = ops.qgemm_prepack_weights(_dev(W3), ops.FMT_INT8_SYM, ops.GRAN_ROW)
    w4 = ops.qgemm_prepack_weights(_dev(W4), ops.FMT_INT8_SYM, ops.GRAN_ROW)
    w4i = ops.qgemm_prepack_weights(_dev(W4), ops.FMT_INT4_SYM, ops.GRAN_GROUP64)
    w5 = ops.qgemm_prepack_weights(_dev(W5), ops.FMT_MXFP8_E4M3, ops.GRAN_BLOCK32)
    We = make_inputs("c5_mxfp8", M=1, K=256, N=4 * 200, seed=5)[1].reshape(4, 200, 256)
    we = ops.qgemm_prepack_experts(_dev(We), ops.FMT_MXFP8_E4M3)
    Ae = make_inputs("c5_mxfp8", M=500, K=256, N=1, seed=6)[0]
    off = _dev(np.array([0, 130, 130, 371, 500], np.int64))
    ae = ops.qgemm_quantize_rows(_dev(Ae), ops.FMT_MXFP8_E4M3, ops.GRAN_BLOCK32)
    a2 = ops.qgemm_quantize_rows(x2, ops.FMT_INT8_SYM, ops.GRAN_ROW)
    a3 = ops.qgemm_quantize_rows(x3, ops.FMT_UINT8_ASYM, ops.GRAN_ROW)
    a4 = ops.qgemm_quantize_rows(x4, ops.FMT_INT8_SYM, ops.GRAN_ROW)
    a5 = ops.qgemm_quantize_rows(x5, ops.FMT_MXFP8_E4M3, ops.GRAN_BLOCK32)
    torch.cuda.synchronize()

    def quant(x, fmt, gran):
        def f(s):
            r = ops.qgemm_quantize_rows(x, fmt, gran, stream=s)
            return [r.q] + [t for t in (r.scales, r.zero_points, r.mx_scales) if t is not None]
        return f

    def norm(s):
        r = ops.qgemm_rmsnorm_quantize_rows(x2, gamma, 1e-6, ops.FMT_UINT8_ASYM, stream=s)
        return [r.q, r.scales, r.zero_points]

    def gemm(a, w, out_type):
        return lambda s: [ops.qgemm_run(a, w, out_type, stream=s)]

    calls += [("quantize int8", quant(x2, ops.FMT_INT8_SYM, ops.GRAN_ROW)),
              ("quantize uint8 per tensor", quant(x3, ops.FMT_UINT8_ASYM, ops.GRAN_TENSOR)),
              ("quantize mxfp8", quant(x5, ops.FMT_MXFP8_E4M3, ops.GRAN_BLOCK32)),
              ("quantize mxfp4", quant(x5, ops.FMT_MXFP4_E2M1, ops.GRAN_BLOCK32)),
              ("rmsnorm quantize", norm),
              ("gemm tiled", gemm(a2, w2, ops.OUT_F32)),
              ("gemm one tile per CU", gemm(a3, w3, ops.OUT_BF16)),
              ("gemm decode", gemm(a4, w4, ops.OUT_F32)),
              ("gemm mx exact", lambda s: [ops.qgemm_run_mx(a5, w5, mode=ops.MX_EXACT, stream=s)]),
              ("gemm mx scaled", lambda s: [ops.qgemm_run_mx(a5, w5, mode=ops.MX_SCALED_MFMA, stream=s)]),
              ("gemm mx grouped", lambda s: [ops.qgemm_run_mx_grouped(ae, we, off, mode=ops.MX_EXACT, stream=s)]),
              ("gemm w4a8", lambda s: [ops.qgemm_run_w4a8(a4, w4i, ops.OUT_F32, stream=s)])]
    return calls


def test_calls_on_two_streams_at_once_match_one_after_another(ops):
    print_case("two streams")
    calls = _calls(ops)
    main = torch.cuda.current_stream()
    refs = []
    for name, fn in calls:
        outs = fn(main)
        torch.cuda.synchronize()
        refs.append([_bits(t) for t in outs])
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(main)
    for rep in range(3):
        got = []
        # interleave: call i on stream (i + rep) % 2, nothing waits on anything
        for i, (name, fn) in enumerate(calls):
            s = streams[(i + rep) % 2]
            with torch.cuda.stream(s):
                got.append(fn(s))
        torch.cuda.synchronize()
        for (name, _), ref, outs in zip(calls, refs, got):
            for k, (r, t) in enumerate(zip(ref, outs)):
                assert np.array_equal(r, _bits(t)), f"{name} output {k} differs on rep {rep}"
