"""The measured step under HIP graph capture.

bench.py captures K whole steps (quantize + GEMM + epilogue) into one graph
and replays it. Here one step of each kernel family is captured, replayed
several times with eager work and synchronizations between the replays
(the output overwritten, unrelated kernels launched), and every replay must
give the bits of the same calls launched eagerly; after new inputs are
copied into the captured buffers, a replay must give the eager result on
the new inputs. The launches record no allocation and no memset, so nothing
in the captured step depends on state the capture froze.
"""
import numpy as np
import pytest

from block_scaled_quantized_qgemm_amd.inputs import make_inputs
from conftest import print_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

REPLAYS = 3


@pytest.fixture(scope="module")
def ops():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_scaled_quantized_qgemm_amd import ops as _ops
    _ops.L.load()
    return _ops


def _bits(t):
    torch.cuda.synchronize()
    return t.view(torch.int32 if t.element_size() == 4 else torch.int16).cpu().numpy().copy()


def _check_graph(step, A, A_next, out):
    """step() writes `out` from the device buffer A. Eager reference, capture,
    replays with eager work between them, then a replay on new inputs."""
    step()
    ref = _bits(out)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm the stream outside the capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    for r in range(REPLAYS):
        out.fill_(float("nan") if out.is_floating_point() else -1)
        junk = torch.randn(1024, 1024, device="cuda") @ torch.randn(1024, 1024, device="cuda")
        torch.cuda.synchronize()
        g.replay()
        got = _bits(out)
        assert np.array_equal(got, ref), f"replay {r} differs from the eager step"
        del junk
    A.copy_(A_next)
    step()
    ref2 = _bits(out)
    out.zero_()
    torch.cuda.synchronize()
    g.replay()
    assert np.array_equal(_bits(out), ref2), "a replay on new inputs differs from the eager step"
    assert not np.array_equal(ref, ref2)


@pytest.mark.parametrize("fmt,gran,M", [(0, 1, 300), (1, 1, 300), (0, 0, 8), (1, 0, 257)])
def test_graph_int8_step(ops, fmt, gran, M):
    """Per-token and per-tensor (three launches through a workspace) int8 /
    uint8 steps on the tiled and the decode kernels."""
    print_case("graph int8", fmt, gran, M)
    K, N = 1000, 520
    A_np, W_np = make_inputs("c2_per_token", M=2 * M, K=K, N=N, seed=M + K)
    A = torch.from_numpy(A_np[:M]).cuda()
    A2 = torch.from_numpy(A_np[M:]).cuda()
    w = ops.qgemm_prepack_weights(torch.from_numpy(W_np).cuda(), 0, 1)
    q = ops.qgemm_quantize_rows(A, fmt, gran)
    need = ops.qgemm_workspace_bytes(M, K, fmt, gran)
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda") if need else None
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def step():
        ops.qgemm_quantize_rows(A, fmt, gran, out=q, workspace=ws)
        ops.qgemm_run(q, w, ops.OUT_F32, out=out)

    _check_graph(step, A, A2, out)


@pytest.mark.parametrize("mode,fa,fw", [(0, 2, 2), (1, 2, 2), (1, 4, 4), (1, 2, 4)])
def test_graph_mx_step(ops, mode, fa, fw):
    print_case("graph mx", mode, fa, fw)
    M, K, N = 300, 512, 260
    A_np, W_np = make_inputs("c5_mxfp8", M=2 * M, K=K, N=N, seed=7 + mode + fa + fw)
    A = torch.from_numpy(A_np[:M]).cuda()
    A2 = torch.from_numpy(A_np[M:]).cuda()
    w = ops.qgemm_prepack_weights(torch.from_numpy(W_np).cuda(), fw, ops.GRAN_BLOCK32)
    q = ops.qgemm_quantize_rows(A, fa, ops.GRAN_BLOCK32)
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def step():
        ops.qgemm_quantize_rows(A, fa, ops.GRAN_BLOCK32, out=q)
        ops.qgemm_run_mx(q, w, out=out, mode=mode)

    _check_graph(step, A, A2, out)


@pytest.mark.parametrize("M", [8, 300])
def test_graph_w4a8_step(ops, M):
    print_case("graph w4a8", M)
    K, N = 1024, 256
    A_np, W_np = make_inputs("c2_per_token", M=2 * M, K=K, N=N, seed=11 + M)
    A = torch.from_numpy(A_np[:M]).cuda()
    A2 = torch.from_numpy(A_np[M:]).cuda()
    w = ops.qgemm_prepack_weights(torch.from_numpy(W_np).cuda(), ops.FMT_INT4_SYM, ops.GRAN_GROUP64)
    q = ops.qgemm_quantize_rows(A, 0, 1)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def step():
        ops.qgemm_quantize_rows(A, 0, 1, out=q)
        ops.qgemm_run_w4a8(q, w, ops.OUT_BF16, out=out)

    _check_graph(step, A, A2, out)


@pytest.mark.parametrize("mode", [0, 1])
def test_graph_grouped_mx_step(ops, mode):
    print_case("graph grouped mx", mode)
    sizes = [300, 0, 41, 700]
    K, N = 256, 300
    E, M = len(sizes), sum(sizes)
    A_np, W_np = make_inputs("c5_mxfp8", M=2 * M, K=K, N=E * N, seed=23 + mode)
    A = torch.from_numpy(A_np[:M]).cuda()
    A2 = torch.from_numpy(A_np[M:]).cuda()
    w = ops.qgemm_prepack_experts(torch.from_numpy(W_np.reshape(E, N, K)).cuda(), ops.FMT_MXFP8_E4M3)
    off = torch.from_numpy(np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)).cuda()
    q = ops.qgemm_quantize_rows(A, ops.FMT_MXFP8_E4M3, ops.GRAN_BLOCK32)
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def step():
        ops.qgemm_quantize_rows(A, ops.FMT_MXFP8_E4M3, ops.GRAN_BLOCK32, out=q)
        ops.qgemm_run_mx_grouped(q, w, off, out=out, mode=mode)

    _check_graph(step, A, A2, out)
