"""GPU checks of the measured-ceiling calls (include/qgemm_ceiling.h), which
the benchmark runs next to each GEMM: every instruction kind launches and
returns, the per-workgroup clock counters are plausible, the operation count
follows the launch shape, and neither call writes anything but its sink (and
the clock array)."""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ops():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_scaled_quantized_qgemm_amd import ops as _ops
    _ops.L.load()
    return _ops


def _guarded(n, dtype, fill):
    """A device buffer of n elements inside 64 guard elements on each side."""
    g = torch.full((n + 128,), fill, dtype=dtype, device="cuda")
    return g, g[64:64 + n]


@pytest.mark.parametrize("kind", [0, 1, 2, 3])
@pytest.mark.parametrize("waves", [1, 2])
def test_ceiling_mfma_runs_and_counts(ops, kind, waves):
    print(f"[case] ceiling mfma kind {kind} waves/SIMD {waves}", flush=True)
    gen = torch.Generator(device="cpu").manual_seed(7 + kind)
    a = torch.randint(0, 256, (ops.CEILING_A_BYTES,), dtype=torch.uint8, generator=gen).cuda()
    b = torch.randint(0, 256, (ops.CEILING_B_BYTES,), dtype=torch.uint8, generator=gen).cuda()
    trips = 64
    wg, n_ops = ops.qgemm_ceiling_mfma_shape(kind, waves, trips)
    assert wg == torch.cuda.get_device_properties(0).multi_processor_count
    per = {0: 2 * 16 * 16 * 64, 1: 2 * 32 * 32 * 64, 2: 2 * 32 * 32 * 64, 3: 2 * 32 * 32 * 16}[kind]
    assert n_ops == per * 8 * trips * 4 * waves * wg
    sg, sink = _guarded(1, torch.int32, -7)
    cg, clocks = _guarded(2 * wg, torch.int64, -1)
    ops.qgemm_ceiling_mfma(kind, waves, trips, a, b, sink, clocks)
    torch.cuda.synchronize()
    assert (sg[:64] == -7).all() and (sg[65:] == -7).all()
    assert (cg[:64] == -1).all() and (cg[64 + 2 * wg:] == -1).all()
    c = clocks.view(-1, 2).cpu()
    assert (c[:, 0] > 0).all() and (c[:, 1] > 0).all()
    # the loop issues 8 * trips instructions of at least 16 cycles each
    assert (c[:, 0] >= 8 * trips * 16).all()
    ghz = (c[:, 0].double() / (c[:, 1].double() / 1e8)).mean().item() / 1e9
    assert 0.3 < ghz < 4.0, ghz


@pytest.mark.parametrize("block", [16384, 65536, 1 << 20])
def test_ceiling_stream_reads_only(ops, block):
    print(f"[case] ceiling stream block {block}", flush=True)
    n = (3 << 20) + 4096  # a partial last block
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda")
    keep = src.clone()
    sg, sink = _guarded(1, torch.int32, -7)
    ops.qgemm_ceiling_stream(src, n, block, sink)
    ops.qgemm_ceiling_stream(src, 0, block, sink)
    torch.cuda.synchronize()
    assert torch.equal(src, keep)
    assert (sg[:64] == -7).all() and (sg[65:] == -7).all()
