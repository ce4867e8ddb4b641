"""Benchmark of the quantized linear layer on one MI355X.

A step is one pass of the whole hot path over one batch: quantize the float32
activations (qgemm_quantize_rows) and run the GEMM with its fused epilogue
(qgemm_run / qgemm_run_mx, qgemm_run_w4a8 with --w4a8, or qgemm_run_mx_grouped for the
grouped MoE workload). Weights are prepared once beforehand (offline, as
on the pages) and every input is resident in HBM before the timed region.
Activation / weight / output buffers rotate over enough copies that the
256 MB Infinity Cache cannot hold the working set.

Prints one JSON line. Default workload: the large-M GEMM, 2048 tokens x
K=4096 x N=11008 with per-token asymmetric uint8 activations (zero point),
per-channel int8 weights and bfloat16 output; the same line carries, under
"secondary", the decode-shaped GEMM (8 x 4096 x 14336, HBM GB/s) and the
MXFP8 GEMM (8192^3) in both MX modes, each with its own roofline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "quantized GEMM TOPS (quant+GEMM+epilogue) and % of MFMA peak; decode-M HBM GB/s"

PEAK_INT8_TOPS = 5000.0   # dense int8 MFMA, MI355X
PEAK_FP8_TFLOPS = 5000.0  # dense fp8 / MXFP8 MFMA, MI355X
PEAK_BF16_TFLOPS = 2500.0  # dense bf16 MFMA, MI355X (the exact MX mode runs on these)
PEAK_FP4_TFLOPS = 10100.0  # dense fp4 / fp6 MFMA, MI355X
PEAK_HBM_GBS = 8000.0     # HBM3E
MALL_BYTES = 256 << 20


def mx_peak(fp4, wfp4):
    """Dense matrix-core peak of an MX contraction: MXFP4 x MXFP4 runs at the
    fp4 rate, any pair with an e4m3 operand at the fp8 rate. Both MX modes are
    priced against it (the exact mode's bf16 matrix cores reach half of it)."""
    return PEAK_FP4_TFLOPS if fp4 and wfp4 else PEAK_FP8_TFLOPS
MOE = ("c6_moe_mxfp8",)   # grouped (MoE) workloads: bench.main_grouped

# name -> (activation format, granularity, weight granularity, output type, headline unit)
WORKLOADS = {
    "c1_tiny": ("int8_sym", "tensor", "channel", "f32", "TOPS"),
    "c2_per_token": ("int8_sym", "row", "channel", "f32", "TOPS"),
    "c3_asym_uint8": ("uint8_asym", "row", "channel", "bf16", "TOPS"),
    "c4_decode": ("int8_sym", "row", "channel", "f32", "GB/s"),
    "c5_mxfp8": ("mxfp8", "block32", "block32", "f32", "TFLOPS"),
    "c6_moe_mxfp8": ("mxfp8", "block32", "block32", "f32", "TFLOPS"),
}
DESCRIPTION = {
    "c1_tiny": "64x256x64 per-tensor int8 A, per-channel int8 W, fp32 out",
    "c2_per_token": "512x4096x4096 per-token int8 A (outlier channels), per-channel int8 W, fp32 out",
    "c3_asym_uint8": "2048x4096x11008 per-token asymmetric uint8 A with zero point, per-channel int8 W, bf16 out",
    "c4_decode": "8x4096x14336 decode-shaped, per-token int8 A quantized on the fly, prepacked int8 W, fp32 out",
    "c5_mxfp8": "8192x8192x8192 MXFP8 (e4m3 + E8M0 per 32 K) A and W, fp32 out",
    "c6_moe_mxfp8": "grouped (MoE) MXFP8: 8 experts, 8192 routed rows of K=4096 split unevenly over them, "
                    "N=4096 per expert, fp32 out",
}


MX_PAIRS = ["e4m3", "e2m1", "e4m3xe2m1", "e2m1xe4m3"]
MX_NAMES = {"e4m3": "fp8-e4m3", "e2m1": "fp4-e2m1"}


def mx_pair(arg):
    """--mx-format: one element format for A and W, or 'AxW'. Returns
    (A is e2m1, W is e2m1)."""
    fa, _, fw = arg.partition("x")
    return fa == "e2m1", (fw or fa) == "e2m1"


def mx_tags(arg):
    """dtype string, workload note and profile-name suffix of an MX format pair."""
    fa, _, fw = arg.partition("x")
    fw = fw or fa
    dtype = MX_NAMES[fa] if fa == fw else f"{MX_NAMES[fa]} x {MX_NAMES[fw]}"
    note = "" if arg == "e4m3" else (" -- MXFP4: e2m1 A and W, E8M0 per 32" if arg == "e2m1"
                                     else f" -- {fa} A x {fw} W, E8M0 per 32")
    suffix = "" if arg == "e4m3" else ("_fp4" if arg == "e2m1" else "_" + arg)
    return dtype, note, suffix


def algorithmic(name, M, K, N, w4a8=False, fp4=False, wfp4=None):
    """Ops and algorithmic bytes: whole step, and the GEMM kernel alone.

    Whole step: float32 A read once, W codes + per-channel scales/column sums
    (or E8M0 scales, or int4 codes + float32 scales per group of 64 K) read
    once, output written once. GEMM kernel: the same with A as 1-byte codes
    plus its per-row scale (and zero point).
    """
    act, _, _, out, _ = WORKLOADS[name]
    ob = {"f32": 4, "bf16": 2}[out]
    ops = 2.0 * M * N * K
    if w4a8:
        w = N * K / 2 + 4 * N * math.ceil(K / 64)
        a_codes = M * K + 4 * M
    elif act == "mxfp8":
        cb_a = 0.5 if fp4 else 1.0  # code bytes per element: e2m1 packs two per byte
        cb_w = 0.5 if (fp4 if wfp4 is None else wfp4) else 1.0
        w = cb_w * N * K + N * (K // 32)
        a_codes = cb_a * M * K + M * (K // 32)
    else:
        w = N * K + 8 * N
        a_codes = M * K + 8 * M
    step_bytes = 4.0 * M * K + w + ob * M * N
    gemm_bytes = a_codes + w + ob * M * N
    return ops, step_bytes, gemm_bytes


def source_digest(name):
    """Digest of the code of the GEMM kernels a workload's name selects (int4
    weights, MX, or int8): their sources with comments and whitespace
    removed, so only a code change makes the stored counter figures stale."""
    import re
    h = hashlib.sha256()
    if name.endswith("_w4a8"):
        srcs = ("gemm_w4a8.hip",)
    elif "mxfp" in name:
        srcs = ("gemm_mx_dma.hip",)
    else:
        srcs = ("gemm.hip", "gemm_i8_wide.hip")
    for f in srcs + ("common.hpp", "kernels.hpp"):
        with open(os.path.join(ROOT, "block_scaled_quantized_qgemm_amd", "csrc", f)) as fh:
            code = fh.read()
        code = re.sub(r"/\*.*?\*/", " ", code, flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        h.update("".join(code.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(name):
    """HBM bytes per GEMM launch from committed rocprofv3 counter runs, or None.

    profiles/traffic_<workload>.json holds FETCH_SIZE / WRITE_SIZE per dispatch
    (KiB), the copy-kernel calibration factor and the digest of the GEMM
    sources they were taken with; a stale digest means the kernel changed
    since, and the figure is not reported.
    """
    p = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("source_digest") != source_digest(name):
        return None
    return float(t["hbm_bytes_per_launch"])


def host_cpu():
    """The host's CPU model (from /proc/cpuinfo) and its logical CPU count."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "host_logical_cpus": os.cpu_count()}


def cpu_baseline(name, A, W, budget_s=10.0, fused=None, w4a8=False, fp4=False, wfp4=None):
    """The oracle, untuned, on a bounded sample of the same workload.
    fused: (gamma, eps, bias) to time the RMSNorm-fused step with a bias;
    w4a8: int4 per-group-64 weights and the per-group GEMM."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
    act, gran, _, _, _ = WORKLOADS[name]
    M, K = A.shape
    N = W.shape[0]
    if act == "mxfp8":
        rows = min(M, 64)
        wfp4 = fp4 if wfp4 is None else wfp4
        quant = O.quantize_mxfp4 if fp4 else O.quantize_mx
        fmt = "e2m1" if fp4 else "e4m3"
        Wq, We = (O.quantize_mxfp4 if wfp4 else O.quantize_mx)(W)   # offline weight preparation, untimed
        Wd = O.mx_dequantize(Wq, We, "e2m1" if wfp4 else "e4m3")
        sample = f"{rows} of {M} rows of A against all of W (W prepared outside the timing)"
    elif w4a8:
        rows = min(M, 256)
        Wq4, Ws4 = O.quantize_int4_groups(W)
        sample = f"{rows} of {M} rows of A against all of W (W prepared outside the timing)"
    else:
        rows = min(M, 256)
        Wq, Ws, _ = O.prepare_weights_int8(W, per_channel=True)
        sample = f"{rows} of {M} rows of A against all of W (W prepared outside the timing)"
    As = A[:rows]
    reps, t0 = 0, time.perf_counter()
    while True:
        if act == "mxfp8":
            qa, Ea = quant(As)
            _ = O.mx_dequantize(qa, Ea, fmt) @ Wd.T
        elif w4a8:
            if fused is not None:
                qa, sa = O.rmsnorm_quantize(As, fused[0], fused[1], act="sym_row")[:2]
            else:
                qa, sa = O.quantize_sym_int8(As, per_row=(gran == "row"))
            y, _ = O.w4a8_gemm(qa, sa, Wq4, Ws4)
            if fused is not None:
                y = y + fused[2].astype(np.float64)[None, :]
        else:
            if fused is not None:
                r = O.rmsnorm_quantize(As, fused[0], fused[1], act="asym_row" if act == "uint8_asym" else "sym_row")
                qa, sa, za = r[0], r[1], (r[2] if act == "uint8_asym" else 0)
            elif act == "uint8_asym":
                qa, sa, za = O.quantize_asym_uint8(As, per_row=(gran == "row"))
            else:
                qa, sa = O.quantize_sym_int8(As, per_row=(gran == "row"))
                za = 0
            C = O.int_gemm(qa, za, Wq)
            _ = O.add_bias(O.epilogue(C, sa, Ws), None if fused is None else fused[2])
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 1000:
            break
    ops = 2.0 * rows * K * N * reps
    unit = "GB/s" if WORKLOADS[name][4] == "GB/s" else WORKLOADS[name][4]
    if unit == "GB/s":
        _, step_bytes, _ = algorithmic(name, rows, K, N, w4a8, fp4, wfp4)
        value = step_bytes * reps / el / 1e9
    else:
        value = ops / el / 1e12
    return {"value": value, "unit": unit, "cores": int(cores), "kind": "oracle",
            "sample": f"{sample}; {reps} passes in {el:.1f} s", **host_cpu(),
            "threads": "cores = the BLAS thread pool the oracle's matrix products ran on"}


def timed(fn, steps, eager, repeats=None):
    """Milliseconds per call of fn(i), i = 0 .. steps-1, on the current stream,
    and the host wall time. The calls are captured once into a HIP graph and
    replayed (eager: launched from Python), bracketed by events on the stream.
    With a list `repeats`, four further passes are each timed the same way
    afterwards, and every pass's ms per call (the measurement first) is put in
    it: the others only describe the measurement's spread."""
    import torch
    if eager:
        run = lambda: [fn(i) for i in range(steps)]  # noqa: E731
    else:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(steps):
                fn(i)
        run = graph.replay
        run()  # one untimed replay
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    run()
    stop.record()
    torch.cuda.synchronize()
    ms, wall = start.elapsed_time(stop) / steps, time.perf_counter() - t0
    if repeats is not None:
        repeats.append(ms)
        for _ in range(4):
            start.record()
            run()
            stop.record()
            torch.cuda.synchronize()
            repeats.append(start.elapsed_time(stop) / steps)
    return ms, wall


def spread(ms_list):
    """min / median / mean of per-pass ms per step."""
    v = sorted(ms_list)
    return {"passes": len(v), "min_ms": v[0], "median_ms": v[len(v) // 2], "mean_ms": sum(v) / len(v)}


def calibration_copy(mib, dev):
    """A plain device copy of known size after the timed region (its counters
    calibrate the GEMM's FETCH_SIZE / WRITE_SIZE)."""
    import torch
    nb = mib << 20
    src = torch.ones(nb // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def _ceiling_bytes(t, n):
    """The first n bytes of a device tensor (repeated when it is shorter)."""
    import torch
    b = t.reshape(-1).view(torch.uint8)
    if b.numel() < n:
        b = b.repeat((n + b.numel() - 1) // b.numel())
    return b[:n].contiguous()


def mfma_ceiling(kind, a_src, b_src, waves_per_simd=2, target_ms=4.0, reps=5):
    """Measured issue rate of a GEMM kernel's matrix-core instruction
    (qgemm_ceiling_mfma): one workgroup per CU with waves_per_simd waves on
    every SIMD, the workload's own code bytes as operands (the part is
    power-limited and its clock depends on the operand bits), nothing else in
    the loop. Launches of about target_ms, after about 20 ms of warm-up so the
    clock settles. Returns the rate in T(FL)OP/s and the shader clock (GHz)
    the part held, from the probe's own cycle and real-time counters."""
    import torch
    from block_scaled_quantized_qgemm_amd import ops
    a = _ceiling_bytes(a_src, ops.CEILING_A_BYTES)
    b = _ceiling_bytes(b_src, ops.CEILING_B_BYTES)
    sink = torch.zeros(1, dtype=torch.int32, device=a.device)
    trips = 256
    wg, _ = ops.qgemm_ceiling_mfma_shape(kind, waves_per_simd, trips)
    clocks = torch.zeros(2 * wg, dtype=torch.int64, device=a.device)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def run(t, n):
        torch.cuda.synchronize()
        start.record()
        for _ in range(n):
            ops.qgemm_ceiling_mfma(kind, waves_per_simd, t, a, b, sink, clocks)
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / n

    ms = run(trips, 2)
    trips = max(1, min(1 << 24, int(trips * target_ms / max(ms, 1e-3))))
    run(trips, 5)
    ms = run(trips, reps)
    _, n_ops = ops.qgemm_ceiling_mfma_shape(kind, waves_per_simd, trips)
    c = clocks.view(-1, 2).double().cpu()
    ghz = float((c[:, 0] / (c[:, 1] / 1e8)).mean() / 1e9)
    return n_ops / (ms * 1e-3) / 1e12, ghz


CEILING_NAMES = {0: "v_mfma_i32_16x16x64_i8", 1: "v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3)",
                 2: "v_mfma_scale_f32_32x32x64_f8f6f4 (e2m1)", 3: "v_mfma_f32_32x32x16_bf16"}


def add_mfma_ceiling(roof, kind, a_src, b_src):
    """Put the measured matrix-core ceiling of the GEMM's instruction next to
    the published peak in a roofline."""
    rate, ghz = mfma_ceiling(kind, a_src, b_src)
    roof["measured_ceiling"] = {
        "value": rate, "unit": roof["unit"], "clock_ghz": ghz,
        "probe": f"qgemm_ceiling_mfma: {CEILING_NAMES[kind]} back to back, 8 independent accumulators, "
                 "2 waves per SIMD, one workgroup per CU, operands from this workload's codes"}
    roof["frac_of_measured_ceiling"] = roof["achieved"] / rate


def add_stream_ceiling(roof, bufs, steps):
    """Put the measured HBM read rate of a plain stream over the same rotating
    weight buffers (qgemm_ceiling_stream, best of four block sizes) next to
    the published peak in a roofline."""
    import torch
    from block_scaled_quantized_qgemm_amd import ops
    nbytes = min(b.numel() for b in bufs) // 16 * 16
    sink = torch.zeros(1, dtype=torch.int32, device=bufs[0].device)
    best = None
    for bb in (32768, 65536, 131072, 262144):
        ms, _ = timed(lambda i: ops.qgemm_ceiling_stream(bufs[i % len(bufs)], nbytes, bb, sink), steps, False)
        rate = nbytes / (ms * 1e-3) / 1e9
        if best is None or rate > best[0]:
            best = (rate, bb)
    roof["measured_ceiling"] = {
        "value": best[0], "unit": "GB/s",
        "probe": f"qgemm_ceiling_stream: one plain read of the {nbytes / 1e6:.1f} MB prepared weight buffer per "
                 f"launch, {best[1] // 1024} KB per workgroup, over the same rotating buffers"}
    roof["frac_of_measured_ceiling"] = roof["achieved"] / best[0]


def ceiling_kind(ops, act, mx_mode, fp4, wfp4):
    """The matrix-core instruction a workload's GEMM kernel issues."""
    if act != "mxfp8":
        return ops.CEIL_I8
    if mx_mode == ops.MX_EXACT:
        return ops.CEIL_BF16
    return ops.CEIL_F4_SCALED if fp4 and wfp4 else ops.CEIL_F8_SCALED


def cpu_baseline_grouped(A, W, sizes, fp4, budget_s=10.0, wfp4=None):
    """The oracle's grouped reference, untuned, on a bounded sample: up to 16
    rows of every expert against the first 1024 output columns of its weights
    (prepared outside the timing)."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
    wfp4 = fp4 if wfp4 is None else wfp4
    quant = O.quantize_mxfp4 if fp4 else O.quantize_mx
    f = "e2m1" if fp4 else "e4m3"
    fw = "e2m1" if wfp4 else "e4m3"
    W = np.ascontiguousarray(W[:, :1024])
    E, N, K = W.shape
    qw, Ew = (O.quantize_mxfp4 if wfp4 else O.quantize_mx)(W.reshape(E * N, K))
    qw, Ew = qw.reshape(E, N, K), Ew.reshape(E, N, K // 32)
    off = np.concatenate([[0], np.cumsum(sizes)])
    take = [np.arange(off[e], off[e] + min(16, sizes[e])) for e in range(E)]
    As = A[np.concatenate(take)]
    offs = np.concatenate([[0], np.cumsum([len(t) for t in take])])
    reps, t0 = 0, time.perf_counter()
    while True:
        qa, Ea = quant(As)
        O.mx_grouped_gemm_ref(qa, Ea, offs, qw, Ew, f, fw)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 1000:
            break
    return {"value": 2.0 * len(As) * N * K * reps / el / 1e12, "unit": "TFLOPS", "cores": int(cores),
            "kind": "oracle", "sample": f"up to 16 rows of each expert ({len(As)} rows) against {N} columns of its weights "
                                        f"(weights prepared outside the timing); {reps} passes in {el:.1f} s",
            **host_cpu(), "threads": "cores = the BLAS thread pool the oracle's matrix products ran on"}


def main_grouped(args):
    """The grouped (MoE) MX workload: quantize the routed rows, then one
    grouped GEMM over all experts."""
    import numpy as np
    import torch
    from block_scaled_quantized_qgemm_amd import ops
    from block_scaled_quantized_qgemm_amd.inputs import make_moe_inputs

    name = args.workload
    fp4, wfp4 = mx_pair(args.mx_format)
    dtype, note, suffix = mx_tags(args.mx_format)
    mx_mode = ops.MX_EXACT if args.mx_mode == "exact" else ops.MX_SCALED_MFMA
    if args.fused or args.w4a8:
        print("bench.py: --fused and --w4a8 do not apply to the grouped workload", file=sys.stderr)
        sys.exit(2)
    fmt = ops.FMT_MXFP4_E2M1 if fp4 else ops.FMT_MXFP8_E4M3
    wfmt = ops.FMT_MXFP4_E2M1 if wfp4 else ops.FMT_MXFP8_E4M3
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    A_np, W_np, sizes = make_moe_inputs(name)
    E, N, K = W_np.shape
    M = A_np.shape[0]
    A0 = torch.from_numpy(A_np).to(dev)
    W0 = torch.from_numpy(W_np).to(dev)
    w0 = ops.qgemm_prepack_experts(W0, wfmt)
    del W0
    offsets = torch.from_numpy(np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)).to(dev)
    torch.cuda.synchronize()

    ops_count = 2.0 * M * N * K
    cb = 0.5 if wfp4 else 1.0
    w_bytes = E * (cb * N * K + N * (K // 32))
    step_bytes = 4.0 * M * K + w_bytes + 4.0 * M * N
    set_bytes = A0.numel() * 4 + w0.packed.numel() + M * N * 4 + M * K
    nsets = args.rotate or max(1, min(64, math.ceil(3 * MALL_BYTES / set_bytes)))
    sets = []
    for i in range(nsets):
        Ai = A0 if i == 0 else A0.clone()
        wi = w0 if i == 0 else ops.PackedExperts(w0.packed.clone(), w0.desc, E)
        qi = ops.qgemm_quantize_rows(Ai, fmt, ops.GRAN_BLOCK32)
        oi = torch.empty((M, N), dtype=torch.float32, device=dev)
        sets.append((Ai, wi, qi, oi))
    torch.cuda.synchronize()

    def quantize(i):
        Ai, wi, qi, oi = sets[i % nsets]
        ops.qgemm_quantize_rows(Ai, fmt, ops.GRAN_BLOCK32, out=qi)

    def gemm(i):
        Ai, wi, qi, oi = sets[i % nsets]
        ops.qgemm_run_mx_grouped(qi, wi, offsets, out=oi, mode=mx_mode)

    def step(i):
        quantize(i)
        gemm(i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ms_per_step, wall = timed(step, args.steps, args.eager)
    gemm_ms, _ = timed(gemm, args.steps, args.eager)
    peak = mx_peak(fp4, wfp4)
    roof = {"bound": "mfma", "achieved": ops_count / (gemm_ms * 1e-3) / 1e12, "peak": peak, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["step_frac"] = ops_count / (ms_per_step * 1e-3) / 1e12 / peak
    if mx_mode == ops.MX_EXACT:
        roof["exact_mode_ceiling_frac"] = PEAK_BF16_TFLOPS / peak
        roof["frac_of_bf16_cores"] = roof["achieved"] / PEAK_BF16_TFLOPS
    roof["traffic"] = measured_traffic(name + suffix + ("_scaled" if mx_mode != ops.MX_EXACT else ""))
    if not args.no_ceiling:
        add_mfma_ceiling(roof, ceiling_kind(ops, "mxfp8", mx_mode, fp4, wfp4), sets[0][2].q, w0.packed)
    line = {
        "metric": METRIC, "value": ops_count / (ms_per_step * 1e-3) / 1e12, "unit": "TFLOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic (seeded generator with the workload's shapes and distributions)",
        "config": {"workload": f"{name}: {DESCRIPTION[name]} ({args.mx_mode} mode)" + note,
                   "experts": E, "M_total": M, "K": K, "N": N, "rows_per_expert": [int(x) for x in sizes],
                   "rotating_buffer_sets": nsets, "gemm_ms": gemm_ms,
                   "launch": "eager" if args.eager else "hip graph (K steps captured, replayed once)",
                   "step_hbm_gbs": step_bytes / (ms_per_step * 1e-3) / 1e9},
        "roofline": roof,
    }
    if args.calibration_copy:
        calibration_copy(args.calibration_copy, dev)
    print(f"[bench] {name}: {ms_per_step * 1e3:.2f} us/step, gemm {gemm_ms * 1e3:.2f} us, "
          f"wall {wall:.3f} s for {args.steps} steps", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_grouped(A_np, W_np, sizes, fp4, args.cpu_budget, wfp4)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c3_asym_uint8", choices=sorted(WORKLOADS))
    ap.add_argument("--no-secondary", action="store_true",
                    help="measure the chosen workload only (by default the large-M headline also carries the "
                         "decode-shaped and the MXFP8 workloads under 'secondary')")
    ap.add_argument("--rotate", type=int, default=0, help="buffer sets (0: enough to exceed the MALL 3x)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the measured ceilings (matrix-core issue rate of the GEMM's instruction on the "
                         "workload's codes, or a plain HBM stream over the same weight buffers)")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--calibration-copy", type=int, default=0, metavar="MIB",
                    help="after the timed region, copy MIB MiB device-to-device: a plain copy of known size "
                         "whose FETCH_SIZE / WRITE_SIZE counters calibrate the GEMM's traffic")
    ap.add_argument("--fused", action="store_true",
                    help="int8 per-token workloads: RMSNorm fused with the quantizer "
                         "(qgemm_rmsnorm_quantize_rows) and a float32 bias in the GEMM epilogue")
    ap.add_argument("--eager", action="store_true",
                    help="launch every step from Python instead of replaying a captured HIP graph")
    ap.add_argument("--w4a8", action="store_true",
                    help="symmetric int8 workloads: int4 weights with a float32 scale per group of 64 K "
                         "(qgemm_run_w4a8)")
    ap.add_argument("--mx-format", default="e4m3", choices=MX_PAIRS,
                    help="MX workloads: element format of activations and weights (e2m1: MXFP4), or a "
                         "pair 'AxW' (e4m3xe2m1: e4m3 activations, e2m1 weights)")
    ap.add_argument("--mx-mode", default="exact", choices=["exact", "scaled-mfma"],
                    help="MX workload: exact products (bf16 matrix cores) or block-scaled fp8 matrix cores")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the benchmark measures one GPU; the library has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)
    if args.workload in MOE:
        return main_grouped(args)

    line = measure(args, args.workload, args.mx_mode, not args.no_cpu_baseline)
    if (not args.no_secondary and args.workload == "c3_asym_uint8" and not (args.fused or args.w4a8)):
        import torch
        sec = {}
        for key, wl, mode in (("c4_decode", "c4_decode", "exact"),
                              ("c5_mxfp8_exact", "c5_mxfp8", "exact"),
                              ("c5_mxfp8_scaled", "c5_mxfp8", "scaled-mfma")):
            torch.cuda.empty_cache()
            sub = argparse.Namespace(**{**vars(args), "mx_format": "e4m3", "rotate": 0, "calibration_copy": 0})
            l2 = measure(sub, wl, mode, False)
            sec[key] = {"workload": l2["config"]["workload"], "value": l2["value"], "unit": l2["unit"],
                        "ms_per_step": l2["ms_per_step"], "gemm_ms": l2["config"]["gemm_ms"],
                        "step_spread": l2["config"]["step_spread"], "quantize": l2["config"]["quantize"],
                        "prepack_ms": l2["config"]["prepack_ms"], "dtype": l2["dtype"], "roofline": l2["roofline"]}
        line["secondary"] = sec
    print(json.dumps(line), flush=True)


def measure(args, name, mx_mode_arg, with_cpu):
    """Time one workload (K whole steps, then K GEMM launches) and return its
    JSON line (without printing it)."""
    import numpy as np
    import torch
    from block_scaled_quantized_qgemm_amd import ops
    from block_scaled_quantized_qgemm_amd.inputs import make_inputs, WORKLOADS as SHAPES

    act, gran, wgran, out, unit = WORKLOADS[name]
    if args.fused and (act == "mxfp8" or gran != "row"):
        print("bench.py: --fused applies to the per-token int8 / uint8 workloads", file=sys.stderr)
        sys.exit(2)
    if args.w4a8 and act != "int8_sym":
        print("bench.py: --w4a8 applies to the symmetric int8 workloads", file=sys.stderr)
        sys.exit(2)
    fp4, wfp4 = mx_pair(args.mx_format)
    mx_dtype, mx_note, mx_suffix = mx_tags(args.mx_format)
    if args.mx_format != "e4m3" and act != "mxfp8":
        print("bench.py: --mx-format applies to the MX workloads", file=sys.stderr)
        sys.exit(2)
    M, K, N, _, _ = SHAPES[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    A_np, W_np = make_inputs(name)
    fmt = {"int8_sym": ops.FMT_INT8_SYM, "uint8_asym": ops.FMT_UINT8_ASYM,
           "mxfp8": ops.FMT_MXFP4_E2M1 if fp4 else ops.FMT_MXFP8_E4M3}[act]
    agr = {"tensor": ops.GRAN_TENSOR, "row": ops.GRAN_ROW, "block32": ops.GRAN_BLOCK32}[gran]
    wgr = {"tensor": ops.GRAN_TENSOR, "channel": ops.GRAN_ROW, "block32": ops.GRAN_BLOCK32}[wgran]
    otype = {"f32": ops.OUT_F32, "bf16": ops.OUT_BF16}[out]
    odt = {"f32": torch.float32, "bf16": torch.bfloat16}[out]

    mx_mode = ops.MX_EXACT if mx_mode_arg == "exact" else ops.MX_SCALED_MFMA
    A0 = torch.from_numpy(A_np).to(dev)
    W0 = torch.from_numpy(W_np).to(dev)
    wfmt = ((ops.FMT_MXFP4_E2M1 if wfp4 else ops.FMT_MXFP8_E4M3) if act == "mxfp8"
            else ops.FMT_INT8_SYM)   # int8 weights are symmetric
    if args.w4a8:
        wfmt, wgr = ops.FMT_INT4_SYM, ops.GRAN_GROUP64
    w0 = ops.qgemm_prepack_weights(W0, wfmt, wgr)
    torch.cuda.synchronize()
    # weight preparation is offline; one warm call timed with events, reported apart
    pstart, pstop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pstart.record()
    ops.qgemm_prepack_weights(W0, wfmt, wgr)
    pstop.record()
    torch.cuda.synchronize()
    prepack_ms = pstart.elapsed_time(pstop)
    ops_count, step_bytes, gemm_bytes = algorithmic(name, M, K, N, args.w4a8, fp4, wfp4)
    if args.fused:  # the norm weight and the bias are read once more
        step_bytes += 4 * K + 4 * N
        gemm_bytes += 4 * N
    set_bytes = A0.numel() * 4 + w0.packed.numel() + M * ((N + 7) // 8 * 8) * (4 if out == "f32" else 2) + M * K
    nsets = args.rotate or max(1, min(64, math.ceil(3 * MALL_BYTES / set_bytes)))

    # rotation sets: copies of A (float32), prepared W, quantized-A buffers and outputs
    sets = []
    for i in range(nsets):
        Ai = A0 if i == 0 else A0.clone()
        wi = w0 if i == 0 else ops.PackedWeights(w0.packed.clone(), w0.desc)
        qi = ops.qgemm_quantize_rows(Ai, fmt, agr)
        oi = torch.empty((M, (N + 7) // 8 * 8), dtype=odt, device=dev)
        sets.append((Ai, wi, qi, oi))
    rng = np.random.default_rng(1234)
    gamma = torch.from_numpy(rng.normal(1.0, 0.1, size=K).astype(np.float32)).to(dev)
    bias = torch.from_numpy(rng.normal(0.0, 0.5, size=N).astype(np.float32)).to(dev)
    eps = 1e-6
    ws = None
    need = ops.qgemm_workspace_bytes(M, K, fmt, agr)
    if need:
        ws = torch.empty((need,), dtype=torch.uint8, device=dev)
    del W0
    torch.cuda.synchronize()

    def quantize(i):
        Ai, wi, qi, oi = sets[i % nsets]
        if args.fused:
            ops.qgemm_rmsnorm_quantize_rows(Ai, gamma, eps, fmt, out=qi)
        else:
            ops.qgemm_quantize_rows(Ai, fmt, agr, out=qi, workspace=ws)

    def gemm(i):
        Ai, wi, qi, oi = sets[i % nsets]
        if act == "mxfp8":
            ops.qgemm_run_mx(qi, wi, out=oi, mode=mx_mode)
        elif args.w4a8:
            ops.qgemm_run_w4a8(qi, wi, otype, out=oi, bias=bias if args.fused else None)
        else:
            ops.qgemm_run(qi, wi, otype, out=oi, bias=bias if args.fused else None)

    def step(i):
        quantize(i)
        gemm(i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # The timed launches are captured once into HIP graphs (K whole steps, and
    # K GEMM launches) and replayed, so the host's per-call overhead (Python,
    # ctypes) is not charged to the GPU: the library launches onto the current
    # stream, the step allocates nothing and records no memset. --eager
    # launches every step from Python instead.
    K_steps = args.steps

    # Timed region 1: K whole steps (quantize + GEMM + epilogue) back to back.
    # Four more passes afterwards describe the spread (not the value).
    passes = []
    ms_per_step, wall = timed(step, K_steps, args.eager, passes)
    # Timed region 2: the GEMM kernel alone, K launches over the same rotating
    # buffer sets, bracketed by events on the stream it runs on; the average
    # launch duration feeds the roofline.
    gemm_ms, _ = timed(gemm, K_steps, args.eager)
    # The quantizer alone over the same rotation: its bytes (float32 A read,
    # codes and per-row scales / zero points or E8M0 bytes written; the norm
    # weight when fused) against HBM.
    quant_ms, _ = timed(quantize, K_steps, args.eager)
    if act == "mxfp8":
        q_bytes = 4.0 * M * K + (0.5 if fp4 else 1.0) * M * K + M * (K // 32)
    else:
        q_bytes = 4.0 * M * K + M * K + 8.0 * M + (4.0 * K if args.fused else 0.0)
    quant = {"ms": quant_ms, "gbps": q_bytes / (quant_ms * 1e-3) / 1e9, "bytes": q_bytes,
             "frac_of_hbm": q_bytes / (quant_ms * 1e-3) / 1e9 / PEAK_HBM_GBS}

    if unit == "GB/s":
        value = step_bytes / (ms_per_step * 1e-3) / 1e9
        gemm_achieved = gemm_bytes / (gemm_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": gemm_achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        value = ops_count / (ms_per_step * 1e-3) / 1e12
        gemm_achieved = ops_count / (gemm_ms * 1e-3) / 1e12
        peak = mx_peak(fp4, wfp4) if act == "mxfp8" else PEAK_INT8_TOPS
        roof = {"bound": "mfma", "achieved": gemm_achieved, "peak": peak, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # the whole step (quantize + GEMM + epilogue) against the same peak
    roof["step_frac"] = value / roof["peak"]
    if act == "mxfp8" and mx_mode == ops.MX_EXACT:
        # exact products run on the bf16 matrix cores: at most half the MXFP8 peak
        roof["exact_mode_ceiling_frac"] = PEAK_BF16_TFLOPS / roof["peak"]
        roof["frac_of_bf16_cores"] = roof["achieved"] / PEAK_BF16_TFLOPS
    roof["traffic"] = measured_traffic(name + ("_w4a8" if args.w4a8 else "") + mx_suffix
                                       + ("_scaled" if act == "mxfp8" and mx_mode != ops.MX_EXACT else ""))
    if not args.no_ceiling:
        if unit == "GB/s":
            add_stream_ceiling(roof, [st[1].packed for st in sets], K_steps)
        else:
            add_mfma_ceiling(roof, ceiling_kind(ops, act, mx_mode, fp4, wfp4), sets[0][2].q, w0.packed)

    line = {
        "metric": METRIC,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": mx_dtype if act == "mxfp8" else ("i8 x i4" if args.w4a8 else "i8"),
        "data": "synthetic (seeded generator with the workload's shapes and distributions)",
        "config": {"workload": f"{name}: {DESCRIPTION[name]}"
                   + (f" ({mx_mode_arg} mode)" if act == "mxfp8" else "")
                   + (mx_note if act == "mxfp8" else "")
                   + (" with RMSNorm fused into the quantizer and a float32 bias" if args.fused else "")
                   + (" -- W4A8: int4 W with a float32 scale per group of 64 K" if args.w4a8 else ""),
                   "M": M, "K": K, "N": N,
                   "rotating_buffer_sets": nsets, "gemm_ms": gemm_ms,
                   "launch": "eager" if args.eager else "hip graph (K steps captured, replayed once)",
                   "step_hbm_gbs": step_bytes / (ms_per_step * 1e-3) / 1e9,
                   "step_spread": spread(passes), "quantize": quant, "prepack_ms": prepack_ms},
        "roofline": roof,
    }
    if args.calibration_copy:
        calibration_copy(args.calibration_copy, dev)
    print(f"[bench] {name}: {ms_per_step * 1e3:.2f} us/step, gemm {gemm_ms * 1e3:.2f} us, "
          f"wall {wall:.3f} s for {K_steps} steps", file=sys.stderr, flush=True)
    if with_cpu:
        line["cpu_baseline"] = cpu_baseline(name, A_np, W_np, args.cpu_budget,
                                            (gamma.cpu().numpy(), eps, bias.cpu().numpy()) if args.fused else None,
                                            args.w4a8, fp4, wfp4)
    return line


if __name__ == "__main__":
    main()
