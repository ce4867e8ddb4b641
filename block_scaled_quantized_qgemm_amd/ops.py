"""Python binding of the C ABI: the same four calls, on torch tensors.

Marshalling only -- shapes, dtypes, strides, allocation of outputs and the
current HIP stream are turned into the plain pointers and sizes of
include/qgemm.h; every step of the computation runs in the HIP library.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib as L

FMT_INT8_SYM, FMT_UINT8_ASYM, FMT_MXFP8_E4M3, FMT_INT4_SYM, FMT_MXFP4_E2M1 = 0, 1, 2, 3, 4
_MX_FMTS = (FMT_MXFP8_E4M3, FMT_MXFP4_E2M1)
GRAN_TENSOR, GRAN_ROW, GRAN_BLOCK32, GRAN_GROUP64 = 0, 1, 2, 3
OUT_F32, OUT_BF16, OUT_I32 = 0, 1, 2
MX_EXACT, MX_SCALED_MFMA = 0, 1
# include/qgemm_ceiling.h: the matrix-core instruction a ceiling measurement issues
CEIL_I8, CEIL_F8_SCALED, CEIL_F4_SCALED, CEIL_BF16 = 0, 1, 2, 3
CEILING_A_BYTES, CEILING_B_BYTES = 16384, 2048

_OUT_DTYPES = {OUT_F32: torch.float32, OUT_BF16: torch.bfloat16, OUT_I32: torch.int32}


class QgemmError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = L.load().qgemm_status_string(status).decode()
        super().__init__(f"{fn} failed: {msg} ({status})")
        self.status = status


def _check(fn: str, status: int):
    if status != 0:
        raise QgemmError(fn, status)


def _round_up(v: int, m: int) -> int:
    return (v + m - 1) // m * m


def _stream(device: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def unpack_fp4_codes(packed: torch.Tensor, K: int) -> torch.Tensor:
    """One e2m1 code (0..15) per element from two-codes-per-byte rows
    (element 2i in the low nibble of byte i); returns uint8 [rows, K]."""
    lo = packed & 0x0F
    hi = packed >> 4
    return torch.stack([lo, hi], dim=-1).reshape(packed.shape[0], -1)[:, :K]


@dataclass
class QuantizedRows:
    """Codes [M, ld] (the first K columns valid; MXFP4: the first K / 2 bytes,
    two codes per byte) plus scales / zero points / E8M0 scales."""
    q: torch.Tensor
    K: int
    fmt: int
    gran: int
    scales: Optional[torch.Tensor] = None
    zero_points: Optional[torch.Tensor] = None
    mx_scales: Optional[torch.Tensor] = None

    @property
    def M(self) -> int:
        return self.q.shape[0]

    def codes(self) -> torch.Tensor:
        """The stored codes: [M, K] bytes, or [M, K / 2] packed bytes for MXFP4."""
        return self.q[:, : self.K // 2] if self.fmt == FMT_MXFP4_E2M1 else self.q[:, : self.K]

    def element_codes(self) -> torch.Tensor:
        """One code per element, [M, K] (MXFP4 codes unpacked)."""
        if self.fmt == FMT_MXFP4_E2M1:
            return unpack_fp4_codes(self.q[:, : self.K // 2], self.K)
        return self.codes()


def unblock_int8_codes(raw: torch.Tensor, n_pad: int, k_pad: int) -> torch.Tensor:
    """Row-major [n_pad, k_pad] copy of packed int8 codes stored as 1 KB blocks:
    block (n // 16, k // 64) in block-row-major order, and inside it the 16 bytes
    of row n % 16 with k % 64 in [16c, 16c + 16) at 256 c + 16 (n % 16)."""
    b = raw.reshape(n_pad // 16, k_pad // 64, 4, 16, 16)      # [rb, kb, c, r, j]
    return b.permute(0, 3, 1, 2, 4).reshape(n_pad, k_pad)     # [rb, r, kb, c, j]


def unblock_mx8_codes(raw: torch.Tensor, n_pad: int, k_pad: int) -> torch.Tensor:
    """Row-major [n_pad, k_pad] copy of packed e4m3 weight codes stored as 1 KB
    blocks of 16 rows x 64 K in block-row-major order, row n % 16 of a block
    at 64 (n % 16) with its 64 codes in K order."""
    b = raw.reshape(n_pad // 16, k_pad // 64, 16, 64)        # [rb, kb, r, j]
    return b.permute(0, 2, 1, 3).reshape(n_pad, k_pad)        # [rb, r, kb, j]


def unblock_int4_codes(raw: torch.Tensor, n_pad: int, k_pad: int) -> torch.Tensor:
    """Row-major int8 [n_pad, k_pad] codes from the packed int4 layout: 1 KB
    blocks of 16 rows x 128 K; lane 16 c + r of a block owns 16 bytes, 8 per
    group of 64 K; dword d of those 8 holds k % 16 in [8d, 8d + 8), k % 4 in
    its byte, low nibble for k % 8 < 4. Nibbles are sign-extended."""
    b = raw.reshape(n_pad // 16, k_pad // 128, 4, 16, 2, 2, 4)  # [rb, pb, c, r, g, d, byte]
    lo = b & 0x0F
    hi = b >> 4
    nib = torch.stack([lo, hi], dim=6)                        # [rb, pb, c, r, g, d, half, byte]
    nib = nib.to(torch.int16)
    val = torch.where(nib >= 8, nib - 16, nib).to(torch.int8)
    # k = 128 pb + 64 g + 16 c + 8 d + 4 half + byte
    return val.permute(0, 3, 1, 4, 2, 5, 6, 7).reshape(n_pad, k_pad)


@dataclass
class PackedWeights:
    """A prepared weight buffer and its host descriptor."""
    packed: torch.Tensor
    desc: L.WDesc

    @property
    def N(self) -> int:
        return int(self.desc.N)

    @property
    def K(self) -> int:
        return int(self.desc.K)

    def codes(self) -> torch.Tensor:
        """Codes as [N_pad, K_pad], row-major. The int8 and e4m3 buffers store
        1 KB blocks of 16 rows x 64 K (see qgemm_wdesc); those come back as a
        row-major copy."""
        d = self.desc
        if d.fmt == FMT_INT4_SYM:
            raw = self.packed[d.codes_off: d.codes_off + d.N_pad * d.K_pad // 2]
            return unblock_int4_codes(raw, d.N_pad, d.K_pad)
        if d.fmt == FMT_MXFP4_E2M1:  # one code per element, [N_pad, K_pad]
            raw = self.packed[d.codes_off: d.codes_off + d.N_pad * d.K_pad // 2]
            return unpack_fp4_codes(raw.view(d.N_pad, d.K_pad // 2), d.K_pad)
        raw = self.packed[d.codes_off: d.codes_off + d.N_pad * d.K_pad]
        if d.fmt == FMT_MXFP8_E4M3:
            return unblock_mx8_codes(raw, d.N_pad, d.K_pad)
        return unblock_int8_codes(raw, d.N_pad, d.K_pad).view(torch.int8)

    def scales(self) -> torch.Tensor:
        d = self.desc
        if d.fmt == FMT_INT8_SYM:
            n = 1 if d.gran == GRAN_TENSOR else d.N_pad
            return self.packed[d.scales_off: d.scales_off + 4 * n].view(torch.float32)
        if d.fmt == FMT_INT4_SYM:  # [N_pad, K_pad / 64] from 64 per 16 rows x 256 K: [rb, qb, r, g]
            n = d.N_pad * (d.K_pad // 64)
            raw = self.packed[d.scales_off: d.scales_off + 4 * n].view(torch.float32)
            return raw.reshape(d.N_pad // 16, d.K_pad // 256, 16, 4).permute(0, 2, 1, 3).reshape(d.N_pad, d.K_pad // 64)
        return self.packed[d.scales_off: d.scales_off + d.N_pad * (d.K_pad // 32)].view(d.N_pad, d.K_pad // 32)

    def colsum(self) -> torch.Tensor:
        d = self.desc
        return self.packed[d.colsum_off: d.colsum_off + 4 * d.N_pad].view(torch.int32)


@dataclass
class PackedExperts:
    """E experts' prepared weights back to back (expert e at byte
    e * desc.bytes) and the descriptor they share."""
    packed: torch.Tensor
    desc: L.WDesc
    E: int

    @property
    def N(self) -> int:
        return int(self.desc.N)

    def expert(self, e: int) -> PackedWeights:
        nb = int(self.desc.bytes)
        return PackedWeights(self.packed[e * nb:(e + 1) * nb], self.desc)


def qgemm_workspace_bytes(rows: int, K: int, fmt: int, gran: int) -> int:
    return int(L.load().qgemm_workspace_bytes(rows, K, fmt, gran))


def qgemm_packed_weight_bytes(N: int, K: int, fmt: int, gran: int) -> int:
    return int(L.load().qgemm_packed_weight_bytes(N, K, fmt, gran))


def _quantized_rows_out(x: torch.Tensor, fmt: int, gran: int) -> QuantizedRows:
    """Output buffers of a row quantization of the float32 [M, K] matrix x."""
    M, K = x.shape
    dev = x.device
    ld = _round_up(max(K // 2 if fmt == FMT_MXFP4_E2M1 else K, 1), 16)
    q = torch.empty((M, ld), dtype=torch.int8 if fmt == FMT_INT8_SYM else torch.uint8, device=dev)
    scales = zeros = mx = None
    if fmt in _MX_FMTS:
        # E8M0 rows padded to a multiple of 4 bytes: the GEMM's DMA path
        # fetches them a dword at a time
        mx = torch.empty((M, _round_up(max(K // 32, 1), 4)), dtype=torch.uint8, device=dev)
    else:
        scales = torch.empty((1 if gran == GRAN_TENSOR else M,), dtype=torch.float32, device=dev)
        if fmt == FMT_UINT8_ASYM:
            zeros = torch.empty_like(scales, dtype=torch.int32)
    return QuantizedRows(q, K, fmt, gran, scales, zeros, mx)


def qgemm_quantize_rows_noalloc(x: torch.Tensor, fmt: int = FMT_INT8_SYM, gran: int = GRAN_ROW,
                                out: Optional[QuantizedRows] = None, stream=None) -> QuantizedRows:
    """qgemm_quantize_rows without a workspace: the library keeps per-tensor
    statistics in its own static device array (see qgemm.h). With ``out``
    given, nothing is allocated on the device."""
    lib = L.load()
    assert x.dtype == torch.float32 and x.dim() == 2 and x.stride(1) == 1
    M, K = x.shape
    if out is None:
        out = _quantized_rows_out(x, fmt, gran)
    st = lib.qgemm_quantize_rows_noalloc(
        _ptr(x), M, K, x.stride(0), fmt, gran, _ptr(out.q), out.q.stride(0),
        _ptr(out.scales), _ptr(out.zero_points), _ptr(out.mx_scales),
        0 if out.mx_scales is None else out.mx_scales.stride(0), ctypes.c_void_p(_stream(x.device, stream)))
    _check("qgemm_quantize_rows_noalloc", st)
    return out


def qgemm_quantize_rows(x: torch.Tensor, fmt: int = FMT_INT8_SYM, gran: int = GRAN_ROW,
                        out: Optional[QuantizedRows] = None, workspace: Optional[torch.Tensor] = None,
                        stream=None) -> QuantizedRows:
    """Quantize the rows of a float32 [M, K] device matrix (see qgemm.h)."""
    lib = L.load()
    assert x.dtype == torch.float32 and x.dim() == 2 and x.stride(1) == 1
    M, K = x.shape
    dev = x.device
    if out is None:
        out = _quantized_rows_out(x, fmt, gran)
    need = qgemm_workspace_bytes(M, K, fmt, gran)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.qgemm_quantize_rows(
        _ptr(x), M, K, x.stride(0), fmt, gran, _ptr(out.q), out.q.stride(0),
        _ptr(out.scales), _ptr(out.zero_points), _ptr(out.mx_scales),
        0 if out.mx_scales is None else out.mx_scales.stride(0),
        _ptr(workspace), ws_bytes, ctypes.c_void_p(_stream(dev, stream)))
    _check("qgemm_quantize_rows", st)
    return out


def qgemm_rmsnorm_quantize_rows(x: torch.Tensor, gamma: torch.Tensor, eps: float, fmt: int = FMT_INT8_SYM,
                                out: Optional[QuantizedRows] = None, stream=None) -> QuantizedRows:
    """RMSNorm of the float32 [M, K] rows with weight gamma [K], then per-row quantization (see qgemm.h)."""
    lib = L.load()
    assert x.dtype == torch.float32 and x.dim() == 2 and x.stride(1) == 1
    assert gamma.dtype == torch.float32 and gamma.dim() == 1 and gamma.is_contiguous()
    M, K = x.shape
    assert gamma.shape[0] == K
    dev = x.device
    if out is None:
        ld = _round_up(max(K, 1), 16)
        q = torch.empty((M, ld), dtype=torch.int8 if fmt == FMT_INT8_SYM else torch.uint8, device=dev)
        scales = torch.empty((M,), dtype=torch.float32, device=dev)
        zeros = torch.empty_like(scales, dtype=torch.int32) if fmt == FMT_UINT8_ASYM else None
        out = QuantizedRows(q, K, fmt, GRAN_ROW, scales, zeros, None)
    st = lib.qgemm_rmsnorm_quantize_rows(
        _ptr(x), M, K, x.stride(0), _ptr(gamma), ctypes.c_float(eps), fmt, GRAN_ROW, _ptr(out.q), out.q.stride(0),
        _ptr(out.scales), _ptr(out.zero_points), ctypes.c_void_p(_stream(dev, stream)))
    _check("qgemm_rmsnorm_quantize_rows", st)
    return out


def qgemm_prepack_weights(w: torch.Tensor, fmt: int = FMT_INT8_SYM, gran: int = GRAN_ROW,
                          stream=None) -> PackedWeights:
    """Prepare a float32 [N, K] weight (per-channel / per-tensor int8, MXFP8,
    or int4 with a scale per group of 64 K)."""
    lib = L.load()
    assert w.dtype == torch.float32 and w.dim() == 2 and w.stride(1) == 1
    N, K = w.shape
    dev = w.device
    nbytes = qgemm_packed_weight_bytes(N, K, fmt, gran)
    if nbytes == 0:
        raise QgemmError("qgemm_prepack_weights", -2)
    packed = torch.empty((nbytes,), dtype=torch.uint8, device=dev)
    need = qgemm_workspace_bytes(N, K, fmt, gran)
    ws = torch.empty((need,), dtype=torch.uint8, device=dev) if need else None
    desc = L.WDesc()
    st = lib.qgemm_prepack_weights(_ptr(w), N, K, w.stride(0), fmt, gran, _ptr(packed), nbytes,
                                   ctypes.byref(desc), _ptr(ws), need, ctypes.c_void_p(_stream(dev, stream)))
    _check("qgemm_prepack_weights", st)
    return PackedWeights(packed, desc)


def qgemm_unpack_weights(w: PackedWeights, stream=None) -> dict:
    """Plain copies of what a prepared weight buffer holds (see qgemm.h), as a
    dict of device tensors: 'codes' [N, K] (int8 for int8 and int4 weights,
    uint8 bytes for MX; e2m1 two per byte, [N, K / 2]); 'scales' float32 [N]
    or [1] (int8) or [N, ceil(K / 64)] (int4); 'colsums' int32 [N] (int8);
    'mx_scales' uint8 [N, K / 32] (MX). Only what the format has."""
    lib = L.load()
    d = w.desc
    dev = w.packed.device
    N, K = int(d.N), int(d.K)
    mx = d.fmt in (FMT_MXFP8_E4M3, FMT_MXFP4_E2M1)
    out = {}
    code_cols = K // 2 if d.fmt == FMT_MXFP4_E2M1 else K
    out["codes"] = torch.empty((N, code_cols), dtype=torch.uint8 if mx else torch.int8, device=dev)
    if d.fmt == FMT_INT8_SYM:
        out["scales"] = torch.empty((1 if d.gran == GRAN_TENSOR else N,), dtype=torch.float32, device=dev)
        out["colsums"] = torch.empty((N,), dtype=torch.int32, device=dev)
    elif d.fmt == FMT_INT4_SYM:
        out["scales"] = torch.empty((N, (K + 63) // 64), dtype=torch.float32, device=dev)
    else:
        out["mx_scales"] = torch.empty((N, K // 32), dtype=torch.uint8, device=dev)
    sc = out.get("scales")
    mxs = out.get("mx_scales")
    st = lib.qgemm_unpack_weights(ctypes.byref(d), _ptr(w.packed), _ptr(out["codes"]), out["codes"].stride(0),
                                  _ptr(sc), sc.stride(0) if sc is not None and sc.dim() == 2 else 1,
                                  _ptr(out.get("colsums")), _ptr(mxs), mxs.stride(0) if mxs is not None else 0,
                                  ctypes.c_void_p(_stream(dev, stream)))
    _check("qgemm_unpack_weights", st)
    return out


def qgemm_prepack_experts(w: torch.Tensor, fmt: int = FMT_MXFP8_E4M3, stream=None) -> PackedExperts:
    """Prepare E experts' float32 [E, N, K] MX weights into one buffer for
    qgemm_run_mx_grouped (one qgemm_prepack_weights call per expert slice)."""
    lib = L.load()
    assert w.dtype == torch.float32 and w.dim() == 3 and w.stride(2) == 1
    E, N, K = w.shape
    dev = w.device
    nb = qgemm_packed_weight_bytes(N, K, fmt, GRAN_BLOCK32)
    if nb == 0:
        raise QgemmError("qgemm_prepack_weights", -2)
    packed = torch.empty((E * nb,), dtype=torch.uint8, device=dev)
    desc = L.WDesc()
    for e in range(E):
        st = lib.qgemm_prepack_weights(_ptr(w[e]), N, K, w.stride(1), fmt, GRAN_BLOCK32, _ptr(packed[e * nb:]), nb,
                                       ctypes.byref(desc), None, 0, ctypes.c_void_p(_stream(dev, stream)))
        _check("qgemm_prepack_weights", st)
    return PackedExperts(packed, desc, E)


def _alloc_out(M: int, N: int, dtype, dev):
    buf = torch.empty((M, _round_up(N, 8)), dtype=dtype, device=dev)
    return buf


def _bias_ptr(bias: Optional[torch.Tensor], N: int):
    if bias is None:
        return None
    assert bias.dtype == torch.float32 and bias.dim() == 1 and bias.shape[0] == N and bias.is_contiguous()
    return _ptr(bias)


def qgemm_run(a: QuantizedRows, w: PackedWeights, out_type: int = OUT_F32,
              out: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
              stream=None) -> torch.Tensor:
    """int8 GEMM with the fused dequantization epilogue (plus an optional
    float32 bias [N]); returns out[:, :N]."""
    lib = L.load()
    dev = a.q.device
    N = w.N
    if out is None:
        out = _alloc_out(a.M, N, _OUT_DTYPES[out_type], dev)
    st = lib.qgemm_run(_ptr(a.q), a.q.stride(0), _ptr(a.scales), _ptr(a.zero_points), a.fmt, a.gran, a.M,
                       ctypes.byref(w.desc), _ptr(w.packed), _ptr(out), out.stride(0), out_type,
                       _bias_ptr(bias, N), None, 0, ctypes.c_void_p(_stream(dev, stream)))
    _check("qgemm_run", st)
    return out[:, :N]


def qgemm_run_mx(a: QuantizedRows, w: PackedWeights, out: Optional[torch.Tensor] = None,
                 mode: int = MX_EXACT, bias: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Block-scaled GEMM of e4m3 or e2m1 activations and weights (float32
    out, plus an optional float32 bias [N]); returns out[:, :N]."""
    lib = L.load()
    dev = a.q.device
    N = w.N
    if out is None:
        out = _alloc_out(a.M, N, torch.float32, dev)
    st = lib.qgemm_run_mx(_ptr(a.q), a.q.stride(0), _ptr(a.mx_scales), a.mx_scales.stride(0), a.fmt, a.M,
                          ctypes.byref(w.desc), _ptr(w.packed), _ptr(out), out.stride(0), mode,
                          _bias_ptr(bias, N), None, 0, ctypes.c_void_p(_stream(dev, stream)))
    _check("qgemm_run_mx", st)
    return out[:, :N]


def qgemm_run_mx_grouped(a: QuantizedRows, w: PackedExperts, offsets: torch.Tensor,
                         out: Optional[torch.Tensor] = None, mode: int = MX_EXACT,
                         bias: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Grouped (MoE) block-scaled GEMM: rows offsets[e] .. offsets[e+1] - 1
    of A times expert e's weights (offsets: device int64 [E + 1]); float32
    out, plus an optional float32 bias [E, N]. Returns out[:, :N]."""
    lib = L.load()
    dev = a.q.device
    N = w.N
    assert offsets.dtype == torch.int64 and offsets.dim() == 1 and offsets.numel() == w.E + 1
    assert offsets.is_contiguous() and offsets.device == dev
    if bias is not None:
        assert bias.dtype == torch.float32 and bias.shape == (w.E, N) and bias.is_contiguous()
    if out is None:
        out = _alloc_out(a.M, N, torch.float32, dev)
    st = lib.qgemm_run_mx_grouped(_ptr(a.q), a.q.stride(0), _ptr(a.mx_scales), a.mx_scales.stride(0), a.fmt, a.M,
                                  _ptr(offsets), w.E, ctypes.byref(w.desc), _ptr(w.packed), _ptr(out), out.stride(0),
                                  mode, _ptr(bias), None, 0, ctypes.c_void_p(_stream(dev, stream)))
    _check("qgemm_run_mx_grouped", st)
    return out[:, :N]


def qgemm_run_w4a8(a: QuantizedRows, w: PackedWeights, out_type: int = OUT_F32,
                   out: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    """int8 activations x int4 weights with per-group-64 scales (float32 or
    bfloat16 out, plus an optional float32 bias [N]); returns out[:, :N]."""
    lib = L.load()
    dev = a.q.device
    N = w.N
    if out is None:
        out = _alloc_out(a.M, N, _OUT_DTYPES[out_type], dev)
    st = lib.qgemm_run_w4a8(_ptr(a.q), a.q.stride(0), _ptr(a.scales), a.gran, a.M,
                            ctypes.byref(w.desc), _ptr(w.packed), _ptr(out), out.stride(0), out_type,
                            _bias_ptr(bias, N), None, 0, ctypes.c_void_p(_stream(dev, stream)))
    _check("qgemm_run_w4a8", st)
    return out[:, :N]


# ---- measured ceilings (include/qgemm_ceiling.h; not part of the GEMM path) ----

def qgemm_ceiling_mfma_shape(kind: int, waves_per_simd: int, trips: int):
    """(workgroups, operations) of one qgemm_ceiling_mfma launch on the current device."""
    lib = L.load()
    wg, ops_ = ctypes.c_int64(0), ctypes.c_double(0.0)
    st = lib.qgemm_ceiling_mfma_shape(kind, waves_per_simd, trips, ctypes.byref(wg), ctypes.byref(ops_))
    _check("qgemm_ceiling_mfma_shape", st)
    return int(wg.value), float(ops_.value)


def qgemm_ceiling_mfma(kind: int, waves_per_simd: int, trips: int, a_ops: torch.Tensor, b_ops: torch.Tensor,
                       sink: torch.Tensor, clocks: Optional[torch.Tensor] = None, stream=None) -> None:
    """Issue trips * 8 matrix-core instructions of `kind` per wave on every CU
    (see qgemm_ceiling.h). a_ops / b_ops: device byte tensors of at least
    CEILING_A_BYTES / CEILING_B_BYTES; sink: int32 [1]; clocks: int64
    [2 * workgroups] or None."""
    lib = L.load()
    assert a_ops.is_contiguous() and a_ops.numel() * a_ops.element_size() >= CEILING_A_BYTES
    assert b_ops.is_contiguous() and b_ops.numel() * b_ops.element_size() >= CEILING_B_BYTES
    assert sink.dtype == torch.int32 and sink.numel() >= 1
    if clocks is not None:
        wg, _ = qgemm_ceiling_mfma_shape(kind, waves_per_simd, trips)
        assert clocks.dtype == torch.int64 and clocks.is_contiguous() and clocks.numel() >= 2 * wg
    st = lib.qgemm_ceiling_mfma(kind, waves_per_simd, trips, _ptr(a_ops), _ptr(b_ops), _ptr(sink), _ptr(clocks),
                                ctypes.c_void_p(_stream(a_ops.device, stream)))
    _check("qgemm_ceiling_mfma", st)


def qgemm_ceiling_stream(src: torch.Tensor, nbytes: int, block_bytes: int, sink: torch.Tensor, stream=None) -> None:
    """Read the first nbytes of the device tensor src once, one workgroup per
    block_bytes (see qgemm_ceiling.h)."""
    lib = L.load()
    assert src.is_contiguous() and nbytes <= src.numel() * src.element_size()
    assert sink.dtype == torch.int32 and sink.numel() >= 1
    st = lib.qgemm_ceiling_stream(_ptr(src), nbytes, block_bytes, _ptr(sink), ctypes.c_void_p(_stream(src.device, stream)))
    _check("qgemm_ceiling_stream", st)
