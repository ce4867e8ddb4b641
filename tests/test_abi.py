"""CPU-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects invalid arguments before touching any device."""
import ctypes
import os
import re

import pytest

from conftest import ROOT

torch = pytest.importorskip("torch")

from block_scaled_quantized_qgemm_amd import _lib as L  # noqa: E402

HEADER = os.path.join(ROOT, "include", "qgemm.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))

OK, E_NULL, E_SHAPE, E_MODE, E_ALIGN, E_OVERFLOW, E_DEVICE, E_DESC, E_WS = 0, -1, -2, -3, -4, -5, -6, -7, -8
INT8, UINT8, MX, INT4, MX4 = 0, 1, 2, 3, 4
TENSOR, ROW, BLK, G64 = 0, 1, 2, 3
ABI = 9


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libqgemm.so is not built (run __graft_entry__.build())")
    return L.load()


def _declared_functions():
    src = "".join(open(h).read() for h in HEADERS)
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?[\w\*\s]+?\b(qgemm_\w+)\s*\(", src, flags=re.M))


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert names == set(L.SIGNATURES), names ^ set(L.SIGNATURES)
    for n in names:
        assert hasattr(lib, n)


def test_version_and_status_strings(lib):
    assert lib.qgemm_abi_version() == ABI
    for s in range(-9, 1):
        assert lib.qgemm_status_string(s).startswith(b"QGEMM_")
    assert lib.qgemm_status_string(-100) == b"unknown qgemm status"


def test_sizes(lib):
    # int8: codes [256][128] + scales 4*256 + colsum 4*256
    assert lib.qgemm_packed_weight_bytes(1, 1, INT8, ROW) == 256 * 256 + 1024 + 1024
    assert lib.qgemm_packed_weight_bytes(4096, 4096, INT8, ROW) == 4096 * 4096 + 4 * 4096 * 2
    assert lib.qgemm_packed_weight_bytes(8192, 8192, MX, BLK) == 8192 * 8192 + 8192 * 256
    assert lib.qgemm_packed_weight_bytes(64, 100, MX, BLK) == 0       # K % 32
    assert lib.qgemm_packed_weight_bytes(64, 96, UINT8, ROW) == 0     # weights are symmetric
    assert lib.qgemm_packed_weight_bytes(0, 96, INT8, ROW) == 0
    assert lib.qgemm_workspace_bytes(64, 256, INT8, TENSOR) == 256
    assert lib.qgemm_workspace_bytes(64, 256, UINT8, TENSOR) == 512
    assert lib.qgemm_workspace_bytes(64, 256, INT8, ROW) == 0
    assert lib.qgemm_workspace_bytes(64, 256, MX, BLK) == 0
    # int4: codes [256][512 / 2], then float32 scales [256][512 / 64]
    assert lib.qgemm_packed_weight_bytes(100, 300, INT4, G64) == 256 * 256 + 4 * 256 * 8
    assert lib.qgemm_packed_weight_bytes(14336, 4096, INT4, G64) == 14336 * 2048 + 4 * 14336 * 64
    assert lib.qgemm_packed_weight_bytes(100, 300, INT4, ROW) == 0
    assert lib.qgemm_packed_weight_bytes(100, 300, INT8, G64) == 0
    assert lib.qgemm_workspace_bytes(64, 256, INT4, G64) == 0
    # MXFP4: codes [256][512 / 2], E8M0 [256][512 / 32]
    assert lib.qgemm_packed_weight_bytes(100, 320, MX4, BLK) == 256 * 256 + 256 * 16
    assert lib.qgemm_packed_weight_bytes(64, 100, MX4, BLK) == 0      # K % 32
    assert lib.qgemm_packed_weight_bytes(64, 96, MX4, ROW) == 0


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def _q(lib, x=FAKE, M=4, K=64, ldx=64, fmt=INT8, gran=ROW, q=FAKE, ldq=64, s=FAKE, z=None, mx=None,
       ldmx=0, ws=None, wsb=0):
    return lib.qgemm_quantize_rows(x, M, K, ldx, fmt, gran, q, ldq, s, z, mx, ldmx, ws, wsb, None)


def test_quantize_rows_validation(lib):
    assert _q(lib, fmt=7) == E_MODE
    assert _q(lib, fmt=MX, gran=ROW) == E_MODE
    assert _q(lib, fmt=INT8, gran=BLK) == E_MODE
    assert _q(lib, K=0) == E_SHAPE
    assert _q(lib, M=-1) == E_SHAPE
    assert _q(lib, M=0, x=None, q=None, s=None) == OK           # empty call
    assert _q(lib, x=None) == E_NULL
    assert _q(lib, s=None) == E_NULL
    assert _q(lib, fmt=UINT8, z=None) == E_NULL
    assert _q(lib, ldx=32) == E_SHAPE
    assert _q(lib, ldq=63) == E_SHAPE
    assert _q(lib, ldq=80 + 8) == E_ALIGN
    assert _q(lib, x=FAKE + 2) == E_ALIGN
    assert _q(lib, q=FAKE + 4) == E_ALIGN
    assert _q(lib, fmt=MX, gran=BLK, K=48, ldx=48, ldq=48, s=None, mx=FAKE, ldmx=2) == E_SHAPE
    assert _q(lib, fmt=MX, gran=BLK, s=None, mx=None) == E_NULL
    assert _q(lib, fmt=MX, gran=BLK, s=None, mx=FAKE, ldmx=1) == E_SHAPE
    assert _q(lib, gran=TENSOR) == E_WS
    assert _q(lib, gran=TENSOR, ws=FAKE, wsb=15) == E_WS
    assert _q(lib, fmt=MX4, gran=ROW) == E_MODE
    assert _q(lib, fmt=MX4, gran=BLK, s=None, mx=FAKE, ldmx=2, ldq=16) == E_SHAPE   # K / 2 = 32 bytes
    assert _q(lib, fmt=MX4, gran=BLK, s=None, mx=FAKE, ldmx=2, ldq=40) == E_ALIGN


def _qn(lib, x=FAKE, M=4, K=64, ldx=64, fmt=INT8, gran=ROW, q=FAKE, ldq=64, s=FAKE, z=None, mx=None, ldmx=0):
    return lib.qgemm_quantize_rows_noalloc(x, M, K, ldx, fmt, gran, q, ldq, s, z, mx, ldmx, None)


def test_quantize_rows_noalloc_validation(lib):
    """The allocation-free entry point validates like qgemm_quantize_rows
    (before any device call) and refuses per-tensor sizes beyond its 1 MiB
    static array: 2^18 rows of int8 statistics, 2^17 of uint8."""
    assert _qn(lib, fmt=7) == E_MODE
    assert _qn(lib, fmt=MX, gran=ROW) == E_MODE
    assert _qn(lib, K=0) == E_SHAPE
    assert _qn(lib, M=0, x=None, q=None, s=None) == OK
    assert _qn(lib, x=None) == E_NULL
    assert _qn(lib, fmt=UINT8, z=None) == E_NULL
    assert _qn(lib, ldq=63) == E_SHAPE
    assert _qn(lib, q=FAKE + 4) == E_ALIGN
    assert _qn(lib, fmt=MX, gran=BLK, s=None, mx=FAKE, ldmx=1) == E_SHAPE
    assert _qn(lib, gran=TENSOR, M=(1 << 18) + 1) == E_WS
    assert _qn(lib, gran=TENSOR, fmt=UINT8, z=FAKE, M=(1 << 17) + 1) == E_WS
    assert lib.qgemm_workspace_bytes(1 << 18, 64, INT8, TENSOR) == 1 << 20
    assert lib.qgemm_workspace_bytes(1 << 17, 64, UINT8, TENSOR) == 1 << 20


def _wdesc(**kw):
    d = L.WDesc(magic=0x51474D57, version=ABI, fmt=INT8, gran=ROW, N=100, K=300, N_pad=256, K_pad=512,
                codes_off=0, scales_off=256 * 512, colsum_off=256 * 512 + 1024, bytes=256 * 512 + 2048)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def _run(lib, d, a=FAKE, lda=304, s=FAKE, z=None, fmt=INT8, gran=ROW, M=8, w=FAKE, out=FAKE, ldo=100,
         ot=0, bias=None):
    return lib.qgemm_run(a, lda, s, z, fmt, gran, M, ctypes.byref(d), w, out, ldo, ot, bias, None, 0, None)


def test_run_validation(lib):
    good = _wdesc()
    assert lib.qgemm_packed_weight_bytes(100, 300, INT8, ROW) == good.bytes
    assert _run(lib, _wdesc(magic=1)) == E_DESC
    assert _run(lib, _wdesc(version=2)) == E_DESC
    assert _run(lib, _wdesc(fmt=MX)) == E_DESC
    assert _run(lib, _wdesc(K_pad=384)) == E_DESC
    assert _run(lib, _wdesc(bytes=5)) == E_DESC
    assert lib.qgemm_run(FAKE, 304, FAKE, None, INT8, ROW, 8, None, FAKE, FAKE, 100, 0, None, None, 0, None) == E_NULL
    assert _run(lib, good, fmt=MX) == E_MODE
    assert _run(lib, good, ot=3) == E_MODE
    assert _run(lib, good, ot=2, bias=FAKE) == E_MODE     # the int32 export takes no bias
    assert _run(lib, good, bias=FAKE + 2) == E_ALIGN
    assert _run(lib, good, M=-1) == E_SHAPE
    assert _run(lib, good, M=0, a=None, s=None, w=None, out=None) == OK
    assert _run(lib, good, a=None) == E_NULL
    assert _run(lib, good, fmt=UINT8) == E_NULL            # missing zero points
    assert _run(lib, good, lda=288) == E_SHAPE
    assert _run(lib, good, lda=312) == E_ALIGN
    assert _run(lib, good, ldo=99) == E_SHAPE
    assert _run(lib, good, ldo=102) == E_ALIGN
    assert _run(lib, good, w=FAKE + 16) == E_ALIGN
    # exact-int32 limits on K
    nb = lib.qgemm_packed_weight_bytes(8, 133145, INT8, ROW)
    big = _wdesc(N=8, K=133145, K_pad=133376, scales_off=256 * 133376, colsum_off=256 * 133376 + 1024,
                 bytes=nb)
    assert _run(lib, big, lda=133152) == E_OVERFLOW
    nb = lib.qgemm_packed_weight_bytes(8, 66312, INT8, ROW)
    mid = _wdesc(N=8, K=66312, K_pad=66560, scales_off=256 * 66560, colsum_off=256 * 66560 + 1024, bytes=nb)
    assert _run(lib, mid, lda=66320, fmt=UINT8, z=FAKE) == E_OVERFLOW


def test_run_mx_validation(lib):
    nb = lib.qgemm_packed_weight_bytes(100, 320, MX, BLK)
    d = L.WDesc(magic=0x51474D57, version=ABI, fmt=MX, gran=BLK, N=100, K=320, N_pad=256, K_pad=512,
                codes_off=0, scales_off=256 * 512, colsum_off=-1, bytes=nb)
    call = lambda **kw: lib.qgemm_run_mx(kw.get("a", FAKE), kw.get("lda", 320), kw.get("e", FAKE),
                                         kw.get("ldas", 10), kw.get("af", MX), kw.get("M", 4),
                                         ctypes.byref(kw.get("d", d)),
                                         FAKE, kw.get("out", FAKE), kw.get("ldo", 100), kw.get("mode", 0),
                                         kw.get("bias", None), None, 0, None)
    assert call(d=_wdesc()) == E_DESC                     # an int8 descriptor
    assert call(e=None) == E_NULL
    assert call(ldas=9) == E_SHAPE
    assert call(lda=304) == E_SHAPE
    assert call(lda=328) == E_ALIGN
    assert call(M=0, a=None, e=None, out=None) == OK
    assert call(mode=2) == E_MODE
    assert call(bias=FAKE + 1) == E_ALIGN
    assert call(af=INT8) == E_MODE
    # the block-scaled matrix cores take any e4m3 / e2m1 pair (M = 0: validation only)
    assert call(af=MX4, lda=160, mode=1, M=0, a=None, e=None, out=None) == OK
    assert call(af=MX4, lda=160, M=0, a=None, e=None, out=None) == OK
    assert call(af=MX4, lda=144) == E_SHAPE               # packed e2m1 rows need K / 2 bytes
    nb4 = lib.qgemm_packed_weight_bytes(100, 320, MX4, BLK)
    d4 = L.WDesc(magic=0x51474D57, version=ABI, fmt=MX4, gran=BLK, N=100, K=320, N_pad=256, K_pad=512,
                 codes_off=0, scales_off=256 * 256, colsum_off=-1, bytes=nb4)
    assert call(d=d4, mode=1, M=0, a=None, e=None, out=None) == OK
    assert call(d=d4, mode=2) == E_MODE
    assert call(d=_w4desc()) == E_DESC                    # int4 weights are not MX


def _mxdesc(N=100, K=320, fmt=MX):
    nb = L.load().qgemm_packed_weight_bytes(N, K, fmt, BLK)
    kp = (K + 255) // 256 * 256
    np_ = (N + 255) // 256 * 256
    cb = kp // 2 if fmt == MX4 else kp
    return L.WDesc(magic=0x51474D57, version=ABI, fmt=fmt, gran=BLK, N=N, K=K, N_pad=np_, K_pad=kp,
                   codes_off=0, scales_off=(np_ * cb + 255) // 256 * 256, colsum_off=-1, bytes=nb)


def _grouped(lib, **kw):
    d = kw.get("d", _mxdesc(K=kw.get("K", 320)))
    return lib.qgemm_run_mx_grouped(kw.get("a", FAKE), kw.get("lda", d.K), kw.get("e", FAKE), kw.get("ldas", 12),
                                    kw.get("af", MX), kw.get("M", 40), kw.get("off", FAKE), kw.get("E", 3),
                                    ctypes.byref(d), kw.get("w", FAKE), kw.get("out", FAKE), kw.get("ldo", d.N),
                                    kw.get("mode", 0), kw.get("bias", None), None, 0, None)


def test_run_mx_grouped_validation(lib):
    assert _grouped(lib, d=_wdesc()) == E_DESC                 # an int8 descriptor
    assert _grouped(lib, mode=2) == E_MODE
    assert _grouped(lib, af=INT8) == E_MODE
    # any e4m3 / e2m1 pair in either mode (M = 0: validation only)
    assert _grouped(lib, af=MX4, lda=160, mode=1, M=0, a=None, e=None, off=None, out=None) == OK
    assert _grouped(lib, af=MX4, lda=160, mode=0, M=0, a=None, e=None, off=None, out=None) == OK
    d4 = _mxdesc(K=384, fmt=MX4)
    assert _grouped(lib, d=d4, af=MX4, lda=192, ldas=12, mode=0, M=0, a=None, e=None, off=None, out=None) == OK
    assert _grouped(lib, d=d4, af=MX4, lda=192, ldas=12, mode=2) == E_MODE
    assert _grouped(lib, E=0) == E_SHAPE
    assert _grouped(lib, E=4097) == E_SHAPE
    assert _grouped(lib, M=-1) == E_SHAPE
    assert _grouped(lib, d=_mxdesc(K=96), lda=96, ldas=4) == E_SHAPE         # K % 64 != 0 (e4m3)
    assert _grouped(lib, d=_mxdesc(K=320, fmt=MX4), af=MX4, lda=160, ldas=12, mode=1) == E_SHAPE  # K % 128
    assert _grouped(lib, M=0, a=None, e=None, off=None, out=None) == OK
    assert _grouped(lib, off=None) == E_NULL
    assert _grouped(lib, w=None) == E_NULL
    assert _grouped(lib, ldas=9) == E_SHAPE
    assert _grouped(lib, ldas=14) == E_ALIGN                   # scale rows are read a dword at a time
    assert _grouped(lib, e=FAKE + 2) == E_ALIGN
    assert _grouped(lib, off=FAKE + 4) == E_ALIGN
    assert _grouped(lib, lda=328) == E_ALIGN
    assert _grouped(lib, w=FAKE + 16) == E_ALIGN
    assert _grouped(lib, bias=FAKE + 2) == E_ALIGN


def test_rmsnorm_quantize_validation(lib):
    f = lambda **kw: lib.qgemm_rmsnorm_quantize_rows(
        kw.get("x", FAKE), kw.get("M", 4), kw.get("K", 64), kw.get("ldx", 64), kw.get("g", FAKE),
        kw.get("eps", 1e-6), kw.get("fmt", INT8), kw.get("gran", ROW), kw.get("q", FAKE), kw.get("ldq", 64),
        kw.get("s", FAKE), kw.get("z", None), None)
    assert f(fmt=MX, gran=BLK) == E_MODE
    assert f(gran=TENSOR) == E_MODE
    assert f(eps=-1.0) == E_MODE
    assert f(eps=float("nan")) == E_MODE
    assert f(eps=float("inf")) == E_MODE
    assert f(K=0) == E_SHAPE
    assert f(M=0, x=None, g=None, q=None, s=None) == OK
    assert f(g=None) == E_NULL
    assert f(fmt=UINT8) == E_NULL                         # missing zero points
    assert f(ldx=32) == E_SHAPE
    assert f(ldq=72) == E_ALIGN
    assert f(g=FAKE + 2) == E_ALIGN


def test_prepack_validation(lib):
    d = L.WDesc()
    f = lambda **kw: lib.qgemm_prepack_weights(kw.get("w", FAKE), kw.get("N", 64), kw.get("K", 64),
                                               kw.get("ldw", 64), kw.get("fmt", INT8), kw.get("gran", ROW),
                                               kw.get("p", 0x100000), kw.get("pb", 1 << 20), ctypes.byref(d),
                                               kw.get("ws", None), kw.get("wsb", 0), None)
    assert f(fmt=UINT8) == E_MODE
    assert f(fmt=MX, gran=ROW) == E_MODE
    assert f(fmt=MX, gran=BLK, K=40, ldw=40) == E_SHAPE
    assert f(N=0) == E_SHAPE
    assert f(w=None) == E_NULL
    assert f(ldw=32) == E_SHAPE
    assert f(p=0x100000 + 128) == E_ALIGN
    assert f(pb=100) == E_SHAPE
    assert f(gran=TENSOR) == E_WS
    assert f(fmt=INT4, gran=ROW) == E_MODE
    assert f(fmt=MX4, gran=ROW) == E_MODE
    assert f(fmt=MX4, gran=BLK, K=40, ldw=40) == E_SHAPE
    assert f(fmt=INT8, gran=G64) == E_MODE
    assert f(fmt=INT4, gran=G64, pb=100) == E_SHAPE
    assert d.magic == 0                                   # untouched on error


def _w4desc(**kw):
    nb = 256 * 256 + 4 * 256 * 8
    d = L.WDesc(magic=0x51474D57, version=ABI, fmt=INT4, gran=G64, N=100, K=300, N_pad=256, K_pad=512,
                codes_off=0, scales_off=256 * 256, colsum_off=-1, bytes=nb)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def _run4(lib, d, a=FAKE, lda=304, s=FAKE, gran=ROW, M=8, w=FAKE, out=FAKE, ldo=100, ot=0, bias=None):
    return lib.qgemm_run_w4a8(a, lda, s, gran, M, ctypes.byref(d), w, out, ldo, ot, bias, None, 0, None)


def test_unpack_weights_validation(lib):
    """qgemm_unpack_weights rejects bad arguments before any launch: a missing
    descriptor or buffer, a damaged descriptor, an output the format does not
    have, a leading dimension too small, a misaligned buffer."""
    d = L.WDesc()
    dev = 0x10000000
    un = lib.qgemm_unpack_weights
    assert un(None, dev, dev, 64, None, 0, None, None, 0, None) == E_NULL
    assert un(ctypes.byref(d), None, dev, 64, None, 0, None, None, 0, None) == E_NULL
    assert un(ctypes.byref(d), dev, dev, 64, None, 0, None, None, 0, None) == E_DESC  # zero descriptor
    # a descriptor as qgemm_prepack_weights fills it, for checks that come before the device
    def desc(N, K, fmt, gran, colsum=True):
        nb = lib.qgemm_packed_weight_bytes(N, K, fmt, gran)
        assert nb > 0
        x = L.WDesc()
        x.magic, x.version, x.fmt, x.gran, x.N, x.K = 0x51474D57, ABI, fmt, gran, N, K
        x.N_pad, x.K_pad = (N + 255) // 256 * 256, (K + 255) // 256 * 256
        x.codes_off = 0
        if fmt == INT4:
            x.scales_off = (x.N_pad * x.K_pad // 2 + 255) // 256 * 256
            x.colsum_off = -1
        elif fmt == INT8:
            x.scales_off = (x.N_pad * x.K_pad + 255) // 256 * 256
            x.colsum_off = (x.scales_off + 4 * x.N_pad + 255) // 256 * 256
        else:
            cb = x.K_pad // 2 if fmt == MX4 else x.K_pad
            x.scales_off = (x.N_pad * cb + 255) // 256 * 256
            x.colsum_off = -1
        x.bytes = nb
        return x
    d8, d4, dmx = desc(64, 256, INT8, ROW), desc(64, 256, INT4, G64), desc(64, 256, MX, BLK)
    assert un(ctypes.byref(d8), dev, None, 0, None, 0, None, dev, 8, None) == E_MODE     # no E8M0 in int8
    assert un(ctypes.byref(dmx), dev, None, 0, dev, 0, None, None, 0, None) == E_MODE   # no float scales in MX
    assert un(ctypes.byref(d4), dev, None, 0, None, 0, dev, None, 0, None) == E_MODE    # no column sums in int4
    assert un(ctypes.byref(d8), dev, dev, 255, None, 0, None, None, 0, None) == E_SHAPE   # ld_codes < K
    assert un(ctypes.byref(d4), dev, None, 0, dev, 3, None, None, 0, None) == E_SHAPE     # ld_scales < 4 groups
    assert un(ctypes.byref(dmx), dev, None, 0, None, 0, None, dev, 7, None) == E_SHAPE    # ld_mx < K / 32
    assert un(ctypes.byref(d8), dev + 16, dev, 256, None, 0, None, None, 0, None) == E_ALIGN
    assert un(ctypes.byref(d8), dev, None, 0, dev + 2, 0, None, None, 0, None) == E_ALIGN
    assert un(ctypes.byref(d8), dev, None, 0, None, 0, None, None, 0, None) == OK        # nothing requested
    bad = L.WDesc.from_buffer_copy(d8)
    bad.bytes += 256
    assert un(ctypes.byref(bad), dev, dev, 256, None, 0, None, None, 0, None) == E_DESC


def test_run_w4a8_validation(lib):
    good = _w4desc()
    assert lib.qgemm_packed_weight_bytes(100, 300, INT4, G64) == good.bytes
    assert _run4(lib, _wdesc()) == E_DESC                 # an int8 descriptor
    assert _run4(lib, _w4desc(colsum_off=0)) == E_DESC
    assert _run4(lib, _w4desc(scales_off=256 * 512)) == E_DESC
    assert lib.qgemm_run_w4a8(FAKE, 304, FAKE, ROW, 8, None, FAKE, FAKE, 100, 0, None, None, 0, None) == E_NULL
    assert _run(lib, good) == E_DESC                      # int4 weights through the int8 call
    assert _run4(lib, good, gran=BLK) == E_MODE
    assert _run4(lib, good, ot=2) == E_MODE               # no single integer sum to export
    assert _run4(lib, good, M=-1) == E_SHAPE
    assert _run4(lib, good, M=16 * 65535 + 1) == E_SHAPE
    assert _run4(lib, good, M=0, a=None, s=None, w=None, out=None) == OK
    assert _run4(lib, good, s=None) == E_NULL
    assert _run4(lib, good, lda=288) == E_SHAPE
    assert _run4(lib, good, lda=312) == E_ALIGN
    assert _run4(lib, good, ldo=99) == E_SHAPE
    assert _run4(lib, good, ldo=102) == E_ALIGN
    assert _run4(lib, good, w=FAKE + 16) == E_ALIGN
    assert _run4(lib, good, bias=FAKE + 2) == E_ALIGN
    assert _run4(lib, good, lda=1 << 29, M=17) == E_SHAPE  # 32-bit offsets over a 16-row band
    K = (1 << 27) + 1
    kp = (K + 255) // 256 * 256
    huge = _w4desc(N=16, K=K, K_pad=kp, scales_off=256 * kp // 2,
                   bytes=lib.qgemm_packed_weight_bytes(16, K, INT4, G64))
    assert _run4(lib, huge, lda=kp, M=1) == E_SHAPE


def test_ceiling_validation(lib):
    """The measured-ceiling calls (qgemm_ceiling.h) reject bad arguments before
    any launch: missing buffers, an unknown instruction kind, waves per SIMD
    or trips out of range, misaligned buffers, stream sizes that are not whole
    16-byte loads or whole 16 KB blocks."""
    dev = 0x10000000
    wg, ops_ = ctypes.c_int64(0), ctypes.c_double(0.0)
    shape = lib.qgemm_ceiling_mfma_shape
    assert shape(0, 2, 16, None, ctypes.byref(ops_)) == E_NULL
    assert shape(4, 2, 16, ctypes.byref(wg), ctypes.byref(ops_)) == E_MODE
    assert shape(-1, 2, 16, ctypes.byref(wg), ctypes.byref(ops_)) == E_MODE
    assert shape(0, 3, 16, ctypes.byref(wg), ctypes.byref(ops_)) == E_SHAPE
    assert shape(0, 0, 16, ctypes.byref(wg), ctypes.byref(ops_)) == E_SHAPE
    assert shape(0, 2, 0, ctypes.byref(wg), ctypes.byref(ops_)) == E_SHAPE
    assert shape(0, 2, (1 << 24) + 1, ctypes.byref(wg), ctypes.byref(ops_)) == E_SHAPE
    mf = lib.qgemm_ceiling_mfma
    assert mf(0, 2, 16, None, dev, dev, None, None) == E_NULL
    assert mf(0, 2, 16, dev, dev, None, None, None) == E_NULL
    assert mf(5, 2, 16, dev, dev, dev, None, None) == E_MODE
    assert mf(1, 2, 0, dev, dev, dev, None, None) == E_SHAPE
    assert mf(1, 2, 16, dev + 16, dev, dev, None, None) == E_ALIGN
    assert mf(1, 2, 16, dev, dev + 8, dev, None, None) == E_ALIGN
    assert mf(1, 2, 16, dev, dev, dev + 2, None, None) == E_ALIGN
    assert mf(1, 2, 16, dev, dev, dev, dev + 4, None) == E_ALIGN
    st = lib.qgemm_ceiling_stream
    assert st(None, 1024, 16384, dev, None) == E_NULL
    assert st(dev, 1024, 16384, None, None) == E_NULL
    assert st(dev, 1000, 16384, dev, None) == E_SHAPE      # not whole 16-byte loads
    assert st(dev, -16, 16384, dev, None) == E_SHAPE
    assert st(dev, 1024, 8192, dev, None) == E_SHAPE       # block under 16 KB
    assert st(dev, 1024, 20000, dev, None) == E_SHAPE      # not whole 16 KB
    assert st(dev, 1024, (1 << 20) + 16384, dev, None) == E_SHAPE
    assert st(dev + 8, 1024, 16384, dev, None) == E_ALIGN
    assert st(dev, 0, 16384, dev, None) == OK                # nothing to read


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_no_device_is_an_error_not_a_fallback(lib):
    # fully valid arguments: the only thing missing is a gfx950
    assert _q(lib) == E_DEVICE
    assert _run(lib, _wdesc()) == E_DEVICE
    assert _run4(lib, _w4desc()) == E_DEVICE
    assert _grouped(lib) == E_DEVICE
    assert lib.qgemm_rmsnorm_quantize_rows(FAKE, 4, 64, 64, FAKE, 1e-6, INT8, ROW, FAKE, 64, FAKE, None,
                                           None) == E_DEVICE
    wg, ops_ = ctypes.c_int64(0), ctypes.c_double(0.0)
    assert lib.qgemm_ceiling_mfma_shape(0, 2, 16, ctypes.byref(wg), ctypes.byref(ops_)) == E_DEVICE
    assert lib.qgemm_ceiling_mfma(0, 2, 16, FAKE, FAKE, FAKE, None, None) == E_DEVICE
    assert lib.qgemm_ceiling_stream(FAKE, 1024, 16384, FAKE, None) == E_DEVICE


def test_packed_int8_block_layout_round_trip():
    """The Python view of packed int8 codes inverts the documented block layout:
    block (n // 16, k // 64) at ((n // 16) * (K_pad // 64) + k // 64) KB, code (n, k)
    at 256 * ((k % 64) // 16) + 16 * (n % 16) + k % 16 inside it."""
    import torch
    from block_scaled_quantized_qgemm_amd.ops import unblock_int8_codes
    n_pad, k_pad = 32, 256
    ref = torch.randint(0, 256, (n_pad, k_pad), dtype=torch.int32).to(torch.uint8)
    raw = torch.zeros(n_pad * k_pad, dtype=torch.uint8)
    kb = k_pad // 64
    for n in range(n_pad):
        for k in range(k_pad):
            off = ((n // 16) * kb + k // 64) * 1024 + 256 * ((k % 64) // 16) + 16 * (n % 16) + k % 16
            raw[off] = ref[n, k]
    assert torch.equal(unblock_int8_codes(raw, n_pad, k_pad), ref)


def test_packed_mx8_block_layout_round_trip():
    """The Python view of packed e4m3 weight codes inverts the documented block
    layout: code (n, k) at ((n // 16) * (K_pad // 64) + k // 64) KB + 64 * (n % 16)
    + k % 64."""
    import torch
    from block_scaled_quantized_qgemm_amd.ops import unblock_mx8_codes
    n_pad, k_pad = 48, 256
    ref = torch.randint(0, 256, (n_pad, k_pad), dtype=torch.int32).to(torch.uint8)
    raw = torch.zeros(n_pad * k_pad, dtype=torch.uint8)
    kb = k_pad // 64
    for n in range(n_pad):
        for k in range(k_pad):
            raw[((n // 16) * kb + k // 64) * 1024 + 64 * (n % 16) + k % 64] = ref[n, k]
    assert torch.equal(unblock_mx8_codes(raw, n_pad, k_pad), ref)


def test_packed_int4_block_layout_round_trip():
    """The Python view of packed int4 codes inverts the documented layout:
    block (n // 16, k // 128) at ((n // 16) * (K_pad // 128) + k // 128) KB;
    lane 16 c + n % 16 (c = (k % 64) // 16) owns 16 bytes, 8 per group of 64;
    code kk = k % 16 in byte 4 (kk // 8) + kk % 4, low nibble iff kk % 8 < 4."""
    import torch
    from block_scaled_quantized_qgemm_amd.ops import unblock_int4_codes
    n_pad, k_pad = 32, 256
    ref = torch.randint(-8, 8, (n_pad, k_pad), dtype=torch.int32)
    raw = [0] * (n_pad * k_pad // 2)
    pb = k_pad // 128
    for n in range(n_pad):
        for k in range(k_pad):
            c, kk = (k % 64) // 16, k % 16
            off = ((n // 16) * pb + k // 128) * 1024 + 16 * (16 * c + n % 16) + 8 * ((k % 128) // 64) \
                + 4 * (kk // 8) + kk % 4
            nib = int(ref[n, k]) & 0xF
            raw[off] |= nib if kk % 8 < 4 else nib << 4
    got = unblock_int4_codes(torch.tensor(raw, dtype=torch.uint8), n_pad, k_pad)
    assert torch.equal(got.to(torch.int32), ref)
