"""Drive the C ABI built with the sanitizers against the stubbed HIP runtime
(tests/asan/hip_stubs.cpp) as if a GPU were present: valid calls must reach
exactly one launcher (and the memsets the layout needs), invalid ones none.
Device pointers are fake aligned addresses; nothing dereferences them.

usage: python device_checks.py LIB.so {gfx950|other} DESC_FILE
(gfx950 writes the weight descriptors it prepares to DESC_FILE; another
device reads them from there, since its prepack calls are refused.)
"""
import ctypes
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import block_scaled_quantized_qgemm_amd._lib as L  # noqa: E402

L.LIB_PATH = sys.argv[1]
MODE = sys.argv[2]
DESC_FILE = sys.argv[3]
lib = L.load()
launches = ctypes.c_int.in_dll(lib, "qg_stub_launches")
memsets = ctypes.c_int.in_dll(lib, "qg_stub_memsets")

OK, E_NULL, E_SHAPE, E_MODE, E_ALIGN, E_OVERFLOW, E_DEVICE, E_DESC, E_WS = 0, -1, -2, -3, -4, -5, -6, -7, -8
INT8, UINT8, MX, INT4, MX4 = 0, 1, 2, 3, 4
TENSOR, ROW, BLK, G64 = 0, 1, 2, 3
DEV = [0x10000000 + 0x1000000 * i for i in range(16)]  # fake, 256-byte aligned device buffers
failures = []


def expect(name, rc, want, n_launch, n_memset=0):
    """rc must be `want` (on a non-gfx950 device every valid call is E_DEVICE)
    and the call must have launched n_launch kernels and n_memset memsets."""
    if MODE != "gfx950" and want == OK and n_launch > 0:
        want, n_launch, n_memset = E_DEVICE, 0, 0
    got_l, got_m = launches.value, memsets.value
    launches.value = memsets.value = 0
    if rc != want or got_l != n_launch or got_m != n_memset:
        failures.append(f"{name}: rc {rc} (want {want}), launches {got_l} (want {n_launch}), "
                        f"memsets {got_m} (want {n_memset})")


def quant(M, K, fmt, gran, zp=None, mx=None, ld_mx=0, ws=None, wsb=0, ldq=None, x=DEV[0]):
    return lib.qgemm_quantize_rows(x, M, K, K, fmt, gran, DEV[1], ldq or (K + 15) // 16 * 16, DEV[2], zp, mx,
                                   ld_mx, ws, wsb, None)


expect("int8 per row", quant(4, 256, INT8, ROW), OK, 1)
expect("uint8 per row", quant(4, 256, UINT8, ROW, zp=DEV[3]), OK, 1)
expect("uint8 per row without zero points", quant(4, 256, UINT8, ROW), E_NULL, 0)
need = lib.qgemm_workspace_bytes(4, 256, INT8, TENSOR)
expect("int8 per tensor", quant(4, 256, INT8, TENSOR, ws=DEV[4], wsb=need), OK, 1)
expect("int8 per tensor, short workspace", quant(4, 256, INT8, TENSOR, ws=DEV[4], wsb=need - 4), E_WS, 0)
expect("empty M", quant(0, 256, INT8, ROW), OK, 0)
expect("K % 32 for MX", quant(4, 100, MX, BLK, mx=DEV[5], ld_mx=4), E_SHAPE, 0)
expect("MX e4m3", quant(4, 256, MX, BLK, mx=DEV[5], ld_mx=8), OK, 1)
expect("MX e2m1", quant(4, 256, MX4, BLK, mx=DEV[5], ld_mx=8, ldq=128), OK, 1)
expect("null x", quant(4, 256, INT8, ROW, x=None), E_NULL, 0)

na = lib.qgemm_quantize_rows_noalloc
expect("no-alloc per tensor", na(DEV[0], 4, 256, 256, UINT8, TENSOR, DEV[1], 256, DEV[2], DEV[3], None, 0, None), OK, 1)
expect("no-alloc beyond its array", na(DEV[0], 300000, 256, 256, INT8, TENSOR, DEV[1], 256, DEV[2], None, None, 0,
                                       None), E_WS, 0)

rq = lib.qgemm_rmsnorm_quantize_rows
expect("rmsnorm int8", rq(DEV[0], 4, 256, 256, DEV[6], ctypes.c_float(1e-6), INT8, ROW, DEV[1], 256, DEV[2], None,
                          None), OK, 1)
expect("rmsnorm without gamma", rq(DEV[0], 4, 256, 256, None, ctypes.c_float(1e-6), INT8, ROW, DEV[1], 256, DEV[2],
                                   None, None), E_NULL, 0)


def prepack(N, K, fmt, gran, short=0):
    d = L.WDesc()
    nb = lib.qgemm_packed_weight_bytes(N, K, fmt, gran)
    rc = lib.qgemm_prepack_weights(DEV[7], N, K, K, fmt, gran, DEV[8], nb - short, ctypes.byref(d), None, 0, None)
    return rc, d, nb


# prepack clears the packed buffer's padding (int8, int4) and sets the E8M0
# padding (MX) before its one quantize launch
rc, d8, nb = prepack(64, 256, INT8, ROW)
expect("prepack int8", rc, OK, 1, 1)
if MODE == "gfx950" and not (d8.N == 64 and d8.K == 256 and d8.K_pad == 256 and d8.bytes == nb):
    failures.append(f"int8 descriptor: N {d8.N} K {d8.K} K_pad {d8.K_pad} bytes {d8.bytes} (packed size {nb})")
expect("prepack int8, short buffer", prepack(64, 256, INT8, ROW, short=256)[0], E_SHAPE, 0)
rc, dmx, _ = prepack(64, 256, MX, BLK)
expect("prepack MX", rc, OK, 1, 2)
rc, d4, _ = prepack(64, 256, INT4, G64)
expect("prepack int4", rc, OK, 1, 1)
rc, dbig, _ = prepack(16, 70000, INT8, ROW)
expect("prepack int8, K = 70000", rc, OK, 1, 1)
descs = [d8, dmx, d4, dbig]
if MODE == "gfx950":
    with open(DESC_FILE, "wb") as f:
        for d in descs:
            f.write(bytes(d))
else:
    with open(DESC_FILE, "rb") as f:
        raw = f.read()
    n = ctypes.sizeof(L.WDesc)
    d8, dmx, d4, dbig = [L.WDesc.from_buffer_copy(raw[i * n:(i + 1) * n]) for i in range(4)]


def run(desc, fmt=INT8, zp=None, M=4, lda=None, out_type=0, bias=None):
    return lib.qgemm_run(DEV[9], lda or desc.K_pad, DEV[10], zp, fmt, ROW, M, ctypes.byref(desc), DEV[8], DEV[11], 64,
                         out_type, bias, None, 0, None)


expect("run int8", run(d8), OK, 1)
expect("run uint8", run(d8, UINT8, DEV[3]), OK, 1)
expect("run int32 with a bias", run(d8, out_type=2, bias=DEV[12]), E_MODE, 0)
expect("run lda < K", run(d8, lda=128), E_SHAPE, 0)
bad = L.WDesc.from_buffer_copy(d8)
bad.magic ^= 1
expect("run with a damaged descriptor", run(bad), E_DESC, 0)
expect("run MX weights through the int8 call", run(dmx), E_DESC, 0)
expect("run int8, K = 70000", run(dbig), OK, 1)
expect("run uint8, K = 70000 (int32 overflow)", run(dbig, UINT8, DEV[3]), E_OVERFLOW, 0)

rm = lib.qgemm_run_mx
expect("run MX exact", rm(DEV[9], 256, DEV[5], 8, MX, 4, ctypes.byref(dmx), DEV[8], DEV[11], 64, 0, None, None, 0,
                          None), OK, 1)
expect("run MX with int8 weights", rm(DEV[9], 256, DEV[5], 8, MX, 4, ctypes.byref(d8), DEV[8], DEV[11], 64, 0, None,
                                      None, 0, None), E_DESC, 0)
rg = lib.qgemm_run_mx_grouped
expect("grouped MX", rg(DEV[9], 256, DEV[5], 8, MX, 4, DEV[13], 2, ctypes.byref(dmx), DEV[8], DEV[11], 64, 0, None,
                        None, 0, None), OK, 1)
expect("grouped MX without offsets", rg(DEV[9], 256, DEV[5], 8, MX, 4, None, 2, ctypes.byref(dmx), DEV[8], DEV[11],
                                        64, 0, None, None, 0, None), E_NULL, 0)
rw = lib.qgemm_run_w4a8
expect("run W4A8", rw(DEV[9], 256, DEV[10], ROW, 4, ctypes.byref(d4), DEV[8], DEV[11], 64, 0, None, None, 0, None),
       OK, 1)
expect("run W4A8 int32 out", rw(DEV[9], 256, DEV[10], ROW, 4, ctypes.byref(d4), DEV[8], DEV[11], 64, 2, None, None, 0,
                                None), E_MODE, 0)

un = lib.qgemm_unpack_weights
expect("unpack int8: codes, scales, column sums",
       un(ctypes.byref(d8), DEV[8], DEV[14], 256, DEV[15], 0, DEV[13], None, 0, None), OK, 3)
expect("unpack int4: codes, scales", un(ctypes.byref(d4), DEV[8], DEV[14], 256, DEV[15], 4, None, None, 0, None),
       OK, 2)
expect("unpack MX: codes, E8M0", un(ctypes.byref(dmx), DEV[8], DEV[14], 256, None, 0, None, DEV[15], 8, None), OK, 2)
expect("unpack nothing requested", un(ctypes.byref(d8), DEV[8], None, 0, None, 0, None, None, 0, None), OK, 0)
expect("unpack MX with float scales", un(ctypes.byref(dmx), DEV[8], None, 0, DEV[15], 0, None, None, 0, None),
       E_MODE, 0)

# measured ceilings: one launch each; the shape call launches nothing and
# reports one workgroup per CU (the stub has 256) and the operation count
wg, ops_ = ctypes.c_int64(0), ctypes.c_double(0.0)
expect("ceiling shape", lib.qgemm_ceiling_mfma_shape(0, 2, 100, ctypes.byref(wg), ctypes.byref(ops_)),
       OK if MODE == "gfx950" else E_DEVICE, 0)
if MODE == "gfx950" and (wg.value != 256 or ops_.value != 2.0 * 16 * 16 * 64 * 8 * 100 * 4 * 2 * 256):
    failures.append(f"ceiling shape: {wg.value} workgroups, {ops_.value} operations")
expect("ceiling mfma", lib.qgemm_ceiling_mfma(1, 2, 100, DEV[0], DEV[1], DEV[2], DEV[3], None), OK, 1)
expect("ceiling mfma, bad kind", lib.qgemm_ceiling_mfma(7, 2, 100, DEV[0], DEV[1], DEV[2], None, None), E_MODE, 0)
expect("ceiling stream", lib.qgemm_ceiling_stream(DEV[0], 1 << 20, 1 << 16, DEV[2], None), OK, 1)
expect("ceiling stream, empty", lib.qgemm_ceiling_stream(DEV[0], 0, 1 << 16, DEV[2], None), OK, 0)

if failures:
    print("\n".join(failures))
    sys.exit(1)
print(f"device checks passed ({MODE})")
