"""ctypes loader for libqgemm.so (the C ABI declared in include/qgemm.h, and
the measured-ceiling calls of include/qgemm_ceiling.h).

torch is imported first on purpose: the library then binds to the HIP runtime
torch already loaded (same soname), so torch's streams and allocations are
valid handles for it. A missing library is an error, never a fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede loading the HIP library)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqgemm.so")

c_i64 = ctypes.c_int64
c_int = ctypes.c_int
c_size = ctypes.c_size_t
c_vp = ctypes.c_void_p


class WDesc(ctypes.Structure):
    """Mirror of ``qgemm_wdesc``."""
    _fields_ = [
        ("magic", ctypes.c_uint32), ("version", ctypes.c_uint32),
        ("fmt", ctypes.c_int32), ("gran", ctypes.c_int32),
        ("N", c_i64), ("K", c_i64), ("N_pad", c_i64), ("K_pad", c_i64),
        ("codes_off", c_i64), ("scales_off", c_i64), ("colsum_off", c_i64), ("bytes", c_i64),
    ]


# every symbol include/*.h declares, with its C signature
SIGNATURES = {
    "qgemm_abi_version": (c_int, []),
    "qgemm_status_string": (ctypes.c_char_p, [c_int]),
    "qgemm_packed_weight_bytes": (c_size, [c_i64, c_i64, c_int, c_int]),
    "qgemm_workspace_bytes": (c_size, [c_i64, c_i64, c_int, c_int]),
    "qgemm_quantize_rows": (c_int, [c_vp, c_i64, c_i64, c_i64, c_int, c_int, c_vp, c_i64,
                                    c_vp, c_vp, c_vp, c_i64, c_vp, c_size, c_vp]),
    "qgemm_quantize_rows_noalloc": (c_int, [c_vp, c_i64, c_i64, c_i64, c_int, c_int, c_vp, c_i64,
                                            c_vp, c_vp, c_vp, c_i64, c_vp]),
    "qgemm_prepack_weights": (c_int, [c_vp, c_i64, c_i64, c_i64, c_int, c_int, c_vp, c_size,
                                      ctypes.POINTER(WDesc), c_vp, c_size, c_vp]),
    "qgemm_rmsnorm_quantize_rows": (c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, ctypes.c_float, c_int, c_int,
                                            c_vp, c_i64, c_vp, c_vp, c_vp]),
    "qgemm_unpack_weights": (c_int, [ctypes.POINTER(WDesc), c_vp, c_vp, c_i64, c_vp, c_i64, c_vp, c_vp, c_i64,
                                     c_vp]),
    "qgemm_run": (c_int, [c_vp, c_i64, c_vp, c_vp, c_int, c_int, c_i64, ctypes.POINTER(WDesc), c_vp,
                          c_vp, c_i64, c_int, c_vp, c_vp, c_size, c_vp]),
    "qgemm_run_mx": (c_int, [c_vp, c_i64, c_vp, c_i64, c_int, c_i64, ctypes.POINTER(WDesc), c_vp,
                             c_vp, c_i64, c_int, c_vp, c_vp, c_size, c_vp]),
    "qgemm_run_mx_grouped": (c_int, [c_vp, c_i64, c_vp, c_i64, c_int, c_i64, c_vp, c_i64,
                                     ctypes.POINTER(WDesc), c_vp, c_vp, c_i64, c_int, c_vp, c_vp, c_size, c_vp]),
    "qgemm_run_w4a8": (c_int, [c_vp, c_i64, c_vp, c_int, c_i64, ctypes.POINTER(WDesc), c_vp,
                               c_vp, c_i64, c_int, c_vp, c_vp, c_size, c_vp]),
    # include/qgemm_ceiling.h
    "qgemm_ceiling_mfma_shape": (c_int, [c_int, c_int, c_i64, ctypes.POINTER(c_i64), ctypes.POINTER(ctypes.c_double)]),
    "qgemm_ceiling_mfma": (c_int, [c_int, c_int, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "qgemm_ceiling_stream": (c_int, [c_vp, c_i64, c_i64, c_vp, c_vp]),
}

_lib = None


def load():
    """Load libqgemm.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                "(or python -m block_scaled_quantized_qgemm_amd.build)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib
