"""MI355X-native quantized linear layer (int8 per-token / per-channel, MXFP8,
and int8 x int4 with per-group-64 weight scales).

The compute path is the HIP library ``libqgemm.so`` (C ABI in
``include/qgemm.h``); ``ops`` is its thin torch binding with the same names:
``qgemm_quantize_rows``, ``qgemm_rmsnorm_quantize_rows``,
``qgemm_prepack_weights``, ``qgemm_run``, ``qgemm_run_mx``, ``qgemm_run_w4a8``. Importing this package loads neither torch nor the library;
the names below resolve on first use.
"""

_BINDING = {
    "qgemm_quantize_rows", "qgemm_rmsnorm_quantize_rows", "qgemm_prepack_weights", "qgemm_run", "qgemm_run_mx", "qgemm_run_w4a8",
    "qgemm_workspace_bytes", "qgemm_packed_weight_bytes", "QgemmError", "QuantizedRows", "PackedWeights",
    "FMT_INT8_SYM", "FMT_UINT8_ASYM", "FMT_MXFP8_E4M3", "FMT_INT4_SYM", "FMT_MXFP4_E2M1", "GRAN_TENSOR", "GRAN_ROW",
    "GRAN_BLOCK32", "GRAN_GROUP64",
    "OUT_F32", "OUT_BF16", "OUT_I32", "MX_EXACT", "MX_SCALED_MFMA",
}


def __getattr__(name):
    if name in _BINDING:
        from . import ops
        return getattr(ops, name)
    raise AttributeError(name)
