"""CPU oracle for the quantized linear layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package. It imports nothing from the
HIP product path (``block_scaled_quantized_qgemm_amd``), and the product
path never imports it. See ``qgemm_oracle`` for the definitions and the page
passages each one follows.
"""
from .qgemm_oracle import *  # noqa: F401,F403
from .qgemm_oracle import (  # noqa: F401
    quantize_sym_int8, quantize_asym_uint8, prepare_weights_int8, k_limit,
    int_gemm, int_gemm_entries, epilogue, quantized_linear, bf16_to_f32,
    ceil_to_ue8m0, e8m0_value, e4m3_decode, e4m3_encode_rne, quantize_mx,
    mx_dequantize, mx_gemm_ref, mx_gemm_ref_entries, mx_grouped_gemm_ref, E4M3_VALUES,
)
from . import metrics  # noqa: F401
