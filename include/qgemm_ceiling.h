/*
 * qgemm_ceiling.h -- measured ceilings for the roofline report.
 *
 * Not part of the quantized GEMM path. A roofline divides a kernel's
 * achieved rate by the part's published peak; these calls measure, on the
 * device at hand, what the two resources the GEMM kernels are bound by
 * deliver when nothing else runs:
 *   - how fast the matrix cores issue the instruction a GEMM kernel uses, on
 *     that GEMM's own operand bytes, in the same wave arrangement (the part
 *     is power-limited, so the clock it holds depends on the operand bits);
 *   - how fast a plain stream reads a buffer out of HBM.
 * Both launch on `stream` and return at once; the caller times them (HIP
 * events) and divides qgemm_ceiling_mfma_shape's operation count, or the
 * streamed bytes, by the time. Status codes are those of qgemm.h; every
 * argument is validated before anything is launched. Only the library's own
 * static LDS is used: nothing is allocated.
 */
#ifndef QGEMM_CEILING_H
#define QGEMM_CEILING_H

#include "qgemm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* The matrix-core instruction a ceiling measurement issues. */
typedef enum {
  QGEMM_CEIL_I8 = 0,        /* v_mfma_i32_16x16x64_i8: the int8 GEMM kernels' instruction        */
  QGEMM_CEIL_F8_SCALED = 1, /* v_mfma_scale_f32_32x32x64_f8f6f4, e4m3 x e4m3 (MX on the fp8 cores) */
  QGEMM_CEIL_F4_SCALED = 2, /* the same instruction, e2m1 x e2m1 (MXFP4 on the fp4 cores)          */
  QGEMM_CEIL_BF16 = 3       /* v_mfma_f32_32x32x16_bf16: the exact MX mode's instruction            */
} qgemm_ceiling_kind;

/* Bytes qgemm_ceiling_mfma reads from its operand buffers. */
#define QGEMM_CEILING_A_BYTES 16384
#define QGEMM_CEILING_B_BYTES 2048

/*
 * qgemm_ceiling_mfma_shape -- the launch qgemm_ceiling_mfma makes on the
 * current device: `*workgroups` (one per compute unit; qgemm_ceiling_mfma's
 * `clocks` holds 2 * *workgroups entries) and `*ops`, the operations
 * (2 * M * N * K per instruction) one launch performs.
 * Errors: QGEMM_E_NULL, QGEMM_E_MODE (kind), QGEMM_E_SHAPE (waves_per_simd not
 * 1 or 2, trips outside [1, 2^24]), QGEMM_E_DEVICE.
 */
int qgemm_ceiling_mfma_shape(int kind, int waves_per_simd, int64_t trips, int64_t* workgroups, double* ops);

/*
 * qgemm_ceiling_mfma -- issue trips * 8 independent instructions of `kind` on
 * every wave of one workgroup per compute unit, waves_per_simd waves on each
 * SIMD, with nothing else in the loop.
 *   a_ops   device, QGEMM_CEILING_A_BYTES, 32-byte aligned: lane l of every
 *           wave takes 8 operand sets of 32 bytes at a_ops + 32 * (8 l + q)
 *   b_ops   device, QGEMM_CEILING_B_BYTES, 32-byte aligned: one 32-byte set
 *           at b_ops + 32 l
 *           The bytes are codes as the GEMM stores them: int8 for
 *           QGEMM_CEIL_I8 (the first 16 bytes of a set), e4m3 for
 *           F8_SCALED and BF16 (BF16 converts the first 8 codes of a set to
 *           bf16, as the exact MX mode does), e2m1 pairs for F4_SCALED. The
 *           block scales are 2^0.
 *   sink    device int32, 4-byte aligned: written only if the results hash
 *           to one fixed value, so the work cannot be optimised away.
 *   clocks  device int64 [2 * workgroups] or NULL, 8-byte aligned: per
 *           workgroup, the shader-clock ticks and the 100 MHz real-time ticks
 *           its first wave spent in the loop (their ratio is the clock the
 *           part held).
 * Errors: QGEMM_E_NULL, QGEMM_E_MODE, QGEMM_E_SHAPE (as qgemm_ceiling_mfma_shape),
 * QGEMM_E_ALIGN, QGEMM_E_DEVICE, QGEMM_E_HIP.
 */
int qgemm_ceiling_mfma(int kind, int waves_per_simd, int64_t trips, const void* a_ops, const void* b_ops,
                       int32_t* sink, int64_t* clocks, void* stream);

/*
 * qgemm_ceiling_stream -- read `bytes` of `src` once: one workgroup of 256
 * threads per `block_bytes` (16-byte non-temporal loads, 16 in flight per
 * thread when block_bytes is a multiple of 64 KB, else 4).
 *   src          device, 16-byte aligned, `bytes` long
 *   bytes        a multiple of 16, 0 .. 2^40 (0: nothing is launched)
 *   block_bytes  a multiple of 16384 in [16384, 2^20], with at most 2^31 - 1
 *                blocks
 *   sink         device int32, as in qgemm_ceiling_mfma
 * Errors: QGEMM_E_NULL, QGEMM_E_SHAPE, QGEMM_E_ALIGN, QGEMM_E_DEVICE, QGEMM_E_HIP.
 */
int qgemm_ceiling_stream(const void* src, int64_t bytes, int64_t block_bytes, int32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_CEILING_H */
