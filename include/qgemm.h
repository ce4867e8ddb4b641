/*
 * qgemm.h -- C ABI of the MI355X (gfx950) quantized linear-layer library.
 *
 * One hot path: dynamic per-token activation quantization, an int8 x int8
 * GEMM accumulated exactly in int32, and a dequantization epilogue that
 * applies s_a * s_w once per output and subtracts z_a * colsum(W_q) for
 * asymmetric activations; plus the MX variant (e4m3 or e2m1 data, one E8M0
 * scale per 32 K-elements), by default in an exact mode on the bf16 matrix
 * cores (every product and block scale exact, float32 sums), optionally on
 * the block-scaled fp8/fp4 matrix cores (faster, looser; see qgemm_run_mx).
 *
 * Pages the operations follow (titles as they appear on the pages):
 *   [D98]  "100 Days of GPU -- Day 98: Quantization and sparsity"
 *   [TL27] "TileLang tutorial, chapter 27: low-precision quantization"
 *   [SK]   "Skill: Write an INT8 Quantized Kernel"
 *   [AQ]   "Activation Quantization Architecture, in depth"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named "device" are HIP device allocations on the current
 *   device; the caller allocates and owns every buffer, including the
 *   workspace. The library allocates no device memory and keeps no state
 *   beyond a per-device cache of "is this a gfx950" and of its compute-unit
 *   count, and a 1 MiB static device array per GPU that only
 *   qgemm_quantize_rows_noalloc uses.
 * - Matrices are row-major with an explicit leading dimension in ELEMENTS.
 *   Activations are [M, K] (one row per token); weights are [N, K] (one row
 *   per output channel, K contiguous); outputs are [M, N].
 * - `stream` is a hipStream_t (NULL = the null stream), borrowed for the call.
 *   Every call is asynchronous: a return of QGEMM_OK means the arguments were
 *   valid and the kernels were launched; device faults surface at the
 *   caller's next synchronization.
 * - Every argument is validated before anything is launched, so an error
 *   return leaves every output untouched. Nothing aborts or throws.
 * - M == 0 is a valid empty call (nothing is launched). N and K must be >= 1.
 * - Unsupported devices are an error (QGEMM_E_DEVICE): there is no fallback
 *   path, and a block-scaled call is never served by a kernel that would
 *   drop its scales ([TL27] 4.2(d)).
 * - Non-finite inputs (NaN, Inf) are not supported; outputs are then
 *   unspecified.
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QGEMM_ABI_VERSION 9
#define QGEMM_WDESC_MAGIC 0x51474d57u /* "WMGQ" */

/* Status codes. Every entry point returns one of these. */
typedef enum {
  QGEMM_OK = 0,
  QGEMM_E_NULL = -1,      /* a required pointer is NULL                                    */
  QGEMM_E_SHAPE = -2,     /* a size or leading dimension is out of range                   */
  QGEMM_E_MODE = -3,      /* unsupported format / granularity / output combination         */
  QGEMM_E_ALIGN = -4,     /* a pointer or leading dimension is not aligned as documented   */
  QGEMM_E_OVERFLOW = -5,  /* K too large for an exact int32 accumulator                    */
  QGEMM_E_DEVICE = -6,    /* the current device is not a gfx950                            */
  QGEMM_E_UNSUPPORTED_DEVICE = QGEMM_E_DEVICE, /* the same code under its longer name        */
  QGEMM_E_DESC = -7,      /* the weight descriptor is invalid or does not fit the call     */
  QGEMM_E_WORKSPACE = -8, /* workspace missing or smaller than qgemm_workspace_bytes()     */
  QGEMM_E_HIP = -9        /* a HIP runtime call or a kernel launch failed                  */
} qgemm_status;

/* Quantized formats. */
typedef enum {
  /* Symmetric int8, codes in [-127, 127], x = q * s.
   * [D98] "What a scale actually promises"; [AQ] "The quantizer itself". */
  QGEMM_FMT_INT8_SYM = 0,
  /* Asymmetric uint8 with zero point, codes in [0, 255], x = (q - z) * s.
   * [SK] "Required reasoning process" step 1; [AQ] "The quantizer itself". */
  QGEMM_FMT_UINT8_ASYM = 1,
  /* OCP e4m3fn data with one E8M0 power-of-two scale per 32 K-elements.
   * [TL27] sections 2.2 and 2.3. */
  QGEMM_FMT_MXFP8_E4M3 = 2,
  /* Symmetric int4 weights, codes in [-8, 7], x = q * s with one scale per
   * group of 64 consecutive K-elements of a row (weights only).
   * [TL27] sections 2.4 (s = absmax / 7, clip to [-8, 7]), 3.3(c) and 5.1
   * (int8 activations times int4 weights in groups of 64). */
  QGEMM_FMT_INT4_SYM = 3,
  /* fp4 e2m1 data, two codes per byte (element 2i in the low nibble), with
   * one E8M0 power-of-two scale per 32 K-elements. [TL27] sections 1.2 and 8
   * (e2m1, u = 2^-2), 2.3 (the MX block and E8M0), 3.1 (the packed e2m1 storage). */
  QGEMM_FMT_MXFP4_E2M1 = 4
} qgemm_format;

/* Scale granularity. */
typedef enum {
  QGEMM_GRAN_TENSOR = 0,  /* one scale (and zero point) for the whole matrix          */
  QGEMM_GRAN_ROW = 1,     /* one per row: per token for A, per output channel for W   */
  QGEMM_GRAN_BLOCK32 = 2, /* one per 32 contiguous K-elements of a row (MX only)      */
  QGEMM_GRAN_GROUP64 = 3  /* one per 64 contiguous K-elements of a row (INT4 only)    */
} qgemm_granularity;

/* Output element type of qgemm_run. */
typedef enum {
  QGEMM_OUT_F32 = 0,   /* float32                                                    */
  QGEMM_OUT_BF16 = 1,  /* bfloat16, round to nearest even of the float32 result       */
  QGEMM_OUT_I32 = 2    /* int32: the corrected sum C = sum_k (q_a - z_a) * q_w,
                          before scaling (for exact checks)                          */
} qgemm_out_type;

/*
 * How qgemm_run_mx evaluates the block-scaled product (both apply every
 * 32-element block's own pair of scales inside the K loop).
 */
typedef enum {
  /* Exact products: each e4m3 value is multiplied by its block's power-of-two
   * scale on the way into on-chip memory -- an exact operation whose result a
   * bfloat16 holds exactly -- and the bf16 matrix cores form every product
   * exactly and sum in float32. Error: float32 summation only. */
  QGEMM_MX_EXACT = 0,
  /* gfx950 block-scaled matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4),
   * fed the codes and one E8M0 byte per lane and block. For e4m3: twice the
   * peak rate of QGEMM_MX_EXACT, but inside each group of 8 consecutive K the
   * hardware aligns the products to the largest one and drops the bits more
   * than 13 binades below it (measured), so
   * |out - exact| <= 2^-10 * sum_k |a_k w_k| plus float32 summation. For
   * e2m1 x e2m1: four times the exact mode's peak and float32 sums only. A
   * mixed pair (e4m3 x e2m1 either way) has the e4m3 bound. */
  QGEMM_MX_SCALED_MFMA = 1
} qgemm_mx_mode;

/*
 * Host-side descriptor of a prepared weight buffer ("checkpoint metadata":
 * [TL27] section 7, pitfall 10 -- record the granularity with the weights).
 * Filled by qgemm_prepack_weights; read by qgemm_run / qgemm_run_mx.
 *
 * Layout of the packed device buffer (all offsets in bytes, 256-aligned):
 *   codes   at codes_off:  N_pad x K_pad bytes; rows >= N and columns >= K
 *           are zero. QGEMM_FMT_INT8_SYM: 1 KB blocks of 16 rows x 64 K; block
 *           (n/16, k/64) starts at byte ((n/16)*(K_pad/64) + k/64) * 1024 and
 *           holds, at 256*c + 16*(n%16), the 16 codes of row n with k%64 in
 *           [16c, 16c+16) (so each block is one 16x16x64 int8 matrix-core
 *           operand in lane order and a streamed 1 KB load).
 *           QGEMM_FMT_MXFP8_E4M3: 1 KB blocks of 16 rows x 64 K in the same
 *           block order as INT8; code (n, k) at byte
 *           ((n/16)*(K_pad/64) + k/64) * 1024 + 64*(n%16) + k%64 (each block
 *           holds its 16 rows' 64 codes in K order, so the 16 rows x 64 K a
 *           GEMM stage takes is one contiguous 1 KB load; ABI version 9 and
 *           later).
 *           QGEMM_FMT_MXFP4_E2M1: e2m1 codes [N_pad][K_pad/2] bytes, row-major,
 *           two per byte (element 2i in the low nibble).
 *           QGEMM_FMT_INT4_SYM: N_pad x K_pad / 2 bytes in 1 KB blocks of 16
 *           rows x 128 K; block (n/16, k/128) starts at byte
 *           ((n/16)*(K_pad/128) + k/128) * 1024. Row n%16 and c = (k%64)/16
 *           own the 16 bytes at 16*(16c + n%16): bytes 0-7 for k%128 < 64,
 *           8-15 for the other group; in those 8 bytes, the 16 codes of
 *           kk = k%16 sit in byte 4*(kk/8) + kk%4, in the low nibble when
 *           kk%8 < 4, else the high one; a nibble is the code's low four
 *           two's-complement bits ([TL27] 3.3(b) and pitfall 9).
 *   scales  at scales_off: INT8: float32 [N_pad] (GRAN_ROW; rows >= N are 0)
 *           or float32 [1] (GRAN_TENSOR). MX: E8M0 bytes [N_pad][K_pad/32]
 *           row-major, padding blocks hold 127 (scale 1.0) (the same for
 *           MXFP4). INT4: float32,
 *           64 per 16 rows x 256 K: the scale of row n, group g at float
 *           index ((n/16)*(K_pad/256) + g/4) * 64 + 4*(n%16) + g%4 (one
 *           16-byte load gives a row the scales of four groups); padding is 0.
 *   colsum  at colsum_off: INT8 only: int32 [N_pad], colsum[n] = sum_k q_w[n,k]
 *           ([D98] "The program, and the gate that has to be per column":
 *           computed once, when the weights are quantized). -1 for MX and INT4.
 */
typedef struct qgemm_wdesc {
  uint32_t magic;      /* QGEMM_WDESC_MAGIC                        */
  uint32_t version;    /* QGEMM_ABI_VERSION                        */
  int32_t fmt;         /* qgemm_format                             */
  int32_t gran;        /* qgemm_granularity                        */
  int64_t N, K;        /* logical sizes                            */
  int64_t N_pad;       /* N rounded up to a multiple of 256        */
  int64_t K_pad;       /* K rounded up to a multiple of 256        */
  int64_t codes_off;
  int64_t scales_off;
  int64_t colsum_off;
  int64_t bytes;       /* bytes of the packed buffer that are used */
} qgemm_wdesc;

/* ABI version of the loaded library (QGEMM_ABI_VERSION it was built with). */
int qgemm_abi_version(void);

/* Static, human-readable name of a status code. Never NULL. */
const char* qgemm_status_string(int status);

/*
 * Size in bytes of the packed weight buffer qgemm_prepack_weights needs for
 * an [N, K] weight in format `fmt` with granularity `gran`. Returns 0 for an
 * invalid combination or size.
 */
size_t qgemm_packed_weight_bytes(int64_t N, int64_t K, int fmt, int gran);

/*
 * Workspace bytes the quantize / prepack calls need for these arguments.
 * Per-tensor quantization needs M (or N) float partial results (2x for the
 * asymmetric min/max); per-row and MX quantization need none (0 returned).
 * `rows` is M for activations, N for weights.
 */
size_t qgemm_workspace_bytes(int64_t rows, int64_t K, int fmt, int gran);

/*
 * qgemm_quantize_rows -- dynamic activation quantization (steps Q1-Q3 and MXQ).
 *
 *   INT8_SYM   ([AQ] "The integer GEMM, written out", quantize_per_token;
 *               [D98] "What a scale actually promises" and "Pitfalls"):
 *     amax = max_k |x[m,k]| (per row) or over the whole matrix (TENSOR);
 *     s = max(amax / 127, 1e-8)                         (float32)
 *     q = clamp(rint(x / s), -127, 127)                 (int8)
 *   UINT8_ASYM ([SK] step 1; [AQ] "The quantizer itself"):
 *     s = max((max - min) / 255, 1e-8); z = clamp(rint(-min / s), 0, 255)
 *     q = clamp(rint(x / s) + z, 0, 255)                (uint8)
 *   MXFP8_E4M3 ([TL27] 2.2 item 3 and 2.3; GRAN_BLOCK32 only; K % 32 == 0):
 *     per row and 32-block b: amax = max(max|x|, 1e-4);
 *     E = ceil_to_ue8m0(amax / 448) in [1, 254]  (scale 2^(E-127));
 *     q = e4m3(x * 2^(127-E)), round to nearest even.
 *   MXFP4_E2M1, BLOCK32 (K % 32 == 0): the same with e2m1's largest value 6:
 *     E = ceil_to_ue8m0(amax / 6); q = e2m1(x * 2^(127-E)), round to nearest,
 *     ties to the even code; two codes per byte, element 2i in the low nibble.
 *   Division is the correctly rounded float32 x / s (no reciprocal), rint is
 *   round-half-to-even, so codes, scales and zero points are bit-exact
 *   against a float32 evaluation of the same formulas.
 *
 * Arguments:
 *   x            device, float32 [M][ldx], ldx >= K, 4-byte aligned (rows that start on
 *                16-byte boundaries, ldx % 4 == 0, are read with 16-byte loads).
 *   M, K         M >= 0, K >= 1.
 *   fmt, gran    INT8_SYM or UINT8_ASYM with TENSOR or ROW; MXFP8_E4M3 or
 *                MXFP4_E2M1 with BLOCK32.
 *   q            device, codes [M][ldq] bytes, ldq >= K (MXFP4: ldq >= K/2),
 *                ldq % 16 == 0, 16-byte aligned. Bytes past the row's codes are
 *                not written.
 *   scales       device float32 [M] (ROW) or [1] (TENSOR); NULL for MX.
 *   zero_points  device int32 [M] or [1] for UINT8_ASYM; NULL otherwise.
 *   mx_scales    device E8M0 bytes [M][ld_mx] for MX (ld_mx >= K/32); NULL otherwise.
 *   workspace    device, >= qgemm_workspace_bytes(M, K, fmt, gran) bytes
 *                (may be NULL when that is 0). Contents need no initialization.
 */
int qgemm_quantize_rows(const float* x, int64_t M, int64_t K, int64_t ldx,
                        int fmt, int gran,
                        void* q, int64_t ldq,
                        float* scales, int32_t* zero_points,
                        uint8_t* mx_scales, int64_t ld_mx,
                        void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * qgemm_quantize_rows_noalloc -- qgemm_quantize_rows without a workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.
 *
 *   Same formats, granularities, arguments (minus the workspace), results and
 *   errors as qgemm_quantize_rows. The per-tensor granularity keeps its row
 *   statistics in a static device array of the library (1 MiB on each GPU it
 *   runs on, held until the process ends) instead of a workspace: up to
 *   262,144 rows for INT8_SYM and 131,072 for UINT8_ASYM, beyond which the
 *   call returns QGEMM_E_WORKSPACE before launching anything. The ROW and
 *   BLOCK32 granularities use no scratch memory.
 *   The call allocates nothing: no hipMalloc, no hipFree, no allocating
 *   library routine (its first call on a device looks up that device's copy
 *   of the array once). Every slot it reads was written by the same call, so
 *   nothing needs clearing between calls.
 *   All calls on one GPU share its array: per-tensor calls that overlap on
 *   that GPU (concurrent streams, or threads) race and may return wrong
 *   scales; serialize them.
 */
int qgemm_quantize_rows_noalloc(const float* x, int64_t M, int64_t K, int64_t ldx,
                                int fmt, int gran,
                                void* q, int64_t ldq,
                                float* scales, int32_t* zero_points,
                                uint8_t* mx_scales, int64_t ld_mx,
                                void* stream);

/*
 * qgemm_rmsnorm_quantize_rows -- RMSNorm and per-row quantization in one pass
 * over the rows ([AQ] "Fusion: making quantization nearly free": the norm
 * kernel already holds each row, so it finds the row's amax and writes the
 * codes and one scale per token without another read of the activations).
 *
 *   rms    = sqrt(sum_k x[m,k]^2 / K + eps)   float64 (every square is exact
 *            there, the sum is carried as a double-double and rounded once),
 *            then rounded once to float32
 *   y[m,k] = (x[m,k] / rms) * gamma[k]       the page's order: a correctly
 *            rounded float32 division, then a float32 multiply
 *   then exactly qgemm_quantize_rows on y with gran = ROW: INT8_SYM
 *   (s = max(amax / 127, 1e-8), q = clamp(rint(y / s), -127, 127)) or
 *   UINT8_ASYM (s, z from the row's min and max).
 *
 *   x        device float32 [M][ldx], ldx >= K.
 *   gamma    device float32 [K] (the norm's per-column weight).
 *   eps      finite, >= 0 (else QGEMM_E_MODE).
 *   fmt      QGEMM_FMT_INT8_SYM or QGEMM_FMT_UINT8_ASYM; gran QGEMM_GRAN_ROW
 *            (any other combination: QGEMM_E_MODE).
 *   q, ldq, scales, zero_points as in qgemm_quantize_rows (ROW granularity).
 *   The double-double sum of squares equals the correctly rounded float64
 *   sum unless the exact sum lies within about K * 2^-104 (relative) of the
 *   midpoint between two doubles, so rms is the same float32 value as the
 *   plain definition computed with an exact sum.
 */
int qgemm_rmsnorm_quantize_rows(const float* x, int64_t M, int64_t K, int64_t ldx,
                                const float* gamma, float eps,
                                int fmt, int gran,
                                void* q, int64_t ldq,
                                float* scales, int32_t* zero_points,
                                void* stream);

/*
 * qgemm_prepack_weights -- offline weight preparation (step "W prepack").
 *
 *   INT8_SYM, ROW or TENSOR: per output channel n (or once for the matrix),
 *     s_w = max(amax / 127, 1e-8); q_w = clamp(rint(w / s_w), -127, 127);
 *     colsum[n] = sum_k q_w[n,k]  ([AQ] "The integer GEMM, written out",
 *     quantize_per_channel; [D98] the column sums of the zero-point row).
 *   MXFP8_E4M3 or MXFP4_E2M1, BLOCK32: the MX rule of qgemm_quantize_rows on
 *     each row of W.
 *   INT4_SYM, GROUP64: per row n and group g of 64 K (a last, shorter group
 *     takes the elements it has), s = max(amax / 7, 1e-8) in float32,
 *     q = clamp(rint(w / s), -8, 7) with a correctly rounded quotient
 *     ([TL27] 2.4; 5.1 for the group of 64).
 *   Writes the packed layout described at qgemm_wdesc (including zero padding)
 *   and fills *desc on the host.
 *
 *   w        device float32 [N][ldw], ldw >= K, 4-byte aligned.
 *   packed   device, >= qgemm_packed_weight_bytes(N, K, fmt, gran) bytes, 256-byte aligned.
 *   desc     host, written on success only.
 *   workspace as for qgemm_quantize_rows with rows = N.
 *   The packed buffer is immutable afterwards and may be used on any stream.
 */
int qgemm_prepack_weights(const float* w, int64_t N, int64_t K, int64_t ldw,
                          int fmt, int gran,
                          void* packed, size_t packed_bytes, qgemm_wdesc* desc,
                          void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * qgemm_unpack_weights -- plain copies of what a prepared weight buffer holds:
 * the codes, scales, column sums and E8M0 scales that qgemm_prepack_weights
 * computed ([AQ] quantize_per_channel; [D98] the column sums; [TL27] 2.3 and
 * 2.4 for the MX and int4 scales), read out of the packed layout into plain
 * row-major arrays, for inspection, checkpoints and tests.
 *
 *   desc, packed  a descriptor and its packed device buffer (any format).
 *   Every output is optional (NULL: not written); all are device memory:
 *   codes_out     [N][ld_codes] bytes: int8 codes (INT8_SYM; INT4_SYM as one
 *                 sign-extended int8 per element), e4m3 codes (MXFP8), or e2m1
 *                 codes two per byte as stored (MXFP4, K / 2 bytes per row);
 *                 ld_codes >= the row's bytes.
 *   scales_out    float32 scales: INT8_SYM [N] (ROW) or [1] (TENSOR), ld_scales
 *                 ignored; INT4_SYM [N][ld_scales], ld_scales >= ceil(K / 64),
 *                 one per group of 64 K. Not for MX formats (QGEMM_E_MODE).
 *   colsums_out   int32 [N] column sums (INT8_SYM only, else QGEMM_E_MODE).
 *   mx_scales_out E8M0 bytes [N][ld_mx], ld_mx >= K / 32 (MX formats only,
 *                 else QGEMM_E_MODE).
 * Errors: QGEMM_E_NULL (desc or packed), QGEMM_E_DESC, QGEMM_E_MODE,
 * QGEMM_E_SHAPE (a leading dimension too small), QGEMM_E_ALIGN (packed not
 * 256-byte aligned, scales_out / colsums_out not 4-byte aligned),
 * QGEMM_E_DEVICE, QGEMM_E_HIP. Launches one small kernel per output
 * requested, on `stream`; allocates nothing and records no memset.
 */
int qgemm_unpack_weights(const qgemm_wdesc* desc, const void* packed,
                         void* codes_out, int64_t ld_codes,
                         float* scales_out, int64_t ld_scales,
                         int32_t* colsums_out,
                         uint8_t* mx_scales_out, int64_t ld_mx,
                         void* stream);

/*
 * qgemm_run -- int8 GEMM with the fused dequantization epilogue (steps G, E).
 *
 *   C[m,n]   = sum_k (q_a[m,k] - z_a[m]) * q_w[n,k]        exact int32
 *              ([AQ] "The integer GEMM, written out": the integer dot product
 *              minus z_a * colsum(q_w); [D98] "What a scale actually
 *              promises": int32 accumulation rounds nothing)
 *   out[m,n] = float(C[m,n]) * (s_a[m] * s_w[n])            float32 arithmetic
 *              ([D98] "The program, and the gate that has to be per column":
 *              the scales multiply once per output, after the loop;
 *              [SK] "Correctness requirements": zero point before scaling)
 *   out[m,n] = out[m,n] + bias[n]                           if bias != NULL,
 *              float32 ([AQ] int8_linear: y + bias after the scales; [SK]
 *              step 5: apply the bias in fp32 in the epilogue)
 *   cast to float32, to bfloat16 (round to nearest even), or C itself (I32).
 *
 *   a_q      device codes [M][lda] (int8 for INT8_SYM, uint8 for UINT8_ASYM),
 *            lda >= K, lda % 16 == 0, 16-byte aligned. Row m is read from byte
 *            0 up to the end of the 16-byte chunk holding column K - 1, never
 *            further; (min(M, 256) - 1) * lda + K_pad < 2^32 (QGEMM_E_SHAPE).
 *   a_scales device float32 [M] (ROW) or [1] (TENSOR).
 *   a_zero   device int32 [M] or [1] (UINT8_ASYM, values 0..255); NULL for INT8_SYM.
 *   w_desc   host descriptor from qgemm_prepack_weights (INT8_SYM weights).
 *   w_packed device packed buffer of that descriptor.
 *   out      device [M][ldo] of out_type, ldo >= N, 16-byte aligned, ldo % 4 == 0.
 *   bias     device float32 [N] or NULL; NULL with out_type I32 (else QGEMM_E_MODE).
 *   K limit  (QGEMM_E_OVERFLOW): K <= 133144 for INT8_SYM activations
 *            (127*127*K < 2^31), K <= 66311 for UINT8_ASYM (255*127*K < 2^31)
 *            ([SK] step 2 and "Correctness requirements"; [AQ] about 133,000 terms).
 *   workspace unused by this version (pass NULL, 0).
 */
int qgemm_run(const void* a_q, int64_t lda, const float* a_scales, const int32_t* a_zero,
              int a_fmt, int a_gran, int64_t M,
              const qgemm_wdesc* w_desc, const void* w_packed,
              void* out, int64_t ldo, int out_type, const float* bias,
              void* workspace, size_t workspace_bytes,
              void* stream);

/*
 * qgemm_run_mx -- block-scaled GEMM (step MXG): e4m3 or e2m1 activations
 * times e4m3 or e2m1 weights, each with one E8M0 scale per 32 K-elements.
 *
 *   out[m,n] = sum_b 2^(Ea[m,b]-127) * 2^(Ew[n,b]-127) *
 *              sum_{k in block b} a[m,k] * w[n,k]
 *   Each 32-element K block is multiplied by its own pair of scales inside
 *   the K loop ([TL27] 4.1: (A*scale_A)(B*scale_B); 4.3: a per-K-block scale
 *   cannot be moved out of the sum). float32 accumulation and output; how
 *   exactly the products and sums are formed depends on `mode`. With a bias,
 *   out[m,n] + bias[n] in float32 (the bias term of the MX formula
 *   C = (scale_A x A)(scale_B x B) + bias on the [TL27] pages; [TL27] 4.2
 *   lists e4m3 x e2m1 and e2m1 x e2m1 MX matmuls).
 *
 *   a_codes  device codes [M][lda] bytes: e4m3 (a_fmt QGEMM_FMT_MXFP8_E4M3,
 *            lda >= K) or packed e2m1 (QGEMM_FMT_MXFP4_E2M1, lda >= K/2), as
 *            written by qgemm_quantize_rows; lda % 16 == 0, 16-byte aligned.
 *   a_e8m0   device E8M0 [M][lda_s], lda_s >= K/32. With lda_s % 4 == 0, a
 *            4-byte aligned a_e8m0 and K % 64 == 0 (e2m1 x e2m1 in
 *            QGEMM_MX_SCALED_MFMA mode: K % 128 == 0), the call runs on the
 *            LDS-DMA kernel, which reads each row's scales a dword at a time
 *            (never past lda_s).
 *   a_fmt    QGEMM_FMT_MXFP8_E4M3 or QGEMM_FMT_MXFP4_E2M1 (else QGEMM_E_MODE).
 *   w_desc   descriptor of MXFP8_E4M3 or MXFP4_E2M1 weights with the same K
 *            (K % 32 == 0).
 *   out      device float32 [M][ldo], ldo >= N, ldo % 4 == 0, 16-byte aligned.
 *   mode     qgemm_mx_mode: QGEMM_MX_EXACT (products exact, float32 sums) or
 *            QGEMM_MX_SCALED_MFMA (block-scaled matrix cores, each operand
 *            with its own format code; see the enum -- for e2m1 x e2m1 the
 *            products span under 8 binades, so nothing is dropped and the sums
 *            are float32 sums, as in the exact mode, at twice the e4m3 rate).
 *            Both modes take any pair of the two formats.
 *            Both need E8M0 codes in [3, 240] for exactness of the scaled values,
 *            which qgemm_quantize_rows always produces for inputs below 2^120.
 *   bias     device float32 [N] or NULL.
 *   workspace unused by this version (pass NULL, 0).
 */
int qgemm_run_mx(const uint8_t* a_codes, int64_t lda, const uint8_t* a_e8m0, int64_t lda_s, int a_fmt,
                 int64_t M, const qgemm_wdesc* w_desc, const void* w_packed,
                 float* out, int64_t ldo, int mode, const float* bias,
                 void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * qgemm_run_mx_grouped -- grouped (MoE) block-scaled GEMM: the rows of A
 * routed to expert e, stored one expert after the other, times expert e's
 * weights ([TL27] 6.2, MoE point 3: A is the concatenation of the experts'
 * rows, its scales indexed by the concatenated row; one weight matrix per
 * expert, its scales indexed by expert and output column).
 *
 *   out[m,n] = qgemm_run_mx's out[m,n] for row m of A against the weights of
 *              the expert e whose rows offsets[e] .. offsets[e+1] - 1 hold m,
 *              plus bias[e][n] when bias != NULL.
 *   Row m's result does not depend on the other rows or experts: it is the
 *   bits qgemm_run_mx gives for that row and expert on this kernel.
 *
 *   a_codes, lda, a_e8m0, lda_s, a_fmt, out, ldo, mode: as qgemm_run_mx,
 *            for M_total rows; in addition lda_s % 4 == 0 and a_e8m0 4-byte
 *            aligned (QGEMM_E_ALIGN), and K % 64 == 0, or K % 128 == 0 for
 *            e2m1 x e2m1 in QGEMM_MX_SCALED_MFMA mode (QGEMM_E_SHAPE). Any
 *            pair of the two formats runs in either mode.
 *   M_total  rows of A and out, >= 0 (0: nothing is launched).
 *   offsets  device int64 [E + 1], non-decreasing, offsets[0] = 0 and
 *            offsets[E] = M_total, 8-byte aligned. It stays on the device (a
 *            router on the GPU needs no host copy). Values outside
 *            [0, M_total] are clamped and a decreasing pair is an empty
 *            group, so nothing outside the buffers is accessed; the results
 *            are then unspecified.
 *   E        number of experts, 1 .. 4096 (QGEMM_E_SHAPE).
 *   w_desc   descriptor of one expert's weights (QGEMM_FMT_MXFP8_E4M3 or
 *            QGEMM_FMT_MXFP4_E2M1, N x K), shared by all experts.
 *   w_packed the E experts' prepared weights back to back: expert e's at
 *            w_packed + e * w_desc->bytes (each written by
 *            qgemm_prepack_weights with w_desc's shape and format); 256-byte
 *            aligned.
 *   bias     device float32 [E][N] or NULL.
 *   workspace unused by this version (pass NULL, 0).
 */
int qgemm_run_mx_grouped(const uint8_t* a_codes, int64_t lda, const uint8_t* a_e8m0, int64_t lda_s, int a_fmt,
                         int64_t M_total, const int64_t* offsets, int64_t E,
                         const qgemm_wdesc* w_desc, const void* w_packed,
                         float* out, int64_t ldo, int mode, const float* bias,
                         void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * qgemm_run_w4a8 -- int8 activations times int4 weights with one scale per
 * group of 64 K ([TL27] 3.3(c) and 5.1).
 *
 *   P_g[m,n] = sum_{k in group g} q_a[m,k] * q_w[n,k]            exact int32
 *   out[m,n] = s_a[m] * sum_g s_w[n,g] * P_g[m,n]                float32
 *              (each group's scale multiplies its own partial sum inside
 *              the K loop: [TL27] 4.3, a scale that varies along K cannot
 *              be applied once after the sum)
 *   out[m,n] = out[m,n] + bias[n]                                if bias != NULL
 *   cast to float32 or bfloat16 (round to nearest even).
 *   Rounding: float32 accumulation over the groups; |out - exact| is within
 *   (K_pad / 64 + 16) * 2^-24 * (sum_g |s_a s_w[n,g] P_g| + |bias[n]|) for
 *   float32 output.
 *
 *   a_q      device int8 codes [M][lda] (QGEMM_FMT_INT8_SYM activations from
 *            qgemm_quantize_rows), lda >= K, lda % 16 == 0, 16-byte aligned;
 *            (min(M, 16) - 1) * lda + K_pad + 65536 < 2^32 (QGEMM_E_SHAPE).
 *   a_scales device float32 [M] (a_gran QGEMM_GRAN_ROW) or [1] (TENSOR).
 *   M        0 <= M <= 16 * 65535 (QGEMM_E_SHAPE).
 *   w_desc   host descriptor of QGEMM_FMT_INT4_SYM / QGEMM_GRAN_GROUP64 weights.
 *   out      device [M][ldo] of out_type (QGEMM_OUT_F32 or QGEMM_OUT_BF16;
 *            QGEMM_OUT_I32 is QGEMM_E_MODE: there is no single integer sum),
 *            ldo >= N, ldo % 4 == 0, 16-byte aligned.
 *   bias     device float32 [N] or NULL.
 *   K <= 2^27 (QGEMM_E_SHAPE); no tighter limit: every group's partial sum
 *   is exact in int32 and in float32.
 *   workspace unused by this version (pass NULL, 0).
 */
int qgemm_run_w4a8(const int8_t* a_q, int64_t lda, const float* a_scales, int a_gran, int64_t M,
                   const qgemm_wdesc* w_desc, const void* w_packed,
                   void* out, int64_t ldo, int out_type, const float* bias,
                   void* workspace, size_t workspace_bytes,
                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_H */
