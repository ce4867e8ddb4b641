// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

// Symmetric int8 / asymmetric uint8 row quantization (per row or per tensor).
// Codes go row-major with stride ldq (kblocks == 0) or, for packed weights,
// into 1 KB blocks of 16 rows x 64 K with kblocks blocks along K (see
// GemmArgs::w). `colsum` (may be null) receives the sum of each row's codes.
// `ws` holds rows (2*rows when asym) floats for the per-tensor statistics.
void launch_quantize_int(const float* x, int64_t rows, int64_t K, int64_t ldx, bool asym, bool per_tensor,
                         uint8_t* q, int64_t ldq, int64_t kblocks, float* scales, int32_t* zeros, int32_t* colsum,
                         float* ws, hipStream_t st);

// The library's static scratch array for the allocation-free quantize entry
// point: kScratchFloats floats on each device. scratch_buffer() returns the
// current device's copy (looked up once per device, no allocation).
constexpr int64_t kScratchFloats = int64_t(1) << 18;  // 1 MiB
constexpr int kMaxScratchDevices = 64;
hipError_t scratch_buffer(float** ptr);

// RMSNorm (double-double sum of squares, float32 rms, normalized row
// (x / rms) * gamma in float32)
// fused with per-row symmetric int8 / asymmetric uint8 quantization.
void launch_rmsnorm_quantize(const float* x, int64_t rows, int64_t K, int64_t ldx, const float* gamma, float eps,
                             bool asym, uint8_t* q, int64_t ldq, float* scales, int32_t* zeros, hipStream_t st);

// MXFP8 (e4m3 codes) or, fp4, MXFP4 (e2m1 codes, two per byte, element 2i
// in the low nibble) row quantization with E8M0 per 32 K-elements; K % 32 == 0.
// Codes go row-major with stride ldq, except e4m3 weights being prepared
// (wblk_kpad = their K_pad > 0): those go to the blocked layout of
// mx8_code_off.
void launch_quantize_mx(const float* x, int64_t rows, int64_t K, int64_t ldx, bool fp4, uint8_t* q, int64_t ldq,
                        uint8_t* e8, int64_t lde, int64_t wblk_kpad, hipStream_t st);

// int4 weights, symmetric, one scale per group of 64 K of each row, into the
// packed layout of GemmArgs::w (INT4). The buffer must be zero beforehand.
void launch_quantize_int4(const float* w, int64_t rows, int64_t K, int64_t ldw, int64_t K_pad, uint8_t* codes,
                          float* scales, hipStream_t st);

// Compute units of the current device (cached per device).
int cu_count();

// One output of qgemm_unpack_weights: a plain copy of a section of a packed
// weight buffer. Codes go one 16-byte piece of an output row per thread (int8
// and int4 codes as one int8 per element, MX codes as stored), the other
// outputs one element per thread.
enum { UNPACK_CODES = 0, UNPACK_WORDS = 1, UNPACK_INT4_SCALES = 2, UNPACK_E8M0 = 3 };
enum { UNPACK_FMT_INT8 = 0, UNPACK_FMT_INT4 = 1, UNPACK_FMT_MX = 2, UNPACK_FMT_MX8 = 3 };
struct UnpackArgs {
  const uint8_t* src;   // the section of the packed buffer the output comes from
  int64_t src_pitch;    // bytes per source row (MX codes, E8M0)
  void* out;
  int64_t ld;           // output row pitch in elements (bytes for codes)
  int64_t rows, cols;   // output rows; elements (16-byte pieces for codes) per row
  int64_t row_bytes;    // codes: the bytes of one output row
  int64_t K_pad;
  int what, fmt;
};
hipError_t launch_unpack(const UnpackArgs& a, hipStream_t st);

// Measured ceilings (qgemm_ceiling_mfma, qgemm_ceiling_stream; not part of
// the GEMM path). Matrix cores: one workgroup per CU, 256 * waves_per_simd
// threads; lane l of every wave takes kCeilSets 32-byte operand sets from
// a_ops + 32 * (kCeilSets * l + q) and one from b_ops + 32 * l, then issues
// trips * kCeilSets instructions of the kind. `clocks` (may be null) gets,
// per workgroup, the shader-clock and 100 MHz real-time ticks of its loop.
// Stream: one workgroup of 256 threads per block_bytes (a multiple of 16 KB)
// of src, 16-byte loads clamped to the last 16 bytes.
enum { CEIL_I8 = 0, CEIL_F8_SCALED = 1, CEIL_F4_SCALED = 2, CEIL_BF16 = 3 };
constexpr int kCeilSets = 8;
constexpr int kCeilHoldWords = 24 * 1024;  // 96 KB of LDS: one workgroup per CU
constexpr int kCeilSinkMagic = 0x5eed5eed;
hipError_t launch_ceiling_mfma(int kind, int waves_per_simd, int64_t trips, const uint8_t* a_ops,
                               const uint8_t* b_ops, int32_t* sink, int64_t* clocks, hipStream_t st);
hipError_t launch_ceiling_stream(const uint8_t* src, int64_t bytes, int64_t block_bytes, int32_t* sink,
                                 hipStream_t st);

struct GemmArgs {
  const uint8_t* a;     // activation codes [M][lda]
  int64_t lda;
  const float* sa;      // int8: per-row or [1] scales
  const int32_t* za;    // int8 asym: zero points
  const uint8_t* ea;    // mx: E8M0 [M][lda_s]
  int64_t lda_s;
  int a_per_tensor;
  // packed codes, N_pad x K_pad. int8: 1 KB blocks of 16 rows x 64 K, block
  // (n / 16, k / 64) at byte ((n / 16) * (K_pad / 64) + k / 64) * 1024, and in
  // it the 16 bytes k % 64 in [16c, 16c + 16) of row n % 16 at 256 c + 16 (n % 16)
  // (one v_mfma_i32_16x16x64_i8 B operand in lane order). MX e4m3: 1 KB
  // blocks of 16 rows x 64 K in the same block order, row n % 16 at byte
  // 64 (n % 16) in K order (mx8_code_off). MX e2m1: row-major, K_pad / 2
  // bytes per row.
  // INT4: N_pad x K_pad / 2 bytes in 1 KB blocks of 16 rows x 128 K, block
  // (n / 16, k / 128) at ((n / 16) * (K_pad / 128) + k / 128) * 1024; lane
  // l = 16 c + n % 16 owns the 16 bytes at 16 l: bytes 0-7 hold k % 128 in
  // [16c, 16c + 16), bytes 8-15 the same chunk of the next group; in each
  // 8 bytes, dword d holds kk = k % 16 in [8d, 8d + 8), kk % 4 in its byte,
  // the low nibble for kk % 8 < 4 and the high one otherwise.
  const uint8_t* w;
  const float* sw;      // int8: [N_pad] or [1]; INT4: 64 per 16 rows x 256 K, at
                        // ((n / 16) * (K_pad / 256) + g / 4) * 64 + 4 (n % 16) + g % 4
  const int32_t* colsum;
  const uint8_t* ew;    // mx: E8M0 [N_pad][K_pad/32]
  int w_per_tensor;
  int a_fp4, w_fp4;     // mx: e2m1 codes (two per byte) instead of e4m3
  int64_t M, N, K, K_pad;
  void* out;
  int64_t ldo;
  const float* bias;    // [N] added to each output row after the scales (float32), or null
  // grouped MX GEMM: rows groups[e] .. groups[e + 1] - 1 of A belong to
  // expert e, whose packed weights start w_stride bytes after expert e - 1's
  // (w and ew point into expert 0's); the bias is [num_groups][N]
  const int64_t* groups;
  int num_groups;
  int64_t w_stride;
};

// The large-M int8 GEMM (gemm_i8_wide.hip): the W-block count FN of its
// 256 x 32 FN tiles for this shape on `cus` compute units, or 0 when the shape
// is better served by the tilings of gemm.hip; and its launcher.
int wide_tile_fn(int64_t M, int64_t N, int64_t cus);
template <bool ASYM, int OUT>
hipError_t launch_gemm_i8_wide(const GemmArgs& a, int fn, hipStream_t st);

// qgemm_run: int8 GEMM + epilogue. out_type: 0 f32, 1 bf16, 2 i32 (no bias).
hipError_t launch_gemm_i8(const GemmArgs& a, bool asym, int out_type, hipStream_t st);
// qgemm_run_mx: block-scaled GEMM of any e4m3 / e2m1 pair, float32 output.
// mode 0: exact products (bf16 matrix cores on dequantized values), mode 1:
// block-scaled fp8 / fp4 matrix cores.
hipError_t launch_gemm_mx(const GemmArgs& a, int mode, hipStream_t st);
// The block-scaled GEMM on an LDS-DMA ring (gemm_mx_dma.hip), any pair in
// either mode: whether it takes these arguments (K % 64 == 0, e2m1 x e2m1 in
// mode 1: K % 128 == 0; dword-aligned activation scale rows), and its launcher.
bool mx_dma_eligible(const GemmArgs& a, int mode);
hipError_t launch_gemm_mx_dma(const GemmArgs& a, int mode, hipStream_t st);
// qgemm_run_mx_grouped: the same kernel over E experts' row groups (a.M is
// the total row count, a.groups device offsets; mx_dma_eligible must hold).
hipError_t launch_gemm_mx_grouped(const GemmArgs& a, int mode, hipStream_t st);
// qgemm_run_w4a8: int8 activations x int4 weights, per-group scales inside
// the K loop, float32 sums. out_type: 0 f32, 1 bf16.
hipError_t launch_gemm_w4a8(const GemmArgs& a, int out_type, hipStream_t st);

}  // namespace qg
