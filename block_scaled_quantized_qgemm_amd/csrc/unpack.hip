// Plain copies of what a prepared weight buffer holds (qgemm_unpack_weights):
// the codes, scales, column sums and E8M0 scales of the weight preparation
// step ("Activation Quantization Architecture, in depth", quantize_per_channel;
// "100 Days of GPU -- Day 98", the column sums of the zero-point row; "TileLang
// tutorial, chapter 27", 2.3 and 2.4 for the MX and int4 scales), read back out
// of the packed layout into row-major arrays. One gather kernel; each launch
// fills one output, one thread per element (per 16 bytes for codes).
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace qg {

namespace {

// the int4 code of (row n, column k) in the packed layout of GemmArgs::w
// (INT4), sign-extended
__device__ inline int int4_code(const uint8_t* codes, int64_t n, int64_t k, int64_t K_pad) {
  const int64_t blk = ((n / 16) * (K_pad / 128) + k / 128) * 1024;
  const int kr = (int)(k % 128), g2 = kr / 64, c = (kr % 64) / 16, kk = kr % 16;
  const uint8_t b = codes[blk + 16 * (16 * c + (int)(n % 16)) + 8 * g2 + 4 * (kk / 8) + (kk % 4)];
  const int v = (kk % 8) < 4 ? (b & 15) : (b >> 4);
  return (v ^ 8) - 8;
}

__global__ __launch_bounds__(256) void unpack_kernel(UnpackArgs a) {
  const int64_t total = a.rows * a.cols, step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += step) {
    const int64_t n = t / a.cols, c = t % a.cols;
    switch (a.what) {
      case UNPACK_CODES: {  // c: 16-byte piece of the output row's a.row_bytes bytes
        uint8_t* dst = static_cast<uint8_t*>(a.out) + n * a.ld + 16 * c;
        const int64_t b0 = 16 * c;
        const int cnt = (int)min((int64_t)16, a.row_bytes - b0);
        for (int i = 0; i < cnt; ++i) {
          const int64_t b = b0 + i;
          uint8_t v;
          if (a.fmt == UNPACK_FMT_INT8)  // 16-row x 64-K blocks, chunk (k % 64) / 16 of row n % 16
            v = a.src[((n / 16) * (a.K_pad / 64) + b / 64) * 1024 + 256 * ((b % 64) / 16) + 16 * (n % 16) + b % 16];
          else if (a.fmt == UNPACK_FMT_INT4)
            v = (uint8_t)int4_code(a.src, n, b, a.K_pad);
          else if (a.fmt == UNPACK_FMT_MX8)  // e4m3: 1 KB blocks of 16 rows x 64 K
            v = a.src[mx8_code_off(n, b, a.K_pad)];
          else  // e2m1: row-major, K_pad / 2 bytes per row
            v = a.src[n * a.src_pitch + b];
          dst[i] = v;
        }
        break;
      }
      case UNPACK_WORDS:  // float32 scales or int32 column sums, [rows] from a word array
        static_cast<uint32_t*>(a.out)[n] = reinterpret_cast<const uint32_t*>(a.src)[n];
        break;
      case UNPACK_INT4_SCALES:  // group c of row n: 64 scales per 16 rows x 256 K, a row's four contiguous
        static_cast<float*>(a.out)[n * a.ld + c] =
            reinterpret_cast<const float*>(a.src)[((n / 16) * (a.K_pad / 256) + c / 4) * 64 + 4 * (n % 16) + c % 4];
        break;
      default:  // UNPACK_E8M0: [N_pad][K_pad / 32] bytes
        static_cast<uint8_t*>(a.out)[n * a.ld + c] = a.src[n * a.src_pitch + c];
        break;
    }
  }
}

}  // namespace

hipError_t launch_unpack(const UnpackArgs& a, hipStream_t st) {
  const int64_t total = a.rows * a.cols;
  if (total <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<int64_t>((total + 255) / 256, int64_t(1) << 16);
  hipLaunchKernelGGL(unpack_kernel, dim3(blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace qg
