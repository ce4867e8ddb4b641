// int8 activations x int4 weights with one float32 scale per group of 64 K
// ("TileLang tutorial, chapter 27", sections 3.3(c), 4.3 and 5.1) for gfx950.
#include "common.hpp"
#include "kernels.hpp"

namespace qg {

constexpr int kW4Waves = 8;  // waves per workgroup, each on its own K range

// ---------------------------------------------------------------------------
// W4A8: int8 activations x int4 weights with one float32 scale per group of
// 64 K ("TileLang tutorial, chapter 27", sections 3.3(c) and 5.1), for 16-row
// bands of A: the decode kernel's stream over W at half the bytes. A
// workgroup owns 16 weight rows over all of K; its eight waves take
// contiguous ranges of 128-deep steps (two groups). Per step a lane loads 16
// bytes of codes (its 16-K chunk of both groups) and its activation chunks;
// per two steps, the four group scales of its weight row (16 bytes).
//
// With at most 8 activation rows, rows 8-15 of the 16-row operand only feed
// output rows that are never stored, so one 16-byte load per lane carries
// both groups of a step (lanes 16c + r: the first group's chunk c of row r;
// lanes 16c + 8 + r: the second group's) and a DPP rotate by 8 lanes within
// each row of 16 lanes gives the second group's operand. The activation loads
// are the kernel's main cost beyond the weight stream, so this halves them.
//
// Sign extension without a shift back: a nibble moved to the top of its byte
// (masking with 0xF0 per byte after a 4-bit shift for the low nibble) is the
// int8 value 16 q exactly, so the int8 matrix cores give 16 P_g exactly
// (|16 P_g| <= 16 * 64 * 127 * 8 < 2^24, also exact as a float32). Each group
// then enters a float32 sum through one FMA with its own scale (section 4.3:
// a scale that changes along K is applied per block inside the loop, never
// after the sum); 1/16 is folded into the final s_a multiply, which is exact
// because it is a power of two.
// ---------------------------------------------------------------------------
constexpr int kW4Batch = 4;        // 128-deep steps per load batch (even: scales come in pairs of steps)
constexpr int kStreamLoad = 2;     // cache policy of the once-read weight stream: non-temporal

template <int OUT, bool ONE, bool MLE8>
__global__ __launch_bounds__(kW4Waves * 64) void gemm_w4a8_kernel(GemmArgs p) {
  constexpr int U = kW4Batch;
  constexpr int kHi = (int)0xF0F0F0F0u;
  __shared__ v4f red[kW4Waves][64];
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t m0 = (int64_t)blockIdx.y * 16;
  const int64_t mrows = p.M - m0 < 16 ? p.M - m0 : 16;
  const int pairs = (int)(p.K_pad / 128);
  // steps of each wave, a whole number of batches; steps at or past K_pad
  // read zero codes and zero scales from outside the block's ranges
  const int per = ONE ? U : (pairs + kW4Waves * U - 1) / (kW4Waves * U) * U;
  const int pbeg = wid * per;
  const int row = lane & 15;
  constexpr uint32_t kOff = 0x80000000u;
  const int64_t blk0 = (n0 >> 4) * pairs;  // first code block of the workgroup's rows
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.w + blk0 * 1024), (short)0, (int)(pairs * 1024), kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.sw + blk0 * 32), (short)0, (int)(pairs * 128), kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.a + m0 * p.lda), (short)0, (int)((mrows - 1) * p.lda + ((p.K + 15) & ~(int64_t)15)),
      kRawBufferWord3);
  const uint32_t woff = (uint32_t)pbeg * 1024u + (uint32_t)(lane * 16);
  const uint32_t soff = (uint32_t)pbeg * 128u + (uint32_t)(row * 16);
  const int arow = MLE8 ? (lane & 7) : row;
  const int akin = (MLE8 ? ((lane >> 3) & 1) * 64 : 0) + (lane >> 4) * 16;
  const uint32_t aoff = arow < mrows ? (uint32_t)(arow * p.lda + pbeg * 128 + akin) : kOff;

  v4f y = {0.f, 0.f, 0.f, 0.f};
  for (int b = 0; b < (ONE ? U : per); b += U) {
    v4i wv[U], a0[U], a1[MLE8 ? 1 : U];
    v4f sv[U / 2];
    // per step: activations, codes, and every second step the scales
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t st = (uint32_t)(b + u);
      a0[u] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(ars, (int)(aoff + st * 128u), 0, 0));
      if (!MLE8)
        a1[u] = __builtin_bit_cast(
            v4i, __builtin_amdgcn_raw_buffer_load_b128(ars, (int)(aoff + st * 128u + 64u), 0, 0));
      wv[u] = __builtin_bit_cast(
          v4i, __builtin_amdgcn_raw_buffer_load_b128(wrs, (int)(woff + st * 1024u), 0, kStreamLoad));
      if (u % 2 == 0)
        sv[u / 2] = __builtin_bit_cast(
            v4f, __builtin_amdgcn_raw_buffer_load_b128(srs, (int)(soff + st * 128u), 0, kStreamLoad));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      v4i x1;
      if constexpr (MLE8) {
#pragma unroll
        for (int d = 0; d < 4; ++d) x1[d] = __builtin_amdgcn_update_dpp(0, a0[u][d], 0x128, 0xF, 0xF, false);  // row_ror:8
      } else {
        x1 = a1[MLE8 ? 0 : u];
      }
      const v4i w = wv[u];
      const v4i w0 = {(w.x << 4) & kHi, w.x & kHi, (w.y << 4) & kHi, w.y & kHi};
      const v4i w1 = {(w.z << 4) & kHi, w.z & kHi, (w.w << 4) & kHi, w.w & kHi};
      const v4i zero = {0, 0, 0, 0};
      const v4i c0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0[u], w0, zero, 0, 0, 0);
      const v4i c1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(x1, w1, zero, 0, 0, 0);
      const float s0 = (u & 1) ? sv[u / 2].z : sv[u / 2].x;
      const float s1 = (u & 1) ? sv[u / 2].w : sv[u / 2].y;
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = __builtin_fmaf(s0, (float)c0[i], y[i]);
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = __builtin_fmaf(s1, (float)c1[i], y[i]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  red[wid][lane] = y;
  __syncthreads();

  // thread t < 256 finishes item t / 64 of lane t % 64: row 4 * (l / 16) + item, column l % 16
  for (int t = threadIdx.x; t < 256; t += kW4Waves * 64) {
    const int l = t & 63, item = t >> 6;
    const int64_t m = m0 + 4 * (l >> 4) + item;
    const int64_t n = n0 + (l & 15);
    if (m < p.M && n < p.N) {
      float acc = red[0][l][item];
#pragma unroll
      for (int w = 1; w < kW4Waves; ++w) acc += red[w][l][item];
      const float sa = p.a_per_tensor ? p.sa[0] : p.sa[m];
      float yv = acc * (sa * 0.0625f);  // the codes entered as 16 q
      if (p.bias) yv = yv + p.bias[n];
      store_one<OUT>(p.out, m * p.ldo + n, 0, yv);
    }
  }
}

template <int OUT, bool MLE8>
static void launch_w4a8_rows(const GemmArgs& a, const dim3 grid, hipStream_t st) {
  if (a.K_pad <= 128 * kW4Batch * kW4Waves)
    hipLaunchKernelGGL((gemm_w4a8_kernel<OUT, true, MLE8>), grid, dim3(kW4Waves * 64), 0, st, a);
  else
    hipLaunchKernelGGL((gemm_w4a8_kernel<OUT, false, MLE8>), grid, dim3(kW4Waves * 64), 0, st, a);
}

template <int OUT>
static hipError_t launch_w4a8(const GemmArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((a.N + 15) / 16), (unsigned)((a.M + 15) / 16));
  if (a.M <= 8)
    launch_w4a8_rows<OUT, true>(a, grid, st);
  else
    launch_w4a8_rows<OUT, false>(a, grid, st);
  return hipGetLastError();
}

hipError_t launch_gemm_w4a8(const GemmArgs& a, int out_type, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  if (out_type == 1) return launch_w4a8<1>(a, st);
  return launch_w4a8<0>(a, st);
}

}  // namespace qg
