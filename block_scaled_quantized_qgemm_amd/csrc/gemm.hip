// Matrix-core GEMMs for gfx950: the int8 path (v_mfma_i32_32x32x32_i8, exact
// int32 accumulation, fused dequantization epilogue) and the MX path
// (v_mfma_scale_f32_32x32x64_f8f6f4, e4m3 operands with one E8M0 scale per
// 32 K-elements fed per lane, float32 accumulation).
//
// Structure (one template for both):
//  * a workgroup owns a BM x BN output tile and walks K in BK-byte steps;
//  * the A and W tiles of the next step are fetched from global memory into
//    registers (16-byte loads, consecutive lanes on consecutive bytes of a
//    row) while the matrix cores work on the current step out of LDS;
//  * LDS holds two stages; rows are stored with their 16-byte chunks XOR-
//    swizzled by row so that the 16-byte fragment reads of 32 consecutive rows
//    spread over all banks;
//  * each wave owns a (BM/WM) x (BN/WN) sub-tile made of 32x32 MFMA blocks.
//
// Semantics followed:
//  * int8: C = sum_k (q_a - z_a) q_w exactly in int32 ("Activation
//    Quantization Architecture, in depth", section "The integer GEMM, written
//    out"), then out = float(C) * (s_a * s_w) once per output ("100 Days of
//    GPU -- Day 98", section "The program, and the gate that has to be per
//    column"). uint8 codes enter the signed matrix cores as q - 128 (a byte
//    XOR with 0x80) and the epilogue subtracts (z - 128) * colsum instead of
//    z * colsum, which yields the same exact C.
//  * MX: each 32-element K block is scaled by its own pair of E8M0 factors
//    inside the K loop ("TileLang tutorial, chapter 27", sections 4.1 and 4.3).
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace qg {

template <int BK>
__device__ inline int swz(int row) {
  constexpr int CPR = BK / 16;            // 16-byte chunks per row
  constexpr int RPL = 128 / BK > 0 ? 128 / BK : 1;  // rows sharing one 128-byte line
  return (row / RPL) % CPR;
}

template <int BK>
__device__ inline int lds_off(int row, int chunk) {
  return row * BK + ((chunk ^ swz<BK>(row)) << 4);
}

template <int BM, int BN, int BK, int WM, int WN, bool MX, bool ASYM, int OUT>
__global__ __launch_bounds__(WM* WN * 64) void gemm_kernel(GemmArgs p) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  constexpr int FM = TM / 32, FN = TN / 32;  // 32x32 blocks per wave
  constexpr int CPR = BK / 16;
  constexpr int A_CH = BM * CPR / NT;        // 16-byte chunks per thread per stage
  constexpr int B_CH = BN * CPR / NT;
  static_assert(BM * CPR % NT == 0 && BN * CPR % NT == 0, "tile / thread mismatch");
  static_assert(!MX || BK % 64 == 0, "MX steps are 64 deep");
  constexpr int STAGE = (BM + BN) * BK;

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WN, wn = wid % WN;

  // Tile order: workgroups are dealt round-robin over the 8 XCDs; give each
  // XCD a contiguous run of tiles, walked column-block-major within groups of
  // 8 tile-rows so that neighbours share A rows and W columns in that L2.
  const int tiles_m = (int)((p.M + BM - 1) / BM);
  const int tiles_n = (int)((p.N + BN - 1) / BN);
  const int ntiles = tiles_m * tiles_n;
  int pid = blockIdx.x;
  {
    const int per = ntiles / 8;
    if (per > 0 && pid < per * 8) pid = (pid % 8) * per + pid / 8;
  }
  constexpr int GROUP = 8;
  const int group_tiles = GROUP * tiles_n;
  const int g = pid / group_tiles;
  const int first_m = g * GROUP;
  const int gsize = min(tiles_m - first_m, GROUP);
  const int tile_m = first_m + (pid % group_tiles) % gsize;
  const int tile_n = (pid % group_tiles) / gsize;
  const int64_t m0 = (int64_t)tile_m * BM, n0 = (int64_t)tile_n * BN;

  const int nkt = (int)(p.K_pad / BK);

  // ---- global -> register staging, register -> LDS stores
  v4i ra[A_CH], rb[B_CH];
#define QG_LOAD_STAGE(KT)                                                                     \
  {                                                                                           \
    const int64_t k0_ = (int64_t)(KT) * BK;                                                   \
    _Pragma("unroll") for (int i = 0; i < A_CH; ++i) {                                        \
      const int id = tid + i * NT;                                                            \
      const int r = id / CPR, c = id % CPR;                                                   \
      const int64_t m = m0 + r, k = k0_ + c * 16;                                             \
      ra[i] = (m < p.M && k < p.K) ? *reinterpret_cast<const v4i*>(p.a + m * p.lda + k)       \
                                   : v4i{0, 0, 0, 0};                                         \
    }                                                                                         \
    _Pragma("unroll") for (int i = 0; i < B_CH; ++i) {                                        \
      const int id = tid + i * NT;                                                            \
      const int r = id / CPR, c = id % CPR;                                                   \
      rb[i] = *reinterpret_cast<const v4i*>(p.w + (n0 + r) * p.K_pad + k0_ + c * 16);         \
    }                                                                                         \
  }
#define QG_STORE_STAGE(S)                                                                     \
  {                                                                                           \
    uint8_t* sa_ = smem + (S) * STAGE;                                                        \
    uint8_t* sb_ = sa_ + BM * BK;                                                             \
    _Pragma("unroll") for (int i = 0; i < A_CH; ++i) {                                        \
      const int id = tid + i * NT;                                                            \
      const int r = id / CPR, c = id % CPR;                                                   \
      v4i v = ra[i];                                                                          \
      if (ASYM) v ^= (int)0x80808080u;                                                        \
      *reinterpret_cast<v4i*>(sa_ + lds_off<BK>(r, c)) = v;                                   \
    }                                                                                         \
    _Pragma("unroll") for (int i = 0; i < B_CH; ++i) {                                        \
      const int id = tid + i * NT;                                                            \
      const int r = id / CPR, c = id % CPR;                                                   \
      *reinterpret_cast<v4i*>(sb_ + lds_off<BK>(r, c)) = rb[i];                               \
    }                                                                                         \
  }

  // ---- MX scales: per lane, one E8M0 byte per (fragment, 64-deep step)
  constexpr int KS = MX ? BK / 64 : 1;
  int esa[MX ? FM * KS : 1], esb[MX ? FN * KS : 1];
  const int64_t kblocks = p.K / 32;
#define QG_LOAD_SCALES(KT)                                                                    \
  if constexpr (MX) {                                                                         \
    _Pragma("unroll") for (int ks = 0; ks < KS; ++ks) {                                       \
      const int64_t blk = ((int64_t)(KT) * BK + ks * 64) / 32 + (lane >> 5);                  \
      _Pragma("unroll") for (int i = 0; i < FM; ++i) {                                        \
        const int64_t m = m0 + wm * TM + i * 32 + (lane & 31);                                \
        esa[ks * FM + i] = (m < p.M && blk < kblocks) ? (int)p.ea[m * p.lda_s + blk] : 127;   \
      }                                                                                       \
      _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                        \
        const int64_t n = n0 + wn * TN + j * 32 + (lane & 31);                                \
        esb[ks * FN + j] = (int)p.ew[n * (p.K_pad / 32) + blk];                               \
      }                                                                                       \
    }                                                                                         \
  }

  typedef typename std::conditional<MX, v16f, v16i>::type acc_t;
  acc_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  QG_LOAD_STAGE(0)
  QG_STORE_STAGE(0)
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1;
    QG_LOAD_SCALES(kt)
    if (kt + 1 < nkt) QG_LOAD_STAGE(kt + 1)
    const uint8_t* sa = smem + cur * STAGE;
    const uint8_t* sb = sa + BM * BK;
    if constexpr (!MX) {
#pragma unroll
      for (int kk = 0; kk < BK / 32; ++kk) {
        const int ch = kk * 2 + (lane >> 5);
        v4i af[FM], bf[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
          af[i] = *reinterpret_cast<const v4i*>(sa + lds_off<BK>(wm * TM + i * 32 + (lane & 31), ch));
#pragma unroll
        for (int j = 0; j < FN; ++j)
          bf[j] = *reinterpret_cast<const v4i*>(sb + lds_off<BK>(wn * TN + j * 32 + (lane & 31), ch));
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        // lane 32h + r: bytes 0..15 = K 16h.., bytes 16..31 = K 32+16h.. of this 64-deep step
        const int c0 = ks * 4 + (lane >> 5), c1 = c0 + 2;
        v8i af[FM], bf[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int r = wm * TM + i * 32 + (lane & 31);
          v4i lo = *reinterpret_cast<const v4i*>(sa + lds_off<BK>(r, c0));
          v4i hi = *reinterpret_cast<const v4i*>(sa + lds_off<BK>(r, c1));
          af[i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int r = wn * TN + j * 32 + (lane & 31);
          v4i lo = *reinterpret_cast<const v4i*>(sb + lds_off<BK>(r, c0));
          v4i hi = *reinterpret_cast<const v4i*>(sb + lds_off<BK>(r, c1));
          bf[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                af[i], bf[j], acc[i][j], 0, 0, 0, esa[ks * FM + i], 0, esb[ks * FN + j]);
      }
    }
    if (kt + 1 < nkt) QG_STORE_STAGE(cur ^ 1)
    __syncthreads();
  }
#undef QG_LOAD_STAGE
#undef QG_STORE_STAGE
#undef QG_LOAD_SCALES

  // ---- epilogue: lane l of a 32x32 block holds column l%32 and rows
  // 8*(e/4) + 4*(l/32) + e%4 for its 16 values e. The tile's per-row scale
  // and zero point are staged in LDS (free after the last barrier).
  float* s_sa = reinterpret_cast<float*>(smem);
  int* s_z = reinterpret_cast<int*>(smem + BM * 4);
  if constexpr (!MX && OUT != 2) {
    for (int r = tid; r < BM; r += NT) {
      const int64_t m = m0 + r;
      s_sa[r] = m < p.M ? (p.a_per_tensor ? p.sa[0] : p.sa[m]) : 0.f;
    }
  }
  if constexpr (!MX && ASYM) {
    for (int r = tid; r < BM; r += NT) {
      const int64_t m = m0 + r;
      s_z[r] = m < p.M ? (p.a_per_tensor ? p.za[0] : p.za[m]) : 0;
    }
  }
  if constexpr (!MX && (ASYM || OUT != 2)) __syncthreads();

#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int64_t n = n0 + wn * TN + j * 32 + (lane & 31);
    const bool n_ok = n < p.N;
    float sw = 0.f;
    int cs = 0;
    if constexpr (!MX) {
      if (n_ok) {
        sw = p.w_per_tensor ? p.sw[0] : p.sw[n];
        if (ASYM) cs = p.colsum[n];
      }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = wm * TM + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int64_t m = m0 + r;
        if (!(n_ok && m < p.M)) continue;
        if constexpr (MX) {
          reinterpret_cast<float*>(p.out)[m * p.ldo + n] = acc[i][j][e];
        } else {
          int c = acc[i][j][e];
          if (ASYM) {
            // wrap-around int32 arithmetic: the true C fits, so the result is exact
            c = (int)((uint32_t)c - (uint32_t)(s_z[r] - 128) * (uint32_t)cs);
          }
          if constexpr (OUT == 2) {
            reinterpret_cast<int32_t*>(p.out)[m * p.ldo + n] = c;
          } else {
            const float y = (float)c * (s_sa[r] * sw);
            if constexpr (OUT == 0)
              reinterpret_cast<float*>(p.out)[m * p.ldo + n] = y;
            else
              reinterpret_cast<uint16_t*>(p.out)[m * p.ldo + n] = f32_to_bf16_rne(y);
          }
        }
      }
    }
  }
}

template <int BM, int BN, int BK, int WM, int WN, bool MX, bool ASYM, int OUT>
static hipError_t launch_cfg(const GemmArgs& a, hipStream_t st) {
  auto kern = gemm_kernel<BM, BN, BK, WM, WN, MX, ASYM, OUT>;
  const size_t lds = (size_t)2 * (BM + BN) * BK;
  if (lds > 65536) {  // above the default dynamic-LDS limit (gfx950 has 160 KiB)
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(WM * WN * 64), lds, st, a);
  return hipGetLastError();
}

template <bool MX, bool ASYM, int OUT>
static hipError_t launch_pick(const GemmArgs& a, hipStream_t st) {
  // Large problems: 256x256 tiles (4 waves of 128x128); otherwise 128x128.
  const int64_t big_tiles = ((a.M + 255) / 256) * ((a.N + 255) / 256);
  if (big_tiles >= 256) return launch_cfg<256, 256, 64, 2, 2, MX, ASYM, OUT>(a, st);
  return launch_cfg<128, 128, 64, 2, 2, MX, ASYM, OUT>(a, st);
}

hipError_t launch_gemm_i8(const GemmArgs& a, bool asym, int out_type, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  if (asym) {
    if (out_type == 0) return launch_pick<false, true, 0>(a, st);
    if (out_type == 1) return launch_pick<false, true, 1>(a, st);
    return launch_pick<false, true, 2>(a, st);
  }
  if (out_type == 0) return launch_pick<false, false, 0>(a, st);
  if (out_type == 1) return launch_pick<false, false, 1>(a, st);
  return launch_pick<false, false, 2>(a, st);
}

hipError_t launch_gemm_mx(const GemmArgs& a, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  return launch_pick<true, false, 0>(a, st);
}

}  // namespace qg
