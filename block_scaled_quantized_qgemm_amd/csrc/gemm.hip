// Matrix-core GEMMs for gfx950.
//
// int8 x int8 (exact int32 sums, fused dequantization epilogue):
//  * gemm_i8_dma_kernel -- tiled, v_mfma_i32_32x32x32_i8, tiles fetched from
//    global memory straight into an LDS ring; for M > 16.
//  * gemm_i8_decode_kernel -- M <= 16: a stream over the weights with
//    v_mfma_i32_16x16x64_i8, every weight byte read once into registers.
//
// (int8 x int4 with per-group scales lives in gemm_w4a8.hip.)
//
// MX (e4m3 or e2m1 + E8M0 per 32 K), float32 output, gemm_mx_kernel in two modes:
//  * MXB -- exact products: each e4m3 value is multiplied by its block's
//           power-of-two scale while the tile is moved into LDS
//           (v_cvt_scalef32_pk_bf16_fp8; e4m3 times a power of two is exactly
//           representable in bf16), then v_mfma_f32_32x32x16_bf16 forms exact
//           products and float32 sums.
//  * MXF -- the block-scaled fp8 matrix cores
//           (v_mfma_scale_f32_32x32x64_f8f6f4), one E8M0 byte per lane and
//           block. Inside each group of 8 consecutive K the hardware aligns the
//           products to the largest one and drops bits more than 13 binades
//           below it, so sums are not float32-exact.
//  The MX tiling: a workgroup owns a BM x BN tile and walks K in BK-deep
//  steps; the next step's A and W tiles are fetched from global memory into
//  registers (16-byte loads, consecutive lanes on consecutive bytes of a row)
//  while the matrix cores consume the current step out of LDS; LDS holds two
//  stages whose rows store 16-byte chunks XOR-swizzled by row, so the 16-byte
//  fragment reads of 32 consecutive rows spread over all banks. Each wave owns
//  a (BM/WM) x (BN/WN) sub-tile of 32x32 matrix-core blocks. The epilogue goes
//  through LDS so that every lane stores 16 contiguous bytes of a row.
//
// Semantics followed:
//  * int8: C = sum_k (q_a - z_a) q_w exactly in int32 ("Activation
//    Quantization Architecture, in depth", section "The integer GEMM, written
//    out"), then out = float(C) * (s_a * s_w) once per output ("100 Days of
//    GPU -- Day 98", section "The program, and the gate that has to be per
//    column"). uint8 codes enter the signed matrix cores as q - 128 (a byte
//    XOR with 0x80) and the epilogue subtracts (z - 128) * colsum instead of
//    z * colsum, which yields the same exact C.
//  * MX: every 32-element K block carries its own pair of E8M0 factors inside
//    the K loop ("TileLang tutorial, chapter 27", sections 4.1 and 4.3).
#include <atomic>

#include "common.hpp"
#include "kernels.hpp"

namespace qg {

enum MxMode { MXB = 1, MXF = 2 };

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// The exact MX mode's bf16 tiles have 128-byte rows, written as converted
// 16-byte chunks (four lanes per row: chunks 2c or 2c + 1, c = lane % 4) and
// read as MFMA fragments (16 lanes on 16 consecutive rows at one chunk).
// gfx950 serves 16-byte reads 16 consecutive lanes per cycle over its 64
// four-byte banks, and 16-byte writes 8 consecutive lanes per cycle over a
// 128-byte window (fitted to bank-conflict counter measurements). Reads then
// need the row's chunk XOR to be a bijection on row bits 1-3 (the 8 rows of
// one parity share a bank half), and writes need it to flip chunk parity
// between the two rows of a cycle: XOR with (row / 2) % 8 and with row % 2.
__device__ inline int lds_off_bf16(int row, int chunk) {
  return row * 128 + (((chunk ^ ((row >> 1) & 7) ^ (row & 1)) & 7) << 4);
}

// LDS offset of the 16-byte chunk `chunk` (K bytes [16 chunk, 16 chunk + 16)
// of the stage) of W tile row `row` when the stage holds the packed weight
// blocks of 16 rows x 64 K in order (row block major, BK / 64 blocks per row
// block). The 16 lanes that read one chunk of 16 consecutive rows cover 256
// contiguous bytes, i.e. every bank once.
template <int BK>
__device__ inline int w_blk_off(int row, int chunk) {
  return (((row >> 4) * (BK / 64) + (chunk >> 2)) << 10) + ((chunk & 3) << 8) + ((row & 15) << 4);
}

// Sixteen e4m3 codes times 2^(E-127) as sixteen bf16 (exact for E in [3, 240]).
__device__ inline void fp8x16_to_bf16(const v4i& q, float scale, v4i& lo, v4i& hi) {
  v2bf t[8];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    t[2 * d] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)q[d], scale, false);
    t[2 * d + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)q[d], scale, true);
  }
  int w[8];
  __builtin_memcpy(w, t, 32);
  lo = v4i{w[0], w[1], w[2], w[3]};
  hi = v4i{w[4], w[5], w[6], w[7]};
}

// Sixteen e2m1 codes (8 bytes, element 2i in the low nibble of byte i) times
// 2^(E-127) as sixteen bf16 (exact: two significant bits).
__device__ inline void fp4x16_to_bf16(const v4i& q, float scale, v4i& lo, v4i& hi) {
  v2bf t[8];
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    t[4 * d + 0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((unsigned)q[d], scale, 0);
    t[4 * d + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((unsigned)q[d], scale, 1);
    t[4 * d + 2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((unsigned)q[d], scale, 2);
    t[4 * d + 3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((unsigned)q[d], scale, 3);
  }
  int w[8];
  __builtin_memcpy(w, t, 32);
  lo = v4i{w[0], w[1], w[2], w[3]};
  hi = v4i{w[4], w[5], w[6], w[7]};
}

// FA4 / FW4 in the scaled mode: that operand's e2m1 codes are staged raw, 32
// codes per 16-byte chunk (so its LDS rows are half as long as e4m3 rows).
template <int BM, int BN, int BK, int WM, int WN, int MODE, bool FA4 = false, bool FW4 = false>
struct MxCfg {
  static constexpr int NT = WM * WN * 64;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr bool A4 = MODE == MXF && FA4, W4 = MODE == MXF && FW4;  // raw e2m1 staging
  static constexpr int KPCA = A4 ? 32 : 16, KPCW = W4 ? 32 : 16;          // K per global chunk
  static constexpr int CPRA = BK / KPCA, CPRW = BK / KPCW;                 // global chunks per row and K step
  // LDS bytes per row: bf16 in the exact mode, the codes as they are otherwise
  static constexpr int RBA = MODE == MXB ? 2 * BK : (A4 ? BK / 2 : BK);
  static constexpr int RBW = MODE == MXB ? 2 * BK : (W4 ? BK / 2 : BK);
  static constexpr int A_CH = BM * CPRA / NT, B_CH = BN * CPRW / NT;
  static constexpr int STAGE = BM * RBA + BN * RBW;
  static constexpr int RS = TN + 8;  // epilogue staging row stride in words: rows r and r+4
                                     // (the two half-waves) start 32 banks apart
  static constexpr int EPI = WM * WN * 32 * RS * 4;      // per-wave 32 x TN float staging
  static constexpr int LDS = 2 * STAGE > EPI ? 2 * STAGE : EPI;
  static_assert(BM * CPRA % NT == 0 && BN * CPRW % NT == 0, "tile / thread mismatch");
  static_assert(MODE != MXF || BK % 64 == 0, "scaled fp8 steps are 64 deep");
  static_assert(MODE != MXB || (RBA == 128 && RBW == 128), "exact-mode staging: 128-byte bf16 rows");
  static_assert(TN % 4 == 0 && (TN / 4) <= 64 && 64 % (TN / 4) == 0, "epilogue lane map");
};

// FA4 / FW4: the activations / weights are e2m1, two codes per byte. In the
// exact mode a 16-K chunk is then 8 bytes, converted to the same two bf16 LDS
// chunks as sixteen e4m3 codes. In the scaled mode the codes go to LDS as they
// are, each operand in its own format: an e2m1 lane operand for a 64-deep step
// is the 16 bytes holding K 32h .. 32h + 31 of its row (lane 32h + r;
// measured), an e4m3 one the 32 bytes of K 16h .. and 32 + 16h .., and each
// operand's format code goes to the instruction (so e4m3 x e2m1 pairs run
// too). e2m1 x e2m1 products span under 8 binades, so the hardware's
// 8-product alignment drops nothing and the sums are float32 sums; a pair
// with an e4m3 operand has the e4m3 bound of the scaled mode.
template <int BM, int BN, int BK, int WM, int WN, int MODE, bool FA4 = false, bool FW4 = false>
__global__ __launch_bounds__(WM* WN * 64) void gemm_mx_kernel(GemmArgs p) {
  using C = MxCfg<BM, BN, BK, WM, WN, MODE, FA4, FW4>;
  constexpr bool A4 = C::A4, W4 = C::W4;
  constexpr int NT = C::NT, TM = C::TM, TN = C::TN, FM = C::FM, FN = C::FN;
  constexpr int CPRA = C::CPRA, CPRW = C::CPRW, RBA = C::RBA, RBW = C::RBW, KPCA = C::KPCA, KPCW = C::KPCW;
  constexpr int A_CH = C::A_CH, B_CH = C::B_CH, STAGE = C::STAGE;

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WN, wn = wid % WN;

  // Tile order: workgroups are dealt round-robin over the 8 XCDs; give each
  // XCD a contiguous run of tiles, walked in groups of 8 tile-rows so that
  // neighbours share A rows and W columns in that XCD's L2.
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
  const int64_t kblocks = p.K / 32;
  const int64_t wblocks = p.K_pad / 32;

  // ---- global -> register staging (and, for MXB, the scale of each chunk).
  // Two register sets: while the matrix cores consume stage kt from LDS, set
  // (kt+1)&1 already holds stage kt+1 and stage kt+2 is in flight into the
  // other set, so global latency is covered by two stages of matrix work.
  v4i ra0[A_CH], rb0[B_CH], ra1[A_CH], rb1[B_CH];
  int ea0[MODE == MXB ? A_CH : 1], eb0[MODE == MXB ? B_CH : 1];
  int ea1[MODE == MXB ? A_CH : 1], eb1[MODE == MXB ? B_CH : 1];
#define QG_LOAD_STAGE(KT, RA, RB_, EA, EB)                                                      \
  {                                                                                             \
    const int64_t k0_ = (int64_t)(KT) * BK;                                                     \
    _Pragma("unroll") for (int i = 0; i < A_CH; ++i) {                                          \
      const int id = tid + i * NT;                                                              \
      const int r = id / CPRA, c = id % CPRA;                                                   \
      /* Unconditional load from a clamped address: no branch and no use of the */             \
      /* value before the LDS store, so the loads stay in flight. Rows >= M only */             \
      /* feed outputs that are never stored; columns >= K meet zero weights (and */             \
      /* are zeroed at the store for MX, where a stray code could be NaN). */                   \
      const int64_t m = min(m0 + r, p.M - 1), k = k0_ + c * KPCA;                                \
      const int64_t kc = k < p.K ? k : 0;                                                       \
      if constexpr (A4) {                                                                       \
        RA[i] = *reinterpret_cast<const v4i*>(p.a + m * p.lda + (kc >> 1));                     \
      } else if constexpr (FA4) {                                                               \
        const uint2 h_ = *reinterpret_cast<const uint2*>(p.a + m * p.lda + (kc >> 1));          \
        RA[i] = v4i{(int)h_.x, (int)h_.y, 0, 0};                                                \
      } else {                                                                                  \
        RA[i] = *reinterpret_cast<const v4i*>(p.a + m * p.lda + kc);                            \
      }                                                                                         \
      if constexpr (MODE == MXB) EA[i] = (int)p.ea[m * p.lda_s + (kc >> 5)];                    \
    }                                                                                           \
    _Pragma("unroll") for (int i = 0; i < B_CH; ++i) {                                          \
      const int id = tid + i * NT;                                                              \
      const int r = id / CPRW, c = id % CPRW;                                                   \
      const int64_t n = n0 + r, k = k0_ + c * KPCW;                                             \
      if constexpr (W4) {                                                                       \
        RB_[i] = *reinterpret_cast<const v4i*>(p.w + n * (p.K_pad >> 1) + (k >> 1));            \
      } else if constexpr (FW4) {                                                               \
        const uint2 h_ = *reinterpret_cast<const uint2*>(p.w + n * (p.K_pad >> 1) + (k >> 1));  \
        RB_[i] = v4i{(int)h_.x, (int)h_.y, 0, 0};                                               \
      } else {                                                                                  \
        RB_[i] = *reinterpret_cast<const v4i*>(p.w + mx8_code_off(n, k, p.K_pad));              \
      }                                                                                         \
      if constexpr (MODE == MXB) EB[i] = (int)p.ew[n * wblocks + (k >> 5)];                     \
    }                                                                                           \
  }
#define QG_STORE_STAGE(KT, S, RA, RB_, EA, EB)                                                  \
  {                                                                                             \
    uint8_t* sa_ = smem + (S) * STAGE;                                                          \
    uint8_t* sb_ = sa_ + BM * RBA;                                                              \
    _Pragma("unroll") for (int i = 0; i < A_CH; ++i) {                                          \
      const int id = tid + i * NT;                                                              \
      const int r = id / CPRA, c = id % CPRA;                                                   \
      if ((int64_t)(KT) * BK + c * KPCA >= p.K) RA[i] = v4i{0, 0, 0, 0};                        \
      if constexpr (MODE == MXB) {                                                              \
        v4i lo, hi;                                                                             \
        if constexpr (FA4)                                                                      \
          fp4x16_to_bf16(RA[i], e8m0_to_f32(EA[i]), lo, hi);                                    \
        else                                                                                    \
          fp8x16_to_bf16(RA[i], e8m0_to_f32(EA[i]), lo, hi);                                    \
        *reinterpret_cast<v4i*>(sa_ + lds_off_bf16(r, 2 * c)) = lo;                             \
        *reinterpret_cast<v4i*>(sa_ + lds_off_bf16(r, 2 * c + 1)) = hi;                         \
      } else {                                                                                  \
        *reinterpret_cast<v4i*>(sa_ + lds_off<RBA>(r, c)) = RA[i];                              \
      }                                                                                         \
    }                                                                                           \
    _Pragma("unroll") for (int i = 0; i < B_CH; ++i) {                                          \
      const int id = tid + i * NT;                                                              \
      const int r = id / CPRW, c = id % CPRW;                                                   \
      if constexpr (MODE == MXB) {                                                              \
        v4i lo, hi;                                                                             \
        if constexpr (FW4)                                                                      \
          fp4x16_to_bf16(RB_[i], e8m0_to_f32(EB[i]), lo, hi);                                   \
        else                                                                                    \
          fp8x16_to_bf16(RB_[i], e8m0_to_f32(EB[i]), lo, hi);                                   \
        *reinterpret_cast<v4i*>(sb_ + lds_off_bf16(r, 2 * c)) = lo;                             \
        *reinterpret_cast<v4i*>(sb_ + lds_off_bf16(r, 2 * c + 1)) = hi;                         \
      } else {                                                                                  \
        *reinterpret_cast<v4i*>(sb_ + lds_off<RBW>(r, c)) = RB_[i];                             \
      }                                                                                         \
    }                                                                                           \
  }

  // ---- MXF: per lane one E8M0 byte per (fragment, 64-deep step)
  constexpr int KS = MODE == MXF ? BK / 64 : 1;
  // Scales travel with the stage data: loaded into the register set of the
  // stage (fs*0 / fs*1), copied to the LDS buffer's set (es*0 / es*1) when the
  // stage is stored, used two steps after their load.
  constexpr int SA = MODE == MXF ? FM * KS : 1, SB = MODE == MXF ? FN * KS : 1;
  int fsa0[SA], fsb0[SB], fsa1[SA], fsb1[SB], esa0[SA], esb0[SB], esa1[SA], esb1[SB];
#define QG_LOAD_SCALES(KT, DA, DB)                                                              \
  if constexpr (MODE == MXF) {                                                                  \
    _Pragma("unroll") for (int ks = 0; ks < KS; ++ks) {                                         \
      const int64_t blk = ((int64_t)(KT) * BK + ks * 64) / 32 + (lane >> 5);                    \
      _Pragma("unroll") for (int i = 0; i < FM; ++i) {                                          \
        /* clamped row and block: a valid E8M0 byte; rows >= M are never stored */            \
        /* and the data of blocks >= K/32 are zeroed */                                        \
        const int64_t m = min(m0 + wm * TM + i * 32 + (lane & 31), p.M - 1);                    \
        DA[ks * FM + i] = (int)p.ea[m * p.lda_s + min(blk, kblocks - 1)];                       \
      }                                                                                         \
      _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                          \
        const int64_t n = n0 + wn * TN + j * 32 + (lane & 31);                                  \
        DB[ks * FN + j] = (int)p.ew[n * wblocks + blk];                                         \
      }                                                                                         \
    }                                                                                           \
  }

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

#define QG_COMPUTE(S)                                                                           \
  {                                                                                             \
    const uint8_t* sa = smem + (S) * STAGE;                                                     \
    const uint8_t* sb = sa + BM * RBA;                                                          \
    if constexpr (MODE == MXB) {                                                                \
      /* 16-deep bf16 steps: lane 32h + r holds K 8h..8h+7 of the step */                      \
      _Pragma("unroll") for (int kk = 0; kk < BK / 16; ++kk) {                                  \
        const int ch = kk * 2 + (lane >> 5);                                                    \
        v8bf af[FM], bf[FN];                                                                    \
        _Pragma("unroll") for (int i = 0; i < FM; ++i) af[i] =                                  \
            *reinterpret_cast<const v8bf*>(sa + lds_off_bf16(wm * TM + i * 32 + (lane & 31), ch)); \
        _Pragma("unroll") for (int j = 0; j < FN; ++j) bf[j] =                                  \
            *reinterpret_cast<const v8bf*>(sb + lds_off_bf16(wn * TN + j * 32 + (lane & 31), ch)); \
        _Pragma("unroll") for (int i = 0; i < FM; ++i)                                          \
          _Pragma("unroll") for (int j = 0; j < FN; ++j)                                        \
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0); \
        __builtin_amdgcn_sched_barrier(0);                                                      \
      }                                                                                         \
    } else {                                                                                    \
      /* 64-deep scaled steps: e4m3, lane 32h + r holds K 16h.. and 32+16h..; */                \
      /* e2m1, lane 32h + r holds K 32h .. 32h+31 in its first 16 bytes */                      \
      _Pragma("unroll") for (int ks = 0; ks < KS; ++ks) {                                       \
        const int ca = A4 ? ks * 2 + (lane >> 5) : ks * 4 + (lane >> 5);                        \
        const int cw = W4 ? ks * 2 + (lane >> 5) : ks * 4 + (lane >> 5);                        \
        v8i af[FM], bf[FN];                                                                     \
        _Pragma("unroll") for (int i = 0; i < FM; ++i) {                                        \
          const int r = wm * TM + i * 32 + (lane & 31);                                         \
          const v4i lo = *reinterpret_cast<const v4i*>(sa + lds_off<RBA>(r, ca));               \
          const v4i hi = A4 ? v4i{0, 0, 0, 0} : *reinterpret_cast<const v4i*>(sa + lds_off<RBA>(r, ca + 2)); \
          af[i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};                  \
        }                                                                                       \
        _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                        \
          const int r = wn * TN + j * 32 + (lane & 31);                                         \
          const v4i lo = *reinterpret_cast<const v4i*>(sb + lds_off<RBW>(r, cw));               \
          const v4i hi = W4 ? v4i{0, 0, 0, 0} : *reinterpret_cast<const v4i*>(sb + lds_off<RBW>(r, cw + 2)); \
          bf[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};                  \
        }                                                                                       \
        _Pragma("unroll") for (int i = 0; i < FM; ++i)                                          \
          _Pragma("unroll") for (int j = 0; j < FN; ++j)                                        \
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                        \
                af[i], bf[j], acc[i][j], A4 ? 4 : 0, W4 ? 4 : 0, 0,                             \
                (S) == 0 ? esa0[ks * FM + i] : esa1[ks * FM + i], 0,                            \
                (S) == 0 ? esb0[ks * FN + j] : esb1[ks * FN + j]);                              \
        __builtin_amdgcn_sched_barrier(0);                                                      \
      }                                                                                         \
    }                                                                                           \
  }
#define QG_KEEP_SCALES(DA, DB, SA_, SB_)                                                        \
  if constexpr (MODE == MXF) {                                                                  \
    _Pragma("unroll") for (int t = 0; t < FM * KS; ++t) DA[t] = SA_[t];                         \
    _Pragma("unroll") for (int t = 0; t < FN * KS; ++t) DB[t] = SB_[t];                         \
  }

  QG_LOAD_SCALES(0, esa0, esb0)
  QG_LOAD_STAGE(0, ra0, rb0, ea0, eb0)
  QG_STORE_STAGE(0, 0, ra0, rb0, ea0, eb0)
  QG_LOAD_STAGE(1, ra1, rb1, ea1, eb1)
  QG_LOAD_SCALES(min(1, nkt - 1), fsa1, fsb1)
  __syncthreads();

  // nkt is even: the packed K is a multiple of 256 and BK divides 128. The
  // body is branch-free (the last stage is simply fetched again at the end),
  // so the compiler can wait for exactly the older register set.
  for (int kt = 0; kt < nkt; kt += 2) {
    // even stage kt: LDS buffer 0; set 1 holds stage kt+1; stage kt+2 goes into set 0
    QG_LOAD_STAGE(min(kt + 2, nkt - 1), ra0, rb0, ea0, eb0)
    QG_LOAD_SCALES(min(kt + 2, nkt - 1), fsa0, fsb0)
    QG_COMPUTE(0)
    QG_STORE_STAGE(kt + 1, 1, ra1, rb1, ea1, eb1)
    QG_KEEP_SCALES(esa1, esb1, fsa1, fsb1)
    __syncthreads();
    // odd stage kt+1: LDS buffer 1; set 0 holds stage kt+2; stage kt+3 goes into set 1
    QG_LOAD_STAGE(min(kt + 3, nkt - 1), ra1, rb1, ea1, eb1)
    QG_LOAD_SCALES(min(kt + 3, nkt - 1), fsa1, fsb1)
    QG_COMPUTE(1)
    QG_STORE_STAGE(kt + 2, 0, ra0, rb0, ea0, eb0)
    QG_KEEP_SCALES(esa0, esb0, fsa0, fsb0)
    __syncthreads();
  }
#undef QG_LOAD_STAGE
#undef QG_STORE_STAGE
#undef QG_LOAD_SCALES
#undef QG_COMPUTE
#undef QG_KEEP_SCALES

  // ---- epilogue through LDS. Lane l of a 32x32 block holds column l%32 and
  // rows 8*(e/4) + 4*(l/32) + e%4 of its 16 values e. Each wave writes one
  // 32-row slab of its sub-tile to its own LDS region, then reads it back row
  // by row so that every lane finishes 4 consecutive columns of one row.
  constexpr int LPR = TN / 4;        // lanes per row on the way out
  constexpr int RPI = 64 / LPR;      // rows per read-back pass
  constexpr int RS = C::RS;
  uint8_t* wreg = smem + wid * (32 * RS * 4);
  const int cq = (lane % LPR) * 4;   // this lane's first column inside the wave tile
  const int64_t nq = n0 + wn * TN + cq;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        reinterpret_cast<float*>(wreg)[r * RS + j * 32 + (lane & 31)] = acc[i][j][e];
      }
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < 32 / RPI; ++pass) {
      const int r = pass * RPI + lane / LPR;
      const int64_t m = m0 + wm * TM + i * 32 + r;
      v4f y = *reinterpret_cast<const v4f*>(wreg + (r * RS + cq) * 4);
      if (m < p.M && nq < p.N) {
        if (p.bias) {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (nq + t < p.N) y[t] = y[t] + p.bias[nq + t];
        }
        float* o = reinterpret_cast<float*>(p.out) + m * p.ldo + nq;
        if (nq + 3 < p.N)
          *reinterpret_cast<v4f*>(o) = y;
        else
          for (int t = 0; t < 4 && nq + t < p.N; ++t) o[t] = y[t];
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Deep pipeline for the 1-byte operand path (int8): the tiles travel from
// global memory straight into an NS-stage LDS ring (global_load_lds_dwordx4:
// each lane's 16 bytes land at the wave's LDS block + 16 * lane), so no
// registers hold staged data and NS - 1 stages are in flight. One explicit
// vmcnt wait and one barrier per K step; the fragments of sub-step kk + 1 are
// read while the matrix cores work on sub-step kk.
// ---------------------------------------------------------------------------
template <int BM, int BN, int BK, int WM, int WN, int NS, bool ASYM, int OUT>
struct DmaCfg {
  static constexpr int NT = WM * WN * 64, NW = WM * WN;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int RB = BK;                       // one byte per element
  static constexpr int STAGE = (BM + BN) * RB;
  static constexpr int IPS = STAGE / 1024;            // 1 KB wave loads per stage
  static constexpr int IPW = IPS / NW;                // ... per wave
  static constexpr int IA = BM * RB / 1024;           // the first IA loads of a stage carry A
  static constexpr int NKK = BK / 32;                 // matrix-core sub-steps per stage
  static constexpr int SLOTS = (NKK - 1) * FM * FN;   // MFMAs the stage's loads are spread over
  static constexpr int RS = TN + 8;
  static constexpr int EPI = NW * 32 * RS * 4;
  static constexpr int EPI_ALL = EPI + BM * 8;        // + per-row scale and zero point
  static constexpr int LDS = NS * STAGE > EPI_ALL ? NS * STAGE : EPI_ALL;
  static_assert(STAGE % 1024 == 0 && IPS % NW == 0 && (BM * RB) % 1024 == 0, "stage / wave-load mismatch");
  static_assert(NKK >= 2 && NKK % 2 == 0 && SLOTS >= IPW, "load slots");
  static_assert(NS >= 2 && (NS - 2) * IPW < 64, "vmcnt range");
  static_assert(TN % 4 == 0 && (TN / 4) <= 64 && 64 % (TN / 4) == 0, "epilogue lane map");
};

template <int BM, int BN, int BK, int WM, int WN, int NS, bool ASYM, int OUT>
__global__ __launch_bounds__(WM* WN * 64) void gemm_i8_dma_kernel(GemmArgs p) {
  using C = DmaCfg<BM, BN, BK, WM, WN, NS, ASYM, OUT>;
  constexpr int TM = C::TM, TN = C::TN, FM = C::FM, FN = C::FN, RB = C::RB;
  constexpr int STAGE = C::STAGE, IPW = C::IPW, NKK = C::NKK, SLOTS = C::SLOTS;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wid / WN, wn = wid % WN;

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

  // Stage loads (buffer_load ... lds, 16 bytes per lane). Wave wid issues the
  // stage's 1 KB loads wid*IPW .. wid*IPW+IPW-1. For A,
  // lane l fetches the 16-byte chunk that belongs at LDS slot l of the
  // swizzled row-major tile (row * lda + chunk); for W, one load copies one
  // packed 16 x 64 weight block (1 KB contiguous) as it is. The lane offsets
  // do not change along K: they are computed once, and the stage's K offset
  // goes in the scalar offset.
  // A rows >= M are clamped to row M - 1 (their outputs are never stored). The
  // buffer's byte range ends at the 16-byte chunk holding A column K - 1 of
  // the last row, so nothing past it is read: the hardware returns zeros for
  // every dword outside the range (the weights are zero there). A stage past
  // the last one gets an empty range, so its loads move no data and still
  // count in vmcnt. Load j = wid * IPW + i of a stage carries A when j < IA,
  // else W (the test is uniform over the wave).
  const uint8_t* const abase = p.a + m0 * p.lda;
  const uint8_t* const wbase = p.w + n0 * p.K_pad;
  const int64_t last_a_row = min((int64_t)BM - 1, p.M - 1 - m0);
  const uint32_t nrec_a = (uint32_t)(last_a_row * p.lda + ((p.K + 15) & ~(int64_t)15));
  // W rows end at N_pad (N rounded up to 256): a tile width that does not
  // divide 256 must not read past the packed codes
  const int64_t n_pad = (p.N + 255) / 256 * 256;
  const uint32_t nrec_w = (uint32_t)(min((int64_t)BN, n_pad - n0) * p.K_pad);
  uint32_t voff[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int j = wid * IPW + i;
    if (j < C::IA) {  // swizzled row-major A tile: slot P holds chunk c of row r
      const int P = j * 1024 + lane * 16;
      const int r = P / RB;
      const int c = ((P % RB) >> 4) ^ ((r / (RB >= 256 ? 1 : 256 / RB)) % (RB / 16));
      voff[i] = (uint32_t)(min((int64_t)r, last_a_row) * p.lda) + (uint32_t)(c * 16);
    } else {  // W tile: the weight blocks (16 rows x 64 K, 1 KB) copied whole, in order
      const int jw = j - C::IA;
      voff[i] = (uint32_t)(((jw / (BK / 64)) * (p.K_pad >> 6) + jw % (BK / 64)) << 10) + (uint32_t)(lane * 16);
    }
  }
  auto dma = [&](int kt, int s, int i, bool live) {
    const bool ja = wid * IPW + i < C::IA;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(ja ? abase : wbase), (short)0, live ? (int)(ja ? nrec_a : nrec_w) : 0, kRawBufferWord3);
    // bytes per stage along the operand's K order: A rows are plain, W blocks hold 16 rows
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, QG_LDSP(smem + s * STAGE + (wid * IPW + i) * 1024), 16, (int)voff[i],
                                             kt * (ja ? BK : BK * 16), 0, 0);
  };

  v16i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

#define QG_LOAD_FRAGS(BUF, KK, FA, FB)                                                            \
  {                                                                                               \
    const uint8_t* sa_ = smem + (BUF) * STAGE;                                                    \
    const int ch_ = (KK) * 2 + (lane >> 5);                                                       \
    _Pragma("unroll") for (int i = 0; i < FM; ++i) FA[i] =                                        \
        *reinterpret_cast<const v4i*>(sa_ + lds_off<RB>(wm * TM + i * 32 + (lane & 31), ch_));    \
    _Pragma("unroll") for (int j = 0; j < FN; ++j) FB[j] = *reinterpret_cast<const v4i*>(         \
        sa_ + BM * RB + w_blk_off<BK>(wn * TN + j * 32 + (lane & 31), ch_));                      \
  }
  v4i fa[2][FM], fb[2][FN];

  // prologue: stages 0 .. NS-2 in flight
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
#pragma unroll
    for (int i = 0; i < IPW; ++i) dma(s, s, i, s < nkt);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * IPW));
  __builtin_amdgcn_s_barrier();
  QG_LOAD_FRAGS(0, 0, fa[0], fb[0])

  for (int kt = 0; kt < nkt; ++kt) {
    // Stage kt + NS - 1 refills the slot every wave finished reading before the
    // last barrier; its loads are spread between the matrix-core instructions
    // of the first NKK - 1 sub-steps.
    const int ks = kt + NS - 1;
    const bool live = ks < nkt;
    const int cur = kt % NS, nxt = (kt + 1) % NS, sl = ks % NS;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int pb = kk & 1, qb = pb ^ 1;
      if (kk + 1 < NKK) {
        QG_LOAD_FRAGS(cur, kk + 1, fa[qb], fb[qb])
      } else {
        // next stage: its loads landed (vmcnt counts the loads issued after
        // it), this wave's reads of the current stage are done (lgkmcnt 0);
        // after the barrier everyone's are
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * IPW) & ~(15 << 8));
        __builtin_amdgcn_s_barrier();
        QG_LOAD_FRAGS(nxt, 0, fa[qb], fb[qb])
      }
      __builtin_amdgcn_sched_barrier(0);
      if (ASYM) {  // uint8 codes enter the signed matrix cores as q - 128
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[pb][i] ^= (int)0x80808080u;
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[pb][i], fb[pb][j], acc[i][j], 0, 0, 0);
          if (kk + 1 < NKK) {
            const int slot = kk * FM * FN + i * FN + j;
#pragma unroll
            for (int d = 0; d < IPW; ++d)
              if ((d * SLOTS) / IPW == slot) dma(ks, sl, d, live);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
    }
  }
#undef QG_LOAD_FRAGS
  // the empty loads past the last stage may still be in flight
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();

  // ---- epilogue through LDS (the scheme of gemm_mx_kernel); the tile's row
  // scales and zero points are fetched once into LDS after the staging area
  constexpr int LPR = TN / 4;
  constexpr int RPI = 64 / LPR;
  constexpr int RS = C::RS;
  uint8_t* wreg = smem + wid * (32 * RS * 4);
  float* rsa = reinterpret_cast<float*>(smem + C::EPI);
  int* rza = reinterpret_cast<int*>(smem + C::EPI + BM * 4);
  for (int r = tid; r < BM; r += C::NT) {
    const int64_t m = min(m0 + r, p.M - 1);
    rsa[r] = p.a_per_tensor ? p.sa[0] : p.sa[m];
    if (ASYM) rza[r] = p.a_per_tensor ? p.za[0] : p.za[m];
  }
  const int cq = (lane % LPR) * 4;
  const int64_t nq = n0 + wn * TN + cq;
  float sw4[4] = {0.f, 0.f, 0.f, 0.f}, bs4[4] = {0.f, 0.f, 0.f, 0.f};
  int cs4[4] = {0, 0, 0, 0};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if (nq + t < p.N) {
      sw4[t] = p.w_per_tensor ? p.sw[0] : p.sw[nq + t];
      if (ASYM) cs4[t] = p.colsum[nq + t];
      if (p.bias) bs4[t] = p.bias[nq + t];
    }
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        reinterpret_cast<int*>(wreg)[r * RS + j * 32 + (lane & 31)] = acc[i][j][e];
      }
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < 32 / RPI; ++pass) {
      const int r = pass * RPI + lane / LPR;
      const int64_t m = m0 + wm * TM + i * 32 + r;
      const v4i raw = *reinterpret_cast<const v4i*>(wreg + (r * RS + cq) * 4);
      if (m < p.M && nq < p.N) {
        float y[4];
        int ci[4];
        const float sam = rsa[wm * TM + i * 32 + r];
        const int zm = ASYM ? rza[wm * TM + i * 32 + r] : 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          int c = raw[t];
          // wrap-around int32 arithmetic: the true C fits, so the result is exact
          if (ASYM) c = (int)((uint32_t)c - (uint32_t)(zm - 128) * (uint32_t)cs4[t]);
          ci[t] = c;
          y[t] = (float)c * (sam * sw4[t]);
          if (p.bias) y[t] = y[t] + bs4[t];  // the bias after the scales, in float32
        }
        const bool full = nq + 3 < p.N;
        if constexpr (OUT == 2) {
          int32_t* o = reinterpret_cast<int32_t*>(p.out) + m * p.ldo + nq;
          if (full)
            *reinterpret_cast<v4i*>(o) = v4i{ci[0], ci[1], ci[2], ci[3]};
          else
            for (int t = 0; t < 4 && nq + t < p.N; ++t) o[t] = ci[t];
        } else if constexpr (OUT == 0) {
          float* o = reinterpret_cast<float*>(p.out) + m * p.ldo + nq;
          if (full)
            *reinterpret_cast<v4f*>(o) = v4f{y[0], y[1], y[2], y[3]};
          else
            for (int t = 0; t < 4 && nq + t < p.N; ++t) o[t] = y[t];
        } else {
          uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + m * p.ldo + nq;
          uint16_t h[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) h[t] = f32_to_bf16_rne(y[t]);
          if (full) {
            uint2 v;
            v.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
            v.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
            *reinterpret_cast<uint2*>(o) = v;
          } else {
            for (int t = 0; t < 4 && nq + t < p.N; ++t) o[t] = h[t];
          }
        }
      }
    }
    __syncthreads();
  }
}

int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int BM, int BN, int BK, int WM, int WN, int NS, bool ASYM, int OUT>
static hipError_t launch_dma(const GemmArgs& a, hipStream_t st) {
  using C = DmaCfg<BM, BN, BK, WM, WN, NS, ASYM, OUT>;
  auto kern = gemm_i8_dma_kernel<BM, BN, BK, WM, WN, NS, ASYM, OUT>;
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(C::NT), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Decode-shaped GEMM (M <= 16 rows): the time is the stream of W out of HBM,
// so every byte of W is read once, straight into registers, and the matrix
// cores only need to keep up. A workgroup owns kDecCols blocks of 16 weight
// rows (v_mfma_i32_16x16x64_i8 column blocks) over all of K; its eight waves
// take contiguous ranges of K. A wave works through its range in batches of
// eight 64-deep steps: each step is one contiguous 1 KB load of W per block
// (a 16 x 64 weight block already in the operand's lane order) and one
// 16-byte load per lane of the activation rows, which then feeds every
// block's instruction. Weight loads are non-temporal (each byte is used
// once). Every load of a batch is issued before any is used (24 loads in
// flight per wave, two workgroups per CU). The activation rows ride in the
// other operand. Rows >= M, steps at or past K_pad (each block has its own
// buffer range) and columns past the last 16-byte chunk holding column K - 1
// come back as zeros from the range-checked buffer loads. The eight partial
// int32 tiles are summed through LDS before the epilogue, so the result is
// exact.
// ---------------------------------------------------------------------------
constexpr int kDecWaves = 8;  // waves per workgroup, each on its own K range
constexpr int kDecBatch = 8;  // 64-deep steps per load batch
constexpr int kDecCols = 2;   // 16-row weight blocks per workgroup
constexpr int kDecWAux = 2;   // non-temporal weight loads

// ONE: K_pad <= 512 * kDecWaves, one batch per wave (no loop).
// MLE8 (M <= 8): rows 8-15 of the 16-row activation operand only feed output
// rows that are never stored, so one 16-byte load per lane carries two steps
// (lanes 16c + r: chunk c of step s for row r; lanes 16c + 8 + r: chunk c of
// step s + 1) and a DPP rotate by 8 lanes within each row of 16 lanes gives
// the second step's operand. Half the activation loads, and 16 fewer VGPRs
// per batch.
template <bool ASYM, int OUT, bool ONE, bool MLE8>
__global__ __launch_bounds__(kDecWaves * 64) void gemm_i8_decode_kernel(GemmArgs p) {
  constexpr int U = kDecBatch;
  constexpr int UA = MLE8 ? U / 2 : U;  // activation loads per batch
  __shared__ v4i red[kDecWaves][kDecCols][64];
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n0 = (int64_t)blockIdx.x * 16 * kDecCols;
  const int steps = (int)(p.K_pad / 64);
  // steps of each wave: a whole number of batches. Steps at or past K_pad
  // fall outside the block's W range and read as zeros, so no load is tested;
  // the A bytes they meet (the next row's, or zeros past A's end) are
  // multiplied by those zeros.
  const int per = ONE ? U : (steps + kDecWaves * U - 1) / (kDecWaves * U) * U;
  const int sbeg = wid * per;

  // operand lanes: lane l carries weight row l % 16 and the 16-byte K chunk
  // l / 16 of every 64-deep step; the activation lanes as described above.
  // Rows >= M read A as zeros through an offset beyond its range.
  const int arow = MLE8 ? (lane & 7) : (lane & 15);
  const int akin = (MLE8 ? ((lane >> 3) & 1) * 64 : 0) + (lane >> 4) * 16;
  constexpr uint32_t kOff = 0x80000000u;
  // one range per 16-row block, so its steps past K_pad read zeros (the
  // packed rows are padded to a multiple of 256, so every block exists)
  __amdgpu_buffer_rsrc_t wrs[kDecCols];
#pragma unroll
  for (int c = 0; c < kDecCols; ++c)
    wrs[c] = __builtin_amdgcn_make_buffer_rsrc((void*)(p.w + (n0 + 16 * c) * p.K_pad), (short)0, (int)(16 * p.K_pad),
                                               kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.a, (short)0, (int)((p.M - 1) * p.lda + ((p.K + 15) & ~(int64_t)15)), kRawBufferWord3);
  const uint32_t woff = (uint32_t)sbeg * 1024u + (uint32_t)(lane * 16);  // 16 x 64 blocks, lane order
  const uint32_t aoff = arow < p.M ? (uint32_t)(arow * p.lda + sbeg * 64 + akin) : kOff;

  // one batch at a time: its loads are all issued before the first MFMA
  v4i acc[kDecCols];
#pragma unroll
  for (int c = 0; c < kDecCols; ++c) acc[c] = v4i{0, 0, 0, 0};
  for (int b = 0; b < (ONE ? U : per); b += U) {
    v4i av[UA], wv[kDecCols][U];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int c = 0; c < kDecCols; ++c)
        wv[c][u] = __builtin_bit_cast(
            v4i, __builtin_amdgcn_raw_buffer_load_b128(wrs[c], (int)(woff + (uint32_t)((b + u) * 1024)), 0, kDecWAux));
#pragma unroll
    for (int u = 0; u < UA; ++u)
      av[u] = __builtin_bit_cast(
          v4i, __builtin_amdgcn_raw_buffer_load_b128(
                   ars, (int)(aoff + (uint32_t)((b + (MLE8 ? 2 * u : u)) * 64)), 0, 0));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      v4i a;
      if (MLE8 && (u & 1)) {
#pragma unroll
        for (int d = 0; d < 4; ++d) a[d] = __builtin_amdgcn_update_dpp(0, av[u / 2][d], 0x128, 0xF, 0xF, false);  // row_ror:8
      } else {
        a = av[MLE8 ? u / 2 : u];
      }
      if (ASYM) a ^= (int)0x80808080u;  // uint8 codes enter as q - 128 (a dead step still meets zero weights)
#pragma unroll
      for (int c = 0; c < kDecCols; ++c) acc[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, wv[c][u], acc[c], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int c = 0; c < kDecCols; ++c) red[wid][c][lane] = acc[c];
  __syncthreads();

  // thread t < 256 kDecCols finishes item (t / 64) % 4 of lane t % 64 of block
  // t / 256: row 4 * (l / 16) + item, column 16 * block + l % 16
  for (int t = threadIdx.x; t < 256 * kDecCols; t += kDecWaves * 64) {
    const int cb = t >> 8, l = t & 63, item = (t >> 6) & 3;
    const int m = 4 * (l >> 4) + item;
    const int64_t n = n0 + 16 * cb + (l & 15);
    if (m < p.M && n < p.N) {
      int c = 0;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) c += red[w][cb][l][item];
      const float sa = p.a_per_tensor ? p.sa[0] : p.sa[m];
      const int z = ASYM ? (p.a_per_tensor ? p.za[0] : p.za[m]) : 0;
      if (ASYM) c = (int)((uint32_t)c - (uint32_t)(z - 128) * (uint32_t)p.colsum[n]);
      const float sw = p.w_per_tensor ? p.sw[0] : p.sw[n];
      float yv = (float)c * (sa * sw);
      if (p.bias) yv = yv + p.bias[n];  // the bias after the scales, in float32
      store_one<OUT>(p.out, m * p.ldo + n, c, yv);
    }
  }
}

template <bool ASYM, int OUT, bool MLE8>
static void launch_decode_rows(const GemmArgs& a, hipStream_t st) {
  const int64_t groups = (a.N + 16 * kDecCols - 1) / (16 * kDecCols);
  if (a.K_pad <= 64 * kDecBatch * kDecWaves)
    hipLaunchKernelGGL((gemm_i8_decode_kernel<ASYM, OUT, true, MLE8>), dim3((unsigned)groups), dim3(kDecWaves * 64),
                       0, st, a);
  else
    hipLaunchKernelGGL((gemm_i8_decode_kernel<ASYM, OUT, false, MLE8>), dim3((unsigned)groups),
                       dim3(kDecWaves * 64), 0, st, a);
}

template <bool ASYM, int OUT>
static hipError_t launch_decode(const GemmArgs& a, hipStream_t st) {
  if (a.M <= 8)
    launch_decode_rows<ASYM, OUT, true>(a, st);
  else
    launch_decode_rows<ASYM, OUT, false>(a, st);
  return hipGetLastError();
}

template <bool ASYM, int OUT>
static hipError_t launch_i8(const GemmArgs& a, hipStream_t st) {
  if (a.M <= 16) return launch_decode<ASYM, OUT>(a, st);
  // The largest tile whose count still fills every CU once: bigger tiles
  // reuse each loaded byte more, but a round of tiles that leaves CUs idle
  // costs a whole tile time. 256 x 256 tiles (one 160 KB workgroup per CU)
  // when they come in whole rounds; when they would end in a partial round,
  // 128 x 256 tiles with a 72 KB ring, two workgroups per CU, whose finer
  // grain fills the last round and whose barriers overlap each other's
  // matrix-core work.
  const int64_t cus = cu_count();
  if (const int fn = wide_tile_fn(a.M, a.N, cus)) return launch_gemm_i8_wide<ASYM, OUT>(a, fn, st);
  auto tiles = [&](int64_t bm, int64_t bn) { return ((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn); };
  if (tiles(256, 256) >= cus) {
    if (tiles(256, 256) % cus == 0) return launch_dma<256, 256, 64, 2, 4, 5, ASYM, OUT>(a, st);
    return launch_dma<128, 256, 64, 2, 4, 3, ASYM, OUT>(a, st);
  }
  if (tiles(128, 128) >= cus) return launch_dma<128, 128, 128, 2, 4, 4, ASYM, OUT>(a, st);
  return launch_dma<64, 128, 128, 2, 4, 6, ASYM, OUT>(a, st);
}

template <int BM, int BN, int BK, int WM, int WN, int MODE, bool FA4, bool FW4>
static hipError_t launch_mx_cfg(const GemmArgs& a, hipStream_t st) {
  using C = MxCfg<BM, BN, BK, WM, WN, MODE, FA4, FW4>;
  auto kern = gemm_mx_kernel<BM, BN, BK, WM, WN, MODE, FA4, FW4>;
  const size_t lds = C::LDS;
  if (lds > 65536) {  // above the default dynamic-LDS limit (gfx950 has 160 KiB)
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(C::NT), lds, st, a);
  return hipGetLastError();
}

template <int MODE, bool FA4 = false, bool FW4 = false>
static hipError_t launch_mx(const GemmArgs& a, hipStream_t st) {
  // Large problems: 256x256 tiles (8 waves of 128x64); otherwise 128x128 (4
  // waves of 64x64). The bf16 staging of the exact mode doubles the LDS row,
  // so it steps 64 deep; the scaled-fp8 mode steps 128 deep on small tiles
  // and 64 deep on large ones (its scales need registers too).
  constexpr int BK = MODE == MXB ? 64 : 128;
  const int64_t big_tiles = ((a.M + 255) / 256) * ((a.N + 255) / 256);
  if (big_tiles >= 256) return launch_mx_cfg<256, 256, 64, 2, 4, MODE, FA4, FW4>(a, st);
  return launch_mx_cfg<128, 128, BK, 2, 2, MODE, FA4, FW4>(a, st);
}

hipError_t launch_gemm_i8(const GemmArgs& a, bool asym, int out_type, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  if (asym) {
    if (out_type == 0) return launch_i8<true, 0>(a, st);
    if (out_type == 1) return launch_i8<true, 1>(a, st);
    return launch_i8<true, 2>(a, st);
  }
  if (out_type == 0) return launch_i8<false, 0>(a, st);
  if (out_type == 1) return launch_i8<false, 1>(a, st);
  return launch_i8<false, 2>(a, st);
}


hipError_t launch_gemm_mx(const GemmArgs& a, int mode, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  if (mx_dma_eligible(a, mode)) return launch_gemm_mx_dma(a, mode, st);
  if (mode == 1) {  // any pair of e4m3 / e2m1 operands, each with its own format code
    if (a.a_fp4 && a.w_fp4) return launch_mx<MXF, true, true>(a, st);
    if (a.a_fp4) return launch_mx<MXF, true, false>(a, st);
    if (a.w_fp4) return launch_mx<MXF, false, true>(a, st);
    return launch_mx<MXF>(a, st);
  }
  if (a.a_fp4 && a.w_fp4) return launch_mx<MXB, true, true>(a, st);
  if (a.a_fp4) return launch_mx<MXB, true, false>(a, st);
  if (a.w_fp4) return launch_mx<MXB, false, true>(a, st);
  return launch_mx<MXB>(a, st);
}

}  // namespace qg
