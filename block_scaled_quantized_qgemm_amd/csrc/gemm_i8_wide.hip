// Large-M int8 x int8 GEMM for gfx950: one 256 x BN output tile per
// workgroup, BN chosen per shape so that the tiles come in whole rounds over
// the compute units (for 2048 x 11008: 8 row bands x 32 column strips of 352
// = 256 tiles, one per CU), which moves the fewest operand bytes per
// multiply-add that one workgroup per CU can hold.
//
// Semantics are those of gemm_i8_dma_kernel ("Activation Quantization
// Architecture, in depth", section "The integer GEMM, written out"; "100 Days
// of GPU -- Day 98", section "The program, and the gate that has to be per
// column"): C = sum_k (q_a - z_a) q_w exactly in int32, then
// out = float(C) * (s_a * s_w) (+ bias) once per output; uint8 codes enter the
// signed matrix cores as q - 128 and the epilogue subtracts (z - 128) * colsum.
//
// Structure:
//  * 8 waves as 4 (rows) x 2 (columns); wave tiles of 64 x 16 FN, computed as
//    4 x FN blocks of v_mfma_i32_16x16x64_i8 (a 16-row block of A and a
//    16-row block of W, 64 K deep, per instruction).
//  * 64-deep K stages travel global -> LDS by buffer_load ... lds into an
//    NS-stage ring (NS - 1 stages in flight): A as swizzled row-major 64-byte
//    rows, W as the packed 1 KB blocks (16 rows x 64 K, already in operand lane
//    order), each copied by one wave instruction. A wave issues the same number
//    of loads every stage (spare ones read nothing into a spare 1 KB), so one
//    vmcnt count serves every stage.
//  * W fragments are read three block columns ahead of their MFMAs. One
//    barrier per stage, placed after the stage's last W fragment read: the
//    next stage's A fragments and first three W fragments are read after it
//    while the stage's last four block columns of MFMAs run, so the barrier
//    and the fragment latency are covered by matrix-core work.
//  * Epilogue through LDS: per wave and 16-row block, the int32 block is staged,
//    then each lane finishes four consecutive columns of a row with the tile's
//    row scales / zero points and column scales / sums / bias staged in LDS.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace qg {

// A stage rows are 64 bytes (four 16-byte K chunks); chunk c of row r sits at
// 64 r + 16 (c ^ a_swz(r)). A fragment read has lanes 0-15 on rows r0 .. r0+15
// at one chunk; with this XOR (row bits 1-2) gfx950 serves those reads at the
// full 256 bytes per clock (measured; XOR-ing with row bits 2-3 instead halves
// the rate). The DMA's four lanes of a row still fetch its 64 contiguous bytes.
__device__ inline int a_swz(int r) { return (r >> 1) & 3; }

template <int FN>
struct WideCfg {
  static constexpr int BM = 256, BK = 64, WM = 4, WN = 2, NW = WM * WN, NT = NW * 64;
  static constexpr int FM = 4;                   // 16-row blocks of a wave's 64 rows
  static constexpr int TN = 16 * FN, BN = WN * TN;
  static constexpr int A_BYTES = BM * BK;        // 16 KB of A per stage
  static constexpr int STAGE = A_BYTES + BN * BK;
  static constexpr int LOADS = STAGE / 1024;     // 1 KB wave loads per stage: A first, then W blocks
  static constexpr int IA = A_BYTES / 1024;
  static constexpr int IPW = (LOADS + NW - 1) / NW;
  static constexpr bool SPARE = LOADS % NW != 0;  // some waves issue an empty load per stage
  static constexpr int LDS_MAX = 160 * 1024;
  static constexpr int NS_FIT = (LDS_MAX - (SPARE ? 1024 : 0)) / STAGE;
  static constexpr int NS = NS_FIT > 5 ? 5 : NS_FIT;
  static constexpr int RING = NS * STAGE;
  static constexpr int SPARE_OFF = RING;         // the spare 1 KB for empty loads
  // epilogue: per wave a 16-row int32 slab, rows RS words apart (RS % 16 == 4:
  // the four row groups a 16x16 block writes at once fall on distinct banks)
  static constexpr int RS = TN + 4;
  static constexpr int EPI_W = 16 * RS * 4;
  static constexpr int EPI_ROWS = NW * EPI_W;    // row params after the slabs
  static constexpr int EPI_COLS = EPI_ROWS + BM * 8;
  static constexpr int EPI_END = EPI_COLS + BN * 12;
  static constexpr int LDS = (RING + (SPARE ? 1024 : 0)) > EPI_END ? (RING + (SPARE ? 1024 : 0)) : EPI_END;
  static_assert(FN >= 5 && NS >= 3, "ring");
  static_assert(LDS <= LDS_MAX, "LDS");
  static_assert((NS - 2) * IPW < 64, "vmcnt range");
  static constexpr int PD = 3;                   // W fragments are read PD block columns ahead
  static_assert(IPW <= FN - 1 - PD, "loads are issued before the stage's barrier");
};

template <int FN, bool ASYM, int OUT>
__global__ __launch_bounds__(512) void gemm_i8_wide_kernel(GemmArgs p) {
  using C = WideCfg<FN>;
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, TN = C::TN, FM = C::FM, NS = C::NS;
  constexpr int STAGE = C::STAGE, IPW = C::IPW, IA = C::IA, LOADS = C::LOADS;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid / C::WN, wn = wid % C::WN;

  // Tile order (as in gemm_i8_dma_kernel): each XCD gets a contiguous run of
  // tile ids, walked in groups of 8 row bands so that the tiles running at
  // once on an XCD share A rows and W columns in its L2.
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

  // ---- stage loads. Load j of a stage (j = wid + NW * i) carries A rows
  // 16 j .. 16 j + 15 when j < IA (lane l: row 16 j + l / 4, the chunk that
  // belongs at LDS slot l of the swizzled rows), W block j - IA otherwise (1 KB
  // contiguous, copied as it is), nothing when j >= LOADS (an empty range into
  // the spare KB). A rows >= M are clamped to row M - 1 (never stored); the A
  // range ends at the 16-byte chunk holding column K - 1 of the last row and W
  // rows end at N_pad, so nothing past either is read (zeros come back). The
  // stage's K offset goes in the scalar offset.
  const uint8_t* const abase = p.a + m0 * p.lda;
  const uint8_t* const wbase = p.w + n0 * p.K_pad;
  const int64_t last_a_row = min((int64_t)BM - 1, p.M - 1 - m0);
  const uint32_t nrec_a = (uint32_t)(last_a_row * p.lda + ((p.K + 15) & ~(int64_t)15));
  const int64_t n_pad = (p.N + 255) / 256 * 256;
  const uint32_t nrec_w = (uint32_t)(max((int64_t)0, min((int64_t)BN, n_pad - n0)) * p.K_pad);
  uint32_t voff[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int j = wid + C::NW * i;
    if (j < IA) {
      const int r = 16 * j + lane / 4;
      const int c = (lane & 3) ^ a_swz(r);
      voff[i] = (uint32_t)(min((int64_t)r, last_a_row) * p.lda) + (uint32_t)(c * 16);
    } else {
      const int b = j - IA;  // W row block of the tile (16 rows)
      voff[i] = (uint32_t)((int64_t)b * (p.K_pad >> 6) << 10) + (uint32_t)(lane * 16);
    }
  }
  auto dma = [&](int kt, int s, int i, bool live) {
    const int j = wid + C::NW * i;
    const bool ja = j < IA;
    const bool real = j < LOADS;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(ja ? abase : wbase), (short)0, (live && real) ? (int)(ja ? nrec_a : nrec_w) : 0, kRawBufferWord3);
    uint8_t* dst = real ? smem + s * STAGE + j * 1024 : smem + C::SPARE_OFF;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, QG_LDSP(dst), 16, (int)voff[i], kt * (ja ? BK : BK * 16), 0, 0);
  };

  v4i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  // fragment reads: A block i of this wave (16 rows, lane l: row l % 16, K
  // chunk l / 16 of the stage), W block j (the packed 1 KB in lane order)
  auto read_a = [&](int s, int i) {
    const int r = wm * 64 + i * 16 + (lane & 15);
    return *reinterpret_cast<const v4i*>(smem + s * STAGE + r * 64 + (((lane >> 4) ^ a_swz(r)) << 4));
  };
  auto read_w = [&](int s, int j) {
    return *reinterpret_cast<const v4i*>(smem + s * STAGE + C::A_BYTES + ((wn * FN + j) << 10) + lane * 16);
  };

  // prologue: stages 0 .. NS-2 in flight, then stage 0's first fragments
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
#pragma unroll
    for (int i = 0; i < IPW; ++i) dma(s, s, i, s < nkt);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * IPW));
  __builtin_amdgcn_s_barrier();
  constexpr int PD = C::PD, NB = PD + 1;
  v4i af[2][FM], wf[NB], nw[PD];
#pragma unroll
  for (int i = 0; i < FM; ++i) af[0][i] = read_a(0, i);
#pragma unroll
  for (int q = 0; q < PD; ++q) wf[q] = read_w(0, q);

  // one stage: MFMA block column j uses W fragment j (slot j % NB), read PD
  // columns ahead; the loads of stage kt + NS - 1 go out with the first IPW
  // columns; after the column that reads the stage's last W fragment, the
  // wait for stage kt + 1 and the barrier, then its A fragments (set PB ^ 1)
  // and first PD W fragments are read under the stage's last PD + 1 columns
  // of MFMAs.
  auto stage = [&](int kt, auto pbc) {
    constexpr int PB = decltype(pbc)::value;
    const int cur = kt % NS, nxt = (kt + 1) % NS, ks = kt + NS - 1, sl = ks % NS;
    const bool live = ks < nkt;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      if (j + PD < FN) wf[(j + PD) % NB] = read_w(cur, j + PD);
      if (j == FN - 1 - PD) {
        // this wave's reads of stage kt are issued (lgkmcnt 0: landed) and its
        // loads of stage kt + 1 have arrived; after the barrier everyone's have
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * IPW) & ~(15 << 8));
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int i = 0; i < FM; ++i) af[PB ^ 1][i] = read_a(nxt, i);
      }
      if (j >= FN - PD) nw[j - (FN - PD)] = read_w(nxt, j - (FN - PD));
      if (ASYM && j == 0) {  // uint8 codes enter the signed matrix cores as q - 128
#pragma unroll
        for (int i = 0; i < FM; ++i) af[PB][i] ^= (int)0x80808080u;
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[PB][i], wf[j % NB], acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (j < IPW) dma(ks, sl, j, live);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < PD; ++q) wf[q] = nw[q];
  };

  // nkt is even (K_pad is a multiple of 256): two stages per trip keep the A
  // fragment sets in fixed registers
  for (int kt = 0; kt < nkt; kt += 2) {
    stage(kt, std::integral_constant<int, 0>{});
    stage(kt + 1, std::integral_constant<int, 1>{});
  }
  // the empty loads past the last stage may still be in flight
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();

  // ---- epilogue. The tile's row scales / zero points and column scales /
  // column sums / bias go to LDS once; then each wave stages one 16-row block
  // of its int32 sums at a time in its own slab and finishes it in passes of
  // 64 four-column groups: one 16-byte read of the sums and 16-byte reads of
  // the four columns' parameters per lane, all issued before the arithmetic.
  float* rsa = reinterpret_cast<float*>(smem + C::EPI_ROWS);
  int* rza = reinterpret_cast<int*>(smem + C::EPI_ROWS + BM * 4);
  float* csw = reinterpret_cast<float*>(smem + C::EPI_COLS);
  int* ccs = reinterpret_cast<int*>(smem + C::EPI_COLS + BN * 4);
  float* cbs = reinterpret_cast<float*>(smem + C::EPI_COLS + BN * 8);
  for (int r = tid; r < BM; r += C::NT) {
    const int64_t m = min(m0 + r, p.M - 1);
    rsa[r] = p.a_per_tensor ? p.sa[0] : p.sa[m];
    rza[r] = ASYM ? (p.a_per_tensor ? p.za[0] : p.za[m]) : 0;
  }
  for (int c = tid; c < BN; c += C::NT) {
    const int64_t n = n0 + c;
    const bool in = n < p.N;
    csw[c] = in ? (p.w_per_tensor ? p.sw[0] : p.sw[n]) : 0.0f;
    ccs[c] = (ASYM && in) ? p.colsum[n] : 0;
    cbs[c] = (p.bias && in) ? p.bias[n] : 0.0f;  // a missing bias adds +0, which changes no result
  }
  // The parameters are read by every wave: one barrier, waiting for LDS only
  // (a __syncthreads would also wait for this wave's earlier global stores).
  // After it each wave works in its own slab: a wave's LDS operations complete
  // in order, so its staging writes and reads need no further barrier, and the
  // output stores of a block drain while the next block is staged.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(63) & ~(15 << 8));
  __builtin_amdgcn_s_barrier();
  int* slab = reinterpret_cast<int*>(smem + wid * C::EPI_W);
  constexpr int GPR = TN / 4;  // four-column groups per slab row
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    // block (i, j): lane l, item t is row 4 (l / 16) + t, column 16 j + l % 16
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) slab[(4 * (lane >> 4) + t) * C::RS + 16 * j + (lane & 15)] = acc[i][j][t];
#pragma unroll
    for (int pass = 0; pass < FN; ++pass) {
      const int gq = pass * 64 + lane;
      const int r = gq / GPR, cg = gq % GPR;
      const int lr = wm * 64 + i * 16 + r;   // row inside the tile
      const int lc = wn * TN + 4 * cg;       // column inside the tile
      const v4i raw = *reinterpret_cast<const v4i*>(slab + r * C::RS + 4 * cg);
      const v4f sw4 = *reinterpret_cast<const v4f*>(csw + lc);
      const v4f bs4 = *reinterpret_cast<const v4f*>(cbs + lc);
      const float sam = rsa[lr];
      v4i cs4 = v4i{0, 0, 0, 0};
      int nz = 0;
      if (ASYM) {
        cs4 = *reinterpret_cast<const v4i*>(ccs + lc);
        nz = 128 - rza[lr];  // C = raw + (128 - z) * colsum
      }
      float y[4];
      int ci[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        int c = raw[t];
        if (ASYM) {
          // exact (128 - z) * colsum with 24-bit multiplies: |128 - z| <= 128 and
          // colsum = 4096 hi + lo with lo in [0, 4095] and |hi| < 2^12
          const int lo = cs4[t] & 4095, hi = cs4[t] >> 12;
          c = (int)((uint32_t)c + (uint32_t)__mul24(nz, lo));   // wrap-around int32: the true C fits
          c = (int)((uint32_t)c + ((uint32_t)__mul24(nz, hi) << 12));
        }
        ci[t] = c;
        y[t] = (float)c * (sam * sw4[t]) + bs4[t];  // the bias after the scales, in float32
      }
      const int64_t m = m0 + lr, n = n0 + lc;
      if (m < p.M && n < p.N) {
        const bool full = n + 3 < p.N;
        if constexpr (OUT == 2) {
          int32_t* o = reinterpret_cast<int32_t*>(p.out) + m * p.ldo + n;
          if (full)
            *reinterpret_cast<v4i*>(o) = v4i{ci[0], ci[1], ci[2], ci[3]};
          else
            for (int t = 0; t < 4 && n + t < p.N; ++t) o[t] = ci[t];
        } else if constexpr (OUT == 0) {
          float* o = reinterpret_cast<float*>(p.out) + m * p.ldo + n;
          if (full)
            *reinterpret_cast<v4f*>(o) = v4f{y[0], y[1], y[2], y[3]};
          else
            for (int t = 0; t < 4 && n + t < p.N; ++t) o[t] = y[t];
        } else {
          uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + m * p.ldo + n;
          // round to nearest even (v_cvt_pk_bf16_f32; the outputs are never denormal)
          const __bf16 h0 = (__bf16)y[0], h1 = (__bf16)y[1], h2 = (__bf16)y[2], h3 = (__bf16)y[3];
          const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
          const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, h2) | ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16);
          if (full) {
            *reinterpret_cast<uint2*>(o) = make_uint2(w0, w1);
          } else {
            const uint16_t hv[4] = {(uint16_t)w0, (uint16_t)(w0 >> 16), (uint16_t)w1, (uint16_t)(w1 >> 16)};
            for (int t = 0; t < 4 && n + t < p.N; ++t) o[t] = hv[t];
          }
        }
      }
    }
  }
}

template <int FN, bool ASYM, int OUT>
static hipError_t launch_wide_fn(const GemmArgs& a, hipStream_t st) {
  using C = WideCfg<FN>;
  const int64_t tiles = ((a.M + C::BM - 1) / C::BM) * ((a.N + C::BN - 1) / C::BN);
  hipLaunchKernelGGL((gemm_i8_wide_kernel<FN, ASYM, OUT>), dim3((unsigned)tiles), dim3(C::NT), 0, st, a);
  return hipGetLastError();
}

// Tile widths built: BN = 32 FN.
static constexpr int kWideFN[] = {8, 11};

int wide_tile_fn(int64_t M, int64_t N, int64_t cus) {
  // Row bands of 256 rows; among the built strip widths, those whose tiles
  // fill at least 90% of their rounds over the CUs, the one with the least
  // rounds x tile width (the time of the busiest CU). None for fewer than
  // four row bands or when no width fills its rounds: the tilings of
  // gemm.hip serve those shapes.
  const int64_t bands = (M + 255) / 256;
  if (bands < 4 || cus < 8) return 0;
  int best = 0;
  int64_t best_cost = 0;
  for (int fn : kWideFN) {
    const int64_t bn = 32 * fn;
    const int64_t tiles = bands * ((N + bn - 1) / bn);
    const int64_t rounds = (tiles + cus - 1) / cus;
    if (tiles * 10 < rounds * cus * 9) continue;
    const int64_t cost = rounds * bn;
    if (!best || cost < best_cost) {
      best = fn;
      best_cost = cost;
    }
  }
  return best;
}

template <bool ASYM, int OUT>
hipError_t launch_gemm_i8_wide(const GemmArgs& a, int fn, hipStream_t st) {
  if (fn == 11) return launch_wide_fn<11, ASYM, OUT>(a, st);
  return launch_wide_fn<8, ASYM, OUT>(a, st);
}

template hipError_t launch_gemm_i8_wide<false, 0>(const GemmArgs&, int, hipStream_t);
template hipError_t launch_gemm_i8_wide<false, 1>(const GemmArgs&, int, hipStream_t);
template hipError_t launch_gemm_i8_wide<false, 2>(const GemmArgs&, int, hipStream_t);
template hipError_t launch_gemm_i8_wide<true, 0>(const GemmArgs&, int, hipStream_t);
template hipError_t launch_gemm_i8_wide<true, 1>(const GemmArgs&, int, hipStream_t);
template hipError_t launch_gemm_i8_wide<true, 2>(const GemmArgs&, int, hipStream_t);

}  // namespace qg
