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
// signed matrix cores as q - 128, and (128 - z) * colsum restores C.
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
//  * The MFMAs take the W fragment as their first operand, so a lane's four
//    accumulators of a block are four consecutive columns of one output row.
//    For asymmetric A they start at (128 - z) colsum, so they end at C; the
//    epilogue finishes them in registers with the row and column scales and
//    the bias that the prologue put in LDS and stores each lane's four
//    outputs with one instruction.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace qg {

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

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
  // the epilogue's parameters, written once in the prologue past the ring:
  // row scales (BM), column scales and bias (BN each)
  static constexpr int PAR = BM * 4 + BN * 8;
  static constexpr int NS_FIT = (LDS_MAX - (SPARE ? 1024 : 0) - PAR) / STAGE;
  static constexpr int NS = NS_FIT > 5 ? 5 : NS_FIT;
  static constexpr int RING = NS * STAGE;
  static constexpr int SPARE_OFF = RING;         // the spare 1 KB for empty loads
  static constexpr int PAR_ROWS = RING + (SPARE ? 1024 : 0);
  static constexpr int PAR_COLS = PAR_ROWS + BM * 4;
  static constexpr int LDS = PAR_ROWS + PAR;
  static_assert(FN >= 5 && NS >= 3, "ring");
  static_assert(BM <= NT && BN <= NT, "one parameter per thread");
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

  // fragment reads: A block i of this wave (16 rows, lane l: row l % 16, K
  // chunk l / 16 of the stage), W block j (the packed 1 KB in lane order)
  auto read_a = [&](int s, int i) {
    const int r = wm * 64 + i * 16 + (lane & 15);
    return *reinterpret_cast<const v4i*>(smem + s * STAGE + r * 64 + (((lane >> 4) ^ a_swz(r)) << 4));
  };
  auto read_w = [&](int s, int j) {
    return *reinterpret_cast<const v4i*>(smem + s * STAGE + C::A_BYTES + ((wn * FN + j) << 10) + lane * 16);
  };

  // The epilogue's parameters go to LDS in the prologue, loaded before the
  // stage loads (so the first stage's wait covers them): thread t < BM loads
  // row t's scale, thread t < BN column t's scale and bias. Rows past M are
  // clamped to M - 1 and columns past N get zeros; neither is stored. A
  // missing bias is never read.
  float par_f = 0.0f, par_sw = 0.0f, par_b = 0.0f;
  if (tid < BM) par_f = p.a_per_tensor ? p.sa[0] : p.sa[min(m0 + tid, p.M - 1)];
  if (tid < BN && n0 + tid < p.N) {
    par_sw = p.w_per_tensor ? p.sw[0] : p.sw[n0 + tid];
    if (p.bias) par_b = p.bias[n0 + tid];
  }
  float* const rsa = reinterpret_cast<float*>(smem + C::PAR_ROWS);
  float* const csw = reinterpret_cast<float*>(smem + C::PAR_COLS);
  float* const cbs = reinterpret_cast<float*>(smem + C::PAR_COLS + BN * 4);
  // Accumulator block (i, j) holds, in lane l, row 16 i + l % 16 of the wave's
  // rows and columns 16 j + 4 (l / 16) .. + 3 of its columns (the MFMAs take
  // the W fragment as their first operand, so they compute W times A^T).
  const int64_t nw0 = n0 + wn * TN;               // the wave's first column (uniform)
  const int lc0 = wn * TN + 4 * (lane >> 4);      // the lane's first column in the tile
  // Asymmetric A: the accumulators start at (128 - z) colsum and so end at C
  // itself. Each partial sum is then the sum over the K columns done of
  // (q - z) w plus (128 - z) times the sum of the remaining w, every term at
  // most 255 * 127 in magnitude, so the K limit keeps all of them in int32.
  int zrow[FM];
  v4i cs_j[FN];
  if constexpr (ASYM) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t m = min(m0 + wm * 64 + 16 * i + (lane & 15), p.M - 1);
      zrow[i] = p.a_per_tensor ? p.za[0] : p.za[m];
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t n = nw0 + 16 * j + 4 * (lane >> 4);  // colsum has N_pad >= n + 4 entries
      cs_j[j] = n < p.N ? *reinterpret_cast<const v4i*>(p.colsum + n) : v4i{0, 0, 0, 0};
    }
  }

  // prologue: stages 0 .. NS-2 in flight, then stage 0's first fragments
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
#pragma unroll
    for (int i = 0; i < IPW; ++i) dma(s, s, i, s < nkt);
  if constexpr (ASYM) {
    // 128 - z in [-127, 128]; |colsum| <= 127 K_pad, below 2^23 up to K_pad = 65536:
    // one exact 24-bit multiply per accumulator, else a 32-bit one
    int nz[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) nz[i] = ((128 - zrow[i]) << 20) >> 20;
    if (p.K_pad <= 65536) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int cs = (cs_j[j][t] << 8) >> 8;
#pragma unroll
          for (int i = 0; i < FM; ++i) acc[i][j][t] = nz[i] * cs;
        }
    } else {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < FM; ++i) acc[i][j][t] = nz[i] * cs_j[j][t];
    }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = v4i{0, 0, 0, 0};
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * IPW));
  // (visible to every wave after the first stage barrier, which waits for LDS)
  if (tid < BM) rsa[tid] = par_f;
  if (tid < BN) {
    csw[tid] = par_sw;
    cbs[tid] = par_b;
  }
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
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf[j % NB], af[PB][i], acc[i][j], 0, 0, 0);
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
  // The ring becomes the epilogue's staging area once every wave is past its
  // last fragment read and its loads (the empty ones past the last stage
  // included) have landed.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __builtin_amdgcn_s_barrier();

  // ---- epilogue. Each lane finishes, in registers, the four consecutive
  // outputs of one row that an accumulator block holds (the parameters were
  // written to LDS in the prologue). A 16-row block of the wave's outputs is
  // then staged in the wave's own LDS slab, row-major, and leaves as 16-byte
  // chunks, each row's TN columns contiguous, so every output line is written
  // whole by one wave (16-byte row pieces from the lanes alone would leave
  // half-written lines to be merged, or not, in L2). A wave's LDS operations
  // complete in order, so the slab needs no barrier between its uses.
  using OutT = std::conditional_t<OUT == 2, int32_t, std::conditional_t<OUT == 0, float, uint16_t>>;
  constexpr int OB = sizeof(OutT);
  constexpr int SROW = TN * OB + 16;        // slab row pitch: 4 banks of skew per row
  constexpr int CPR = TN * OB / 16;         // 16-byte chunks per slab row
  constexpr int EPR = 16 / OB;              // outputs per chunk
  constexpr int PASSES = (16 * CPR + 63) / 64;
  static_assert(C::NW * 16 * SROW <= C::RING, "slabs fit in the ring");
  static_assert((TN * OB) % 16 == 0, "whole chunks");
  uint8_t* const slab = smem + wid * 16 * SROW;
  float sam[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) sam[i] = rsa[wm * 64 + 16 * i + (lane & 15)];
  const int64_t mw0 = m0 + wm * 64;  // the wave's first row (uniform)
  // rows start 16-byte aligned (out is; the tile and wave column offsets are
  // multiples of 16 bytes) unless a bf16 ldo is 4 mod 8
  const bool a16 = OB == 4 || p.ldo % 8 == 0;

  // EDGE: the wave's outputs reach past M or N (checks per chunk and lane)
  auto finish = [&](auto has_bias, auto edge) {
    constexpr bool BIAS = decltype(has_bias)::value, EDGE = decltype(edge)::value;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      // block column j's parameters; those of j + 1 are read while j is finished
      v4f sw4 = *reinterpret_cast<const v4f*>(csw + lc0), bs4{}, sw_n{}, bs_n{};
      if (BIAS) bs4 = *reinterpret_cast<const v4f*>(cbs + lc0);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if (j + 1 < FN) {
          sw_n = *reinterpret_cast<const v4f*>(csw + lc0 + 16 * (j + 1));
          if (BIAS) bs_n = *reinterpret_cast<const v4f*>(cbs + lc0 + 16 * (j + 1));
        }
        const v4i ci = acc[i][j];
        v4f y;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          y[t] = (float)ci[t] * (sam[i] * sw4[t]);
          if (BIAS) y[t] = y[t] + bs4[t];  // the bias after the scales, in float32
        }
        uint8_t* const dst = slab + (lane & 15) * SROW + (16 * j + 4 * (lane >> 4)) * OB;
        if constexpr (OUT == 2) {
          *reinterpret_cast<v4i*>(dst) = ci;
        } else if constexpr (OUT == 0) {
          *reinterpret_cast<v4f*>(dst) = y;
        } else {
          // round to nearest even (v_cvt_pk_bf16_f32; the outputs are never denormal)
          const uint32_t w0 = __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{y[0], y[1]}, v2bf));
          const uint32_t w1 = __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{y[2], y[3]}, v2bf));
          *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
        }
        sw4 = sw_n;
        bs4 = bs_n;
      }
      // the block's 16 rows x TN columns, 16 bytes per lane and pass
#pragma unroll
      for (int pass = 0; pass < PASSES; ++pass) {
        const int q = pass * 64 + lane;
        if (16 * CPR % 64 != 0 && q >= 16 * CPR) break;
        const int r = q / CPR, c = q % CPR;
        const v4i v = *reinterpret_cast<const v4i*>(slab + r * SROW + 16 * c);
        const int64_t m = mw0 + 16 * i + r, n = nw0 + c * EPR;
        OutT* const o = reinterpret_cast<OutT*>(p.out) + m * p.ldo + n;
        if (!EDGE || (m < p.M && n + EPR <= p.N)) {
          if (a16) {
            *reinterpret_cast<v4i*>(o) = v;
          } else {  // bf16 rows that start 8 bytes into a 16-byte unit
            reinterpret_cast<uint2*>(o)[0] = make_uint2((uint32_t)v[0], (uint32_t)v[1]);
            reinterpret_cast<uint2*>(o)[1] = make_uint2((uint32_t)v[2], (uint32_t)v[3]);
          }
        } else if (m < p.M) {
          const OutT* e = reinterpret_cast<const OutT*>(&v);
          for (int t = 0; t < EPR && n + t < p.N; ++t) o[t] = e[t];
        }
      }
    }
  };
  const bool interior = mw0 + 64 <= p.M && nw0 + TN <= p.N;  // uniform
  if (p.bias) {
    if (interior)
      finish(std::true_type{}, std::false_type{});
    else
      finish(std::true_type{}, std::true_type{});
  } else {
    if (interior)
      finish(std::false_type{}, std::false_type{});
    else
      finish(std::false_type{}, std::true_type{});
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
