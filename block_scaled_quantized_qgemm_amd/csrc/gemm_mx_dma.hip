// MX GEMM (e4m3 or e2m1 activations and weights, one E8M0 scale per 32 K of
// each row of A and W, float32 output) on an LDS-DMA ring, for gfx950.
//
// The block-scaled product ("TileLang tutorial, chapter 27", sections 4.1 and
// 4.3): out[m][n] = sum over 32-blocks b of 2^(Ea[m][b]-127) 2^(Ew[n][b]-127)
// times the block's sum of e4m3 products; a scale that changes along K is
// applied per block inside the K loop, never after the sum.
//
// e4m3 codes are bytes, so the tiles travel like the int8 GEMM's: global
// memory -> LDS directly (buffer_load ... lds), each lane fetching the
// 16-byte chunk that belongs at its slot of the XOR-swizzled row-major tile,
// NS stages in a ring so NS - 1 are in flight without holding registers. The
// E8M0 bytes travel with the stages too: every SS-th stage also brings 16
// scale bytes of each tile row (its own stage and the next SS - 1) into one of
// two scale slots, a 16-byte lane per row, so one 1 KB load covers 64 rows
// (a dword per row and stage would touch 64 cache lines per 256 bytes and
// double the stage's line requests); the scale layout in global memory stays
// the public row-major [rows][K/32].
//
// Per 64-deep stage a wave reads, per 32-row fragment, the two 16-byte chunks
// the 32x32x64 operand wants (lane 32h + r: K 16h .. 16h+15 and 32 + 16h ..
// 32 + 16h + 15 of row r) and the E8M0 byte of (row r, block h), and issues
// v_mfma_scale_f32_32x32x64_f8f6f4 (the block-scaled fp8 matrix cores; the
// hardware aligns the products of each group of 8 consecutive K to the
// largest and drops bits more than 13 binades below it, so the sums are not
// float32-exact). Each stage starts with the wait and barrier for the next
// stage; that stage's fragment reads and the refill of the slot just consumed
// are then spread between all of the stage's MFMAs, which use fragments read
// during the previous stage.
//
// EXACT (the exact mode): the same ring and fragment reads, then each lane
// turns its 32 e4m3 codes per fragment into bf16 times the block's scale
// (v_cvt_scalef32_pk_bf16_fp8; exact, since e4m3 times a power of two in the
// quantizer's range is a bf16) and feeds v_mfma_f32_32x32x16_bf16: exact
// products, float32 sums. The 64-deep step becomes four 16-deep ones: chunk t
// of a lane's fragment (its codes 8t .. 8t + 7) is the MFMA's 8 K values for
// that lane, the same K positions for A and W, so the four MFMAs together form
// every product of the step once.
//
// A4 / W4 (e2m1 activations / weights): two codes per byte, so that
// operand's stage rows hold KPS / 2 bytes. Scaled mode: its lane operand for
// a 64-deep step is the 16 bytes holding K 32h .. 32h + 31 of its row (the
// upper half of the operand unused), and the instruction gets each operand's
// own format code, so e4m3 x e2m1 pairs run as well. e2m1 x e2m1 products
// span under 8 binades, so the hardware's 8-product alignment drops nothing
// and the sums are float32 sums; a pair with an e4m3 operand has the e4m3
// bound. Exact mode: a lane reads the e2m1 codes of the same K positions as
// an e4m3 fragment (K 16h .. 16h + 15 and 32 + 16h .., two 8-byte halves of
// the step's two chunks), so chunk t is again the K of the t-th 16-deep
// MFMA for any pair, and converts them with v_cvt_scalef32_pk_bf16_fp4.
//
// GROUPED (the grouped MoE GEMM, same section 6.2 of the tutorial): the rows
// routed to each expert are stored one expert after the other; the experts'
// tile-rows are listed in expert order, each workgroup finds its expert from
// the device-resident row offsets, and the tile's rows, weights, scales and
// bias are that expert's. The rest of the kernel is unchanged.
//
// Taken when every stage lies inside K (K % 64 == 0; e2m1 x e2m1 in the
// scaled mode: K % 128 == 0) and the activation scale rows are
// dword-aligned; the register-staged kernel in gemm.hip covers the rest.
#include "common.hpp"
#include "kernels.hpp"

namespace qg {

typedef __bf16 v8bf_t __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));

// Eight e4m3 codes (dwords d0, d1; code i in byte i % 4 of dword i / 4) times
// `scale` as eight bf16, in order.
__device__ inline v8bf_t fp8x8_to_bf16(int d0, int d1, float scale) {
  const v2bf_t t0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)d0, scale, false);
  const v2bf_t t1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)d0, scale, true);
  const v2bf_t t2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)d1, scale, false);
  const v2bf_t t3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)d1, scale, true);
  return v8bf_t{t0[0], t0[1], t1[0], t1[1], t2[0], t2[1], t3[0], t3[1]};
}

// Eight e2m1 codes (dword d; code i in nibble i % 2 of byte i / 2, low
// nibble first) times `scale` as eight bf16, in order.
__device__ inline v8bf_t fp4x8_to_bf16(int d, float scale) {
  const v2bf_t t0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((unsigned)d, scale, 0);
  const v2bf_t t1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((unsigned)d, scale, 1);
  const v2bf_t t2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((unsigned)d, scale, 2);
  const v2bf_t t3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((unsigned)d, scale, 3);
  return v8bf_t{t0[0], t0[1], t1[0], t1[1], t2[0], t2[1], t3[0], t3[1]};
}

template <int BM, int BN, int KPS, int WM, int WN, int NS, bool EXACT, bool A4, bool W4>
struct MxDmaCfg {
  static constexpr int NT = WM * WN * 64, NW = WM * WN;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int RBA = A4 ? KPS / 2 : KPS;     // code bytes per A row and stage (KPS K)
  static constexpr int RBW = W4 ? KPS / 2 : KPS;     // ... per W row
  static constexpr int NKK = KPS / 64;               // 64-deep matrix-core steps per stage
  static constexpr int DATA = BM * RBA + BN * RBW;   // code bytes per stage
  static constexpr int STAGE = DATA;
  static constexpr int SPS = KPS / 32;               // E8M0 bytes per row and stage
  static constexpr int SS = 16 / SPS;                // stages whose scales one 16-byte row load brings
  static constexpr int SUPER = (BM + BN) * 16;       // one scale slot: 16 bytes per tile row
  static constexpr int SCALES = NS * STAGE;          // two scale slots after the ring
  static constexpr int IA = BM * RBA / 1024;         // the first IA 1 KB data loads carry A
  static constexpr int IPD = DATA / 1024 / NW;       // 1 KB data loads per wave and stage
  static constexpr int NSL = (BM + BN) / 64;         // 1 KB scale loads per scale slot
  static constexpr int IPS = (NSL + NW - 1) / NW;    // ... per wave and stage (see the loads)
  static constexpr int IPW = IPD + IPS;
  static constexpr int MPS = (EXACT ? 4 : 1) * FM * FN;  // matrix-core instructions per 64-deep step
  // instructions the stage's loads are spread over: all of the only step
  // (KPS 64), or every step before the last (KPS 128)
  static constexpr int SLOTS = NKK == 1 ? MPS : (NKK - 1) * MPS;
  // stages the prologue puts in flight: with one step per stage the ring is
  // refilled after the stage's barrier, so all NS slots start full
  static constexpr int PRO = NKK == 1 ? NS : NS - 1;
  static constexpr int RS = TN + 8;                  // epilogue staging row stride (words)
  static constexpr int EPI = NW * 32 * RS * 4;
  static constexpr int SINK = SCALES + 2 * SUPER;   // 1 KB that the empty scale loads target
  static constexpr int LDS = SINK + 1024 > EPI ? SINK + 1024 : EPI;
  static_assert(KPS == 64 || KPS == 128, "stage depth");
  static_assert(W4 || RBW == 64, "e4m3 weight stages are one 64-K block column");
  static_assert(!(EXACT && KPS != 64), "exact-mode stages are 64 deep");
  static_assert(DATA % (1024 * NW) == 0 && (BM * RBA) % 1024 == 0 && (BM + BN) % 64 == 0 && BM % 64 == 0,
                "loads per wave");
  static_assert(FM >= 1 && FN >= 1, "fragments");
  static_assert(NS >= 2 && (PRO - 1) * IPW < 64, "vmcnt range");
  // a scale slot is refilled NS (KPS 64) or NS - 1 (KPS 128) stages before
  // its first stage, after every read of its previous contents
  static_assert(NS <= SS + 1, "scale slot reuse");
  static_assert(TN % 4 == 0 && (TN / 4) <= 64 && 64 % (TN / 4) == 0, "epilogue lane map");
};

// Grouped GEMM: the tile-rows of all experts, in expert order. Expert e owns
// rows [off[e], off[e+1]) of A (offsets clamped to [0, M]; a decreasing pair
// is empty) and ceil(rows / BM) tile-rows. Wave-cooperative, 64 experts per
// pass (an inclusive scan of the tile-row counts across the lanes); every
// lane returns the total count and, for tile-row tm, its expert, first row
// and the expert's row end (e = -1 when tm is not below the total).
struct GroupTile {
  int e;
  int64_t row0, row_end;
};
__device__ inline int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
template <int BM>
__device__ inline int group_tiles(const int64_t* off, int E, int64_t M, int tm, GroupTile& gt) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  gt.e = -1;
  gt.row0 = gt.row_end = 0;
  for (int c = 0; c < E; c += 64) {
    const int e = c + lane;
    int64_t lo = 0, hi = 0;
    if (e < E) {
      lo = min(max(off[e], (int64_t)0), M);
      hi = min(max(off[e + 1], (int64_t)0), M);
      hi = hi < lo ? lo : hi;
    }
    const int cnt = (int)((hi - lo + BM - 1) / BM);
    int inc = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int t = __shfl_up(inc, d, 64);
      if (lane >= d) inc += t;
    }
    const int excl = inc - cnt;
    const bool mine = e < E && tm >= base + excl && tm < base + inc;
    const unsigned long long ball = __ballot(mine);
    if (ball) {
      const int L = __ffsll((long long)ball) - 1;
      gt.e = c + L;
      gt.row0 = __shfl(lo + (int64_t)(tm - base - excl) * BM, L, 64);
      gt.row_end = __shfl(hi, L, 64);
    }
    base += __shfl(inc, 63, 64);
  }
  // wave-uniform: keep them in scalar registers
  gt.e = __builtin_amdgcn_readfirstlane(gt.e);
  gt.row0 = uniform64(gt.row0);
  gt.row_end = uniform64(gt.row_end);
  return __builtin_amdgcn_readfirstlane(base);
}

template <int BM, int BN, int KPS, int WM, int WN, int NS, bool EXACT, bool A4, bool W4, bool GROUPED>
__global__ __launch_bounds__(WM* WN * 64) void gemm_mx_dma_kernel(GemmArgs p) {
  using C = MxDmaCfg<BM, BN, KPS, WM, WN, NS, EXACT, A4, W4>;
  constexpr int RBA = C::RBA, RBW = C::RBW;
  constexpr int TM = C::TM, TN = C::TN, FM = C::FM, FN = C::FN, NKK = C::NKK, MPS = C::MPS;
  constexpr int STAGE = C::STAGE, IPD = C::IPD, IPS = C::IPS, IPW = C::IPW, SLOTS = C::SLOTS;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wid / WN, wn = wid % WN;
  const int h = lane >> 5;

  // Tile order (as the int8 GEMM): workgroups are dealt round-robin over the 8
  // XCDs; each XCD gets a contiguous run of tiles, walked in groups of 8
  // tile-rows so that neighbours share A rows and W columns in its L2. The
  // grouped GEMM lists the experts' tile-rows one after the other; the grid
  // is an upper bound on the tiles, and the workgroups past the real count
  // leave before touching memory or a barrier.
  GroupTile gt{0, 0, p.M};
  const int tiles_m =
      GROUPED ? group_tiles<BM>(p.groups, p.num_groups, p.M, -1, gt) : (int)((p.M + BM - 1) / BM);
  const int tiles_n = (int)((p.N + BN - 1) / BN);
  const int ntiles = tiles_m * tiles_n;
  int pid = blockIdx.x;
  if (GROUPED && pid >= ntiles) return;
  {
    const int per = ntiles / 8;
    if (per > 0 && pid < per * 8) pid = (pid % 8) * per + pid / 8;
  }
  constexpr int GROUP = 8;
  const int group_size = GROUP * tiles_n;
  const int first_m = pid / group_size * GROUP;
  const int gsize = min(tiles_m - first_m, GROUP);
  const int tile_m = first_m + (pid % group_size) % gsize;
  const int tile_n = (pid % group_size) / gsize;
  if (GROUPED) {
    group_tiles<BM>(p.groups, p.num_groups, p.M, tile_m, gt);
  } else {
    gt.row0 = (int64_t)tile_m * BM;
  }
  const int64_t m0 = gt.row0, m_end = gt.row_end, n0 = (int64_t)tile_n * BN;
  // the expert's weights, scales and bias (expert 0 for the plain GEMM)
  const uint8_t* const wexp = GROUPED ? p.w + gt.e * p.w_stride : p.w;
  const uint8_t* const ewexp = GROUPED ? p.ew + gt.e * p.w_stride : p.ew;
  const float* const bias = GROUPED && p.bias ? p.bias + gt.e * p.N : p.bias;
  const int nkt = (int)(p.K / KPS);  // every stage inside K (the launcher checks K % KPS == 0)
  const int64_t kbytes = A4 ? p.K / 2 : p.K;  // code bytes of an A row's K
  const int64_t ldw = W4 ? p.K_pad / 2 : p.K_pad, ldws = p.K_pad / 32;

  // Loads of a stage. Data: wave wid issues the stage's 1 KB loads
  // wid*IPD .. wid*IPD+IPD-1; lane l of load j fetches the 16-byte chunk that
  // belongs at LDS slot 16 l of the swizzled row-major tile (A for j < IA,
  // then W). Scales: every SS-th stage also brings the E8M0 bytes of itself and
  // the next SS - 1 stages, 16 per tile row (one 16-byte lane per row, so a
  // 1 KB load covers 64 rows instead of 64 cache lines per 256 bytes), into
  // one of two scale slots; load js (wave wid issues wid*IPS ..) covers tile
  // rows 64 js .. 64 js + 63 (A rows, then W rows). The other stages (and
  // js >= NSL) issue the same number of loads with an empty range into a
  // spare 1 KB, so every wave counts IPW loads per stage. Per-lane offsets do
  // not change along K; the stage's K offset goes in the scalar offset. A rows
  // >= M are clamped to row M - 1 (their outputs are never stored); the buffer
  // ranges end at the last row's K (codes) and at its last scale dword
  // (dwords past a range read as zero: only bytes of blocks past K/32 or of
  // the next row fall there, and they are never used), so nothing past them
  // is read. Stages past the last one get an empty range: their loads move no
  // data and still count in vmcnt.
  const int64_t last_a_row = min((int64_t)BM - 1, m_end - 1 - m0);
  const uint8_t* const abase = p.a + m0 * p.lda;
  const uint8_t* const wbase = wexp + n0 * ldw;
  const uint8_t* const eabase = p.ea + m0 * p.lda_s;
  const uint8_t* const ewbase = ewexp + n0 * ldws;
  const uint32_t nrec_a = (uint32_t)(last_a_row * p.lda + kbytes);
  const uint32_t nrec_w = (uint32_t)(BN * ldw);
  const uint32_t nrec_ea = (uint32_t)(last_a_row * p.lda_s + ((p.K / 32 + 3) & ~(int64_t)3));
  const uint32_t nrec_ew = (uint32_t)(BN * ldws);
  uint32_t voff[IPW];
#pragma unroll
  for (int i = 0; i < IPD; ++i) {
    const int j = wid * IPD + i;
    const bool ja = j < C::IA;
    // the (row, chunk) whose slot is P under the chunk swizzle of lds_off<RB>
    if (ja) {
      const int P = j * 1024 + lane * 16;
      const int r = P / RBA;
      const int c = ((P % RBA) >> 4) ^ ((r / (256 / RBA)) % (RBA / 16));
      voff[i] = (uint32_t)(min((int64_t)r, last_a_row) * p.lda) + (uint32_t)(c * 16);
    } else {
      const int P = (j - C::IA) * 1024 + lane * 16;
      const int r = P / RBW;
      const int c = ((P % RBW) >> 4) ^ ((r / (256 / RBW)) % (RBW / 16));
      // e2m1 weights are row-major; e4m3 weights come in 1 KB blocks of 16
      // rows x 64 K (mx8_code_off), so this load, rows 16 (j - IA) .. + 15 of
      // the tile, reads one whole block (the stage's K offset: kt KB)
      voff[i] = W4 ? (uint32_t)(r * ldw) + (uint32_t)(c * 16)
                   : (uint32_t)((r >> 4) * 16 * ldw) + (uint32_t)((r & 15) * 64 + c * 16);
    }
  }
#pragma unroll
  for (int i = 0; i < IPS; ++i) {
    const int js = wid * IPS + i;
    const int r = min(js * 64 + lane, BM + BN - 1);
    voff[IPD + i] = r < BM ? (uint32_t)(min((int64_t)r, last_a_row) * p.lda_s) : (uint32_t)((r - BM) * ldws);
  }
  auto dma = [&](int kt, int s, int i, bool live) {
    if (i < IPD) {
      const int j = wid * IPD + i;
      const bool ja = j < C::IA;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(ja ? abase : wbase), (short)0, live ? (int)(ja ? nrec_a : nrec_w) : 0, kRawBufferWord3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, QG_LDSP(smem + s * STAGE + j * 1024), 16, (int)voff[i],
                                               kt * (ja ? RBA : (W4 ? RBW : 1024)), 0, 0);
    } else {
      const int js = wid * IPS + (i - IPD);
      const bool ja = js * 64 < BM, real = js < C::NSL && kt % C::SS == 0;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(ja ? eabase : ewbase), (short)0, live && real ? (int)(ja ? nrec_ea : nrec_ew) : 0, kRawBufferWord3);
      // (the scalar offset goes through a named variable: written inline in
      // the call, this hipcc dropped the kernel's host stub without a message)
      const int soff = (kt / C::SS) * 16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, QG_LDSP(smem + (real ? C::SCALES + ((kt / C::SS) & 1) * C::SUPER + js * 1024 : C::SINK)), 16, (int)voff[i],
          soff, 0, 0);
    }
  };
  // the stage's loads that go after matrix-core instruction `slot` of the
  // instructions before its barrier
  auto dma_slot = [&](int slot, int ks, int sl, bool live) {
#pragma unroll
    for (int d = 0; d < IPW; ++d)
      if ((d * SLOTS) / IPW == slot) dma(ks, sl, d, live);
  };

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  // Fragments and scale bytes of one 64-deep step kk of stage kt. The step's
  // block h sits in byte 2 kk + h of dword (kt % SS) * SPS / 4 of the row's 16
  // scale bytes, shifted by b0 = (kt % SS) * SPS % 4 bytes. load_frags keeps
  // the dwords as read and their shift `sh`; unpack() then leaves the lane's
  // block in the low byte (scaled mode) or both blocks of the step (exact
  // mode; low byte: K 0-31 of the step, next byte: K 32-63). The shift is
  // done apart from the reads so that it can wait where the fragments are
  // waited for anyway, not between the reads and the next MFMAs.
  struct Frag {
    v8i a[FM], b[FN];
    int sa[FM], sb[FN];
    int sh;
  };
  auto load_frags = [&](int kt, int kk, Frag& f) {
    const uint8_t* sa = smem + (kt % NS) * STAGE;
    const uint8_t* sb = sa + BM * RBA;
    const int q = kt % C::SS;
    const int* ssa = reinterpret_cast<const int*>(smem + C::SCALES + ((kt / C::SS) & 1) * C::SUPER) + q * C::SPS / 4;
    const int* ssb = ssa + 4 * BM;
    const int sh = 8 * (q * C::SPS % 4 + 2 * kk) + (EXACT ? 0 : 8 * h);
    // e4m3: chunks 4 kk + h and 4 kk + h + 2 (K 16h .. and 32 + 16h ..);
    // e2m1: chunk 2 kk + h (K 32h .. 32h + 31)
    const int ca = A4 ? 2 * kk + h : 4 * kk + h, cw = W4 ? 2 * kk + h : 4 * kk + h;
    // the scale dwords of the wave's row blocks first, from one base each:
    // rows 32 apart are 512 bytes apart, so the compiler pairs them into
    // two-address LDS reads
    const int* pa = ssa + 4 * (wm * TM + (lane & 31));
    const int* pb = ssb + 4 * (wn * TN + (lane & 31));
    int wa[FM], wb[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) wa[i] = pa[128 * i];
#pragma unroll
    for (int j = 0; j < FN; ++j) wb[j] = pb[128 * j];
    // exact mode, e2m1: the 8-byte halves h of chunks 2 kk and 2 kk + 1 (K
    // 16h .. 16h + 15 and 32 + 16h ..), one dword per 16-deep chunk t
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = wm * TM + i * 32 + (lane & 31);
      if constexpr (EXACT && A4) {
        const uint2 x0 = *reinterpret_cast<const uint2*>(sa + lds_off<RBA>(r, 2 * kk) + 8 * h);
        const uint2 x1 = *reinterpret_cast<const uint2*>(sa + lds_off<RBA>(r, 2 * kk + 1) + 8 * h);
        f.a[i] = v8i{(int)x0.x, (int)x0.y, (int)x1.x, (int)x1.y, 0, 0, 0, 0};
      } else {
        const v4i lo = *reinterpret_cast<const v4i*>(sa + lds_off<RBA>(r, ca));
        const v4i hi = A4 ? v4i{0, 0, 0, 0} : *reinterpret_cast<const v4i*>(sa + lds_off<RBA>(r, ca + 2));
        f.a[i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      f.sa[i] = wa[i];
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int r = wn * TN + j * 32 + (lane & 31);
      if constexpr (EXACT && W4) {
        const uint2 x0 = *reinterpret_cast<const uint2*>(sb + lds_off<RBW>(r, 2 * kk) + 8 * h);
        const uint2 x1 = *reinterpret_cast<const uint2*>(sb + lds_off<RBW>(r, 2 * kk + 1) + 8 * h);
        f.b[j] = v8i{(int)x0.x, (int)x0.y, (int)x1.x, (int)x1.y, 0, 0, 0, 0};
      } else {
        const v4i lo = *reinterpret_cast<const v4i*>(sb + lds_off<RBW>(r, cw));
        const v4i hi = W4 ? v4i{0, 0, 0, 0} : *reinterpret_cast<const v4i*>(sb + lds_off<RBW>(r, cw + 2));
        f.b[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      f.sb[j] = wb[j];
    }
    f.sh = sh;
  };
  auto unpack = [&](Frag& f) {
    constexpr int mask = EXACT ? 0xffff : 0xff;
#pragma unroll
    for (int i = 0; i < FM; ++i) f.sa[i] = (f.sa[i] >> f.sh) & mask;
#pragma unroll
    for (int j = 0; j < FN; ++j) f.sb[j] = (f.sb[j] >> f.sh) & mask;
  };

  // The matrix-core instructions m0_ .. m1_ - 1 of one 64-deep step (index
  // (i, j) in the scaled mode; (t, i, j) in the exact mode, t the 16-deep
  // chunk), the stage's loads after those with slot (index - first) when
  // first >= 0. Exact mode: chunk t (codes 8t .. 8t + 7 of each lane's
  // fragment, dwords 2t and 2t + 1) as bf16 times its block's scale (chunks
  // 0-1: the step's first block, 2-3: its second); the W chunks are converted
  // first, each A chunk just before its MFMAs.
  auto mfmas = [&](const Frag& f, int m0_, int m1_, int first, int ks, int sl, bool live) {
    if constexpr (EXACT) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t * FM * FN < m0_ || t * FM * FN >= m1_) continue;
        v8bf_t bb[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j)
          bb[j] = W4 ? fp4x8_to_bf16(f.b[j][t], e8m0_to_f32((f.sb[j] >> (t < 2 ? 0 : 8)) & 0xff))
                     : fp8x8_to_bf16(f.b[j][2 * t], f.b[j][2 * t + 1], e8m0_to_f32((f.sb[j] >> (t < 2 ? 0 : 8)) & 0xff));
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const float sc = e8m0_to_f32((f.sa[i] >> (t < 2 ? 0 : 8)) & 0xff);
          const v8bf_t ab = A4 ? fp4x8_to_bf16(f.a[i][t], sc) : fp8x8_to_bf16(f.a[i][2 * t], f.a[i][2 * t + 1], sc);
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, bb[j], acc[i][j], 0, 0, 0);
            if (first >= 0) dma_slot(t * FM * FN + i * FN + j - first, ks, sl, live);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int x = i * FN + j;
          if (x < m0_ || x >= m1_) continue;
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], f.b[j], acc[i][j], A4 ? 4 : 0, W4 ? 4 : 0,
                                                                       0, f.sa[i], 0, f.sb[j]);
          if (first >= 0) dma_slot(x - first, ks, sl, live);
          __builtin_amdgcn_sched_barrier(0);
        }
    }
  };

  // stage kt + 1 landed (vmcnt counts the loads issued after it), this wave's
  // LDS reads are done (lgkmcnt 0); after the barrier everyone's are
  auto stage_barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * IPW) & ~(15 << 8));
    __builtin_amdgcn_s_barrier();
  };

  // One stage kt: `fa` holds the fragments of its first step (unpacked).
  //
  // One step per stage (KPS 64): the barrier comes first. After it, stage
  // kt + 1 has landed and every wave has finished reading slot kt % NS (its
  // fragments were read during stage kt - 1), so the stage reads stage
  // kt + 1's fragments into `fb` and refills slot kt % NS with stage kt + NS,
  // both under all of its MFMAs; the stage ends by unpacking fb's scale
  // bytes. The matrix cores thus never wait on the barrier's fragment reads,
  // and NS - 1 stages stay in flight.
  //
  // Two steps per stage (KPS 128): step 0 (fragments in fa) with the loads of
  // stage kt + NS - 1 (into the slot every wave finished reading before the
  // previous barrier) while step 1's fragments are read into fb; barrier;
  // step 1 while the next stage's step 0 is read into fa.
  Frag f0, f1;
  auto stage = [&](int kt, Frag& fa, Frag& fb) {
    if constexpr (NKK == 1) {
      const int ks = kt + NS;
      stage_barrier();
      load_frags(kt + 1, 0, fb);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(fa, 0, MPS, 0, ks, kt % NS, ks < nkt);
      __builtin_amdgcn_sched_barrier(0);
      unpack(fb);
    } else {
      const int ks = kt + NS - 1;
      const bool live = ks < nkt;
      const int sl = ks % NS;
      load_frags(kt, 1, fb);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(fa, 0, MPS, 0, ks, sl, live);
      stage_barrier();
      unpack(fb);
      __builtin_amdgcn_sched_barrier(0);
      load_frags(kt + 1, 0, fa);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(fb, 0, MPS, -1, ks, sl, live);
      __builtin_amdgcn_sched_barrier(0);
      unpack(fa);
    }
  };

  // prologue: stages 0 .. PRO - 1 in flight
#pragma unroll
  for (int s = 0; s < C::PRO; ++s)
#pragma unroll
    for (int i = 0; i < IPW; ++i) dma(s, s, i, s < nkt);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm((C::PRO - 1) * IPW));
  __builtin_amdgcn_s_barrier();
  load_frags(0, 0, f0);
  unpack(f0);

  if constexpr (NKK == 1) {
    // two stages per trip so the fragment sets alternate without copies
    int kt = 0;
    for (; kt + 1 < nkt; kt += 2) {
      stage(kt, f0, f1);
      stage(kt + 1, f1, f0);
    }
    if (kt < nkt) stage(kt, f0, f1);
  } else {
    for (int kt = 0; kt < nkt; ++kt) stage(kt, f0, f1);
  }

  // the empty loads past the last stage may still be in flight
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();

  // ---- epilogue through LDS. Lane l of a 32x32 block holds column l%32 and
  // rows 8*(e/4) + 4*(l/32) + e%4 of its 16 values e. Each wave writes one
  // 32-row slab of its sub-tile to its own LDS region, then reads it back row
  // by row so that every lane finishes 4 consecutive columns of one row.
  constexpr int LPR = TN / 4;
  constexpr int RPI = 64 / LPR;
  constexpr int RS = C::RS;
  uint8_t* wreg = smem + wid * (32 * RS * 4);
  const int cq = (lane % LPR) * 4;
  const int64_t nq = n0 + wn * TN + cq;
  float bs4[4] = {0.f, 0.f, 0.f, 0.f};
  if (bias) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (nq + t < p.N) bs4[t] = bias[nq + t];
  }
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
      if (m < m_end && nq < p.N) {
        if (bias) {
#pragma unroll
          for (int t = 0; t < 4; ++t) y[t] = y[t] + bs4[t];  // the bias after the scales, in float32
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

template <int BM, int BN, int KPS, int WM, int WN, int NS, bool EXACT, bool A4, bool W4, bool GROUPED>
static hipError_t launch_mx_dma_cfg(const GemmArgs& a, hipStream_t st) {
  using C = MxDmaCfg<BM, BN, KPS, WM, WN, NS, EXACT, A4, W4>;
  // grouped: each expert adds at most one partial tile-row
  const int64_t tiles = ((a.M + BM - 1) / BM + (GROUPED ? a.num_groups : 0)) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_mx_dma_kernel<BM, BN, KPS, WM, WN, NS, EXACT, A4, W4, GROUPED>), dim3((unsigned)tiles),
                     dim3(C::NT), 0, st, a);
  return hipGetLastError();
}

bool mx_dma_eligible(const GemmArgs& a, int mode) {
  if (mode != 0 && mode != 1) return false;
  // any pair of e4m3 / e2m1 operands in either mode; stages of 64 K, of 128 K
  // for e2m1 x e2m1 in the scaled mode
  const int kps = a.a_fp4 && a.w_fp4 && mode == 1 ? 128 : 64;
  if (a.K % kps != 0 || a.lda_s % 4 != 0 || ((uintptr_t)a.ea & 3) != 0) return false;
  // one 256-row band of A (codes and scales) and of W in 32-bit byte offsets
  const int64_t rows = a.M < 256 ? a.M : 256;
  return (rows - 1) * a.lda + a.K < (int64_t(1) << 31) && (rows - 1) * a.lda_s + a.K / 32 + 4 < (int64_t(1) << 31) &&
         256 * a.K_pad < (int64_t(1) << 31);
}

template <bool EXACT, bool A4, bool W4, bool GROUPED>
static hipError_t launch_mx_dma(const GemmArgs& a, hipStream_t st) {
  // 256 x 256 tiles (one workgroup per CU, a 4-stage ring) when they fill
  // every CU; otherwise 128 x 128 tiles (4 waves of 64 x 64, two workgroups
  // per CU). Stages of 64 K (rows of 64 bytes of e4m3, 32 of e2m1), or 128 K
  // when both operands are e2m1 in the scaled mode (64-byte rows).
  // On the 256 x 256 tiles the exact mode with e4m3 x e4m3 runs 4 waves of
  // 128 x 128 (one wave per SIMD, its 256 accumulators in AGPRs): one wave
  // with that many independent bf16 matrix-core instructions keeps its SIMD's
  // matrix core busy, and per SIMD it reads half the fragments and converts a
  // third fewer codes (8192^3: 834-837 us against 840-853 us on 8 waves, in
  // alternating runs). With an e2m1 operand the 4 waves were 4-6% slower; in
  // the scaled mode they matched the 8 waves with operands streamed from HBM
  // (8192^3: 517-519 us against 517-518 us) and were 5% slower on the grouped
  // MoE shape, so those keep 8 waves of 128 x 64.
  // The grouped exact mode keeps the 128 x 128 tiles when the average expert
  // has under 2048 rows: its partial last tile-rows then waste a large share
  // of 256-row tiles, and the exact mode, bound by its matrix cores and
  // conversions, gains from the finer grain (8 experts of about 1024 rows:
  // 299 us against 321 us; the scaled fp8 mode, bound by data movement,
  // keeps the larger tiles).
  constexpr int KPS = A4 && W4 && !EXACT ? 128 : 64;
  const bool small_groups = GROUPED && EXACT && a.M < 2048 * (int64_t)a.num_groups;
  const int64_t big = ((a.M + 255) / 256) * ((a.N + 255) / 256);
  if (big >= cu_count() && !small_groups) {
    if constexpr (EXACT && !A4 && !W4)
      return launch_mx_dma_cfg<256, 256, KPS, 2, 2, 4, EXACT, A4, W4, GROUPED>(a, st);
    else
      return launch_mx_dma_cfg<256, 256, KPS, 2, 4, 4, EXACT, A4, W4, GROUPED>(a, st);
  }
  return launch_mx_dma_cfg<128, 128, KPS, 2, 2, 4, EXACT, A4, W4, GROUPED>(a, st);
}

template <bool EXACT, bool GROUPED>
static hipError_t launch_pair(const GemmArgs& a, hipStream_t st) {
  if (a.a_fp4 && a.w_fp4) return launch_mx_dma<EXACT, true, true, GROUPED>(a, st);
  if (a.a_fp4) return launch_mx_dma<EXACT, true, false, GROUPED>(a, st);
  if (a.w_fp4) return launch_mx_dma<EXACT, false, true, GROUPED>(a, st);
  return launch_mx_dma<EXACT, false, false, GROUPED>(a, st);
}

template <bool GROUPED>
static hipError_t launch_mode(const GemmArgs& a, int mode, hipStream_t st) {
  return mode == 0 ? launch_pair<true, GROUPED>(a, st) : launch_pair<false, GROUPED>(a, st);
}

hipError_t launch_gemm_mx_dma(const GemmArgs& a, int mode, hipStream_t st) { return launch_mode<false>(a, mode, st); }

hipError_t launch_gemm_mx_grouped(const GemmArgs& a, int mode, hipStream_t st) {
  return launch_mode<true>(a, mode, st);
}

}  // namespace qg
