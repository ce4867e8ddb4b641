// int8 activations x int4 weights with one float32 scale per group of 64 K
// ("TileLang tutorial, chapter 27", sections 3.3(c), 4.3 and 5.1) for gfx950.
#include "common.hpp"
#include "kernels.hpp"

namespace qg {

constexpr int kW4Waves = 8;  // waves per workgroup, each on its own K range
constexpr int kW4Cols = 2;   // 16-row weight blocks per workgroup (row kernel)

// ---------------------------------------------------------------------------
// W4A8: int8 activations x int4 weights with one float32 scale per group of
// 64 K ("TileLang tutorial, chapter 27", sections 3.3(c) and 5.1), for 16-row
// bands of A: the decode kernel's stream over W at half the bytes. A
// workgroup owns kW4Cols blocks of 16 weight rows over all of K; its eight
// waves take contiguous ranges of 128-deep steps (two groups). Per step a
// lane loads its activation chunks once for all blocks and, per block, 16
// bytes of codes (its 16-K chunk of both groups); per two steps, the four
// group scales of its weight row in each block (16 bytes). Each block has its
// own buffer ranges, so a block's steps past K_pad read zeros, never the next
// block's codes. Two blocks per workgroup share each activation load between
// twice the weight bytes: the activation loads, identical in every
// workgroup, were 40% of a wave's loads with one block (8 x 4096 x 14336:
// 8.9 -> 8.0 us; four blocks, 224 workgroups: 8.4 us).
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
  constexpr int NC = kW4Cols;
  __shared__ v4f red[kW4Waves][NC][64];
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n0 = (int64_t)blockIdx.x * 16 * NC;
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
  __amdgpu_buffer_rsrc_t wrs[NC], srs[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    wrs[c] = __builtin_amdgcn_make_buffer_rsrc((void*)(p.w + (blk0 + c * pairs) * 1024), (short)0, (int)(pairs * 1024),
                                               kRawBufferWord3);
    srs[c] = __builtin_amdgcn_make_buffer_rsrc((void*)(p.sw + (blk0 + c * pairs) * 32), (short)0, (int)(pairs * 128),
                                               kRawBufferWord3);
  }
  const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.a + m0 * p.lda), (short)0, (int)((mrows - 1) * p.lda + ((p.K + 15) & ~(int64_t)15)),
      kRawBufferWord3);
  const uint32_t woff = (uint32_t)pbeg * 1024u + (uint32_t)(lane * 16);
  const uint32_t soff = (uint32_t)pbeg * 128u + (uint32_t)(row * 16);
  const int arow = MLE8 ? (lane & 7) : row;
  const int akin = (MLE8 ? ((lane >> 3) & 1) * 64 : 0) + (lane >> 4) * 16;
  const uint32_t aoff = arow < mrows ? (uint32_t)(arow * p.lda + pbeg * 128 + akin) : kOff;

  v4f y[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) y[c] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int b = 0; b < (ONE ? U : per); b += U) {
    v4i wv[NC][U], a0[U], a1[MLE8 ? 1 : U];
    v4f sv[NC][U / 2];
    // per step: activations, codes, and every second step the scales
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t st = (uint32_t)(b + u);
      a0[u] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(ars, (int)(aoff + st * 128u), 0, 0));
      if (!MLE8)
        a1[u] = __builtin_bit_cast(
            v4i, __builtin_amdgcn_raw_buffer_load_b128(ars, (int)(aoff + st * 128u + 64u), 0, 0));
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        wv[c][u] = __builtin_bit_cast(
            v4i, __builtin_amdgcn_raw_buffer_load_b128(wrs[c], (int)(woff + st * 1024u), 0, kStreamLoad));
        if (u % 2 == 0)
          sv[c][u / 2] = __builtin_bit_cast(
              v4f, __builtin_amdgcn_raw_buffer_load_b128(srs[c], (int)(soff + st * 128u), 0, kStreamLoad));
      }
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
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const v4i w = wv[c][u];
        const v4i w0 = {(w.x << 4) & kHi, w.x & kHi, (w.y << 4) & kHi, w.y & kHi};
        const v4i w1 = {(w.z << 4) & kHi, w.z & kHi, (w.w << 4) & kHi, w.w & kHi};
        const v4i zero = {0, 0, 0, 0};
        const v4i c0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0[u], w0, zero, 0, 0, 0);
        const v4i c1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(x1, w1, zero, 0, 0, 0);
        const float s0 = (u & 1) ? sv[c][u / 2].z : sv[c][u / 2].x;
        const float s1 = (u & 1) ? sv[c][u / 2].w : sv[c][u / 2].y;
#pragma unroll
        for (int i = 0; i < 4; ++i) y[c][i] = __builtin_fmaf(s0, (float)c0[i], y[c][i]);
#pragma unroll
        for (int i = 0; i < 4; ++i) y[c][i] = __builtin_fmaf(s1, (float)c1[i], y[c][i]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) red[wid][c][lane] = y[c];
  __syncthreads();

  // thread t < 256 NC finishes item (t % 256) / 64 of lane t % 64 of block t / 256:
  // row 4 * (l / 16) + item, column 16 * block + l % 16
  for (int t = threadIdx.x; t < 256 * NC; t += kW4Waves * 64) {
    const int l = t & 63, item = (t >> 6) & 3, cb = t >> 8;
    const int64_t m = m0 + 4 * (l >> 4) + item;
    const int64_t n = n0 + 16 * cb + (l & 15);
    if (m < p.M && n < p.N) {
      float acc = red[0][cb][l][item];
#pragma unroll
      for (int w = 1; w < kW4Waves; ++w) acc += red[w][cb][l][item];
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

// ---------------------------------------------------------------------------
// W4A8 for more than 16 rows: output tiles of BM x BN over all of K, the
// tiles moved into an LDS ring by global -> LDS DMA as in the int8 GEMM. A
// stage is 128 K (two groups of 64): the A rows (128 bytes each, XOR-swizzled
// 16-byte chunks) and the BN / 16 packed weight blocks (1 KB each, copied
// whole; lane l's 16 bytes of a block are its v_mfma_i32_16x16x64_i8 operand
// for both groups). Every second stage also brings the weights' group scales
// of the next 256 K (16 bytes per weight row: a 16-byte lane per row) into a
// scale slot; the other stages issue the same number of loads with an empty
// range into a spare 1 KB, so every wave counts IPW loads per stage.
//
// Per group a wave forms, for each 16 x 16 block of its sub-tile, the exact
// integer sum 16 P_g with one MFMA from a zero accumulator (the nibbles enter
// as 16 q, as in the row kernel above) and adds s_w[n, g] * 16 P_g to its
// float32 accumulator ("TileLang tutorial, chapter 27", section 4.3: a scale
// that varies along K multiplies its own group's partial sum inside the K
// loop), groups in K order. The epilogue multiplies by s_a / 16 and adds the
// bias.
//
// Schedule per stage: group 1's activation fragments are read, group 0's
// MFMAs run with the next ring stage's DMA between them, then the wait and
// barrier for the next stage, its group-0 fragments, weights and scales are
// read, and group 1's MFMAs hide those reads.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, int NS>
struct W4Cfg {
  static constexpr int NT = WM * WN * 64, NW = WM * WN;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 16, FN = TN / 16;      // 16 x 16 blocks per wave
  static constexpr int A_BYTES = BM * 128;              // 128 K of int8 per row
  static constexpr int W_BYTES = BN * 64;               // 128 K of int4 per row
  static constexpr int STAGE = A_BYTES + W_BYTES;
  static constexpr int IA = A_BYTES / 1024;             // the first IA 1 KB loads carry A
  static constexpr int IPD = STAGE / 1024 / NW;         // data loads per wave and stage
  static constexpr int NSL = BN / 64;                   // 1 KB scale loads per scale slot
  static constexpr int IPS = (NSL + NW - 1) / NW;
  static constexpr int IPW = IPD + IPS;
  static constexpr int SLOTSN = (NS + 2) / 2;           // scale slots: >= (NS + 1) / 2
  static constexpr int SUPER = BN * 16;                 // one slot: 16 bytes (4 group scales) per weight row
  static constexpr int SCALES = NS * STAGE;
  static constexpr int SINK = SCALES + SLOTSN * SUPER;
  static constexpr int LDS = SINK + 1024;
  static constexpr int SLOTS = FM * FN;                 // group-0 MFMAs the stage's loads are spread over
  static_assert(STAGE % (1024 * NW) == 0 && BN % 64 == 0 && BM % 16 == 0, "loads per wave");
  static_assert(FM >= 1 && FN >= 1 && SLOTS >= IPW, "load slots");
  static_assert(NS >= 3 && (NS - 2) * IPW < 64, "vmcnt range");
};

template <int BM, int BN, int WM, int WN, int NS, int OUT>
__global__ __launch_bounds__(WM* WN * 64) void gemm_w4a8_tiled_kernel(GemmArgs p) {
  using C = W4Cfg<BM, BN, WM, WN, NS>;
  constexpr int TM = C::TM, TN = C::TN, FM = C::FM, FN = C::FN;
  constexpr int STAGE = C::STAGE, IPD = C::IPD, IPS = C::IPS, IPW = C::IPW, SLOTS = C::SLOTS;
  constexpr int kHi = (int)0xF0F0F0F0u;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid / WN, wn = wid % WN;

  // tile order as the int8 GEMM (XCD-aware runs, groups of 8 tile-rows)
  const int tiles_m = (int)((p.M + BM - 1) / BM);
  const int tiles_n = (int)((p.N + BN - 1) / BN);
  const int ntiles = tiles_m * tiles_n;
  int pid = blockIdx.x;
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
  const int64_t m0 = (int64_t)tile_m * BM, n0 = (int64_t)tile_n * BN;
  const int nkt = (int)(p.K_pad / 128);
  const int64_t kb128 = p.K_pad / 128, kb256 = p.K_pad / 256;

  // Loads. A rows >= M are clamped to row M - 1 (never stored); A's range ends
  // at the 16-byte chunk holding column K - 1 of the last row, and what lies
  // past K in a row meets zero weights. W blocks and scales are padded to
  // N_pad and K_pad with zeros.
  const int64_t last_a_row = min((int64_t)BM - 1, p.M - 1 - m0);
  const uint8_t* const abase = p.a + m0 * p.lda;
  const uint8_t* const wbase = p.w + (n0 >> 4) * kb128 * 1024;
  const uint8_t* const sbase = reinterpret_cast<const uint8_t*>(p.sw) + (n0 >> 4) * kb256 * 256;
  const uint32_t nrec_a = (uint32_t)(last_a_row * p.lda + ((p.K + 15) & ~(int64_t)15));
  const uint32_t nrec_w = (uint32_t)((BN / 16) * kb128 * 1024);
  const uint32_t nrec_s = (uint32_t)((BN / 16) * kb256 * 256);
  uint32_t voff[IPW];
#pragma unroll
  for (int i = 0; i < IPD; ++i) {
    const int j = wid * IPD + i;
    if (j < C::IA) {  // swizzled row-major A tile, 128-byte rows
      const int P = j * 1024 + lane * 16;
      const int r = P / 128;
      const int c = ((P % 128) >> 4) ^ ((r / 2) % 8);
      voff[i] = (uint32_t)(min((int64_t)r, last_a_row) * p.lda) + (uint32_t)(c * 16);
    } else {  // weight block row j - IA of the tile, stage kt at + kt KB
      voff[i] = (uint32_t)((j - C::IA) * kb128 * 1024) + (uint32_t)(lane * 16);
    }
  }
#pragma unroll
  for (int i = 0; i < IPS; ++i) {  // scale rows 64 js + lane: block (64 js + lane) / 16, row lane % 16
    const int js = min(wid * IPS + i, C::NSL - 1);
    const int row = js * 64 + lane;
    voff[IPD + i] = (uint32_t)((row >> 4) * kb256 * 256) + (uint32_t)((row & 15) * 16);
  }
  auto dma = [&](int kt, int s, int i, bool live) {
    if (i < IPD) {
      const int j = wid * IPD + i;
      const bool ja = j < C::IA;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(ja ? abase : wbase), (short)0, live ? (int)(ja ? nrec_a : nrec_w) : 0, kRawBufferWord3);
      const int soff = kt * (ja ? 128 : 1024);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, QG_LDSP(smem + s * STAGE + j * 1024), 16, (int)voff[i], soff, 0, 0);
    } else {
      const int js = wid * IPS + (i - IPD);
      const bool real = js < C::NSL && (kt & 1) == 0;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)sbase, (short)0, live && real ? (int)nrec_s : 0, kRawBufferWord3);
      const int soff = (kt >> 1) * 256;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, QG_LDSP(smem + (real ? C::SCALES + ((kt >> 1) % C::SLOTSN) * C::SUPER + js * 1024 : C::SINK)), 16,
          (int)voff[i], soff, 0, 0);
    }
  };

  // Fragments of one stage: the activation blocks of both groups (lane 16 c + r:
  // row r, K 16 c .. 16 c + 15 of the group), the packed weight blocks (both
  // groups) and the weight column's two group scales.
  struct Frag {
    v4i a[2][FM];
    v4i w[FN];
    v2f s[FN];
  };
  auto load_a = [&](int kt, int g, Frag& f) {
    const uint8_t* sa = smem + (kt % NS) * STAGE;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      f.a[g][i] = *reinterpret_cast<const v4i*>(sa + lds_off<128>(wm * TM + i * 16 + (lane & 15), g * 4 + (lane >> 4)));
  };
  auto load_w = [&](int kt, Frag& f) {
    const uint8_t* sw = smem + (kt % NS) * STAGE + C::A_BYTES;
    const uint8_t* ss = smem + C::SCALES + ((kt >> 1) % C::SLOTSN) * C::SUPER + (kt & 1) * 8;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      f.w[j] = *reinterpret_cast<const v4i*>(sw + (wn * FN + j) * 1024 + lane * 16);
      f.s[j] = *reinterpret_cast<const v2f*>(ss + (wn * TN + j * 16 + (lane & 15)) * 16);
    }
  };

  v4f y[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) y[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // group g of a stage; the loads of stage ks after MFMA `slot` when first.
  // Software-pipelined: the scaling of MFMA k's exact sum is issued after
  // MFMA k + PD, so the conversions and FMAs run while the matrix cores work
  // instead of waiting for each result in turn (the sums are the same, each
  // scaled and added to its own accumulator in the same order).
  auto group = [&](const Frag& f, int g, bool first, int ks, int sl, bool live) {
    const v4i zero = {0, 0, 0, 0};
    constexpr int NM = FN * FM, PD = 4;
    v4i wg[FN];
    float sc[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const v4i w = f.w[j];
      wg[j] = g == 0 ? v4i{(w.x << 4) & kHi, w.x & kHi, (w.y << 4) & kHi, w.y & kHi}
                     : v4i{(w.z << 4) & kHi, w.z & kHi, (w.w << 4) & kHi, w.w & kHi};
      sc[j] = g == 0 ? f.s[j].x : f.s[j].y;
    }
    v4i c[NM];
#pragma unroll
    for (int k = 0; k < NM + PD; ++k) {
      if (k < NM) {
        const int j = k / FM, i = k % FM;
        c[k] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f.a[g][i], wg[j], zero, 0, 0, 0);
        if (first) {
#pragma unroll
          for (int d = 0; d < IPW; ++d)
            if ((d * SLOTS) / IPW == k) dma(ks, sl, d, live);
        }
      }
      if (k >= PD) {
        const int q = k - PD, j = q / FM, i = q % FM;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[i][j][e] = __builtin_fmaf(sc[j], (float)c[q][e], y[i][j][e]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  Frag f0, f1;
  auto stage = [&](int kt, Frag& cur, Frag& nxt) {
    const int ks = kt + NS - 1;
    const bool live = ks < nkt;
    load_a(kt, 1, cur);
    __builtin_amdgcn_sched_barrier(0);
    group(cur, 0, true, ks, ks % NS, live);
    // stage kt + 1 landed (vmcnt counts the loads issued after it), this
    // wave's LDS reads are done (lgkmcnt 0); after the barrier everyone's are
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * IPW) & ~(15 << 8));
    __builtin_amdgcn_s_barrier();
    load_a(kt + 1, 0, nxt);
    load_w(kt + 1, nxt);
    __builtin_amdgcn_sched_barrier(0);
    group(cur, 1, false, ks, ks % NS, live);
  };

  // prologue: stages 0 .. NS-2 in flight
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
#pragma unroll
    for (int i = 0; i < IPW; ++i) dma(s, s, i, s < nkt);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * IPW));
  __builtin_amdgcn_s_barrier();
  load_a(0, 0, f0);
  load_w(0, f0);

  int kt = 0;
  for (; kt + 1 < nkt; kt += 2) {
    stage(kt, f0, f1);
    stage(kt + 1, f1, f0);
  }
  if (kt < nkt) stage(kt, f0, f1);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  // epilogue: lane l of a 16 x 16 block holds rows 4 (l / 16) + e of column
  // l % 16; y * (s_a / 16) (the codes entered as 16 q), then the bias
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int64_t n = n0 + wn * TN + j * 16 + (lane & 15);
    const float bn = (p.bias && n < p.N) ? p.bias[n] : 0.f;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t m = m0 + wm * TM + i * 16 + 4 * (lane >> 4) + e;
        if (m < p.M && n < p.N) {
          const float sa = p.a_per_tensor ? p.sa[0] : p.sa[m];
          float v = y[i][j][e] * (sa * 0.0625f);
          if (p.bias) v = v + bn;
          store_one<OUT>(p.out, m * p.ldo + n, 0, v);
        }
      }
  }
}

template <int BM, int BN, int WM, int WN, int NS, int OUT>
static hipError_t launch_w4a8_tiled(const GemmArgs& a, hipStream_t st) {
  using C = W4Cfg<BM, BN, WM, WN, NS>;
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_w4a8_tiled_kernel<BM, BN, WM, WN, NS, OUT>), dim3((unsigned)tiles), dim3(C::NT), 0, st,
                     a);
  return hipGetLastError();
}

template <int OUT>
static hipError_t launch_w4a8(const GemmArgs& a, hipStream_t st) {
  // the tiled kernel addresses a 128-row band of A and a tile's weight blocks
  // (64 K_pad bytes) with 32-bit offsets; beyond that the row kernel serves
  const int64_t band = (a.M < 128 ? a.M : 128) - 1;
  if (a.M > 16 && a.K_pad <= (int64_t(1) << 24) && band * a.lda + a.K_pad < (int64_t(1) << 31)) {
    // 128 x 128 tiles (8 waves of 64 x 32) when they fill every CU, else 64 x 128
    const int64_t big = ((a.M + 127) / 128) * ((a.N + 127) / 128);
    if (big >= cu_count()) return launch_w4a8_tiled<128, 128, 2, 4, 4, OUT>(a, st);
    return launch_w4a8_tiled<64, 128, 2, 4, 6, OUT>(a, st);
  }
  const dim3 grid((unsigned)((a.N + 16 * kW4Cols - 1) / (16 * kW4Cols)), (unsigned)((a.M + 15) / 16));
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
