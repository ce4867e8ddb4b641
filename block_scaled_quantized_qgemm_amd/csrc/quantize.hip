// Activation quantization and weight preparation kernels for gfx950.
//
// Row kernels: one 256-thread workgroup per row. Each thread keeps its share
// of the row in registers as float4 loads (coalesced: consecutive lanes read
// consecutive 16-byte pieces), the row statistic (amax, or min and max) is
// reduced across the wave with lane shuffles and across the four waves
// through LDS, and the codes are written from the registers without a second
// read of the row. This is the "one extra reduction over data already in
// registers" of "Activation Quantization Architecture, in depth", section
// "Fusion: making quantization nearly free".
//
// MX kernel: eight lanes own one 32-element block (a float4 each), so the
// block amax is a three-step shuffle; e4m3 codes are converted two at a time
// with the hardware conversion (round to nearest even, OCP e4m3fn on gfx950),
// e2m1 codes by comparisons with the midpoints of the fp4 grid.
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace qg {

constexpr int kRowThreads = 256;

struct RowStats {
  float lo, hi;  // symmetric: hi = amax (lo unused); asymmetric: min and max
};

template <bool ASYM>
__device__ inline void stats_update(RowStats& st, float v) {
  if (ASYM) {
    st.lo = fminf(st.lo, v);
    st.hi = fmaxf(st.hi, v);
  } else {
    st.hi = fmaxf(st.hi, fabsf(v));
  }
}

template <bool ASYM>
__device__ inline RowStats block_reduce_stats(RowStats st, float* red) {
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  st.hi = wave_max(st.hi);
  if (ASYM) st.lo = wave_min(st.lo);
  if (lane == 0) {
    red[wid] = st.hi;
    red[8 + wid] = st.lo;
  }
  __syncthreads();
  RowStats r;
  r.hi = red[0];
  r.lo = red[8];
#pragma unroll
  for (int w = 1; w < kRowThreads / kWave; ++w) {
    r.hi = fmaxf(r.hi, red[w]);
    r.lo = fminf(r.lo, red[8 + w]);
  }
  return r;
}

__device__ inline int block_sum_int(int v, int* red) {
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  v = wave_sum(v);
  if (lane == 0) red[wid] = v;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int w = 0; w < kRowThreads / kWave; ++w) s += red[w];
  return s;
}

// Sum of squares of a row as a double-double (hi + lo): every square of a
// float32 is exact in float64 (48 significant bits), each addition is an
// error-free TwoSum whose rounding error is kept in lo, and the partial sums of
// the threads are combined the same way. The terms are non-negative, so the
// pair carries the exact sum to a relative error of about K * 2^-104; rounding
// hi + lo once gives the correctly rounded float64 sum unless the exact sum lies
// within that distance of the midpoint between two doubles.
struct DD {
  double hi, lo;
};

__device__ inline DD dd_add(DD a, double b) {
  const double s = a.hi + b;
  const double bb = s - a.hi;
  const double e = (a.hi - (s - bb)) + (b - bb);
  return DD{s, a.lo + e};
}

__device__ inline DD dd_add(DD a, DD b) {
  DD r = dd_add(a, b.hi);
  r.lo += b.lo;
  return r;
}

__device__ inline double block_sum_sq_dd(DD v, double* red) {
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = dd_add(v, DD{__shfl_xor(v.hi, o, kWave), __shfl_xor(v.lo, o, kWave)});
  if (lane == 0) {
    red[2 * wid] = v.hi;
    red[2 * wid + 1] = v.lo;
  }
  __syncthreads();
  DD s{red[0], red[1]};
#pragma unroll
  for (int w = 1; w < kRowThreads / kWave; ++w) s = dd_add(s, DD{red[2 * w], red[2 * w + 1]});
  return s.hi + s.lo;
}

// RMSNorm in front of the quantizer ("Activation Quantization Architecture,
// in depth", section "Fusion: making quantization nearly free": the norm
// kernel already holds the row, so it also finds the amax and writes codes
// and the scale). rms = sqrt(sum_k x_k^2 / K + eps) from the float64 sum of
// squares, in float64, rounded once to float32; the normalized row is
// y_k = (x_k / rms) * gamma_k in float32, the division correctly rounded.
struct RowNorm {
  const float* gamma;  // [K]; null: no normalization
  float eps;
};

__device__ inline float rms_of(double sumsq, int64_t K, float eps) {
  return (float)sqrt(sumsq / (double)K + (double)eps);
}

// Block sum of float64 values, plain float64 additions.
__device__ inline double block_sum_d(double v, double* red) {
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  if (lane == 0) red[wid] = v;
  __syncthreads();
  double s = red[0];
#pragma unroll
  for (int w = 1; w < kRowThreads / kWave; ++w) s += red[w];
  return s;
}

// Whether the float32 rounding of r, a float64 rms whose relative error is at
// most (K + 16) 2^-53 (a sum of K exact squares in float64, then a division by
// K, the addition of eps and the square root, each rounded once), could differ
// from the rounding of the exact value: r lies within that error of the
// midpoint between (float)r and its neighbour on r's side.
__device__ inline bool rms_rounding_unsure(double r, int64_t K) {
  const float f = (float)r;
  const double fd = (double)f;
  const float g = r >= fd ? nextafterf(f, INFINITY) : nextafterf(f, -INFINITY);
  const double mid = 0.5 * (fd + (double)g);
  return fabs(r - mid) <= r * (double)(K + 16) * 0x1p-53;
}

// Scale (and zero point) from the row statistics, in float32 exactly as the
// formulas read: s = max(amax / 127, 1e-8); asymmetric s = max((max - min) /
// 255, 1e-8), z = clamp(rint(-min / s), 0, 255).
template <bool ASYM>
__device__ inline void scale_from_stats(const RowStats& st, float& s, int& z) {
  if (ASYM) {
    s = (st.hi - st.lo) / 255.0f;
    s = fmaxf(s, 1e-8f);
    float zf = rintf(-st.lo / s);
    zf = fminf(fmaxf(zf, 0.0f), 255.0f);
    z = (int)zf;
  } else {
    s = st.hi / 127.0f;
    s = fmaxf(s, 1e-8f);
    z = 0;
  }
}

// The correctly rounded quotient v / s from y = RN(1 / s), taken once per
// row: q0 = RN(v * y) is within an ulp of v / s, the FMA forms the remainder
// v - q0 * s exactly, and RN(q0 + remainder * y) is RN(v / s) (Markstein's
// correction step; it needs normal intermediates, which hold whenever
// |v / s| is above 2^-100, and below that both quotients give the code 0).
// The identity is checked on the CPU against the IEEE division near every
// code boundary (n + 1/2) s over the significands of s.
__device__ inline float div_rn(float v, float s, float y) {
  const float q0 = v * y;
  const float e = __builtin_fmaf(-q0, s, v);
  return __builtin_fmaf(e, y, q0);
}

template <bool ASYM>
__device__ inline uint32_t encode_code(float v, float s, float y, float zf) {
  float r = rintf(div_rn(v, s, y));
  if (ASYM) {
    r = fminf(fmaxf(r + zf, 0.0f), 255.0f);
    return (uint32_t)(int)r & 0xffu;
  } else {
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (uint32_t)(int)r & 0xffu;
  }
}

// Where code (row, k) is stored: row-major with stride ldq, or (kblocks > 0,
// the packed int8 weight layout) in 1 KB blocks of 16 rows x 64 K, block
// (row / 16, k / 64) at ((row / 16) * kblocks + k / 64) KB, and inside a block
// the 16-byte chunk (k / 16) % 4 of row row % 16 at 256 * ((k / 16) % 4) +
// 16 * (row % 16). Four consecutive codes k .. k + 3 (k % 4 == 0) stay
// contiguous in both layouts.
struct CodeDst {
  uint8_t* q;
  int64_t ldq;
  int64_t kblocks;
};

__device__ inline uint8_t* code_ptr(const CodeDst& d, int64_t row, int64_t k) {
  if (d.kblocks)
    return d.q + (((row >> 4) * d.kblocks + (k >> 6)) << 10) + (((k >> 4) & 3) << 8) + ((row & 15) << 4) + (k & 15);
  return d.q + row * d.ldq + k;
}

template <bool ASYM>
__device__ inline int code_value(uint32_t c) {
  return ASYM ? (int)c : (int)(int8_t)(uint8_t)c;
}

// VPT: float4 pieces per thread kept in registers (row length <= 1024 * VPT).
// PRECOMP: scale / zero point were computed for the whole tensor and are read
// from scales[0] / zeros[0] instead of from this row. NORM: the row is
// RMS-normalized (see RowNorm) before it is quantized.
template <bool ASYM, bool PRECOMP, int VPT, bool NORM = false>
__global__ __launch_bounds__(kRowThreads) void quant_rows_kernel(
    const float* __restrict__ x, int64_t ldx, int64_t K, CodeDst qd,
    float* __restrict__ scales, int32_t* __restrict__ zeros, int32_t* __restrict__ colsum, RowNorm nm) {
  __shared__ float red[16];
  __shared__ int redi[8];
  __shared__ double redd[16];
  const int64_t row = blockIdx.x;
  const float* xr = x + row * ldx;
  const int t = threadIdx.x;

  float4 v[VPT];
  RowStats st;
  st.lo = INFINITY;
  st.hi = ASYM ? -INFINITY : 0.0f;
  // All of this thread's loads are issued before any is used (clamped
  // addresses, no branches), so their latencies overlap.
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int64_t k = 4 * ((int64_t)t + (int64_t)kRowThreads * u);
    v[u] = *reinterpret_cast<const float4*>(xr + (k + 4 <= K ? k : 0));
  }
  float4 g[NORM ? VPT : 1];
  if constexpr (NORM) {
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int64_t k = 4 * ((int64_t)t + (int64_t)kRowThreads * u);
      g[u] = *reinterpret_cast<const float4*>(nm.gamma + (k + 4 <= K ? k : 0));
    }
  }
  // the piece holding column K - 1 is re-read element by element; past K: zeros
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int64_t k = 4 * ((int64_t)t + (int64_t)kRowThreads * u);
    if (k + 4 > K) {
      float e[4] = {0.f, 0.f, 0.f, 0.f}, ge[4] = {0.f, 0.f, 0.f, 0.f};
      for (int c = 0; c < 4; ++c)
        if (k + c < K) {
          e[c] = xr[k + c];
          if (NORM) ge[c] = nm.gamma[k + c];
        }
      v[u] = make_float4(e[0], e[1], e[2], e[3]);
      if constexpr (NORM) g[u] = make_float4(ge[0], ge[1], ge[2], ge[3]);
    }
  }
  if constexpr (NORM) {
    // The sum of squares in float64 (every square is exact there); it decides
    // the float32 rms unless the float64 rms is within its error bound of a
    // float32 rounding midpoint, and then (about once in 10^5 rows, the same
    // for every thread of the block) the row is summed again exactly, as a
    // double-double.
    double ssd = 0.0;
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      ssd = __builtin_fma((double)v[u].x, (double)v[u].x, ssd);
      ssd = __builtin_fma((double)v[u].y, (double)v[u].y, ssd);
      ssd = __builtin_fma((double)v[u].z, (double)v[u].z, ssd);
      ssd = __builtin_fma((double)v[u].w, (double)v[u].w, ssd);
    }
    const double r = sqrt(block_sum_d(ssd, redd) / (double)K + (double)nm.eps);
    float rms = (float)r;
    if (rms_rounding_unsure(r, K)) {
      __syncthreads();  // every thread has read the float64 partial sums
      DD ss{0.0, 0.0};
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        ss = dd_add(ss, (double)v[u].x * (double)v[u].x);
        ss = dd_add(ss, (double)v[u].y * (double)v[u].y);
        ss = dd_add(ss, (double)v[u].z * (double)v[u].z);
        ss = dd_add(ss, (double)v[u].w * (double)v[u].w);
      }
      rms = rms_of(block_sum_sq_dd(ss, redd), K, nm.eps);
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u)
      v[u] = make_float4((v[u].x / rms) * g[u].x, (v[u].y / rms) * g[u].y, (v[u].z / rms) * g[u].z,
                         (v[u].w / rms) * g[u].w);
  }
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int64_t k = 4 * ((int64_t)t + (int64_t)kRowThreads * u);
    if (k + 4 <= K) {
      stats_update<ASYM>(st, v[u].x);
      stats_update<ASYM>(st, v[u].y);
      stats_update<ASYM>(st, v[u].z);
      stats_update<ASYM>(st, v[u].w);
    } else {
      const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      for (int c = 0; c < 4; ++c)
        if (k + c < K) stats_update<ASYM>(st, e[c]);
    }
  }

  float s;
  int z;
  if (PRECOMP) {
    s = scales[0];
    z = ASYM ? zeros[0] : 0;
  } else {
    RowStats r = block_reduce_stats<ASYM>(st, red);
    scale_from_stats<ASYM>(r, s, z);
  }
  const float zf = (float)z;
  const float y = 1.0f / s;  // correctly rounded

  int csum = 0;
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int64_t k = 4 * ((int64_t)t + (int64_t)kRowThreads * u);
    if (k + 4 <= K) {
      uint32_t c0 = encode_code<ASYM>(v[u].x, s, y, zf), c1 = encode_code<ASYM>(v[u].y, s, y, zf);
      uint32_t c2 = encode_code<ASYM>(v[u].z, s, y, zf), c3 = encode_code<ASYM>(v[u].w, s, y, zf);
      *reinterpret_cast<uint32_t*>(code_ptr(qd, row, k)) = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
      if (colsum) csum += code_value<ASYM>(c0) + code_value<ASYM>(c1) + code_value<ASYM>(c2) + code_value<ASYM>(c3);
    } else if (k < K) {
      float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      for (int c = 0; c < 4; ++c)
        if (k + c < K) {
          uint32_t cc = encode_code<ASYM>(e[c], s, y, zf);
          *code_ptr(qd, row, k + c) = (uint8_t)cc;
          if (colsum) csum += code_value<ASYM>(cc);
        }
    }
  }
  if (colsum) {
    int tot = block_sum_int(csum, redi);
    if (t == 0) colsum[row] = tot;
  }
  if (!PRECOMP && t == 0) {
    scales[row] = s;
    if (ASYM) zeros[row] = z;
  }
}

// Rows longer than the register-resident kernels hold: two sweeps over the
// row (the second one is served by the caches).
template <bool ASYM, bool PRECOMP, bool NORM = false>
__global__ __launch_bounds__(kRowThreads) void quant_rows_long_kernel(
    const float* __restrict__ x, int64_t ldx, int64_t K, CodeDst qd,
    float* __restrict__ scales, int32_t* __restrict__ zeros, int32_t* __restrict__ colsum, RowNorm nm) {
  __shared__ float red[16];
  __shared__ int redi[8];
  __shared__ double redd[16];
  const int64_t row = blockIdx.x;
  const float* xr = x + row * ldx;
  const int t = threadIdx.x;
  float rms = 1.0f;
  if constexpr (NORM) {
    DD ss{0.0, 0.0};
    for (int64_t k = t; k < K; k += kRowThreads) ss = dd_add(ss, (double)xr[k] * (double)xr[k]);
    rms = rms_of(block_sum_sq_dd(ss, redd), K, nm.eps);
  }
  // element k of the row as quantized: x, or the normalized (x / rms) * gamma
  auto val = [&](int64_t k) { return NORM ? (xr[k] / rms) * nm.gamma[k] : xr[k]; };
  float s;
  int z;
  if (PRECOMP) {
    s = scales[0];
    z = ASYM ? zeros[0] : 0;
  } else {
    RowStats st;
    st.lo = INFINITY;
    st.hi = ASYM ? -INFINITY : 0.0f;
    for (int64_t k = t; k < K; k += kRowThreads) stats_update<ASYM>(st, val(k));
    RowStats rs = block_reduce_stats<ASYM>(st, red);
    scale_from_stats<ASYM>(rs, s, z);
  }
  const float zf = (float)z;
  const float y = 1.0f / s;  // correctly rounded
  int csum = 0;
  for (int64_t k = t; k < K; k += kRowThreads) {
    uint32_t c = encode_code<ASYM>(val(k), s, y, zf);
    *code_ptr(qd, row, k) = (uint8_t)c;
    csum += code_value<ASYM>(c);
  }
  if (colsum) {
    int tot = block_sum_int(csum, redi);
    if (t == 0) colsum[row] = tot;
  }
  if (!PRECOMP && t == 0) {
    scales[row] = s;
    if (ASYM) zeros[row] = z;
  }
}

// Per-tensor granularity, pass 1: statistics of each row into the workspace.
template <bool ASYM>
__global__ __launch_bounds__(kRowThreads) void row_stats_kernel(const float* __restrict__ x, int64_t ldx,
                                                                int64_t K, float* __restrict__ ws) {
  __shared__ float red[16];
  const int64_t row = blockIdx.x;
  const float* xr = x + row * ldx;
  RowStats st;
  st.lo = INFINITY;
  st.hi = ASYM ? -INFINITY : 0.0f;
  for (int64_t k = threadIdx.x; k < K; k += kRowThreads) stats_update<ASYM>(st, xr[k]);
  RowStats r = block_reduce_stats<ASYM>(st, red);
  if (threadIdx.x == 0) {
    if (ASYM) {
      ws[2 * row] = r.lo;
      ws[2 * row + 1] = r.hi;
    } else {
      ws[row] = r.hi;
    }
  }
}

// Per-tensor granularity, pass 2: one workgroup folds the row statistics and
// writes the single scale (and zero point).
template <bool ASYM>
__global__ __launch_bounds__(kRowThreads) void tensor_scale_kernel(const float* __restrict__ ws, int64_t rows,
                                                                   float* __restrict__ scales,
                                                                   int32_t* __restrict__ zeros) {
  __shared__ float red[16];
  RowStats st;
  st.lo = INFINITY;
  st.hi = ASYM ? -INFINITY : 0.0f;
  for (int64_t r = threadIdx.x; r < rows; r += kRowThreads) {
    if (ASYM) {
      st.lo = fminf(st.lo, ws[2 * r]);
      st.hi = fmaxf(st.hi, ws[2 * r + 1]);
    } else {
      st.hi = fmaxf(st.hi, ws[r]);
    }
  }
  RowStats r = block_reduce_stats<ASYM>(st, red);
  if (threadIdx.x == 0) {
    float s;
    int z;
    scale_from_stats<ASYM>(r, s, z);
    scales[0] = s;
    if (ASYM) zeros[0] = z;
  }
}

// e2m1 code of v (|v| <= 6): the nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6,
// ties to the even code, as the count of midpoints below |v| (a midpoint
// whose upper neighbour has the even code counts when reached, the others
// only when passed); sign in bit 3 (negative values and -0 that round to
// zero keep it).
__device__ inline uint32_t e2m1_code(float v) {
  const float a = fabsf(v);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
  return c | (__builtin_signbit(v) ? 8u : 0u);
}

// MX rows: grid (rows, ceil(K / 1024)); each thread one float4, eight
// threads per 32-element block. e4m3 (scale from amax / 448) or, FP4, e2m1
// (amax / 6, two codes per byte).
template <bool VEC, bool FP4>
__global__ __launch_bounds__(kRowThreads) void quant_mx_kernel(const float* __restrict__ x, int64_t ldx,
                                                               int64_t K, uint8_t* __restrict__ q, int64_t ldq,
                                                               uint8_t* __restrict__ e8, int64_t lde,
                                                               int64_t wblk_kpad) {
  const int64_t row = blockIdx.x;
  const int64_t k = (int64_t)blockIdx.y * (4 * kRowThreads) + 4 * threadIdx.x;
  const bool valid = k < K;  // K % 32 == 0: a block's eight lanes agree
  const float* xr = x + row * ldx + (valid ? k : 0);
  float4 v;
  if (VEC) {  // each activation is read once: non-temporal loads
    const v4f t4 = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(xr));
    v = make_float4(t4[0], t4[1], t4[2], t4[3]);
  } else
    v = make_float4(xr[0], xr[1], xr[2], xr[3]);
  if (!valid) v = make_float4(0.f, 0.f, 0.f, 0.f);
  float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  // the block's eight lanes by DPP moves (quad swaps, then the half-row
  // mirror), not through the LDS unit; a >= 0, so lanes read as 0 are harmless
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0xB1, 0xF, 0xF, false)));
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x4E, 0xF, 0xF, false)));
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x141, 0xF, 0xF, false)));
  a = fmaxf(a, 1e-4f);
  const int E = ceil_to_ue8m0(a / (FP4 ? 6.0f : 448.0f));
  const float inv = e8m0_inverse(E);
  if (!valid) return;
  if constexpr (FP4) {
    const uint32_t h = e2m1_code(v.x * inv) | (e2m1_code(v.y * inv) << 4) | (e2m1_code(v.z * inv) << 8) |
                       (e2m1_code(v.w * inv) << 12);
    uint8_t* qr = q + row * ldq + (k >> 1);
    if (VEC) {
      *reinterpret_cast<uint16_t*>(qr) = (uint16_t)h;
    } else {
      qr[0] = (uint8_t)h;
      qr[1] = (uint8_t)(h >> 8);
    }
    if ((threadIdx.x & 7) == 0) e8[row * lde + (k >> 5)] = (uint8_t)E;
    return;
  }
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(v.x * inv, v.y * inv, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(v.z * inv, v.w * inv, w, true);
  // activations row-major; e4m3 weights (wblk_kpad = K_pad) in the blocked
  // layout of mx8_code_off (four codes of one row segment of a block)
  uint8_t* qr = q + (wblk_kpad ? mx8_code_off(row, k, wblk_kpad) : row * ldq + k);
  if (VEC) {
    *reinterpret_cast<uint32_t*>(qr) = (uint32_t)w;
  } else {
    qr[0] = (uint8_t)w;
    qr[1] = (uint8_t)(w >> 8);
    qr[2] = (uint8_t)(w >> 16);
    qr[3] = (uint8_t)(w >> 24);
  }
  if ((threadIdx.x & 7) == 0) e8[row * lde + (k >> 5)] = (uint8_t)E;
}

// int4 weights: one wave per group of 64 K of a row, a lane per element.
// s = max(amax / 7, 1e-8), q = clamp(rint(w / s), -8, 7) ("TileLang
// tutorial, chapter 27", section 2.4, with the groups of 64 of its section
// 5.1). The lane of the lower K of each (k, k + 4) pair takes its partner's
// code and writes the byte holding both (low nibble first); lane 0 writes the
// scale (16 rows x 4 groups of scales per 64 floats, a row's four together). Groups wholly past K exit (their codes and scales stay zero).
__global__ __launch_bounds__(kRowThreads) void quant_int4_groups_kernel(const float* __restrict__ w, int64_t ldw,
                                                                        int64_t K, int64_t K_pad,
                                                                        uint8_t* __restrict__ codes,
                                                                        float* __restrict__ scales) {
  const int64_t n = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t g = (int64_t)blockIdx.y * (kRowThreads / kWave) + (threadIdx.x / kWave);
  if (g * 64 >= K) return;  // the whole wave
  const int64_t k = g * 64 + lane;
  const float v = k < K ? w[n * ldw + k] : 0.0f;
  const float amax = wave_max(fabsf(v));
  const float s = fmaxf(amax / 7.0f, 1e-8f);
  const float y = 1.0f / s;  // correctly rounded
  const float r = fminf(fmaxf(rintf(div_rn(v, s, y)), -8.0f), 7.0f);
  const uint32_t nib = (uint32_t)(int)r & 0xfu;
  const uint32_t up = (uint32_t)__shfl_xor((int)nib, 4, kWave);
  const int64_t blk = (n >> 4) * (K_pad >> 7) + (g >> 1);
  const int kk = lane & 15, c = lane >> 4;
  if ((lane & 4) == 0)
    codes[(blk << 10) + ((16 * c + (n & 15)) << 4) + 8 * (g & 1) + 4 * (kk >> 3) + (kk & 3)] = (uint8_t)(nib | (up << 4));
  if (lane == 0) scales[((n >> 4) * (K_pad >> 8) + (g >> 2)) * 64 + 4 * (n & 15) + (g & 3)] = s;
}

// ---------------------------------------------------------------------------
// Scratch memory for the allocation-free quantize entry point: the per-row
// statistics of the per-tensor quantizer (one float per row, two for the
// asymmetric format). Each GPU holds its own copy of the array; host code
// must use the address looked up for that device, never the array's name.
// ---------------------------------------------------------------------------
static __device__ __align__(256) float scratch[kScratchFloats];

namespace {
std::mutex g_scratch_mu;
float* g_scratch_dev[kMaxScratchDevices];  // per device: its copy of `scratch`, once looked up
}  // namespace

hipError_t scratch_buffer(float** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_dev[dev] = static_cast<float*>(p);
  }
  *ptr = g_scratch_dev[dev];
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
template <bool ASYM, bool PRECOMP, bool NORM>
static void launch_rows(const float* x, int64_t rows, int64_t K, int64_t ldx, CodeDst qd, float* scales,
                        int32_t* zeros, int32_t* colsum, RowNorm nm, hipStream_t st) {
  dim3 grid((unsigned)rows), block(kRowThreads);
  // the register kernels read 16 bytes at a row's start even when K < 4
  const bool vec = K >= 4 && ldx % 4 == 0 && ((uintptr_t)x % 16) == 0 && qd.ldq % 4 == 0 &&
                   ((uintptr_t)qd.q % 4) == 0 && (!NORM || ((uintptr_t)nm.gamma % 16) == 0);
  if (!vec)
    quant_rows_long_kernel<ASYM, PRECOMP, NORM><<<grid, block, 0, st>>>(x, ldx, K, qd, scales, zeros, colsum, nm);
  else if (K <= 1024)
    quant_rows_kernel<ASYM, PRECOMP, 1, NORM><<<grid, block, 0, st>>>(x, ldx, K, qd, scales, zeros, colsum, nm);
  else if (K <= 2048)
    quant_rows_kernel<ASYM, PRECOMP, 2, NORM><<<grid, block, 0, st>>>(x, ldx, K, qd, scales, zeros, colsum, nm);
  else if (K <= 4096)
    quant_rows_kernel<ASYM, PRECOMP, 4, NORM><<<grid, block, 0, st>>>(x, ldx, K, qd, scales, zeros, colsum, nm);
  else if (K <= 8192)
    quant_rows_kernel<ASYM, PRECOMP, 8, NORM><<<grid, block, 0, st>>>(x, ldx, K, qd, scales, zeros, colsum, nm);
  else
    quant_rows_long_kernel<ASYM, PRECOMP, NORM><<<grid, block, 0, st>>>(x, ldx, K, qd, scales, zeros, colsum, nm);
}

void launch_quantize_int(const float* x, int64_t rows, int64_t K, int64_t ldx, bool asym, bool per_tensor,
                         uint8_t* q, int64_t ldq, int64_t kblocks, float* scales, int32_t* zeros, int32_t* colsum,
                         float* ws, hipStream_t st) {
  if (rows == 0) return;
  const CodeDst qd{q, kblocks ? 16 : ldq, kblocks};
  if (!per_tensor) {
    if (asym)
      launch_rows<true, false, false>(x, rows, K, ldx, qd, scales, zeros, colsum, RowNorm{}, st);
    else
      launch_rows<false, false, false>(x, rows, K, ldx, qd, scales, zeros, colsum, RowNorm{}, st);
    return;
  }
  dim3 grid((unsigned)rows), block(kRowThreads);
  if (asym) {
    row_stats_kernel<true><<<grid, block, 0, st>>>(x, ldx, K, ws);
    tensor_scale_kernel<true><<<1, block, 0, st>>>(ws, rows, scales, zeros);
    launch_rows<true, true, false>(x, rows, K, ldx, qd, scales, zeros, colsum, RowNorm{}, st);
  } else {
    row_stats_kernel<false><<<grid, block, 0, st>>>(x, ldx, K, ws);
    tensor_scale_kernel<false><<<1, block, 0, st>>>(ws, rows, scales, zeros);
    launch_rows<false, true, false>(x, rows, K, ldx, qd, scales, zeros, colsum, RowNorm{}, st);
  }
}

void launch_rmsnorm_quantize(const float* x, int64_t rows, int64_t K, int64_t ldx, const float* gamma, float eps,
                             bool asym, uint8_t* q, int64_t ldq, float* scales, int32_t* zeros, hipStream_t st) {
  if (rows == 0) return;
  const CodeDst qd{q, ldq, 0};
  const RowNorm nm{gamma, eps};
  if (asym)
    launch_rows<true, false, true>(x, rows, K, ldx, qd, scales, zeros, nullptr, nm, st);
  else
    launch_rows<false, false, true>(x, rows, K, ldx, qd, scales, zeros, nullptr, nm, st);
}

void launch_quantize_int4(const float* w, int64_t rows, int64_t K, int64_t ldw, int64_t K_pad, uint8_t* codes,
                          float* scales, hipStream_t st) {
  if (rows == 0) return;
  constexpr int gpb = kRowThreads / kWave;  // groups per workgroup
  dim3 grid((unsigned)rows, (unsigned)((K_pad / 64 + gpb - 1) / gpb)), block(kRowThreads);
  quant_int4_groups_kernel<<<grid, block, 0, st>>>(w, ldw, K, K_pad, codes, scales);
}

void launch_quantize_mx(const float* x, int64_t rows, int64_t K, int64_t ldx, bool fp4, uint8_t* q, int64_t ldq,
                        uint8_t* e8, int64_t lde, int64_t wblk_kpad, hipStream_t st) {
  if (rows == 0) return;
  dim3 grid((unsigned)rows, (unsigned)((K + 4 * kRowThreads - 1) / (4 * kRowThreads))), block(kRowThreads);
  const bool vec = ldx % 4 == 0 && ((uintptr_t)x % 16) == 0 && ldq % 4 == 0 && ((uintptr_t)q % 4) == 0;
  const int64_t wb = fp4 ? 0 : wblk_kpad;
  if (fp4) {
    if (vec)
      quant_mx_kernel<true, true><<<grid, block, 0, st>>>(x, ldx, K, q, ldq, e8, lde, wb);
    else
      quant_mx_kernel<false, true><<<grid, block, 0, st>>>(x, ldx, K, q, ldq, e8, lde, wb);
  } else if (vec) {
    quant_mx_kernel<true, false><<<grid, block, 0, st>>>(x, ldx, K, q, ldq, e8, lde, wb);
  } else {
    quant_mx_kernel<false, false><<<grid, block, 0, st>>>(x, ldx, K, q, ldq, e8, lde, wb);
  }
}

}  // namespace qg
