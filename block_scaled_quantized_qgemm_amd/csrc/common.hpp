// Internal helpers shared by the gfx950 kernels of the quantized linear layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// Wave-wide reductions (64 lanes) over a value every lane holds, by DPP moves
// inside the VALU instead of round trips through the LDS unit: two quad
// swaps, the half-row and row mirrors (each lane then holds its row of 16),
// the broadcast of lane 15 into rows 1 and 3 and of lane 31 into rows 2 and 3
// (lanes of the other rows take `id`, the operation's identity), so lane 63
// holds the whole wave's result, which is then read out to every lane. Max,
// min and integer sums do not depend on the order, so the result is exactly
// that of any other reduction order.
template <typename Op>
__device__ inline int wave_reduce_dpp(int v, int id, Op op) {
  v = op(v, __builtin_amdgcn_update_dpp(id, v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x140, 0xF, 0xF, false));  // row_mirror
  v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x142, 0xA, 0xF, false));  // row_bcast:15
  v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}
__device__ inline float wave_max(float v) {
  return __int_as_float(wave_reduce_dpp(__float_as_int(v), __float_as_int(-INFINITY), [](int x, int y) {
    return __float_as_int(fmaxf(__int_as_float(x), __int_as_float(y)));
  }));
}
__device__ inline float wave_min(float v) {
  return __int_as_float(wave_reduce_dpp(__float_as_int(v), __float_as_int(INFINITY), [](int x, int y) {
    return __float_as_int(fminf(__int_as_float(x), __int_as_float(y)));
  }));
}
__device__ inline int wave_sum(int v) {
  return wave_reduce_dpp(v, 0, [](int x, int y) { return x + y; });
}

// dword 3 of a raw buffer descriptor: 32-bit data format, no swizzle
constexpr int kRawBufferWord3 = 0x00020000;

// Round-to-nearest-even of a finite float32 to bfloat16 (the upper half of a
// float32): add 0x7fff plus the lowest kept bit, then drop the low 16 bits.
__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// E8M0 code of the smallest power of two >= t (t > 0, finite): the float32
// biased exponent, plus one when the mantissa is non-zero, clamped to [1, 254].
__device__ inline int ceil_to_ue8m0(float t) {
  uint32_t b = __float_as_uint(t) & 0x7fffffffu;
  int e = (int)(b >> 23) + ((b & 0x7fffffu) != 0u ? 1 : 0);
  return e < 1 ? 1 : (e > 254 ? 254 : e);
}

// 2^(127 - E) as a float32 for E in [1, 254] (2^-127 is the one subnormal).
__device__ inline float e8m0_inverse(int E) {
  int be = 254 - E;  // biased exponent of 2^(127-E)
  return be >= 1 ? __uint_as_float((uint32_t)be << 23) : __uint_as_float(0x00400000u);
}

// LDS row of RB bytes made of 16-byte chunks. gfx950 serves a 16-byte-per-lane
// LDS access 16 lanes at a time over 64 four-byte banks (256 bytes), so the 16
// rows that 16 lanes read at the same logical chunk must land in 16 distinct
// 16-byte slots of a 256-byte bank line: the chunk index is XOR-ed with the
// row's position among the rows that share a bank line.
template <int RB>
__device__ inline int lds_off(int row, int chunk) {
  constexpr int CPR = RB / 16;
  constexpr int RPL = RB >= 256 ? 1 : 256 / RB;  // rows sharing one 256-byte bank line
  return row * RB + ((chunk ^ ((row / RPL) % CPR)) << 4);
}

// Byte offset of e4m3 weight code (n, k) in a prepared MX buffer: 1 KB
// blocks of 16 rows x 64 K in block-row-major order, row n % 16 of a block at
// byte 64 (n % 16), its 64 codes in K order (so the 16 rows x 64 K a GEMM
// stage takes from one block are a single contiguous 1 KB load).
__host__ __device__ inline int64_t mx8_code_off(int64_t n, int64_t k, int64_t K_pad) {
  return ((((n >> 4) * (K_pad >> 6)) + (k >> 6)) << 10) + ((n & 15) << 6) + (k & 63);
}

// E8M0 code E as the float32 2^(E-127) (E in [1, 254]).
__device__ inline float e8m0_to_f32(int E) { return __uint_as_float((uint32_t)E << 23); }

// s_waitcnt immediate that waits until at most n vector-memory loads are
// outstanding (expcnt and lgkmcnt left at "no wait").
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14); }

// an LDS pointer as the address-space-3 pointer the LDS-DMA builtin takes
#define QG_LDSP(x) ((__attribute__((address_space(3))) void*)(x))

// One output element: OUT 0 float32 y, 1 bfloat16 of y, 2 the int32 c.
template <int OUT>
__device__ inline void store_one(void* out, int64_t idx, int c, float y) {
  if constexpr (OUT == 2) {
    reinterpret_cast<int32_t*>(out)[idx] = c;
  } else if constexpr (OUT == 0) {
    reinterpret_cast<float*>(out)[idx] = y;
  } else {
    reinterpret_cast<uint16_t*>(out)[idx] = f32_to_bf16_rne(y);
  }
}

}  // namespace qg
