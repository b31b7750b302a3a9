// lca_device.h -- device-side helpers shared by the liblca kernels (gfx950, wave64).
//
// Number formats are implemented here from their definitions (OCP FP8 E4M3 "fn", OCP FP4 E2M1 with E8M0
// power-of-two scales, bfloat16), with bit manipulation on fp32 values.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/lca.h"

#define LCA_WAVE 64

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
// Plain 16- and 8-byte vectors: unlike HIP's uint4 struct, copies of these stay in registers (no memcpy through
// private memory); the address-space-1 pointer types make loads global rather than flat.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) const u32x4_t gbl_u32x4_t;
typedef __attribute__((address_space(1))) const u32x2_t gbl_u32x2_t;

namespace lca {

// ------------------------------------------------------------------------------------------------
// bfloat16
// ------------------------------------------------------------------------------------------------
// fp32 -> bf16 with round half to even: the hardware conversion (v_cvt_pk_bf16_f32), one instruction per two values.
__device__ __forceinline__ uint16_t f32_to_bf16(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// ------------------------------------------------------------------------------------------------
// OCP FP8 E4M3 (bias 7, max 448, no inf).  `y` must already be clamped to [-448, 448].
// ------------------------------------------------------------------------------------------------
__device__ __forceinline__ uint8_t fp8_encode(float y) {
  uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  float a = fabsf(y);
  uint32_t code;
  if (a < 0.015625f) {                   // below 2^-6: subnormal grid, spacing 2^-9
    code = (uint32_t)rintf(a * 512.0f);  // exact scaling, round half to even; 8 -> 2^-6 (code 0x08)
  } else {
    uint32_t ua = __float_as_uint(a);
    uint32_t r = ua + 0x7FFFFu + ((ua >> 20) & 1u);  // keep 3 mantissa bits, ties to even
    r &= 0xFFF00000u;
    int e = (int)(r >> 23) - 127;
    code = ((uint32_t)(e + 7) << 3) | ((r >> 20) & 7u);
  }
  return (uint8_t)(code | sign);
}

__device__ __forceinline__ float fp8_decode(uint32_t c) {
  uint32_t e = (c >> 3) & 0xFu, mnt = c & 7u;
  float v = (e == 0) ? (float)mnt * 0.001953125f  // m * 2^-9
                     : __uint_as_float(((e + 120u) << 23) | (mnt << 20));
  return (c & 0x80u) ? -v : v;
}

// ------------------------------------------------------------------------------------------------
// OCP FP4 E2M1 with a power-of-two (E8M0) scale per block of kFp4Block consecutive elements.
// ------------------------------------------------------------------------------------------------
// Smallest integer e with amax <= 6 * 2^e, clamped to [-127, 127]; -127 when amax == 0.
__device__ __forceinline__ int fp4_group_exp(float amax) {
  if (amax == 0.0f) return -127;
  int E;
  float f = frexpf(amax, &E);  // amax = f * 2^E, f in [0.5, 1)
  int e = E - 3 + (f > 0.75f ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}
// Magnitude index of |y| (|y| <= 6) on the grid {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even index.
__device__ __forceinline__ uint32_t fp4_mag(float a) {
  return a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u : a <= 2.5f ? 4u : a < 3.5f ? 5u
       : a <= 5.0f ? 6u : 7u;
}
__device__ __forceinline__ uint32_t fp4_encode(float y) {
  return fp4_mag(fabsf(y)) | ((__float_as_uint(y) >> 28) & 8u);
}
// 2^e as a float for e in [-127, 127] (2^-127 is a subnormal; only used with all-zero codes or exact grids).
__device__ __forceinline__ float exp2i(int e) {
  return e >= -126 ? __uint_as_float((uint32_t)(e + 127) << 23) : __uint_as_float(0x00400000u);
}
__device__ __forceinline__ float fp4_value(uint32_t code) {
  // magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}
  uint32_t m = code & 7u;
  float v = (m < 4u) ? 0.5f * (float)m : (float)(2u << ((m - 4u) >> 1)) * ((m & 1u) ? 1.5f : 1.0f);
  return (code & 8u) ? -v : v;
}

// ------------------------------------------------------------------------------------------------
// Rows and positions
// ------------------------------------------------------------------------------------------------
// Storage row of row i of sequence b: b * cap + i in a dense tensor; through the block table in a paged one.
__device__ __forceinline__ long long tensor_row(const lca_tensor& t, int b, long long i) {
  if (!t.block_table) return (long long)b * t.cap + i;
  const int sh = __builtin_ctz((unsigned)t.block_rows);
  const int blk = t.block_table[(long long)b * (t.cap >> sh) + (i >> sh)];
  return (long long)blk * t.block_rows + (i & (t.block_rows - 1));
}
// Position of sequence b: its own in a ragged batch, else the call's.
__device__ __forceinline__ long long seq_position(const long long* pos, long long uniform, int b) {
  return pos ? pos[b] : uniform;
}

// ------------------------------------------------------------------------------------------------
// Order-preserving key of an fp32 score (larger float -> larger key); -0 is folded onto +0.
// ------------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// ------------------------------------------------------------------------------------------------
// Wave / block reductions
// ------------------------------------------------------------------------------------------------
// Cross-lane combines by lane swaps on the VALU (v_permlane32_swap / v_permlane16_swap, no LDS round trip).  With
// both operands equal to x, permlane32_swap returns (x[l & 31], x[(l & 31) + 32]) and permlane16_swap returns the
// even-row and odd-row values of each pair of 16-lane rows, so every lane gets its own and its partner's value;
// fp32 addition is commutative, so the sum equals own + partner in either lane of the pair.
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Inclusive prefix sum over the 64 lanes with DPP: Hillis-Steele shifts 1, 2, 4, 8 inside each 16-lane row (lanes
// shifted in from outside the row read 0), then row 1 and row 3 add the last lane of the row before them
// (row_bcast:15) and rows 2-3 add lane 31 (row_bcast:31).  Masked-off rows add the 0 passed as the old value.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace lca
