// gfx950.h -- small device helpers for the CDNA4 (gfx950) attention kernels:
// vector types for the bf16 matrix-core operands, LDS address-space casts,
// bf16 packing, and the half-wave exchange used by the row reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

#define ATTN_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 32x32x16 bf16 matrix FMA, fp32 accumulate.  Lane layout (checked on gfx950):
//   A (32 x 16):  lane l holds A[l % 32][8 * (l / 32) + e], e = 0..7
//   B (16 x 32):  lane l holds B[8 * (l / 32) + e][l % 32]
//   C (32 x 32):  lane l, register r holds C[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32]
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Two fp32 values to two bf16 (round to nearest even), packed into 32 bits.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

// acc + lo(p) + hi(p) for a packed bf16 pair: exact products by 1.0, fp32 sum.
__device__ __forceinline__ float add_bf16x2(uint32_t p, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p), one, acc, false);
}

// Value held by the lane in the other half of the wave (lane ^ 32), combined.
__device__ __forceinline__ float halfwave_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halfwave_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bool wave_any(bool p) {
  return __builtin_amdgcn_ballot_w64(p) != 0;
}

// 16-byte LDS read (ds_read_b128).
__device__ __forceinline__ bf16x8 lds_read_b128(const ATTN_LDS char* p) {
  return *(const ATTN_LDS bf16x8*)p;
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// output lane 16g+i, element e (e = 0..3) receives the 16-bit word at
// (address supplied by lane 16g + 4e + i/4) + 2*(i % 4) bytes.  With the
// source lanes pointing at four consecutive rows of a row-major bf16 matrix
// (lanes 4e..4e+3 of the group covering 16 consecutive columns of row e),
// every output lane gets one column's four row values.
__device__ __forceinline__ i16x4 lds_read_tr16(const ATTN_LDS char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)p);
}

}  // namespace attn
