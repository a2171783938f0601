// Device helpers shared by the gfx950 kernels: vector types, bf16 packing,
// MFMA wrappers, lane exchanges and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hsk {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kNegInf = -__builtin_huge_valf();

// ---------------------------------------------------------------- bf16 ----
__device__ __forceinline__ float bf16lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((unsigned)h << 16); }

// two fp32 -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32)
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  bf16x2 r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(unsigned, r);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float a) {
  __bf16 r = (__bf16)a;
  return __builtin_bit_cast(uint16_t, r);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  u32x4 t = {v.x, v.y, v.z, v.w};
  return __builtin_bit_cast(bf16x8, t);
}

// ----------------------------------------------------------------- MFMA ----
// 32x32x16 bf16 -> fp32.  Lane l: A[m = l%32][k = 8(l/32)+j], B[k = 8(l/32)+j][n = l%32],
// C/D register r: [m = 8(r/4) + 4(l/32) + r%4][n = l%32].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// 16x16x32 bf16 -> fp32.  Lane l: A[m = l%16][k = 8(l/16)+j], B[k = 8(l/16)+j][n = l%16],
// C/D register r: [m = 4(l/16) + r][n = l%16].
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16x16x16 bf16 -> fp32.  Lane l: A[m = l%16][k = 4(l/16)+j], B[k = 4(l/16)+j][n = l%16],
// C/D as for the 16x16x32 form.
__device__ __forceinline__ f32x4 mfma16k16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                   0, 0, 0);
}

// ------------------------------------------------------- lane exchanges ----
// value held by lane l ^ 32 (v_permlane32_swap).
__device__ __forceinline__ float xor32(float x) {
  unsigned u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  // lanes < 32 receive the upper half's value in r[1]; lanes >= 32 in r[0]
  return __uint_as_float((__lane_id() & 32) ? r[0] : r[1]);
}

// value held by lane l ^ 16 (v_permlane16_swap: rows of 16 lanes trade places
// pairwise; no LDS round trip, unlike a bpermute)
__device__ __forceinline__ float xor16(float x) {
  unsigned u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  // lanes in even rows receive the next row's value in r[1]; odd rows in r[0]
  return __uint_as_float((__lane_id() & 16) ? r[0] : r[1]);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
// DPP controls (gfx9): quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

// sum / max over each aligned group of 16 lanes; every lane receives the result
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  x += dpp<kDppMirror>(x);
  return x;
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp<kDppXor1>(x));
  x = fmaxf(x, dpp<kDppXor2>(x));
  x = fmaxf(x, dpp<kDppHalfMirror>(x));
  x = fmaxf(x, dpp<kDppMirror>(x));
  return x;
}

// whole-wave reductions (64 lanes); result in every lane
__device__ __forceinline__ float wave_max(float x) {
  x = row16_max(x);
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, xor32(x));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  x = row16_sum(x);
  x += __shfl_xor(x, 16);
  x += xor32(x);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace hsk
