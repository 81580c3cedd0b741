// CDNA4 (gfx950) matrix-core helpers.
//
// v_mfma_f32_32x32x16_{bf16,f16}: one wave computes a 32x32 fp32 tile from
// A (32 x 16) and B (16 x 32).  Operand convention used throughout: lane l
// supplies row/column (l % 32) and the 8 consecutive logical k values
// 8*(l/32) .. 8*(l/32)+7.  Any fixed assignment of (lane half, element) to
// k gives the same product as long as A and B agree, which they always do
// here.  Accumulator layout: element i of lane l holds
//   row = (i/4)*8 + (l/32)*4 + (i%4),   col = l % 32.
#pragma once

#include "nkv_common.hpp"

namespace nkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int acc_row(int i, int lane) {
  return (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// bit casts between 16-byte vectors
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16 pair (round-half-even, v_cvt_pk_bf16_f32), low half = a
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  _Float16 ha = (_Float16)a, hb = (_Float16)b;
  return uint32_t(__builtin_bit_cast(uint16_t, ha)) | (uint32_t(__builtin_bit_cast(uint16_t, hb)) << 16);
}

__device__ __forceinline__ u32x4 ld_u32x4(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

}  // namespace nkv
