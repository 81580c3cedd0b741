// Shared device/host helpers of libnanokv (gfx950, HIP).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <hip/hip_fp16.h>

#include "../../include/nanokv.h"

namespace nkv {

// ---------------------------------------------------------------------------
// status plumbing (host)
// ---------------------------------------------------------------------------
void set_error(const char* fmt, ...);

#define NKV_HIP_CHECK(expr)                                              \
  do {                                                                   \
    hipError_t e_ = (expr);                                              \
    if (e_ != hipSuccess) {                                              \
      ::nkv::set_error("%s failed: %s", #expr, hipGetErrorString(e_));   \
      return NKV_EHIP;                                                   \
    }                                                                    \
  } while (0)

#define NKV_LAUNCH_CHECK()                                               \
  do {                                                                   \
    hipError_t e_ = hipGetLastError();                                   \
    if (e_ != hipSuccess) {                                              \
      ::nkv::set_error("kernel launch failed: %s", hipGetErrorString(e_)); \
      return NKV_EHIP;                                                   \
    }                                                                    \
  } while (0)

// ---------------------------------------------------------------------------
// history position tables: compacted index -> history position
// ---------------------------------------------------------------------------
struct RangeTable {
  int32_t n;                                  // number of ranges
  int64_t total;                              // sum of range lengths
  int64_t begin[NKV_MAX_SEGMENTS];
  int64_t prefix[NKV_MAX_SEGMENTS + 1];       // prefix[k] = start in compacted order
};

// The heads one launch serves (a group of equal low-dimensional width in a
// per-head call, or every head), passed by value in kernel arguments.
constexpr int NKV_MAX_HEADS = 128;
struct HeadSet {
  int32_t n;
  int32_t h[NKV_MAX_HEADS];
};

__device__ __forceinline__ int64_t map_index(const RangeTable& t, int64_t j) {
  int k = 0;
  while (k + 1 < t.n && t.prefix[k + 1] <= j) ++k;
  return t.begin[k] + (j - t.prefix[k]);
}

// ---------------------------------------------------------------------------
// element access
// ---------------------------------------------------------------------------
__host__ __device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  union { uint32_t u; float f; } c;
  c.u = uint32_t(b) << 16;
  return c.f;
}

// round-half-even float -> bfloat16 bits (finite inputs; NaN stays NaN)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

template <int DT>
__device__ __forceinline__ float ld(const void* p, int64_t i) {
  if constexpr (DT == NKV_F32) {
    return static_cast<const float*>(p)[i];
  } else {
    return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
  }
}

template <int DT>
__device__ __forceinline__ void st(void* p, int64_t i, float v) {
  if constexpr (DT == NKV_F32) {
    static_cast<float*>(p)[i] = v;
  } else {
    static_cast<uint16_t*>(p)[i] = f32_to_bf16_bits(v);
  }
}

__device__ __forceinline__ float fp16_bits_to_f32(uint16_t b) {
  return __half2float(__builtin_bit_cast(__half, b));
}

// signed INT4 coefficient j of a packed code row
__device__ __forceinline__ int code_at(const uint8_t* row, int j) {
  int byte = row[j >> 1];
  int nib = (j & 1) ? (byte >> 4) : (byte & 15);
  return nib - ((nib & 8) << 1);
}

// ---------------------------------------------------------------------------
// wave (64-lane) reductions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// order-preserving map float -> uint32 (for atomicMin/Max on floats)
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered_bits(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace nkv
