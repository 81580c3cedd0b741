// Center fitting of libnanokv: the update step of Lloyd's k-means.
//
// The NanoKV page fits shared centers separately per K/V branch (Table 5
// caption: 64 centers) without printing the procedure; the library offers
// Lloyd iterations from caller-given centers.  The assignment step is the
// encoder's own nearest-center search; this file holds the update: every
// center that received tokens becomes their mean, stored in the codec dtype.
//
// The update sorts the rows by their center (counting sort: counts, prefix
// sums, scatter of row ids), then one block per (center, 512 columns) sums
// its rows in fp64 and writes the mean: every row is read once and no float
// atomics are needed.  The scatter order within a center varies from run to
// run, but an fp64 sum of bf16 rows (8 significant bits each) is exact, and
// so order-independent, while the addends and partial sums span at most 53
// bits; otherwise only the last bits of the fp64 sum move, which the
// rounding to the storage dtype hides unless the mean lies that close to a
// rounding boundary.  The mean is rounded once to the storage dtype: fp64 ->
// fp32 with round-to-odd, then fp32 -> bf16 round-half-to-even, which equals
// a single round-half-to-even from fp64 (Boldo and Melquiond, "Emulation of
// FMA and correctly rounded sums: proved algorithms using rounding to odd",
// 2008).
#include "kernels.hpp"

namespace nkv {

__global__ void k_fit_zero(int32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

__global__ void k_fit_count(const int32_t* __restrict__ idx, int64_t N, int32_t* __restrict__ counts) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < N) atomicAdd(counts + idx[i], 1);
}

// exclusive prefix sums of the counts (one block of 1024 threads): row
// offsets per center and the scatter cursors
__global__ __launch_bounds__(1024) void k_fit_scan(const int32_t* __restrict__ counts, int A,
                                                   int32_t* __restrict__ offs,
                                                   int32_t* __restrict__ cursor) {
  __shared__ int32_t part[1024];
  const int per = (A + 1023) / 1024;
  const int a0 = threadIdx.x * per;
  int32_t s = 0;
  for (int a = a0; a < a0 + per && a < A; ++a) s += counts[a];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int st = 1; st < 1024; st <<= 1) {  // Hillis-Steele inclusive scan
    const int32_t v = threadIdx.x >= st ? part[threadIdx.x - st] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int32_t run = part[threadIdx.x] - s;
  for (int a = a0; a < a0 + per && a < A; ++a) {
    offs[a] = run;
    cursor[a] = run;
    run += counts[a];
  }
  if (threadIdx.x == 1023) offs[A] = part[1023];
}

__global__ void k_fit_scatter(const int32_t* __restrict__ idx, int64_t N,
                              int32_t* __restrict__ cursor, int32_t* __restrict__ perm) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < N) perm[atomicAdd(cursor + idx[i], 1)] = (int32_t)i;
}

// fp64 -> fp32 rounding to odd: truncate toward zero, then force the last
// bit to 1 when the truncation was inexact
__device__ __forceinline__ float f64_to_f32_odd(double v) {
  float f = (float)v;  // round-half-even
  if (fabs((double)f) > fabs(v)) f = __uint_as_float(__float_as_uint(f) - 1u);  // toward zero
  if ((double)f != v) f = __uint_as_float(__float_as_uint(f) | 1u);
  return f;
}

// 8 consecutive values of a row in their stored form (16 or 32 bytes)
template <int DT>
struct Raw8 {
  uint4 v[DT == NKV_F32 ? 2 : 1];
};

template <int DT>
__device__ __forceinline__ Raw8<DT> load_raw8(const void* x, int64_t off) {
  Raw8<DT> r;
  if constexpr (DT == NKV_F32) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(x) + off);
    r.v[0] = p[0];
    r.v[1] = p[1];
  } else {
    r.v[0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + off);
  }
  return r;
}

template <int DT>
__device__ __forceinline__ void add8(const Raw8<DT>& r, double (&s)[8]) {
  if constexpr (DT == NKV_F32) {
    const uint32_t u[8] = {r.v[0].x, r.v[0].y, r.v[0].z, r.v[0].w,
                           r.v[1].x, r.v[1].y, r.v[1].z, r.v[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] += (double)__uint_as_float(u[i]);
  } else {
    const uint32_t u[4] = {r.v[0].x, r.v[0].y, r.v[0].z, r.v[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[2 * i] += (double)bf16_bits_to_f32(uint16_t(u[i] & 0xffffu));
      s[2 * i + 1] += (double)bf16_bits_to_f32(uint16_t(u[i] >> 16));
    }
  }
}

// grid (centers, column blocks of 512): the 4 waves of a block take every
// 4th row of the center, eight rows in flight per wave (row ids fetched 64
// at a time, one per lane, and broadcast), each lane 8 consecutive columns
// with 16-byte loads; the wave partials are added in a fixed order through
// LDS and the mean is written.  An empty center is left alone.
// W % 8 == 0 (H * d with d >= 16).
template <int DT>
__global__ __launch_bounds__(256) void k_fit_mean(const void* __restrict__ x, int W,
                                                  const int32_t* __restrict__ offs,
                                                  const int32_t* __restrict__ perm,
                                                  void* __restrict__ centers) {
  __shared__ double red[3][64][8];
  const int a = blockIdx.x;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int w = blockIdx.y * 512 + lane * 8;
  const int k0 = offs[a], k1 = offs[a + 1];
  if (k1 == k0) return;  // block-uniform
  const bool col_ok = w < W;
  const int wc = col_ok ? w : 0;
  double s[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) s[i] = 0.0;
  // this wave's rows: k0 + wv + 4 j
  const int nrow = (k1 - k0 - wv + 3) / 4;
  for (int j0 = 0; j0 < nrow; j0 += 64) {
    const int jl = j0 + lane;
    const int my_row = jl < nrow ? perm[k0 + wv + 4 * jl] : 0;
    const int nb = min(64, nrow - j0);
    int j = 0;
    for (; j + 8 <= nb; j += 8) {
      Raw8<DT> r[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int row = __shfl(my_row, j + u, 64);
        r[u] = load_raw8<DT>(x, (int64_t)row * W + wc);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) add8<DT>(r[u], s);
    }
    for (; j < nb; ++j) {
      const int row = __shfl(my_row, j, 64);
      add8<DT>(load_raw8<DT>(x, (int64_t)row * W + wc), s);
    }
  }
  if (wv > 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) red[wv - 1][lane][i] = s[i];
  }
  __syncthreads();
  if (wv > 0 || !col_ok) return;
  const double n = (double)(k1 - k0);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double m = (((s[i] + red[0][lane][i]) + red[1][lane][i]) + red[2][lane][i]) / n;
    const int64_t o = (int64_t)a * W + w + i;
    if constexpr (DT == NKV_F32) {
      static_cast<float*>(centers)[o] = (float)m;
    } else {
      static_cast<uint16_t*>(centers)[o] = f32_to_bf16_bits(f64_to_f32_odd(m));
    }
  }
}

nkv_status launch_fit_counts(const int32_t* idx, int64_t N, int A, int32_t* counts,
                             hipStream_t s) {
  hipLaunchKernelGGL(k_fit_zero, dim3((unsigned)ceil_div(A, 256)), dim3(256), 0, s, counts,
                     (int64_t)A);
  NKV_LAUNCH_CHECK();
  if (N == 0) return NKV_OK;
  hipLaunchKernelGGL(k_fit_count, dim3((unsigned)ceil_div(N, 256)), dim3(256), 0, s, idx, N,
                     counts);
  NKV_LAUNCH_CHECK();
  return NKV_OK;
}

nkv_status launch_fit_update(int dt, const void* x, int64_t N, int W, const int32_t* idx, int A,
                             int32_t* counts, int32_t* offs, int32_t* cursor, int32_t* perm,
                             void* centers, hipStream_t s) {
  if (N == 0) return NKV_OK;
  nkv_status e;
  if ((e = launch_fit_counts(idx, N, A, counts, s))) return e;
  hipLaunchKernelGGL(k_fit_scan, dim3(1), dim3(1024), 0, s, counts, A, offs, cursor);
  NKV_LAUNCH_CHECK();
  hipLaunchKernelGGL(k_fit_scatter, dim3((unsigned)ceil_div(N, 256)), dim3(256), 0, s, idx, N,
                     cursor, perm);
  NKV_LAUNCH_CHECK();
  const dim3 grid((unsigned)A, (unsigned)ceil_div(W, 512));
  if (dt == NKV_F32)
    hipLaunchKernelGGL(k_fit_mean<NKV_F32>, grid, dim3(256), 0, s, x, W, offs, perm, centers);
  else
    hipLaunchKernelGGL(k_fit_mean<NKV_BF16>, grid, dim3(256), 0, s, x, W, offs, perm, centers);
  NKV_LAUNCH_CHECK();
  return NKV_OK;
}

}  // namespace nkv
