// Generic HIP kernels of libnanokv: any supported dtype / head dimension.
//
// These serve the shapes the tuned MFMA kernels do not (fp32 tensors, head
// dimensions other than 128) and the rare low-dimensional rows whose score
// bound is too loose for the tuned kernel.  They compute in fp32 with plain
// wave-level loops: one wave per token (encode / decode) or per
// (query, head) row (attention).
#include <float.h>

#include <algorithm>

#include "kernels.hpp"
#include "quant.hpp"

namespace nkv {

// ---------------------------------------------------------------------------
// encode: nearest center (NanoKV abstract: shared cluster centers)
// ---------------------------------------------------------------------------
// One block of 256 threads per token; each wave scans a quarter of the
// centers with lanes striding the channels.  Distances are
// ||mu_a||^2 - 2 mu_a . x in fp64 (products of fp32 or bf16 values are
// exact in fp64), so near-ties resolve as exact arithmetic does; ties go to
// the lowest index.
template <int DT>
__global__ __launch_bounds__(256) void k_assign_generic(
    const void* __restrict__ x, int64_t N, int W, const void* __restrict__ centers,
    int A, int32_t* __restrict__ idx) {
  extern __shared__ float smem[];
  float* xs = smem;                 // W
  __shared__ double best_d[4];
  __shared__ int best_a[4];
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int w = threadIdx.x; w < W; w += 256) xs[w] = ld<DT>(x, t * W + w);
  __syncthreads();
  double bd = INFINITY;
  int ba = 0x7fffffff;
  for (int a = wave; a < A; a += 4) {
    double m2 = 0.0, dot = 0.0;
    for (int w = lane; w < W; w += 64) {
      const double m = ld<DT>(centers, (int64_t)a * W + w);
      m2 = fma(m, m, m2);
      dot = fma((double)xs[w], m, dot);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      m2 += __shfl_xor(m2, o, 64);
      dot += __shfl_xor(dot, o, 64);
    }
    const double dist = m2 - 2.0 * dot;
    if (dist < bd) { bd = dist; ba = a; }   // a increases: strict < keeps lowest
  }
  if (lane == 0) { best_d[wave] = bd; best_a[wave] = ba; }
  __syncthreads();
  if (threadIdx.x == 0) {
    double d0 = best_d[0];
    int a0 = best_a[0];
    for (int k = 1; k < 4; ++k) {
      if (best_d[k] < d0 || (best_d[k] == d0 && best_a[k] < a0)) { d0 = best_d[k]; a0 = best_a[k]; }
    }
    idx[t] = a0;
  }
}

// ---------------------------------------------------------------------------
// encode: residual, linear encoder, INT4 (Figure 4(b))
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(256) void k_project_quantize_generic(
    const void* __restrict__ x, int64_t N, int W, const void* __restrict__ centers,
    const int32_t* __restrict__ idx, const void* __restrict__ enc, int r, int group,
    uint8_t* __restrict__ codes, uint16_t* __restrict__ scales) {
  extern __shared__ float smem[];
  float* es = smem;        // W residual
  float* zs = smem + W;    // r coefficients
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int a = idx[t];
  for (int w = threadIdx.x; w < W; w += 256)
    es[w] = ld<DT>(x, t * W + w) - ld<DT>(centers, (int64_t)a * W + w);
  __syncthreads();
  for (int j = wave; j < r; j += 4) {
    float acc = 0.f;
    for (int w = lane; w < W; w += 64) acc = fmaf(ld<DT>(enc, (int64_t)j * W + w), es[w], acc);
    acc = wave_sum(acc);
    if (lane == 0) zs[j] = acc;
  }
  __syncthreads();
  const int ng = r / group;
  for (int gi = threadIdx.x; gi < ng; gi += 256)
    quantize_group(zs + gi * group, group, codes + t * (r / 2) + gi * (group / 2),
                   scales + t * ng + gi);
}

// ---------------------------------------------------------------------------
// decode of a compacted token list into fp32 rows (Figure 4(b))
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(256) void k_decode_generic(
    BranchArgs b, int W, int r, int group, RangeTable rows, float* __restrict__ out) {
  extern __shared__ float smem[];
  float* ch = smem;  // r dequantised coefficients
  const int64_t j = blockIdx.x;
  const int64_t t = map_index(rows, j);
  const uint8_t* crow = b.codes + t * (r / 2);
  const uint16_t* srow = b.scales + t * (r / group);
  for (int c = threadIdx.x; c < r; c += 256)
    ch[c] = (float)code_at(crow, c) * fp16_bits_to_f32(srow[c / group]);
  __syncthreads();
  const int a = b.idx[t];
  for (int w = threadIdx.x; w < W; w += 256) {
    float acc = ld<DT>(b.centers, (int64_t)a * W + w);
    for (int c = 0; c < r; ++c) acc = fmaf(ld<DT>(b.decoder, (int64_t)w * r + c), ch[c], acc);
    out[j * W + w] = acc;
  }
}

template <int DT>
__global__ void k_rows_to_f32(const void* __restrict__ src, int64_t n, float* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = ld<DT>(src, i);
}

// ---------------------------------------------------------------------------
// exact attention over fp32 keys/values, one wave per (query, head) row
// ---------------------------------------------------------------------------
template <int DT, bool OUT_F32>
__global__ __launch_bounds__(256) void k_attention_generic(
    const void* __restrict__ q, int64_t Nq, int H, int d, float tau,
    const float* __restrict__ K, const float* __restrict__ V, int64_t Nk,
    void* __restrict__ out, float* __restrict__ lse) {
  __shared__ float qs[4][128];
  __shared__ float ps[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  const bool valid = row < Nq * H;
  const int64_t qi = valid ? row / H : 0;
  const int h = valid ? (int)(row % H) : 0;
  const int W = H * d;
  for (int j = lane; j < d; j += 64) qs[wave][j] = valid ? ld<DT>(q, qi * W + h * d + j) : 0.f;
  __syncthreads();
  float m = -INFINITY, l = 0.f;
  float o0 = 0.f, o1 = 0.f;  // dims lane, lane + 64
  if (valid) {
    for (int64_t t0 = 0; t0 < Nk; t0 += 64) {
      const int64_t t = t0 + lane;
      float s = -INFINITY;
      if (t < Nk) {
        const float* kr = K + t * W + h * d;
        float acc = 0.f;
        for (int j = 0; j < d; ++j) acc = fmaf(qs[wave][j], kr[j], acc);
        s = acc * tau;
      }
      const float mn = fmaxf(m, wave_max(s));
      const float p = (t < Nk) ? expf(s - mn) : 0.f;
      const float sc = (m == -INFINITY) ? 0.f : expf(m - mn);
      l = l * sc + wave_sum(p);
      ps[wave][lane] = p;
      __builtin_amdgcn_wave_barrier();
      o0 *= sc;
      o1 *= sc;
      const int nt = (int)min<int64_t>(64, Nk - t0);
      for (int tt = 0; tt < nt; ++tt) {
        const float* vr = V + (t0 + tt) * W + h * d;
        const float pt = ps[wave][tt];
        if (lane < d) o0 = fmaf(pt, vr[lane], o0);
        if (lane + 64 < d) o1 = fmaf(pt, vr[lane + 64], o1);
      }
      __builtin_amdgcn_wave_barrier();
      m = mn;
    }
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
    const float L = (l > 0.f) ? m + logf(l) : -INFINITY;
    if (OUT_F32) {
      float* of = static_cast<float*>(out);
      if (lane < d) of[qi * W + h * d + lane] = o0 * inv;
      if (lane + 64 < d) of[qi * W + h * d + lane + 64] = o1 * inv;
    } else {
      if (lane < d) st<DT>(out, qi * W + h * d + lane, o0 * inv);
      if (lane + 64 < d) st<DT>(out, qi * W + h * d + lane + 64, o1 * inv);
    }
    if (lane == 0) lse[qi * H + h] = L;
  }
}

// ---------------------------------------------------------------------------
// NanoKV-Fast low-dimensional read (Figure 4(d)), one wave per (query, head)
// ---------------------------------------------------------------------------
// Two passes over the low-routed tokens: the first finds the exact score
// maximum, the second accumulates with it fixed, so the center-mass table in
// LDS never needs rescaling.  `rows` (optional) restricts the work to a list
// of row ids (query * H + head) whose count is *nrows.
template <int DT>
__global__ __launch_bounds__(64) void k_low_generic(
    const void* __restrict__ q, int64_t Nq, int H, int d, int r, int group, int r_low,
    float tau, BranchArgs kb, BranchArgs vb, LowMaps mp, RangeTable low,
    const int32_t* __restrict__ rows, const int32_t* __restrict__ nrows,
    float* __restrict__ o_low, float* __restrict__ lse_low) {
  extern __shared__ float smem[];
  float* T = smem;                       // A_k center scores (tau folded in)
  float* Wm = T + kb.A;                  // A_v center masses
  float* qt = Wm + vb.A;                 // r_low reduced query
  float* qh = qt + r_low;                // d query slice
  float* ps = qh + d;                    // 64 probabilities
  int* pv = reinterpret_cast<int*>(ps + 64);  // 64 history positions
  const int lane = threadIdx.x;
  const int64_t n_rows = rows ? (int64_t)*nrows : Nq * H;
  for (int64_t ri = blockIdx.x; ri < n_rows; ri += gridDim.x) {
  const int64_t row = rows ? (int64_t)rows[ri] : ri;
  const int64_t qi = row / H;
  const int h = (int)(row % H);
  const int W = H * d;
  const int64_t n = low.total;
  for (int j = lane; j < d; j += 64) qh[j] = ld<DT>(q, qi * W + h * d + j);
  __builtin_amdgcn_wave_barrier();
  for (int j = lane; j < r_low; j += 64) {
    float acc = 0.f;
    for (int i = 0; i < d; ++i) acc = fmaf(qh[i], ld<DT>(mp.qmap, (int64_t)(h * d + i) * mp.ld + j), acc);
    qt[j] = acc;
  }
  for (int a = lane; a < kb.A; a += 64) {
    float acc = 0.f;
    for (int i = 0; i < d; ++i) acc = fmaf(qh[i], ld<DT>(kb.centers, (int64_t)a * W + h * d + i), acc);
    T[a] = acc;
  }
  for (int a = lane; a < vb.A; a += 64) Wm[a] = 0.f;
  __builtin_amdgcn_wave_barrier();

  auto score = [&](int64_t t) -> float {
    const uint8_t* crow = kb.codes + t * (r / 2);
    const uint16_t* srow = kb.scales + t * (r / group);
    float acc = 0.f;
    for (int j = 0; j < r_low; ++j)
      acc = fmaf(qt[j], (float)code_at(crow, j) * fp16_bits_to_f32(srow[j / group]), acc);
    return tau * (acc + T[kb.idx[t]]);
  };

  float m = -INFINITY;
  for (int64_t j0 = 0; j0 < n; j0 += 64) {
    const int64_t j = j0 + lane;
    if (j < n) m = fmaxf(m, score(map_index(low, j)));
  }
  m = wave_max(m);

  float l = 0.f;
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  for (int64_t j0 = 0; j0 < n; j0 += 64) {
    const int64_t j = j0 + lane;
    float p = 0.f;
    int64_t t = 0;
    if (j < n) {
      t = map_index(low, j);
      p = expf(score(t) - m);
      atomicAdd(&Wm[vb.idx[t]], p);
    }
    ps[lane] = p;
    pv[lane] = (int)t;
    l += p;
    __builtin_amdgcn_wave_barrier();
    const int nt = (int)min<int64_t>(64, n - j0);
    for (int tt = 0; tt < nt; ++tt) {
      const int64_t tv = pv[tt];
      const float pt = ps[tt];
      const uint8_t* crow = vb.codes + tv * (r / 2);
      const uint16_t* srow = vb.scales + tv * (r / group);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int c = lane + 64 * k;
        if (c < r_low) acc[k] = fmaf(pt, (float)code_at(crow, c) * fp16_bits_to_f32(srow[c / group]), acc[k]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  l = wave_sum(l);
  // coefficient accumulators to LDS (reuse qt) for the restoration
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int c = lane + 64 * k;
    if (c < r_low) qt[c] = acc[k];
  }
  __builtin_amdgcn_wave_barrier();
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
  for (int i = lane; i < d; i += 64) {
    float val = 0.f;
    for (int c = 0; c < r_low; ++c) val = fmaf(ld<DT>(mp.omap, (int64_t)(h * d + i) * mp.ld + c), qt[c], val);
    for (int a = 0; a < vb.A; ++a) val = fmaf(Wm[a], ld<DT>(vb.centers, (int64_t)a * W + h * d + i), val);
    o_low[qi * W + h * d + i] = val * inv;
  }
  if (lane == 0) lse_low[qi * H + h] = (l > 0.f) ? m + logf(l) : -INFINITY;
  __builtin_amdgcn_wave_barrier();
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
#define NKV_DT_DISPATCH(dt, ...)                                  \
  do {                                                            \
    if ((dt) == NKV_F32) { constexpr int DT = NKV_F32; __VA_ARGS__; } \
    else { constexpr int DT = NKV_BF16; __VA_ARGS__; }            \
  } while (0)

nkv_status launch_encode_generic(int dt, const void* x, int64_t N, int W, const void* centers,
                                 int A, const void* enc, int r, int group, int32_t* idx,
                                 uint8_t* codes, uint16_t* scales, hipStream_t s) {
  if (N == 0) return NKV_OK;
  NKV_DT_DISPATCH(dt, {
    hipLaunchKernelGGL(k_assign_generic<DT>, dim3((unsigned)N), dim3(256), W * sizeof(float), s,
                       x, N, W, centers, A, idx);
    NKV_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_project_quantize_generic<DT>, dim3((unsigned)N), dim3(256),
                       (W + r) * sizeof(float), s, x, N, W, centers, idx, enc, r, group, codes,
                       scales);
    NKV_LAUNCH_CHECK();
  });
  return NKV_OK;
}

nkv_status launch_assign_generic(int dt, const void* x, int64_t N, int W, const void* centers,
                                 int A, int32_t* idx, hipStream_t s) {
  if (N == 0) return NKV_OK;
  NKV_DT_DISPATCH(dt, {
    hipLaunchKernelGGL(k_assign_generic<DT>, dim3((unsigned)N), dim3(256), W * sizeof(float), s,
                       x, N, W, centers, A, idx);
    NKV_LAUNCH_CHECK();
  });
  return NKV_OK;
}

nkv_status launch_decode_generic(int dt, const BranchArgs& b, int W, int r, int group,
                                 const RangeTable& rows, float* out, hipStream_t s) {
  if (rows.total == 0) return NKV_OK;
  NKV_DT_DISPATCH(dt, {
    hipLaunchKernelGGL(k_decode_generic<DT>, dim3((unsigned)rows.total), dim3(256),
                       r * sizeof(float), s, b, W, r, group, rows, out);
    NKV_LAUNCH_CHECK();
  });
  return NKV_OK;
}

nkv_status launch_rows_to_f32(int dt, const void* src, int64_t n, float* dst, hipStream_t s) {
  if (n == 0) return NKV_OK;
  NKV_DT_DISPATCH(dt, {
    hipLaunchKernelGGL(k_rows_to_f32<DT>, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s,
                       src, n, dst);
    NKV_LAUNCH_CHECK();
  });
  return NKV_OK;
}

nkv_status launch_attention_generic(int dt, bool out_f32, const void* q, int64_t Nq, int H,
                                    int d, float tau, const float* K, const float* V,
                                    int64_t Nk, void* out, float* lse, hipStream_t s) {
  if (Nq == 0) return NKV_OK;
  const unsigned grid = (unsigned)ceil_div(Nq * H, 4);
  NKV_DT_DISPATCH(dt, {
    if (out_f32)
      hipLaunchKernelGGL((k_attention_generic<DT, true>), dim3(grid), dim3(256), 0, s, q, Nq,
                         H, d, tau, K, V, Nk, out, lse);
    else
      hipLaunchKernelGGL((k_attention_generic<DT, false>), dim3(grid), dim3(256), 0, s, q, Nq,
                         H, d, tau, K, V, Nk, out, lse);
    NKV_LAUNCH_CHECK();
  });
  return NKV_OK;
}

size_t low_generic_lds_bytes(int A_k, int A_v, int r_low, int d) {
  return (size_t)(A_k + A_v + r_low + d + 64) * sizeof(float) + 64 * sizeof(int);
}

// rows (query * H + head) of the heads in `hs`, and their count
__global__ void k_head_rows(int64_t Nq, int H, HeadSet hs, int32_t* __restrict__ rows,
                            int32_t* __restrict__ nrows) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0) *nrows = (int32_t)(Nq * hs.n);
  if (i < Nq * hs.n) rows[i] = (int32_t)((i / hs.n) * H + hs.h[i % hs.n]);
}

nkv_status launch_head_rows(int64_t Nq, int H, const HeadSet& hs, int32_t* rows, int32_t* nrows,
                            hipStream_t s) {
  const int64_t n = std::max<int64_t>(Nq * hs.n, 1);
  hipLaunchKernelGGL(k_head_rows, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, Nq, H, hs,
                     rows, nrows);
  NKV_LAUNCH_CHECK();
  return NKV_OK;
}

nkv_status launch_low_generic(int dt, const void* q, int64_t Nq, int H, int d, int r, int group,
                              int r_low, float tau, const BranchArgs& kb, const BranchArgs& vb,
                              const LowMaps& mp, const RangeTable& low, const int32_t* rows,
                              const int32_t* nrows, int64_t max_rows, float* o_low,
                              float* lse_low, hipStream_t s) {
  if (max_rows == 0) return NKV_OK;
  const size_t lds = low_generic_lds_bytes(kb.A, vb.A, r_low, d);
  NKV_DT_DISPATCH(dt, {
    if (lds > 64 * 1024)
      NKV_HIP_CHECK(hipFuncSetAttribute((const void*)k_low_generic<DT>,
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
    const unsigned grid = (unsigned)std::min<int64_t>(max_rows, rows ? 4096 : max_rows);
    hipLaunchKernelGGL(k_low_generic<DT>, dim3(grid), dim3(64), lds, s, q, Nq, H,
                       d, r, group, r_low, tau, kb, vb, mp, low, rows, nrows, o_low, lse_low);
    NKV_LAUNCH_CHECK();
  });
  return NKV_OK;
}

}  // namespace nkv
