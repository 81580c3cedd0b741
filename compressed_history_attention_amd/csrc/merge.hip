// LSE merging of partial attentions (NanoKV pages, Figure 4(d): the
// low-dimensional part restores output dimensions before LSE merging).
//
// HBM-bound elementwise pass: one block per query row, the per-head weights
// computed once into LDS, then every channel of the row streamed once.
#include "kernels.hpp"
#include "mfma.hpp"

namespace nkv {

// Parts 0..n-1 are the slices p = 0..n-1 of (o_parts, lse_parts) with
// strides Nq W and Nq H; an optional extra part (o_x, lse_x) follows.
// L = logsumexp_p L_p; O = sum_p exp(L_p - L) O_p (a -inf part adds nothing).
// VEC: four channels per thread and step (d % 4 == 0, 16-byte aligned part
// rows, output rows aligned to four elements); otherwise one channel.
// No pointer is __restrict__: an fp32 output may be the same array as a
// part (every element is read and then written by the same thread), and
// lse_out the same array as a part's LSE (read before the block barrier,
// written after it, by the block that owns the row).
template <int DT, bool VEC>
__global__ __launch_bounds__(256) void k_lse_merge(int64_t Nq, int H, int d, int n,
                                                   const float* o_parts, const float* lse_parts,
                                                   const float* o_x, const float* lse_x, void* out,
                                                   float* lse_out) {
  extern __shared__ float sw[];  // weights [n + 1][H], L[H]
  const int np = n + (o_x ? 1 : 0);
  float* Ls = sw + (size_t)np * H;
  const int64_t qi = blockIdx.x;
  const int W = H * d;
  auto part_lse = [&](int p, int h) {
    return p < n ? lse_parts[((int64_t)p * Nq + qi) * H + h] : lse_x[qi * H + h];
  };
  for (int h = threadIdx.x; h < H; h += blockDim.x) {
    float mx = -INFINITY;
    for (int p = 0; p < np; ++p) mx = fmaxf(mx, part_lse(p, h));
    if (mx == -INFINITY) {
      for (int p = 0; p < np; ++p) sw[p * H + h] = 0.f;
      Ls[h] = -INFINITY;
    } else {
      float tot = 0.f;
      for (int p = 0; p < np; ++p) {
        const float e = expf(part_lse(p, h) - mx);
        sw[p * H + h] = e;
        tot += e;
      }
      for (int p = 0; p < np; ++p) sw[p * H + h] /= tot;
      Ls[h] = mx + logf(tot);
    }
  }
  __syncthreads();
  auto src_of = [&](int p, int c) {
    return p < n ? o_parts + ((int64_t)p * Nq + qi) * W + c : o_x + qi * W + c;
  };
  if constexpr (VEC) {
    // four channels (one head: d % 4 == 0) per thread and step
    for (int c = 4 * threadIdx.x; c < W; c += 4 * blockDim.x) {
      const int h = c / d;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      for (int p = 0; p < np; ++p) {
        const float wgt = sw[p * H + h];
        if (wgt > 0.f) {
          const f32x4 o = *reinterpret_cast<const f32x4*>(src_of(p, c));
#pragma unroll
          for (int u = 0; u < 4; ++u) v[u] += wgt * o[u];
        }
      }
      if constexpr (DT == NKV_F32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(out) + qi * W + c) = v;
      } else {
        uint16_t* ob = static_cast<uint16_t*>(out) + qi * W + c;
        *reinterpret_cast<uint2*>(ob) =
            uint2{uint32_t(f32_to_bf16_bits(v[0])) | (uint32_t(f32_to_bf16_bits(v[1])) << 16),
                  uint32_t(f32_to_bf16_bits(v[2])) | (uint32_t(f32_to_bf16_bits(v[3])) << 16)};
      }
    }
  } else {
    for (int c = threadIdx.x; c < W; c += blockDim.x) {
      const int h = c / d;
      float v = 0.f;
      for (int p = 0; p < np; ++p) {
        const float wgt = sw[p * H + h];
        if (wgt > 0.f) v += wgt * *src_of(p, c);
      }
      st<DT>(out, qi * W + c, v);
    }
  }
  __syncthreads();
  for (int h = threadIdx.x; h < H; h += blockDim.x) lse_out[qi * H + h] = Ls[h];
}

nkv_status launch_lse_merge_parts(int64_t Nq, int H, int d, int n, const float* o_parts,
                                  const float* lse_parts, const float* o_x, const float* lse_x,
                                  void* out, int out_dt, float* lse_out, hipStream_t s) {
  if (Nq == 0) return NKV_OK;
  const size_t lds = ((size_t)(n + 1) + 1) * H * sizeof(float);
  auto al = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; };
  const bool vec = d % 4 == 0 && al(o_parts, 16) && (!o_x || al(o_x, 16)) &&
                   al(out, out_dt == NKV_F32 ? 16 : 8);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)Nq), dim3(256), lds, s, Nq, H, d, n, o_parts,
                       lse_parts, o_x, lse_x, out, lse_out);
  };
  if (out_dt == NKV_F32) {
    if (vec) go(k_lse_merge<NKV_F32, true>);
    else go(k_lse_merge<NKV_F32, false>);
  } else {
    if (vec) go(k_lse_merge<NKV_BF16, true>);
    else go(k_lse_merge<NKV_BF16, false>);
  }
  NKV_LAUNCH_CHECK();
  return NKV_OK;
}

nkv_status launch_lse_merge(int64_t Nq, int H, int d, const float* o_a, const float* lse_a,
                            const float* o_b, const float* lse_b, void* out, int out_dt,
                            float* lse_out, hipStream_t s) {
  return launch_lse_merge_parts(Nq, H, d, 1, o_a, lse_a, o_b, lse_b, out, out_dt, lse_out, s);
}

}  // namespace nkv
