// LSE merging of partial attentions (NanoKV pages, Figure 4(d): the
// low-dimensional part restores output dimensions before LSE merging).
//
// HBM-bound elementwise pass: one block per query row, the per-head weights
// computed once into LDS, then every channel of the row streamed once.
#include "kernels.hpp"

namespace nkv {

template <int DT>
__global__ __launch_bounds__(256) void k_lse_merge(int H, int d, const float* __restrict__ o_a,
                                                   const float* __restrict__ lse_a,
                                                   const float* __restrict__ o_b,
                                                   const float* __restrict__ lse_b,
                                                   void* __restrict__ out,
                                                   float* __restrict__ lse_out) {
  extern __shared__ float sw[];  // wa[H], wb[H], L[H]
  float* wa = sw;
  float* wb = sw + H;
  float* Ls = sw + 2 * H;
  const int64_t qi = blockIdx.x;
  const int W = H * d;
  for (int h = threadIdx.x; h < H; h += blockDim.x) {
    const float la = lse_a[qi * H + h], lb = lse_b[qi * H + h];
    const float mx = fmaxf(la, lb);
    if (mx == -INFINITY) {
      wa[h] = 0.f; wb[h] = 0.f; Ls[h] = -INFINITY;
    } else {
      const float ea = expf(la - mx), eb = expf(lb - mx);
      const float tot = ea + eb;
      wa[h] = ea / tot;
      wb[h] = eb / tot;
      Ls[h] = mx + logf(tot);
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < W; c += blockDim.x) {
    const int h = c / d;
    const float va = wa[h] > 0.f ? o_a[qi * W + c] : 0.f;
    const float vb = wb[h] > 0.f ? o_b[qi * W + c] : 0.f;
    st<DT>(out, qi * W + c, wa[h] * va + wb[h] * vb);
  }
  __syncthreads();
  for (int h = threadIdx.x; h < H; h += blockDim.x) lse_out[qi * H + h] = Ls[h];
}

nkv_status launch_lse_merge(int64_t Nq, int H, int d, const float* o_a, const float* lse_a,
                            const float* o_b, const float* lse_b, void* out, int out_dt,
                            float* lse_out, hipStream_t s) {
  if (Nq == 0) return NKV_OK;
  const size_t lds = 3 * (size_t)H * sizeof(float);
  if (out_dt == NKV_F32)
    hipLaunchKernelGGL(k_lse_merge<NKV_F32>, dim3((unsigned)Nq), dim3(256), lds, s, H, d, o_a,
                       lse_a, o_b, lse_b, out, lse_out);
  else
    hipLaunchKernelGGL(k_lse_merge<NKV_BF16>, dim3((unsigned)Nq), dim3(256), lds, s, H, d, o_a,
                       lse_a, o_b, lse_b, out, lse_out);
  NKV_LAUNCH_CHECK();
  return NKV_OK;
}

}  // namespace nkv
