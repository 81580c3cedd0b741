// Tiled bf16 MFMA GEMM skeleton with pluggable operand loaders and
// epilogues:  C[z](m, n) = sum_k A[z](m, k) * B[z](n, k), fp32 accumulation.
//
// Block: 256 threads (4 waves) computing a 128 x 128 tile; wave w owns the
// 64 x 64 quadrant (w / 2, w % 2) as 2 x 2 MFMA 32x32 tiles.  K advances in
// steps of P::BK (32 or 64) through a register-staged, double-buffered LDS
// pipeline.  A problem type P supplies
//   static constexpr int BK;                       (32: more blocks per CU,
//                                                   64: fewer barriers)
//   int M, N, K;                                   (K % 8 == 0)
//   __device__ u32x4 load_a(int z, int m, int k) const;  // 8 k values (bf16)
//   __device__ u32x4 load_b(int z, int n, int k) const;  //   zero if out of range
//   __device__ void epilogue(int z, int m0, int n0, int lane, const f32x16 (&acc)[2][2]) const;
// epilogue receives the wave's 64 x 64 quadrant origin (m0, n0); acc[i][j]
// covers rows m0 + 32 i .., columns n0 + 32 j .. in the MFMA layout.
#pragma once

#include "mfma.hpp"

namespace nkv {

constexpr int GEMM_BM = 128, GEMM_BN = 128;

template <class P>
__global__ __launch_bounds__(256) void k_gemm(const P p) {
  constexpr int GEMM_BK = P::BK;
  constexpr int GEMM_LDS_STRIDE = GEMM_BK + 8;  // bf16 elements per LDS row
  constexpr int GEMM_LD = GEMM_BM * GEMM_BK / 8 / 256;  // 8-value chunks per thread per operand
  constexpr int TPR = GEMM_BK / 8;                       // threads per tile row
  static_assert(GEMM_BK == 32 || GEMM_BK == 64, "K step");
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][GEMM_BM * GEMM_LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][GEMM_BN * GEMM_LDS_STRIDE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int z = blockIdx.z;
  const int m_blk = blockIdx.y * GEMM_BM, n_blk = blockIdx.x * GEMM_BN;
  // global -> register staging: each thread moves GEMM_LD chunks of 8 k for A
  // and for B: rows ld_row0 + (256 / TPR) j, k offset ld_k
  const int ld_row0 = tid / TPR, ld_k = (tid % TPR) * 8;
  u32x4 ra[GEMM_LD], rb[GEMM_LD];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int j = 0; j < GEMM_LD; ++j) {
      ra[j] = p.load_a(z, m_blk + ld_row0 + (256 / TPR) * j, k0 + ld_k);
      rb[j] = p.load_b(z, n_blk + ld_row0 + (256 / TPR) * j, k0 + ld_k);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int j = 0; j < GEMM_LD; ++j) {
      *reinterpret_cast<u32x4*>(&sA[buf][(ld_row0 + (256 / TPR) * j) * GEMM_LDS_STRIDE + ld_k]) = ra[j];
      *reinterpret_cast<u32x4*>(&sB[buf][(ld_row0 + (256 / TPR) * j) * GEMM_LDS_STRIDE + ld_k]) = rb[j];
    }
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = zero16();
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int nk = (p.K + GEMM_BK - 1) / GEMM_BK;
  fetch(0);
  stash(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) fetch((kt + 1) * GEMM_BK);
#pragma unroll
    for (int ks = 0; ks < GEMM_BK; ks += 16) {
      bf16x8 fa[2], fb[2];
      const int kk = ks + 8 * (lane >> 5);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        fa[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(
            &sA[buf][(wm + 32 * i + (lane & 31)) * GEMM_LDS_STRIDE + kk]));
        fb[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(
            &sB[buf][(wn + 32 * i + (lane & 31)) * GEMM_LDS_STRIDE + kk]));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma_bf16(fa[i], fb[j], acc[i][j]);
    }
    if (kt + 1 < nk) {
      stash(buf ^ 1);
      __syncthreads();
    }
  }
  p.epilogue(z, m_blk + wm, n_blk + wn, lane, acc);
}

template <class P>
inline nkv_status launch_gemm(const P& p, int batch, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0 || batch <= 0) return NKV_OK;
  dim3 grid((unsigned)ceil_div(p.N, GEMM_BN), (unsigned)ceil_div(p.M, GEMM_BM), (unsigned)batch);
  hipLaunchKernelGGL(k_gemm<P>, grid, dim3(256), 0, s, p);
  NKV_LAUNCH_CHECK();
  return NKV_OK;
}

}  // namespace nkv
