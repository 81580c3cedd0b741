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

// The same tile and LDS double buffer with the global loads two K steps
// ahead instead of one (two register sets): step kt computes from LDS while
// the loads of step kt + 2 are in flight and step kt + 1 waits in registers
// for the buffer step kt - 1 freed.  For long K with global latency that one
// step's MFMAs do not cover (P::BK == 64).
// Block order of a 1-D grid for a short M (the centers) and a long N (the
// tokens).  N tiles slowest would stream all of B once per M tile.  Here
// the hardware deals consecutive blocks to the 8 XCDs in turn (block b runs
// on XCD b % 8), and with G > 0 the M tiles form mt / G groups of G, each
// group served by 8 / (mt / G) XCDs that split the N tiles between them:
// an XCD runs its N tiles in order, the G blocks of one N tile together, so
// the N tile's B rows are fetched into its L2 once for G products and its
// G M tiles of A rows stay resident; B is read 8 / G times in all.  G = 0:
// M tiles fastest in plain order.
struct TileOrder {
  int mt, nt;   // M and N tiles
  int G;        // M tiles per group, or 0
  int ng, xpg;  // groups; XCDs per group (ng * xpg = 8)
  int blocks;   // grid size (grouped: whole rounds of every XCD, some empty)
  __device__ bool map(int b, int& m_t, int& n_t) const {
    if (G == 0) {
      m_t = b % mt;
      n_t = b / mt;
      return true;
    }
    const int x = b & 7, i = b >> 3;
    n_t = (i / G) * xpg + x / ng;
    m_t = (x % ng) * G + i % G;
    return n_t < nt;
  }
};

// the grouping for mt x nt tiles: the largest G <= gmax that divides mt
// with mt / G dividing 8, else plain order
inline TileOrder make_tile_order(int64_t mt, int64_t nt, int gmax) {
  TileOrder o{(int)mt, (int)nt, 0, 1, 8, (int)(mt * nt)};
  for (int64_t G = std::min<int64_t>(gmax, mt); G >= 2; --G)
    if (mt % G == 0 && 8 % (mt / G) == 0) {
      o.G = (int)G;
      o.ng = (int)(mt / G);
      o.xpg = 8 / o.ng;
      o.blocks = (int)(8 * ((nt + o.xpg - 1) / o.xpg) * G);
      break;
    }
  return o;
}

template <class P>
__global__ __launch_bounds__(256) void k_gemm_pf2(const P p, const TileOrder o) {
  constexpr int BK = P::BK;
  static_assert(BK == 64, "K step");
  constexpr int LS = BK + 8;              // bf16 elements per LDS row
  constexpr int LD = GEMM_BM * BK / 8 / 256;  // 8-value chunks per thread per operand
  constexpr int TPR = BK / 8;
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][GEMM_BM * LS];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][GEMM_BN * LS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int z = blockIdx.z;
  int m_t, n_t;
  if (!o.map((int)blockIdx.x, m_t, n_t)) return;  // the whole block, before any barrier
  const int m_blk = m_t * GEMM_BM, n_blk = n_t * GEMM_BN;
  const int ld_row0 = tid / TPR, ld_k = (tid % TPR) * 8;
  u32x4 ra[2][LD], rb[2][LD];
  auto fetch = [&](int set, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < LD; ++j) {
      ra[set][j] = p.load_a(z, m_blk + ld_row0 + (256 / TPR) * j, k0 + ld_k);
      rb[set][j] = p.load_b(z, n_blk + ld_row0 + (256 / TPR) * j, k0 + ld_k);
    }
  };
  auto stash = [&](int set, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < LD; ++j) {
      *reinterpret_cast<u32x4*>(&sA[buf][(ld_row0 + (256 / TPR) * j) * LS + ld_k]) = ra[set][j];
      *reinterpret_cast<u32x4*>(&sB[buf][(ld_row0 + (256 / TPR) * j) * LS + ld_k]) = rb[set][j];
    }
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = zero16();
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int nk = (p.K + BK - 1) / BK;
  fetch(0, 0);
  fetch(1, min(1, nk - 1) * BK);
  stash(0, 0);
  __syncthreads();
  auto mm = [&](int cur) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < BK; ks += 16) {
      bf16x8 fa[2], fb[2];
      const int kk = ks + 8 * (lane >> 5);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        fa[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(&sA[cur][(wm + 32 * i + (lane & 31)) * LS + kk]));
        fb[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(&sB[cur][(wn + 32 * i + (lane & 31)) * LS + kk]));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma_bf16(fa[i], fb[j], acc[i][j]);
    }
  };
  // a step with a successor: step kt + 2's loads go into the register set
  // step kt emptied into LDS buffer cur (the final steps reload the last
  // tile), the MFMAs read buffer cur, then step kt + 1 moves from the other
  // register set into the other buffer
  auto step = [&](int kt, int cur) __attribute__((always_inline)) {
    fetch(cur, min(kt + 2, nk - 1) * BK);
    mm(cur);
    stash(cur ^ 1, cur ^ 1);
    __syncthreads();
  };
  // two steps per trip (static register sets and buffers) in straight-line
  // code: the same memory operations on every trip let the compiler's waits
  // leave the newest loads in flight
  int kt = 0;
  for (; kt + 2 < nk; kt += 2) {
    step(kt, 0);
    step(kt + 1, 1);
  }
  if (nk - kt == 2) {
    step(kt, 0);
    mm(1);
  } else {
    mm(0);
  }
  p.epilogue(z, m_blk + wm, n_blk + wn, lane, acc);
}

// gmax: the largest M-tile group of the block order (0 or 1: plain order)
template <class P>
inline nkv_status launch_gemm_pf2(const P& p, int batch, hipStream_t s, int gmax) {
  if (p.M <= 0 || p.N <= 0 || batch <= 0) return NKV_OK;
  const int64_t mt = ceil_div(p.M, GEMM_BM), nt = ceil_div(p.N, GEMM_BN);
  if (mt * nt > (int64_t)1 << 30) return NKV_EUNSUPPORTED;  // a grid of whole XCD rounds stays < 2^31
  const TileOrder o = make_tile_order(mt, nt, gmax);
  dim3 grid((unsigned)o.blocks, 1, (unsigned)batch);
  hipLaunchKernelGGL(k_gemm_pf2<P>, grid, dim3(256), 0, s, p, o);
  NKV_LAUNCH_CHECK();
  return NKV_OK;
}

// The same tile (128 x 128, 4 waves of 64 x 64) for problems whose operands
// are plain bf16 rows: K % 32 == 0 and P supplies
//   __device__ const uint16_t* a_ptr(int z, int m, int k) const;  // &A[z](m, k), 8-aligned k
//   __device__ const uint16_t* b_ptr(int z, int n, int k) const;  // &B[z](n, k)
// (rows m < M, n < N; a k step of 32 never crosses a change of source).
// K steps of 32 move by direct-to-LDS loads (1 KiB per wave instruction,
// no staging registers) through a ring of 4 stages, three steps ahead of the
// MFMAs.  Within a stage each operand is 128 rows of 64 bytes; 16-byte block
// j of row r sits at block j ^ ((r >> 2) & 3), so the 32 rows an MFMA
// operand read touches spread over all banks.  Rows past M or N load row
// M - 1 or N - 1 (finite values whose products only reach discarded
// outputs).
constexpr int GD_BK = 32, GD_STAGES = 4;
// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8; all-ones = no wait on that counter)
constexpr int GD_WAIT_VM8 = 8 | (7 << 4) | (15 << 8);           // vmcnt(8)
constexpr int GD_WAIT_VM4 = 4 | (7 << 4) | (15 << 8);           // vmcnt(4)
constexpr int GD_WAIT_LGKM0 = 15 | (7 << 4) | (0 << 8) | (3 << 14);  // lgkmcnt(0)
constexpr int GD_OP = 128 * GD_BK * 2;  // bytes of one operand tile per stage

// Lane state of the direct-to-LDS loads: chunk c = wave + 4 j (j < 2) of
// each operand holds slots 64 c .. 64 c + 63 of a stage, slot s = row 4 r +
// physical block; the lane loads row r of that chunk, logical k block kblk.
struct GdLanes {
  int wave, arow[2], brow[2], kblk[2];
};

// stage kt into dS (A tile at offset 0, B tile at GD_OP); stages past the
// end reload the last one (the ring then issues the same loads on every
// path, which lets the compiler's own waits match the counts in k_gemm_dma;
// their data is never read)
template <class P>
__device__ __forceinline__ void gd_load(const P& p, int z, const GdLanes& L, int kt, int nk,
                                        char* dS) {
  const int k0 = min(kt, nk - 1) * GD_BK;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = L.wave + 4 * j;
    // (sources as plain pointers: a builtin call whose arguments depend on
    // P would be rejected by the host pass of this template)
    const void* sa = p.a_ptr(z, L.arow[j], k0 + 8 * L.kblk[j]);
    const void* sb = p.b_ptr(z, L.brow[j], k0 + 8 * L.kblk[j]);
    __builtin_amdgcn_global_load_lds(sa, (__attribute__((address_space(3))) void*)(dS + c * 1024),
                                     16, 0, 0);
    __builtin_amdgcn_global_load_lds(
        sb, (__attribute__((address_space(3))) void*)(dS + GD_OP + c * 1024), 16, 0, 0);
  }
}

__device__ __forceinline__ bf16x8 gd_frag(const char* base, int r, int b) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(base + r * 64 + ((b ^ ((r >> 2) & 3)) << 4)));
}

// operand fragments of a stage for the wave's 64 x 64 quadrant (wm, wn)
struct GdFrags {
  bf16x8 a[GD_BK / 16][2], b[GD_BK / 16][2];
};
__device__ __forceinline__ void gd_read(const char* cS, int lane, int wm, int wn, GdFrags& f) {
  const int hl = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < GD_BK / 16; ++ks)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      f.a[ks][i] = gd_frag(cS, wm + 32 * i + (lane & 31), 2 * ks + hl);
      f.b[ks][i] = gd_frag(cS + GD_OP, wn + 32 * i + (lane & 31), 2 * ks + hl);
    }
}

// step kt, with stage kt's fragments already in `cur`: wait for stage kt + 1
// (nS1), load stage kt + 3 into nS3, read stage kt + 1's fragments into
// `nxt` while the MFMAs of stage kt run
template <class P>
__device__ __forceinline__ void gd_step(const P& p, int z, const GdLanes& L, int lane, int wm,
                                        int wn, int kt, int nk, const char* nS1, char* nS3,
                                        const GdFrags& cur, GdFrags& nxt, f32x16 (&acc)[2][2]) {
  // stage kt + 1 has landed once at most the next stage's loads (4 per wave)
  // are outstanding (the builtin, unlike inline asm, is seen by the
  // compiler's own wait placement, which then adds none before the reads
  // below) ...
  __builtin_amdgcn_s_waitcnt(GD_WAIT_VM4);
  // ... in every wave, and every wave's reads of stage kt (read during the
  // step before) have returned, so the stage loaded next (kt + 3, the ring
  // slot of kt - 1) is free.  A bare barrier: the fence of __syncthreads
  // would wait for every load in flight
  __builtin_amdgcn_s_waitcnt(GD_WAIT_LGKM0);
  __builtin_amdgcn_s_barrier();
  gd_load(p, z, L, kt + GD_STAGES - 1, nk, nS3);
  __builtin_amdgcn_sched_barrier(0);
  gd_read(nS1, lane, wm, wn, nxt);
  // steps past the end multiply zeros (no branch around the MFMAs: the same
  // straight line on every path)
  const bool live = kt < nk;
#pragma unroll
  for (int ks = 0; ks < GD_BK / 16; ++ks) {
    bf16x8 fa[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) fa[i] = live ? cur.a[ks][i] : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma_bf16(fa[i], cur.b[ks][j], acc[i][j]);
  }
}

template <class P>
__global__ __launch_bounds__(256) void k_gemm_dma(const P p) {
  // one array per stage: the stage of every LDS access is static (the loop
  // below is unrolled by the ring size), so the compiler can see that
  // reading one stage does not alias the loads in flight into another
  __shared__ __attribute__((aligned(1024))) char s0[2 * GD_OP];
  __shared__ __attribute__((aligned(1024))) char s1[2 * GD_OP];
  __shared__ __attribute__((aligned(1024))) char s2[2 * GD_OP];
  __shared__ __attribute__((aligned(1024))) char s3[2 * GD_OP];
  static_assert(GD_STAGES == 4, "ring of four stages");
  const int tid = threadIdx.x, lane = tid & 63;
  const int z = blockIdx.z;
  const int m_blk = blockIdx.y * GEMM_BM, n_blk = blockIdx.x * GEMM_BN;
  const int nk = p.K / GD_BK;  // >= 1
  GdLanes L;
  L.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int sl = (L.wave + 4 * j) * 64 + lane, r = sl >> 2;
    L.kblk[j] = (sl & 3) ^ ((r >> 2) & 3);
    L.arow[j] = min(m_blk + r, p.M - 1);
    L.brow[j] = min(n_blk + r, p.N - 1);
  }
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = zero16();
  const int wm = (L.wave >> 1) * 64, wn = (L.wave & 1) * 64;
  gd_load(p, z, L, 0, nk, s0);
  gd_load(p, z, L, 1, nk, s1);
  gd_load(p, z, L, 2, nk, s2);
  GdFrags f0, f1;
  __builtin_amdgcn_s_waitcnt(GD_WAIT_VM8);  // stage 0 (two newer stages in flight)
  __builtin_amdgcn_s_barrier();
  gd_read(s0, lane, wm, wn, f0);
  for (int kt = 0; kt < nk; kt += 4) {
    gd_step(p, z, L, lane, wm, wn, kt, nk, s1, s3, f0, f1, acc);
    gd_step(p, z, L, lane, wm, wn, kt + 1, nk, s2, s0, f1, f0, acc);
    gd_step(p, z, L, lane, wm, wn, kt + 2, nk, s3, s1, f0, f1, acc);
    gd_step(p, z, L, lane, wm, wn, kt + 3, nk, s0, s2, f1, f0, acc);
  }
  // no load may still be in flight into LDS when the block ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
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

template <class P>
inline nkv_status launch_gemm_dma(const P& p, int batch, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0 || batch <= 0) return NKV_OK;
  if (p.K < GD_BK || p.K % GD_BK != 0) return launch_gemm(p, batch, s);
  dim3 grid((unsigned)ceil_div(p.N, GEMM_BN), (unsigned)ceil_div(p.M, GEMM_BM), (unsigned)batch);
  hipLaunchKernelGGL(k_gemm_dma<P>, grid, dim3(256), 0, s, p);
  NKV_LAUNCH_CHECK();
  return NKV_OK;
}

}  // namespace nkv
