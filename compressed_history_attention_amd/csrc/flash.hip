// Flash attention forward over decoded history and the current chunk
// (NanoKV full-dimensional read, Figure 4(a): attention itself is unchanged
// once K/V are reconstructed).  bf16 MFMA for QK^T and PV, fp32 online
// softmax in base 2 with the softmax scale folded into one FMA, lazy
// rescaling (the running maximum only moves when a tile exceeds it by more
// than 2^8), natural-log LSE out.
//
// Layout: Q [Nq, W] bf16; K_all [Nk_pad, W] bf16 rows; V^T [H][128][ld]
// bf16 (per-head transposed so PV operands are contiguous along keys).
// Keys beyond Nk up to the 64-key padding are zero and masked.
//
// Block = NW waves (8, or 4 when 8-wave blocks would leave the chip's last
// round of blocks under-filled) x 32 queries of one head; each tile of 64 keys
// moves from HBM/L2 into double-buffered LDS with direct-to-LDS loads (1 KiB
// per wave instruction, no registers, no LDS stores).  Per wave and tile: S^T = K Q^T
// is 2 x 8 MFMA 32x32x16 (lane = query column, 32 keys per lane), O^T +=
// V^T P^T is 4 x 4 MFMAs whose B operand is the wave's own P in registers.
//
// LDS layouts (both conflict-free for the MFMA operand reads):
//  * K tile: 64 rows of 256 bytes; 16-byte block j of key row r is stored at
//    block j ^ (r & 15).
//  * V^T tile: 128 rows (dims) of 128 bytes (64 keys); block j of dim row r
//    is stored at block j ^ ((r >> 1) & 7).
// The S MFMA takes its 32 key rows in the order r -> r with bits 2 and 3
// swapped, so that each lane's P values for a 16-key step are 8 consecutive
// keys: the PV A operand is then one 16-byte read per lane.
#include <cmath>

#include "tuned_internal.hpp"

namespace nkv {

constexpr int FA_KB = FA_KT * 256;  // bytes of a K tile (64 keys x 128 bf16)
constexpr int FA_VB = 128 * FA_KT * 2;  // bytes of a V^T tile (128 dims x 64 keys)

// key row of MFMA output row i within a 32-key block: bits 2 and 3 swapped
__device__ __forceinline__ int fa_key_of_row(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

template <bool OUT_F32, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void k_flash(const uint16_t* __restrict__ Q, int64_t Nq, int H,
                                                  float c, const uint16_t* __restrict__ K,
                                                  const uint16_t* __restrict__ VT, int64_t Nk,
                                                  int64_t ld, int nsplit, int ragged_last,
                                                  void* __restrict__ out,
                                                  float* __restrict__ lse) {
  // one array per stage and operand: the stage of every LDS access is static
  __shared__ __attribute__((aligned(1024))) char sK0[FA_KB];
  __shared__ __attribute__((aligned(1024))) char sK1[FA_KB];
  __shared__ __attribute__((aligned(1024))) char sV0[FA_VB];
  __shared__ __attribute__((aligned(1024))) char sV1[FA_VB];
  const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // XCD-aware order: block L runs on XCD L % 8; work unit u (query block
  // fastest, then head, then key-range split) is given to block
  // (u % per) * 8 + u / per, so that each XCD's L2 serves the K/V rows of a
  // few heads instead of slices of all of them
  constexpr int QB = 32 * NW;  // queries per block
  const int nqb = (int)((Nq + QB - 1) / QB);
  const int nunits = nqb * H * nsplit;
  const int per = (nunits + 7) / 8;
  const int u = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (u >= nunits) return;  // the whole block, before any barrier
  // within a split, the ragged last query block of every head comes after
  // all full blocks, so that these shorter blocks fill the last round
  const int split = u / (nqb * H);  // key-range split (partials merged later)
  const int rnk = u - split * nqb * H;
  int h, qb;
  if (ragged_last && nqb > 1 && rnk >= (nqb - 1) * H) {
    qb = nqb - 1;
    h = rnk - (nqb - 1) * H;
  } else {
    const int nq = ragged_last && nqb > 1 ? nqb - 1 : nqb;
    qb = rnk % nq;
    h = rnk / nq;
  }
  const int W = H * 128;
  const int64_t q0 = (int64_t)qb * QB + wave * 32;
  const int64_t qrow = q0 + (lane & 31);
  const bool qok = qrow < Nq;

  bf16x8 qf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    qf[ks] = qok ? as_bf16x8(ld_u32x4(Q + qrow * W + h * 128 + 16 * ks + 8 * hl))
                 : as_bf16x8(u32x4{0u, 0u, 0u, 0u});

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = zero16();
  float m_run = -INFINITY, l_part = 0.f;

  const int64_t ntiles_all = (Nk + FA_KT - 1) / FA_KT;
  const int64_t t_beg = ntiles_all * split / nsplit, t_end = ntiles_all * (split + 1) / nsplit;
  // this wave's 32 / NW of the 32 1-KiB chunks of tile t: K chunks 0..15 (16
  // key rows each), V^T chunks 16..31 (8 dim rows each), each lane one
  // 16-byte block of the swizzled layout
  const char* kbase = reinterpret_cast<const char*>(K + h * 128);
  const char* vbase = reinterpret_cast<const char*>(VT + (int64_t)h * 128 * ld);
  auto dma = [&](int64_t t, char* dk, char* dv) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 16 / NW; ++j) {
      const int ch = wave + NW * j;  // K chunk
      const int s = ch * 64 + lane, r = s >> 4, blk = (s & 15) ^ (r & 15);
      uint32_t off = (uint32_t)(r * W * 2 + blk * 16);
      asm volatile("" : "+v"(off));
      __builtin_amdgcn_global_load_lds(kbase + t * FA_KT * W * 2 + off,
                                       (__attribute__((address_space(3))) void*)(dk + ch * 1024),
                                       16, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 16 / NW; ++j) {
      const int ch = wave + NW * j;  // V^T chunk
      const int s = ch * 64 + lane, r = s >> 3, blk = (s & 7) ^ ((r >> 1) & 7);
      uint32_t off = (uint32_t)(r * ld * 2 + blk * 16);
      asm volatile("" : "+v"(off));
      __builtin_amdgcn_global_load_lds(vbase + t * FA_KT * 2 + off,
                                       (__attribute__((address_space(3))) void*)(dv + ch * 1024),
                                       16, 0, 0);
    }
  };

  const int krow = fa_key_of_row(lane & 31);  // this lane's key row in a 32-key block
  auto body = [&](int64_t tile, const char* cK, const char* cV, char* nK, char* nV)
      __attribute__((always_inline)) {
    if (tile + 1 < t_end) dma(tile + 1, nK, nV);
    // ---- S^T = K Q^T: K fragments read four k-steps ahead of their MFMAs ----
    // (sched_barrier keeps each batch of reads ahead of the MFMAs using it)
    f32x16 s[2] = {zero16(), zero16()};
    auto read_k4 = [&](int ks0, bf16x8 (&kf)[2][4]) __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int uu = 0; uu < 4; ++uu) {
          const int r = kb * 32 + krow, j = 2 * (ks0 + uu) + hl;
          kf[kb][uu] = as_bf16x8(*reinterpret_cast<const u32x4*>(cK + r * 256 + ((j ^ (r & 15)) << 4)));
        }
    };
    auto read_v4 = [&](int j, bf16x8 (&vf)[4]) __attribute__((always_inline)) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int r = db * 32 + (lane & 31), b = 2 * j + hl;
        vf[db] = as_bf16x8(*reinterpret_cast<const u32x4*>(cV + r * 128 + ((b ^ ((r >> 1) & 7)) << 4)));
      }
    };
    {
      bf16x8 k0[2][4], k1[2][4];
      read_k4(0, k0);
      __builtin_amdgcn_sched_barrier(0);
      read_k4(4, k1);
#pragma unroll
      for (int uu = 0; uu < 4; ++uu)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[kb] = mfma_bf16(k0[kb][uu], qf[uu], s[kb]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int uu = 0; uu < 4; ++uu)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[kb] = mfma_bf16(k1[kb][uu], qf[4 + uu], s[kb]);
    }
    bf16x8 va[4], vb[4];
    read_v4(0, va);
    __builtin_amdgcn_sched_barrier(0);
    if ((tile + 1) * FA_KT > Nk) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (tile * FA_KT + kb * 32 + fa_key_of_row(acc_row(e, lane)) >= Nk) s[kb][e] = -INFINITY;
    }
    // ---- online softmax (base 2, lazy rescale) ----------------------------
    // The running maximum only moves when a score exceeds it by more than 2^8.
    // Instead of the tile maximum before the exponentials, the tile's p are
    // formed from the running maximum and the wave checks the lanes' sums: a
    // sum of at most 256 means no p above 256, so nothing moves.  Otherwise
    // (or when the sum is not finite: the first tile meets an empty maximum)
    // the tile maximum is taken and, where it moves, O and l are rescaled
    // and the p formed again.
    // P for 16 keys (step j: key block j/2, half j%2), packed to bf16: the
    // elements 8 (j%2) .. +7 of the lane are the keys 16 j + 8 (lane/32) + 0..7
    auto probs = [&](int j, float& ss) __attribute__((always_inline)) {
      const int kb = j >> 1, half = j & 1;
      u32x4 pk;
      float pair[4];
#pragma unroll
      for (int uu = 0; uu < 4; ++uu) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * half + 2 * uu], c, -m_run));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * half + 2 * uu + 1], c, -m_run));
        pair[uu] = p0 + p1;
        pk[uu] = pack_bf16x2(p0, p1);
      }
      // a tree from the first pair on: seven adds for eight values (a sum
      // started from 0.f keeps an add the compiler may not drop, as 0 + -0 is +0)
      ss = (pair[0] + pair[1]) + (pair[2] + pair[3]);
      return as_bf16x8(pk);
    };
    // all four steps' p first, then one check for the tile (a rescale must
    // come before the tile's first P V MFMA: rescaling accumulators that
    // MFMAs have already written costs registers the kernel does not have)
    float s0s, s1s, s2s, s3s;
    bf16x8 p0 = probs(0, s0s), p1 = probs(1, s1s), p2 = probs(2, s2s), p3 = probs(3, s3s);
    {
      const float ss = (s0s + s1s) + (s2s + s3s);
      if (__ballot(!(ss <= 256.f))) {  // wave-uniform: the maximum needs both lane halves
        float mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) mt = fmaxf(mt, s[kb][e]);
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64)) * c;
        if (mt > m_run + 8.f) {  // per row, the same in both lane halves
          const float alpha = __builtin_amdgcn_exp2f(m_run - mt);
          l_part *= alpha;
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[i][e] *= alpha;
          m_run = mt;
          p0 = probs(0, s0s);
          p1 = probs(1, s1s);
          p2 = probs(2, s2s);
          p3 = probs(3, s3s);
        }
      }
      l_part += (s0s + s1s) + (s2s + s3s);
    }
    // ---- O^T += V^T P^T: V fragments one 16-key step ahead ----------------
    __builtin_amdgcn_sched_barrier(0);
    read_v4(1, vb);
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = mfma_bf16(va[db], p0, o[db]);
    __builtin_amdgcn_sched_barrier(0);
    read_v4(2, va);
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = mfma_bf16(vb[db], p1, o[db]);
    __builtin_amdgcn_sched_barrier(0);
    read_v4(3, vb);
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = mfma_bf16(va[db], p2, o[db]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = mfma_bf16(vb[db], p3, o[db]);
    // tile + 1 has landed (this wave's share) and every wave is done with
    // this stage before it is loaded again
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  if (t_beg < t_end) {
    dma(t_beg, sK0, sV0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  for (int64_t tile = t_beg; tile < t_end; tile += 2) {
    body(tile, sK0, sV0, sK1, sV1);
    if (tile + 1 < t_end) body(tile + 1, sK1, sV1, sK0, sV0);
  }
  // ---- epilogue -------------------------------------------------------------
  const float l = l_part + __shfl_xor(l_part, 32, 64);
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
  // split z writes its partial (normalised O, LSE) at slice z
  out = static_cast<char*>(out) + (size_t)split * Nq * W * (OUT_F32 ? 4 : 2);
  lse += (int64_t)split * Nq * H;
  if (qok) {
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dim = db * 32 + g * 8 + hl * 4;  // 4 consecutive dims e = 4g .. 4g+3
        const int64_t base = qrow * W + h * 128 + dim;
        if (OUT_F32) {
          float* of = static_cast<float*>(out);
          *reinterpret_cast<f32x4*>(of + base) =
              f32x4{o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv,
                    o[db][4 * g + 3] * inv};
        } else {
          uint16_t* ob = static_cast<uint16_t*>(out);
          *reinterpret_cast<u32x2*>(ob + base) =
              u32x2{pack_bf16x2(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                    pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)};
        }
      }
    }
    if (hl == 0)
      lse[qrow * H + h] = (l > 0.f) ? (m_run + __log2f(l)) * 0.69314718055994531f : -INFINITY;
  }
}

namespace {
// fill of the last round of blocks: rounds / ceil(rounds)
double flash_fill(int64_t blocks, double slots) {
  const double rounds = (double)blocks / slots;
  return rounds / std::ceil(rounds);
}
// 8-wave blocks (one per CU; each K/V tile serves 256 queries) unless their
// last round would be under 85 % full
bool flash_wide(int64_t Nq, int H) { return flash_fill(ceil_div(Nq, 256) * H, 256.0) >= 0.85; }
}  // namespace

int flash_splits(int64_t Nq, int H, int64_t Nk) {
  if (flash_wide(Nq, H)) return 1;
  // 4-wave blocks, two per CU.  Splitting costs a merge of S fp32 partials,
  // so split only when the last round of blocks would be under 85 % full,
  // and then take the smallest count that fills it to 90 % (at least 4 key
  // tiles per split)
  const double slots = 512.0;
  const int64_t blocks = ceil_div(Nq, 128) * H, tiles = ceil_div(Nk, FA_KT);
  auto eff = [&](int S) { return flash_fill(blocks * S, slots); };
  if (eff(1) >= 0.85) return 1;
  int best = 1;
  for (int S = 2; S <= 8 && tiles >= 4 * S; ++S) {
    if (eff(S) > eff(best)) best = S;
    if (eff(S) >= 0.9) return S;
  }
  return best;
}

nkv_status launch_flash(const uint16_t* q, int64_t Nq, int H, float tau, const uint16_t* kall,
                        const uint16_t* vt, int64_t Nk, int64_t ld, bool out_f32, void* out,
                        float* lse, int nsplit, hipStream_t st) {
  if (Nq == 0) return NKV_OK;
  const float c = tau * 1.4426950408889634f;
  const bool wide = nsplit == 1 && flash_wide(Nq, H);
  const int nw = wide ? 8 : 4;
  const int64_t units = ceil_div(Nq, 32 * nw) * H * nsplit;
  const dim3 grid((unsigned)(ceil_div(units, 8) * 8)), block((unsigned)(64 * nw));
  const int ragged = Nq % (32 * nw) != 0 ? 1 : 0;
  if (out_f32 && wide)
    hipLaunchKernelGGL((k_flash<true, 8>), grid, block, 0, st, q, Nq, H, c, kall, vt, Nk, ld, nsplit,
                       ragged, out, lse);
  else if (out_f32)
    hipLaunchKernelGGL((k_flash<true, 4>), grid, block, 0, st, q, Nq, H, c, kall, vt, Nk, ld, nsplit,
                       ragged, out, lse);
  else if (wide)
    hipLaunchKernelGGL((k_flash<false, 8>), grid, block, 0, st, q, Nq, H, c, kall, vt, Nk, ld,
                       nsplit, ragged, out, lse);
  else
    hipLaunchKernelGGL((k_flash<false, 4>), grid, block, 0, st, q, Nq, H, c, kall, vt, Nk, ld,
                       nsplit, ragged, out, lse);
  NKV_LAUNCH_CHECK();
  return NKV_OK;
}

}  // namespace nkv
