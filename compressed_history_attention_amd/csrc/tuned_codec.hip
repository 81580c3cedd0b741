// Tuned encoder and decoder of libnanokv (bf16, MFMA).
//
// Encoder (NanoKV abstract; Figure 4(b)):
//   1. ||mu_a||^2 per center (fp32).
//   2. Distance GEMM  d(a, t) = ||mu_a||^2 - 2 mu_a . x_t  on bf16 MFMA (bf16
//      products are exact in fp32); the epilogue reduces each token's
//      column over the wave's 64 centers to its three nearest by
//      (distance, index), one record each per 64-center slot.  A per-token
//      pass takes the best record; when the runner-up lies within a
//      rigorous bound on the fp32 rounding error of the two distances it
//      assigns the token again in fp64 (the same ||mu||^2 - 2 mu . x form)
//      over the candidate centers the slot records leave, so the argmin is
//      the one exact arithmetic gives, ties to the lowest index.
//   3. Projection GEMM z = E (x - mu_a): the fp32 residual (exact for bf16
//      inputs) is split into three bf16 terms hi + mid + lo = e, so three
//      exact-product MFMA passes with fp32 accumulation give the projection
//      at fp32 accuracy.
//   4. INT4 group quantisation of z.
// Decoder (Figure 4(b)): x_hat = mu_a + D (code * scale) as a GEMM whose A
// loader dequantises INT4 on the fly and whose epilogue adds the center and
// writes bf16 rows (K) or per-head transposed columns (V).
#include <atomic>
#include <type_traits>

#include "prof.hpp"
#include "quant.hpp"
#include "tuned_internal.hpp"

namespace nkv {

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------
// ||mu_a||^2 per center (fp32), 16 centers per block (one per wave in four
// rounds), 16-byte loads; each block also writes the largest of its norms,
// so the assignment's error bound needs no atomics and no cleared counter.
constexpr int NORM_CPB = 16;
// Also ||mu_a||^2 in fp64 (out64), summed in the order the exact
// re-assignment of k_argmin_reduce uses (lane partials over its channels
// 8 lane + 512 k .. + 7, then the butterfly), so that pass reads it instead
// of summing it again per token.
__global__ __launch_bounds__(256) void k_center_norms(const uint16_t* __restrict__ mu, int A, int W,
                                                      float* __restrict__ out,
                                                      double* __restrict__ out64,
                                                      float* __restrict__ block_max) {
  __shared__ float smax[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float mx = 0.f;
  for (int k = 0; k < NORM_CPB / 4; ++k) {
    const int a = blockIdx.x * NORM_CPB + k * 4 + wave;
    if (a >= A) break;  // wave-uniform
    const uint16_t* row = mu + (int64_t)a * W;
    float acc = 0.f;
    double acc64 = 0.0;
    for (int w = 8 * lane; w < W; w += 512) {  // W % 8 == 0 on this path
      const u32x4 v = ld_u32x4(row + w);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float lo = bf16_bits_to_f32(uint16_t(v[u] & 0xffffu));
        const float hi = bf16_bits_to_f32(uint16_t(v[u] >> 16));
        acc = fmaf(lo, lo, fmaf(hi, hi, acc));
        acc64 = fma((double)lo, (double)lo, acc64);
        acc64 = fma((double)hi, (double)hi, acc64);
      }
    }
    acc = wave_sum(acc);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc64 += __shfl_xor(acc64, o, 64);
    if (lane == 0) {
      out[a] = acc;
      out64[a] = acc64;
    }
    mx = fmaxf(mx, acc);
  }
  if (lane == 0) smax[wave] = mx;
  __syncthreads();
  if (threadIdx.x == 0)
    block_max[blockIdx.x] = fmaxf(fmaxf(smax[0], smax[1]), fmaxf(smax[2], smax[3]));
}

// Per token (one wave each): the best of its slot records (lowest distance,
// then lowest index) and the runner-up distance over all centers.  The
// computed distance of center a differs from the exact ||mu_a||^2 -
// 2 mu_a . x by at most g (||mu_a||^2 + 2 ||mu_a|| ||x||) + u |d_a|
// (g = (W + 64) u / (1 - (W + 64) u), u = 2^-24: fp32 sums of W exact
// products, the fp32 norm, one rounding of the difference).  With
// M = max_a ||mu_a|| the bound E = 2 (g + u) (M^2 + 2 M ||x||) covers any two
// centers; when the runner-up is more than E above the best, no other center
// can be nearer (or tie) in exact arithmetic.  Otherwise the wave assigns
// the token again in fp64: d(a) = ||mu_a||^2 - 2 mu_a . x with exact bf16
// products summed in fp64, lowest index on ties.  (M and ||x|| are inflated
// by 1 % for their own rounding; ||x||^2 is summed here from 16-byte loads.)
// ||row||^2 of one bf16 row (W % 8 == 0), summed in fp32 by one wave from
// 16-byte loads; every lane returns the total
__device__ __forceinline__ float row_sqnorm_wave(const uint16_t* row, int W, int lane) {
  float xs = 0.f;
  for (int w = 8 * lane; w < W; w += 512) {
    const u32x4 v = ld_u32x4(row + w);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float lo = bf16_bits_to_f32(uint16_t(v[k] & 0xffffu));
      const float hi = bf16_bits_to_f32(uint16_t(v[k] >> 16));
      xs = fmaf(lo, lo, fmaf(hi, hi, xs));
    }
  }
  return wave_sum(xs);
}

// ||x_t||^2 per token, one wave each (rows that several assignments reuse,
// as in center fitting, are summed once)
__global__ __launch_bounds__(256) void k_row_sqnorm(const uint16_t* __restrict__ x, int64_t N,
                                                    int W, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= N) return;
  const float xs = row_sqnorm_wave(x + t * W, W, lane);
  if (lane == 0) out[t] = xs;
}

__global__ __launch_bounds__(256) void k_argmin_reduce(const uint64_t* __restrict__ best,
                                                       const uint64_t* __restrict__ second,
                                                       const uint64_t* __restrict__ third,
                                                       int nslot, int64_t N, int W,
                                                       const uint16_t* __restrict__ x,
                                                       const float* __restrict__ xnorm,
                                                       const uint16_t* __restrict__ mu, int A,
                                                       const double* __restrict__ mu2d,
                                                       const float* __restrict__ block_max,
                                                       int nblock_max,
                                                       int32_t* __restrict__ idx) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= N) return;  // whole waves; no block barrier below
  // ||x_t||^2: given, or summed here (W % 8 == 0 on this path)
  const uint16_t* row = x + t * W;
  const float xs = xnorm ? xnorm[t] : row_sqnorm_wave(row, W, lane);
  float m2 = 0.f;  // max ||mu||^2 from the per-block maxima
  for (int i = lane; i < nblock_max; i += 64) m2 = fmaxf(m2, block_max[i]);
  m2 = wave_max(m2);
  auto dist_of = [](uint64_t k) { return from_ordered_bits(uint32_t(k >> 32)); };
  // nearest over all slots, and the nearest of everything else (every other
  // slot's nearest, the winning slot's runner-up): lane sl holds slots sl,
  // sl + 64, ...
  uint64_t bk = ~0ull, sk = ~0ull;
  for (int sl = lane; sl < nslot; sl += 64) {
    const uint64_t k = best[(int64_t)sl * N + t];
    const uint64_t k2 = second[(int64_t)sl * N + t];
    if (k < bk) {
      sk = bk < k2 ? bk : k2;
      bk = k;
    } else {
      sk = sk < k ? sk : k;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t ob = __shfl_xor(bk, o, 64), os = __shfl_xor(sk, o, 64);
    const uint64_t lose = bk < ob ? ob : bk;
    const uint64_t s1 = sk < os ? sk : os;
    sk = s1 < lose ? s1 : lose;
    bk = bk < ob ? bk : ob;
  }
  const float d1 = dist_of(bk);
  const float d2 = sk == ~0ull ? INFINITY : dist_of(sk);
  const float u = 5.9604645e-8f;  // 2^-24
  const float kw = (float)(W + 64) * u;
  const float g = kw / (1.f - kw);
  const float M = sqrtf(m2) * 1.01f;
  const float X = sqrtf(xs) * 1.01f;
  const float E = 2.f * (g + u) * (M * M + 2.f * M * X);
  int32_t a_out = (int32_t)(bk & 0xffffffffu);
  // (a NaN or infinite distance compares false: such tokens are assigned again too)
  if (!(d2 - d1 > E)) {
    // fp64 assignment, the lane's channels w = 8 lane + 512 k .. + 7.  The
    // exact nearest center has a computed distance within E of d1: in each
    // 64-center slot whose nearest is that close, the nearest is a
    // candidate, so is its runner-up if that close too, and so is every
    // center of the slot if its third is that close as well (the others are
    // no closer than the third).  Candidates are met in increasing center
    // order (ties keep the lowest index); every center when none is found
    // (non-finite distances).
    double bd = INFINITY;
    int ba = 0x7fffffff;
    auto scan = [&](int a0, int a1) {
      for (int a = a0; a < a1; ++a) {
        const uint16_t* mrow = mu + (int64_t)a * W;
        double dot = 0.0;
        for (int w = 8 * lane; w < W; w += 512) {
          const u32x4 xv = ld_u32x4(row + w), mv = ld_u32x4(mrow + w);
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const double xe = bf16_bits_to_f32(uint16_t(xv[k >> 1] >> (16 * (k & 1))));
            const double me = bf16_bits_to_f32(uint16_t(mv[k >> 1] >> (16 * (k & 1))));
            dot = fma(xe, me, dot);
          }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) dot += __shfl_xor(dot, o, 64);
        const double dist = mu2d[a] - 2.0 * dot;  // ||mu_a||^2 in fp64, same order
        if (dist < bd) {  // a increases: strict < keeps the lowest index
          bd = dist;
          ba = a;
        }
      }
    };
    const float lim = d1 + E;
    for (int sl = 0; sl < nslot; ++sl) {
      const int64_t o = (int64_t)sl * N + t;
      const uint64_t kb = best[o], ks = second[o];
      if (!(dist_of(kb) <= lim)) continue;
      const int a = (int)(kb & 0xffffffffu);
      if (ks != ~0ull && dist_of(ks) <= lim) {
        const uint64_t k3 = third[o];
        if (k3 != ~0ull && dist_of(k3) <= lim) {
          scan(sl * 64, min(A, sl * 64 + 64));
        } else {
          const int a2 = (int)(ks & 0xffffffffu);
          scan(min(a, a2), min(a, a2) + 1);
          scan(max(a, a2), max(a, a2) + 1);
        }
      } else {
        scan(a, a + 1);
      }
    }
    if (ba == 0x7fffffff) scan(0, A);
    a_out = ba;
  }
  if (lane == 0) idx[t] = a_out;
}

__device__ __forceinline__ u32x4 load8_bf16(const uint16_t* base, int64_t row, int ld, int k,
                                            bool ok) {
  if (!ok) return u32x4{0u, 0u, 0u, 0u};
  return ld_u32x4(base + row * ld + k);
}

// The same as a load on every path: rows and k clamped into [0, rows) and
// [0, ld - 8], the value zeroed after the load when out of range (a branch
// around the load would make the compiler wait for all loads in flight)
__device__ __forceinline__ u32x4 load8_bf16_always(const uint16_t* base, int64_t row, int rows,
                                                   int ld, int k) {
  const bool ok = row < rows && k < ld;
  const u32x4 v = ld_u32x4(base + min(row, (int64_t)rows - 1) * ld + min(k, ld - 8));
  return ok ? v : u32x4{0u, 0u, 0u, 0u};
}

// ---------------------------------------------------------------------------
// distance GEMM with argmin epilogue: rows = centers, cols = tokens
// ---------------------------------------------------------------------------
struct DistProblem {
  static constexpr int BK = 64;
  int M, N, K;  // M = A centers, N = tokens, K = W
  const uint16_t* mu;
  const uint16_t* x;
  const float* mu2;
  uint64_t* best;    // [slot][N]: (order-preserving distance bits << 32 | a) of the slot's nearest
  uint64_t* second;  // [slot][N]: the same for the slot's runner-up
  uint64_t* third;   // [slot][N]: and for its third
  __device__ u32x4 load_a(int, int m, int k) const { return load8_bf16_always(mu, m, M, K, k); }
  __device__ u32x4 load_b(int, int n, int k) const { return load8_bf16_always(x, n, N, K, k); }
  // one wave = centers m0 .. m0 + 63 (slot m0 / 64) x tokens n0 .. n0 + 63;
  // candidates are ordered by (distance, index)
  __device__ void epilogue(int, int m0, int n0, int lane, const f32x16 (&acc)[2][2]) const {
    if (m0 >= M) return;  // no center in this quadrant
    // the norms of the lane's 32 centers, all requested before any is used
    // (one wait instead of one per center)
    float nm[2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) nm[i][e] = mu2[min(m0 + 32 * i + acc_row(e, lane), M - 1)];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      // the lane's three nearest, k1 < k2 < k3 (keys are distinct: the
      // index is in them)
      uint64_t k1 = ~0ull, k2 = ~0ull, k3 = ~0ull;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int a = m0 + 32 * i + acc_row(e, lane);
          if (a < M) {
            const float dist = nm[i][e] - 2.f * acc[i][j][e];
            const uint64_t k = ((uint64_t)ordered_bits(dist) << 32) | (uint32_t)a;
            if (k < k1) {
              k3 = k2;
              k2 = k1;
              k1 = k;
            } else if (k < k2) {
              k3 = k2;
              k2 = k;
            } else if (k < k3) {
              k3 = k;
            }
          }
        }
      }
      const uint64_t o1 = __shfl_xor(k1, 32, 64), o2 = __shfl_xor(k2, 32, 64),
                     o3 = __shfl_xor(k3, 32, 64);
      // the three nearest of both lanes' (sorted) triples: the smaller first
      // key wins; the rest merge the winner's (k2, k3) with the loser's
      // (o1, o2)
      const bool mine = k1 < o1;
      const uint64_t b = mine ? k1 : o1;
      const uint64_t w2 = mine ? k2 : o2, w3 = mine ? k3 : o3;  // the winner's other two
      const uint64_t l1 = mine ? o1 : k1, l2 = mine ? o2 : k2;  // the loser's first two
      const uint64_t sec = w2 < l1 ? w2 : l1;
      const uint64_t thd = w2 < l1 ? (w3 < l1 ? w3 : l1) : (w2 < l2 ? w2 : l2);
      const int n = n0 + 32 * j + (lane & 31);
      if (lane < 32 && n < N) {
        const int64_t o = (int64_t)(m0 / 64) * N + n;
        best[o] = b;
        second[o] = sec;
        third[o] = thd;
      }
    }
  }
};

// The same product split over K (grid z) when the tiles are too few to fill
// the chip (few tokens or few centers): split z sums its K chunk
// [z K, (z + 1) K) into fp32 partial dot products part[z][token][center],
// which k_dist_reduce adds up before the slot records are formed.  Any
// summation order keeps the rounding bound of the assignment (W + splits
// - 1 additions, splits <= 64).
struct DistSplitProblem {
  static constexpr int BK = 64;
  int M, N, K;  // M = A centers, N = tokens, K = the chunk of one split (multiple of 64)
  int Kfull;    // W
  const uint16_t* mu;
  const uint16_t* x;
  float* part;  // [splits][N][M]
  __device__ u32x4 load_a(int z, int m, int k) const {
    return load8_bf16_always(mu, m, M, Kfull, z * K + k);
  }
  __device__ u32x4 load_b(int z, int n, int k) const {
    return load8_bf16_always(x, n, N, Kfull, z * K + k);
  }
  // lane: token n0 + 32 j + lane % 32, centers m0 + 32 i + acc_row(e): runs of
  // four consecutive centers (e % 4), stored as one 16-byte piece when whole
  __device__ void epilogue(int z, int m0, int n0, int lane, const f32x16 (&acc)[2][2]) const {
    if (m0 >= M) return;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + 32 * j + (lane & 31);
      if (n >= N) continue;
      float* row = part + ((int64_t)z * N + n) * M;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int a = m0 + 32 * i + acc_row(4 * g, lane);
          if ((M & 3) == 0 && a + 4 <= M) {
            *reinterpret_cast<f32x4*>(row + a) =
                f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                      acc[i][j][4 * g + 3]};
          } else {
#pragma unroll
            for (int u = 0; u < 4; ++u)
              if (a + u < M) row[a + u] = acc[i][j][4 * g + u];
          }
        }
    }
  }
};

// Split partials -> the slot records of DistProblem's epilogue: one wave per
// token, lane l holding center 64 slot + l (nearest, runner-up and third of
// each 64-center slot by (distance, index), as there)
__global__ __launch_bounds__(256) void k_dist_reduce(const float* __restrict__ part, int splits,
                                                     int64_t N, int A,
                                                     const float* __restrict__ mu2,
                                                     uint64_t* __restrict__ best,
                                                     uint64_t* __restrict__ second,
                                                     uint64_t* __restrict__ third) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= N) return;  // whole waves
  const int nslot = (A + 63) / 64;
  for (int sl = 0; sl < nslot; ++sl) {
    const int a = sl * 64 + lane;
    uint64_t k = ~0ull;
    if (a < A) {
      float dot = 0.f;
      for (int z = 0; z < splits; ++z) dot += part[((int64_t)z * N + t) * A + a];
      k = ((uint64_t)ordered_bits(mu2[a] - 2.f * dot) << 32) | (uint32_t)a;
    }
    uint64_t b = k;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const uint64_t v = __shfl_xor(b, o, 64);
      b = v < b ? v : b;
    }
    uint64_t r = k == b ? ~0ull : k;  // keys are distinct (the index is in them)
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const uint64_t v = __shfl_xor(r, o, 64);
      r = v < r ? v : r;
    }
    uint64_t q = (k == b || k == r) ? ~0ull : k;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const uint64_t v = __shfl_xor(q, o, 64);
      q = v < q ? v : q;
    }
    if (lane == 0) {
      best[(int64_t)sl * N + t] = b;
      second[(int64_t)sl * N + t] = r;
      third[(int64_t)sl * N + t] = q;
    }
  }
}

// ---------------------------------------------------------------------------
// projection GEMM: rows = tokens, cols = coefficients, K = 3 W (split terms)
// ---------------------------------------------------------------------------
struct ProjProblem {
  static constexpr int BK = 32;
  int M, N, K;  // M = tokens, N = r, K = 3 W / splits (one split per grid z)
  int W;
  const uint16_t* x;
  const uint16_t* mu;
  const int32_t* idx;
  const uint16_t* enc;  // [r, W]
  float* z;             // [splits][tokens, r] partial sums
  __device__ u32x4 load_a(int zs, int m, int k) const {
    if (m >= M || k >= K) return u32x4{0u, 0u, 0u, 0u};
    k += zs * K;
    const int part = k / W, w = k - part * W;
    const u32x4 xv = ld_u32x4(x + (int64_t)m * W + w);
    const u32x4 mv = ld_u32x4(mu + (int64_t)idx[m] * W + w);
    u32x4 out;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float e2[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const float xf = bf16_bits_to_f32(uint16_t(xv[h] >> (16 * s)));
        const float mf = bf16_bits_to_f32(uint16_t(mv[h] >> (16 * s)));
        float e = xf - mf;
        // e = hi + mid + lo, each a bf16 value (round-half-even)
        const float hi = bf16_bits_to_f32(f32_to_bf16_bits(e));
        if (part == 0) { e2[s] = hi; continue; }
        const float r1 = e - hi;
        const float mid = bf16_bits_to_f32(f32_to_bf16_bits(r1));
        e2[s] = (part == 1) ? mid : (r1 - mid);
      }
      out[h] = pack_bf16x2(e2[0], e2[1]);
    }
    return out;
  }
  __device__ u32x4 load_b(int zs, int n, int k) const {
    if (n >= N || k >= K) return u32x4{0u, 0u, 0u, 0u};
    const int w = (k + zs * K) % W;
    return ld_u32x4(enc + (int64_t)n * W + w);
  }
  __device__ void epilogue(int zs, int m0, int n0, int lane, const f32x16 (&acc)[2][2]) const {
    float* zp = z + (int64_t)zs * M * N;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = m0 + 32 * i + acc_row(e, lane), n = n0 + 32 * j + (lane & 31);
          if (m < M && n < N) zp[(int64_t)m * N + n] = acc[i][j][e];
        }
  }
};

// ---------------------------------------------------------------------------
// Projection with the residual computed once: z = E (x - mu_a) for 64 tokens
// and every one of the r outputs per block, over one share of the channels
// (grid y; partial sums per share, added in a fixed order by the quantiser).
// Per 32-channel chunk the block forms the residual e = x - mu_a (exact in
// fp32 for bf16 inputs), splits it into three bf16 terms hi + mid + lo = e
// and stores them in LDS; each wave (32 tokens x r/QW outputs, 2 QW waves)
// multiplies the three terms by the same encoder fragments, read from L2
// one chunk ahead.  Exact products and fp32 sums reproduce an fp32
// projection.
// ---------------------------------------------------------------------------
constexpr int PS_TOK = 64, PS_KC = 32, PS_SHARE = 1024;
constexpr int PS_AS = PS_KC + 8;  // bf16 row stride of a residual term tile

template <int NT, int QW>  // r = 64 NT outputs in QW groups; 2 QW waves
__global__ __launch_bounds__(128 * QW) void k_project_stationary(const uint16_t* __restrict__ x,
                                                            int64_t N, int W,
                                                            const uint16_t* __restrict__ mu,
                                                            const int32_t* __restrict__ idx,
                                                            const uint16_t* __restrict__ enc,
                                                            float* __restrict__ z) {
  constexpr int R = 64 * NT, TW = 2 * NT / QW;  // 32-output tiles per wave
  static_assert(2 * NT % QW == 0, "output groups");
  // [stage][term][64 tokens][32 + 8]
  __shared__ __attribute__((aligned(16))) uint16_t sE[2][3][PS_TOK * PS_AS];
  const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t t0 = (int64_t)blockIdx.x * PS_TOK;
  const int w_beg = blockIdx.y * PS_SHARE, w_end = min(W, w_beg + PS_SHARE);
  const int nchunk = (w_end - w_beg) / PS_KC;
  // residual loads (threads 0..255): thread -> (token tid / 4, channels
  // 8 (tid % 4) .. + 7)
  const bool stager = tid < 256;
  const int rt = (tid & 255) >> 2, rc = (tid & 3) * 8;
  const int64_t rtok = t0 + rt;
  const bool rok = stager && rtok < N;
  const uint16_t* xrow = x + (rok ? rtok : 0) * W;
  const uint16_t* mrow = mu + (int64_t)(rok ? idx[rtok] : 0) * W;
  // Every load is unconditional (a chunk past the share rereads its last
  // chunk; rows past N read row 0 and stage zeros): with loads under
  // run-time conditions the compiler can only wait for all of them, and the
  // residual rows requested two chunks ahead would be waited for at once.
  auto ld_res = [&](int c, u32x4& xv, u32x4& mv) __attribute__((always_inline)) {
    const int w = w_beg + min(c, nchunk - 1) * PS_KC + rc;
    xv = ld_u32x4(xrow + w);
    mv = ld_u32x4(mrow + w);
  };
  auto put_res = [&](int stage, const u32x4& xv, const u32x4& mv) __attribute__((always_inline)) {
    if (!stager) return;
    u32x4 th, tm, tl;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float hi2[2], mid2[2], lo2[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const float e = bf16_bits_to_f32(uint16_t(xv[h] >> (16 * s2))) -
                        bf16_bits_to_f32(uint16_t(mv[h] >> (16 * s2)));
        const float hi = bf16_bits_to_f32(f32_to_bf16_bits(e));
        const float r1 = e - hi;
        const float mid = bf16_bits_to_f32(f32_to_bf16_bits(r1));
        hi2[s2] = hi;
        mid2[s2] = mid;
        lo2[s2] = r1 - mid;
      }
      th[h] = pack_bf16x2(hi2[0], hi2[1]);
      tm[h] = pack_bf16x2(mid2[0], mid2[1]);
      tl[h] = pack_bf16x2(lo2[0], lo2[1]);
    }
    const u32x4 z4 = u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(&sE[stage][0][rt * PS_AS + rc]) = rok ? th : z4;
    *reinterpret_cast<u32x4*>(&sE[stage][1][rt * PS_AS + rc]) = rok ? tm : z4;
    *reinterpret_cast<u32x4*>(&sE[stage][2][rt * PS_AS + rc]) = rok ? tl : z4;
  };
  // wave tile: tokens 32 (wave & 1) .., outputs (wave >> 1) R/QW ..
  const int tw = (wave & 1) * 32, ow = (wave >> 1) * (R / QW);
  // encoder fragments of one chunk: TW tiles x 2 k-steps
  auto ld_enc = [&](int c, u32x4 (&b)[TW][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < TW; ++j)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        b[j][ks] = ld_u32x4(enc + (int64_t)(ow + 32 * j + (lane & 31)) * W + w_beg +
                            min(c, nchunk - 1) * PS_KC + 16 * ks + 8 * hl);
  };
  f32x16 acc[TW];
#pragma unroll
  for (int j = 0; j < TW; ++j) acc[j] = zero16();
  // Inputs are requested two chunks ahead: the residual rows (from HBM) in
  // two register sets, the encoder fragments (from L2) in three buffers.
  // Chunk k uses residual set k % 2, LDS stage k % 2 and buffer k % 3.
  u32x4 xv[2], mv[2];
  u32x4 bb[3][TW][2];
  ld_res(0, xv[0], mv[0]);
  ld_res(1, xv[1], mv[1]);
  ld_enc(0, bb[0]);
  ld_enc(1, bb[1]);
  put_res(0, xv[0], mv[0]);
  __syncthreads();
  auto step = [&](int c, auto RS, auto BS) __attribute__((always_inline)) {
    constexpr int rs = decltype(RS)::value, bs = decltype(BS)::value;
    ld_res(c + 2, xv[rs], mv[rs]);
    ld_enc(c + 2, bb[(bs + 2) % 3]);
#pragma unroll
    for (int term = 0; term < 3; ++term)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(
            &sE[rs][term][(tw + (lane & 31)) * PS_AS + 16 * ks + 8 * hl]));
#pragma unroll
        for (int j = 0; j < TW; ++j) acc[j] = mfma_bf16(a, as_bf16x8(bb[bs][j][ks]), acc[j]);
      }
    // (past the last chunk this stages a reread chunk nobody uses: the
    // same operations on every step keep the compiler's waits exact)
    put_res(rs ^ 1, xv[rs ^ 1], mv[rs ^ 1]);
    __syncthreads();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  // whole groups of six steps in straight-line code (residual sets cycle by
  // two, encoder buffers by three), then the remaining steps
  int c = 0;
  for (; c + 6 <= nchunk; c += 6) {
    step(c, I0{}, I0{});
    step(c + 1, I1{}, I1{});
    step(c + 2, I0{}, I2{});
    step(c + 3, I1{}, I0{});
    step(c + 4, I0{}, I1{});
    step(c + 5, I1{}, I2{});
  }
  if (c < nchunk) step(c, I0{}, I0{});
  if (c + 1 < nchunk) step(c + 1, I1{}, I1{});
  if (c + 2 < nchunk) step(c + 2, I0{}, I2{});
  if (c + 3 < nchunk) step(c + 3, I1{}, I0{});
  if (c + 4 < nchunk) step(c + 4, I0{}, I1{});
  float* zp = z + (int64_t)blockIdx.y * N * R;
#pragma unroll
  for (int j = 0; j < TW; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t t = t0 + tw + acc_row(e, lane);
      if (t < N) zp[t * R + ow + 32 * j + (lane & 31)] = acc[j][e];
    }
}

// the stationary projection serves r = 64 NT (NT in 1..4, 6) and W % 32 == 0;
// its channel shares are fixed per W, so results do not depend on N
inline bool proj_stationary(int W, int r) {
  return r % 64 == 0 && r <= 384 && r != 320 && W % PS_KC == 0;
}
inline int proj_shares(int W) { return (W + PS_SHARE - 1) / PS_SHARE; }

// split-K factor of the projection (fixed per width, so results are
// deterministic): the three residual terms, each possibly halved
inline int proj_splits(int W) {
  if ((3 * W) % (6 * ProjProblem::BK) == 0) return 6;
  if ((3 * W) % (3 * ProjProblem::BK) == 0) return 3;
  return 1;
}

// one thread per coefficient: sum the split partials in a fixed order, then
// quantise its group with lane shuffles (groups never straddle a wave since
// the group size divides 64 and r is a multiple of it)
__global__ __launch_bounds__(256) void k_quantize_rows(const float* __restrict__ z, int splits,
                                                       int64_t N, int r, int group,
                                                       uint8_t* __restrict__ codes,
                                                       uint16_t* __restrict__ scales) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool ok = i < N * r;
  float v = 0.f;
  if (ok) {
    v = z[i];
    for (int sp = 1; sp < splits; ++sp) v += z[(int64_t)sp * N * r + i];
  }
  float m = fabsf(v);
  for (int o = group >> 1; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  const float u = m / 7.0f;  // IEEE division
  const __half sh = __float2half_rn(u);
  const float sf = __half2float(sh);
  int c = 0;
  if (sf > 0.f) c = (int)fminf(7.f, fmaxf(-8.f, rintf(v / sf)));
  const int c1 = __shfl_down(c, 1, 64);
  if (!ok) return;
  const int64_t t = i / r;
  const int j = (int)(i - t * r);
  if ((j & 1) == 0) codes[t * (r / 2) + j / 2] = uint8_t((c & 15) | ((c1 & 15) << 4));
  if (j % group == 0) scales[t * (r / group) + j / group] = __half_as_ushort(sh);
}

namespace {
// workspace of the assignment: ||mu||^2, per-block maxima of it, slot records
// compute units of the current device (cached per device)
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

struct AssignLayout {
  size_t mu2, mu2d, bmax, best, second, third, part, total;
  int nbmax, splits;
};
// K splits of the distance product: one when its 128 x 128 tiles fill the
// chip, else enough for about two blocks per CU, at most 32 and with the
// partials under 8 MiB (the chunk count W / 64 caps it again at launch)
int dist_splits(int64_t N, int32_t A) {
  const int64_t tiles = ceil_div(A, 128) * ceil_div(N, 128);
  if (N <= 0 || tiles >= 256) return 1;
  int64_t s = std::min<int64_t>(32, ceil_div(512, tiles));
  s = std::min<int64_t>(s, (int64_t)(8u << 20) / (sizeof(float) * N * A));
  return (int)std::max<int64_t>(1, s);
}

AssignLayout assign_layout(int64_t N, int32_t A) {
  AssignLayout L{};
  const int64_t nslot = ceil_div(A, 64);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  L.nbmax = (int)ceil_div(A, NORM_CPB);
  L.mu2 = take(sizeof(float) * A);
  L.mu2d = take(sizeof(double) * A);
  L.bmax = take(sizeof(float) * L.nbmax);
  L.best = take(sizeof(uint64_t) * nslot * N);
  L.second = take(sizeof(uint64_t) * nslot * N);
  L.third = take(sizeof(uint64_t) * nslot * N);
  L.splits = dist_splits(N, A);
  L.part = L.splits > 1 ? take(sizeof(float) * L.splits * N * A) : 0;
  L.total = off;
  return L;
}
}  // namespace

size_t tuned_assign_workspace(int64_t N, int32_t A) { return assign_layout(N, A).total; }

nkv_status tuned_row_sqnorm(const nkv_shape* s, const void* x, int64_t N, float* out,
                            hipStream_t st) {
  if (N <= 0) return NKV_OK;
  hipLaunchKernelGGL(k_row_sqnorm, dim3((unsigned)ceil_div(N, 4)), dim3(256), 0, st,
                     static_cast<const uint16_t*>(x), N, s->H * s->d, out);
  NKV_LAUNCH_CHECK();
  return NKV_OK;
}

nkv_status tuned_assign(const nkv_shape* s, const void* x, int64_t N, const void* centers,
                        int32_t A, int32_t* idx, char* ws, hipStream_t st, const float* xnorm) {
  const int W = s->H * s->d;
  const AssignLayout L = assign_layout(N, A);
  float* mu2 = reinterpret_cast<float*>(ws + L.mu2);
  double* mu2d = reinterpret_cast<double*>(ws + L.mu2d);
  float* bmax = reinterpret_cast<float*>(ws + L.bmax);
  uint64_t* best = reinterpret_cast<uint64_t*>(ws + L.best);
  uint64_t* second = reinterpret_cast<uint64_t*>(ws + L.second);
  uint64_t* third = reinterpret_cast<uint64_t*>(ws + L.third);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* mub = static_cast<const uint16_t*>(centers);
  hipLaunchKernelGGL(k_center_norms, dim3((unsigned)L.nbmax), dim3(256), 0, st, mub, A, W, mu2,
                     mu2d, bmax);
  NKV_LAUNCH_CHECK();
  nkv_status e;
  // (register-staged GEMM with 64-wide k steps, loads two steps ahead:
  // measured faster here than the direct-to-LDS one, whose 32-wide steps
  // double the barriers)
  // block order: groups of up to DIST_GROUP center tiles per XCD group
  // (their center rows, 768 KiB per tile at W = 3072, stay in its L2)
  constexpr int DIST_GROUP = 4;
  const int kc = (int)std::min<int64_t>(L.splits, W / 64);
  if (kc <= 1) {
    DistProblem dp{A, (int)N, W, mub, xb, mu2, best, second, third};
    if ((e = launch_gemm_pf2(dp, 1, st, DIST_GROUP))) return e;
  } else {
    const int chunk = (int)ceil_div(ceil_div(W, kc), 64) * 64;
    const int splits = (int)ceil_div(W, chunk);
    float* part = reinterpret_cast<float*>(ws + L.part);
    DistSplitProblem sp{A, (int)N, chunk, W, mub, xb, part};
    if ((e = launch_gemm_pf2(sp, splits, st, DIST_GROUP))) return e;
    hipLaunchKernelGGL(k_dist_reduce, dim3((unsigned)ceil_div(N, 4)), dim3(256), 0, st, part,
                       splits, N, A, mu2, best, second, third);
    NKV_LAUNCH_CHECK();
  }
  hipLaunchKernelGGL(k_argmin_reduce, dim3((unsigned)ceil_div(N, 4)), dim3(256), 0, st, best,
                     second, third, (int)ceil_div(A, 64), N, W, xb, xnorm, mub, A, mu2d, bmax,
                     L.nbmax, idx);
  NKV_LAUNCH_CHECK();
  return NKV_OK;
}

size_t tuned_encode_workspace(const nkv_shape* s, int64_t N, int32_t A) {
  const int W = s->H * s->d;
  const int parts = proj_stationary(W, s->r) ? proj_shares(W) : proj_splits(W);
  size_t off = tuned_assign_workspace(N, A);
  off = align_up(off + sizeof(float) * N * s->r * parts, 256);
  return off;
}

nkv_status tuned_encode(const nkv_shape* s, const void* x, int64_t N, const void* centers,
                        int32_t A, const void* enc, int32_t* idx, uint8_t* codes,
                        uint16_t* scales, char* ws, size_t ws_bytes, hipStream_t st) {
  const int W = s->H * s->d, r = s->r;
  float* z = reinterpret_cast<float*>(ws + tuned_assign_workspace(N, A));
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* mub = static_cast<const uint16_t*>(centers);
  nkv_status e;
  const bool stat = proj_stationary(W, r);
  const int splits = stat ? proj_shares(W) : proj_splits(W);
  {
  ProfScope ps("encode_assign", st);
  if ((e = tuned_assign(s, x, N, centers, A, idx, ws, st))) return e;
  }
  {
  ProfScope ps("encode_project", st);
  const uint16_t* eb = static_cast<const uint16_t*>(enc);
  if (stat) {
    const dim3 grid((unsigned)ceil_div(N, PS_TOK), (unsigned)splits);
    switch (r / 64) {
      case 1: hipLaunchKernelGGL((k_project_stationary<1, 2>), grid, dim3(256), 0, st, xb, N, W, mub, idx, eb, z); break;
      case 2: hipLaunchKernelGGL((k_project_stationary<2, 2>), grid, dim3(256), 0, st, xb, N, W, mub, idx, eb, z); break;
      case 3: hipLaunchKernelGGL((k_project_stationary<3, 2>), grid, dim3(256), 0, st, xb, N, W, mub, idx, eb, z); break;
      case 4: hipLaunchKernelGGL((k_project_stationary<4, 4>), grid, dim3(512), 0, st, xb, N, W, mub, idx, eb, z); break;
      default: hipLaunchKernelGGL((k_project_stationary<6, 4>), grid, dim3(512), 0, st, xb, N, W, mub, idx, eb, z); break;
    }
    NKV_LAUNCH_CHECK();
  } else {
    ProjProblem pp{(int)N, r, 3 * W / splits, W, xb, mub, idx, eb, z};
    if ((e = launch_gemm(pp, splits, st))) return e;
  }
  }
  ProfScope ps("encode_quantize", st);
  hipLaunchKernelGGL(k_quantize_rows, dim3((unsigned)ceil_div(N * r, 256)), dim3(256), 0, st, z,
                     splits, N, r, s->group, codes, scales);
  NKV_LAUNCH_CHECK();
  return NKV_OK;
}

// ---------------------------------------------------------------------------
// decoder GEMM: rows = compacted tokens, cols = channels (128 = one head)
// ---------------------------------------------------------------------------
struct DecodeProblem {
  static constexpr int BK = 32;
  int M, N, K;            // M = tokens in the list, N = W, K = r
  int group;
  BranchArgs b;
  RangeTable rows;
  uint16_t* out;          // K: row-major [*, W] at row offset; V: [H][128][ld]
  int64_t ld;             // V^T key stride
  bool transposed;
  __device__ u32x4 load_a(int, int m, int k) const {
    if (m >= M || k >= K) return u32x4{0u, 0u, 0u, 0u};
    const int64_t t = map_index(rows, m);
    const uint32_t c = *reinterpret_cast<const uint32_t*>(b.codes + t * (K / 2) + k / 2);
    const float sc = fp16_bits_to_f32(b.scales[t * (K / group) + k / group]);
    u32x4 out;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int n0 = (c >> (8 * h)) & 15, n1 = (c >> (8 * h + 4)) & 15;
      const float v0 = (float)(n0 - ((n0 & 8) << 1)) * sc;
      const float v1 = (float)(n1 - ((n1 & 8) << 1)) * sc;
      out[h] = pack_bf16x2(v0, v1);
    }
    return out;
  }
  __device__ u32x4 load_b(int, int n, int k) const {
    if (n >= N || k >= K) return u32x4{0u, 0u, 0u, 0u};
    return ld_u32x4(static_cast<const uint16_t*>(b.decoder) + (int64_t)n * K + k);
  }
  __device__ void epilogue(int, int m0, int n0, int lane, const f32x16 (&acc)[2][2]) const {
    const uint16_t* mu = static_cast<const uint16_t*>(b.centers);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int ai[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + 32 * i + acc_row(e, lane);
        ai[e] = (m < M) ? b.idx[map_index(rows, m)] : 0;
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + 32 * j + (lane & 31);
        if (n >= N) continue;
        if (!transposed) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int m = m0 + 32 * i + acc_row(e, lane);
            if (m < M)
              out[(int64_t)m * N + n] =
                  f32_to_bf16_bits(acc[i][j][e] + bf16_bits_to_f32(mu[(int64_t)ai[e] * N + n]));
          }
        } else {
          const int h = n >> 7, dd = n & 127;
          uint16_t* col = out + ((int64_t)h * 128 + dd) * ld;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int m = m0 + 32 * i + acc_row(e, lane);
            if (m < M)
              col[m] = f32_to_bf16_bits(acc[i][j][e] + bf16_bits_to_f32(mu[(int64_t)ai[e] * N + n]));
          }
        }
      }
    }
  }
};

// V decode in the transposed orientation (rows = channels, cols = tokens):
// lanes own tokens, so the per-head transposed V^T[h][d][token] stores are
// contiguous along tokens.
struct DecodeTProblem {
  static constexpr int BK = 32;
  int M, N, K;            // M = W channels, N = tokens in the list, K = r
  int group;
  BranchArgs b;
  RangeTable rows;
  uint16_t* out;          // [W][ld] (= [H][128][ld])
  int64_t ld;
  __device__ u32x4 load_a(int, int m, int k) const {
    if (m >= M || k >= K) return u32x4{0u, 0u, 0u, 0u};
    return ld_u32x4(static_cast<const uint16_t*>(b.decoder) + (int64_t)m * K + k);
  }
  __device__ u32x4 load_b(int, int n, int k) const {
    if (n >= N || k >= K) return u32x4{0u, 0u, 0u, 0u};
    const int64_t t = map_index(rows, n);
    const uint32_t c = *reinterpret_cast<const uint32_t*>(b.codes + t * (K / 2) + k / 2);
    const float sc = fp16_bits_to_f32(b.scales[t * (K / group) + k / group]);
    u32x4 out;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int n0 = (c >> (8 * h)) & 15, n1 = (c >> (8 * h + 4)) & 15;
      out[h] = pack_bf16x2((float)(n0 - ((n0 & 8) << 1)) * sc, (float)(n1 - ((n1 & 8) << 1)) * sc);
    }
    return out;
  }
  __device__ void epilogue(int, int m0, int n0, int lane, const f32x16 (&acc)[2][2]) const {
    const uint16_t* mu = static_cast<const uint16_t*>(b.centers);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + 32 * j + (lane & 31);
      if (n >= N) continue;
      const int64_t a = b.idx[map_index(rows, n)];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = m0 + 32 * i + acc_row(e, lane);
          if (m < M)
            out[(int64_t)m * ld + n] =
                f32_to_bf16_bits(acc[i][j][e] + bf16_bits_to_f32(mu[a * M + m]));
        }
    }
  }
};

// ---------------------------------------------------------------------------
// Decoder with the codes stationary: one block dequantises the INT4 codes of
// 64 tokens once into LDS (bf16, rows padded against bank conflicts) and
// sweeps every output channel against them, 128 channels per step; wave w
// owns channels 32w..32w+31 of each step and streams its decoder rows from
// L2 into registers eight k-steps ahead (a GEMM tiled over channels would
// dequantise every token once per channel tile).  C[tok][ch] = codes . D^T
// plus the token's center (requested before the step's MFMAs) is rounded to
// bf16 into an LDS tile -- [tok][ch] for K rows, [ch][tok] for the per-head
// transposed V -- and leaves the block as 16-byte row chunks.
// NKS > 0 fixes the number of 16-wide k-steps (r / 16) at compile time: the
// sweep of a step is then straight-line code, every decoder load
// unconditional, and the waits before the MFMAs count exactly the loads they
// need (with k-steps and loads under run-time conditions the compiler waits
// for every load in flight, the centers' included, before each group).
// NKS = 0 takes r / 16 at run time.
// ---------------------------------------------------------------------------
constexpr int DS_TOK = 64, DS_CH = 128;
constexpr int DS_WAIT_VM0 = (7 << 4) | (15 << 8);  // s_waitcnt vmcnt(0) alone

template <bool ROWS, int NKS>
__global__ __launch_bounds__(256) void k_decode_stationary(BranchArgs b, RangeTable rows, int W,
                                                           int r, int group,
                                                           uint16_t* __restrict__ out,
                                                           int64_t ld) {
  extern __shared__ __attribute__((aligned(16))) char dsm[];
  const int rs = r + 8;                                    // bf16 row stride of the codes
  uint16_t* sA = reinterpret_cast<uint16_t*>(dsm);         // [64][r + 8]
  // output tile: K [64][128 + 8], V [128][64 + 8] (bf16)
  uint16_t* sO = reinterpret_cast<uint16_t*>(dsm + DS_TOK * rs * 2);
  constexpr int OS = ROWS ? DS_CH + 8 : DS_TOK + 8;
  __shared__ int64_t sTok[DS_TOK];
  __shared__ int32_t sIdx[DS_TOK];
  const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t m0 = (int64_t)blockIdx.x * DS_TOK;
  const int nvalid = (int)min<int64_t>(DS_TOK, rows.total - m0);
  const uint16_t* D = static_cast<const uint16_t*>(b.decoder);
  const uint16_t* mu = static_cast<const uint16_t*>(b.centers);
  if (tid < DS_TOK) {
    const int64_t t = tid < nvalid ? map_index(rows, m0 + tid) : -1;
    sTok[tid] = t;
    sIdx[tid] = t >= 0 ? b.idx[t] : 0;
  }
  __syncthreads();
  // dequantise: 8 coefficients per item
  const int kc_per_tok = r / 8;
  for (int c = tid; c < DS_TOK * kc_per_tok; c += 256) {
    const int tl = c / kc_per_tok, k = (c - tl * kc_per_tok) * 8;
    const int64_t t = sTok[tl];
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (t >= 0) {
      const uint32_t cw = *reinterpret_cast<const uint32_t*>(b.codes + t * (r / 2) + k / 2);
      const float sc = fp16_bits_to_f32(b.scales[t * (r / group) + k / group]);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int n0 = (cw >> (8 * h)) & 15, n1 = (cw >> (8 * h + 4)) & 15;
        v[h] = pack_bf16x2((float)(n0 - ((n0 & 8) << 1)) * sc, (float)(n1 - ((n1 & 8) << 1)) * sc);
      }
    }
    *reinterpret_cast<u32x4*>(sA + tl * rs + k) = v;
  }
  __syncthreads();
  const int nks = NKS > 0 ? NKS : r / 16;
  auto afrag = [&](int i, int ks) __attribute__((always_inline)) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(sA + (32 * i + (lane & 31)) * rs + 16 * ks +
                                                     8 * hl));
  };
  // this block's share of the sweep (grid y splits the channel steps when
  // there are few token blocks)
  const int nsteps = W / DS_CH, per = (nsteps + gridDim.y - 1) / gridDim.y;
  const int n_beg = blockIdx.y * per * DS_CH, n_end = min(nsteps, (int)(blockIdx.y + 1) * per) * DS_CH;
  // decoder fragments of k-steps ks0..ks0+7 for the rows of sweep step n0
  constexpr int PF = 8;
  auto ldd = [&](int n0, int ks0, u32x4 (&d)[PF]) __attribute__((always_inline)) {
    if constexpr (NKS > 0) {
      // a prefetch past the block's last step rereads that step's rows
      // (n_end >= DS_CH: the grid gives every block at least one step's range)
      const int nn = min(n0, n_end - DS_CH);
      const uint16_t* drow = D + (int64_t)(nn + wave * 32 + (lane & 31)) * r + 8 * hl;
#pragma unroll
      for (int u = 0; u < PF; ++u)
        if (ks0 + u < NKS) d[u] = ld_u32x4(drow + 16 * (ks0 + u));
    } else {
      const uint16_t* drow = D + (int64_t)(n0 + wave * 32 + (lane & 31)) * r + 8 * hl;
#pragma unroll
      for (int u = 0; u < PF; ++u)
        d[u] = (ks0 + u < nks && n0 < n_end) ? ld_u32x4(drow + 16 * (ks0 + u))
                                             : u32x4{0u, 0u, 0u, 0u};
    }
  };
  const int chl = wave * 32 + (lane & 31);  // lane's channel within a step
  // the centers of the lane's 32 elements for sweep step n0 (a step past the
  // block's last rereads that step's channels)
  uint32_t mk[32];
  auto ldmu = [&](int n0) __attribute__((always_inline)) {
    const int nn = min(n0, n_end - DS_CH);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        mk[16 * i + e] = mu[(int64_t)sIdx[32 * i + acc_row(e, lane)] * W + nn + chl];
  };
  u32x4 d0[PF], d1[PF];
  ldd(n_beg, 0, d0);
  // as at the end of every step: the first decoder group is in registers
  // before the loop, so its first MFMAs need no wait on any path
  __builtin_amdgcn_s_waitcnt(DS_WAIT_VM0);
  ldmu(n_beg);
  for (int n0 = n_beg; n0 < n_end; n0 += DS_CH) {
    f32x16 acc[2] = {zero16(), zero16()};
    auto mm = [&](int ks0, const u32x4 (&d)[PF]) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        if (ks0 + u >= nks) break;
        const bf16x8 dv = as_bf16x8(d[u]);
#pragma unroll
        for (int i = 0; i < 2; ++i) acc[i] = mfma_bf16(afrag(i, ks0 + u), dv, acc[i]);
      }
    };
    // d0 holds k-steps 0..PF-1 of this step on entry; the last group's
    // buffer is refilled with the next step's first k-steps
    if constexpr (NKS > 0) {
      constexpr int NG = (NKS + PF - 1) / PF;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        u32x4(&cur)[PF] = (g & 1) ? d1 : d0;
        u32x4(&nxt)[PF] = (g & 1) ? d0 : d1;
        if (g + 1 < NG) ldd(n0, PF * (g + 1), nxt);
        else ldd(n0 + DS_CH, 0, nxt);
#pragma unroll
        for (int u = 0; u < PF; ++u) {
          if (PF * g + u >= NKS) break;
          const bf16x8 dv = as_bf16x8(cur[u]);
#pragma unroll
          for (int i = 0; i < 2; ++i) acc[i] = mfma_bf16(afrag(i, PF * g + u), dv, acc[i]);
        }
      }
      if constexpr (NG % 2 == 1) {
#pragma unroll
        for (int u = 0; u < PF; ++u) d0[u] = d1[u];
      }
    } else {
      for (int ks0 = 0; ks0 < nks; ks0 += 2 * PF) {
        if (ks0 + PF < nks) ldd(n0, ks0 + PF, d1);
        else ldd(n0 + DS_CH, 0, d1);
        mm(ks0, d0);
        if (ks0 + 2 * PF < nks) ldd(n0, ks0 + 2 * PF, d0);
        else if (ks0 + PF < nks) ldd(n0 + DS_CH, 0, d0);
        if (ks0 + PF < nks) mm(ks0 + PF, d1);
      }
      if (((nks + PF - 1) / PF) % 2 == 1) {
#pragma unroll
        for (int u = 0; u < PF; ++u) d0[u] = d1[u];
      }
    }
    __syncthreads();  // the previous step's reads of sO are done
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int tl = 32 * i + acc_row(e, lane);
        const uint16_t v = f32_to_bf16_bits(acc[i][e] + bf16_bits_to_f32(uint16_t(mk[16 * i + e])));
        if constexpr (ROWS) sO[tl * OS + chl] = v;
        else sO[chl * OS + tl] = v;
      }
    __syncthreads();
    // Every load done before the first store: while stores and loads are both
    // in flight the compiler can only wait for a load with vmcnt(0), stores
    // included, and the next step's first MFMAs would wait for this step's
    // stores.  The loads still pending here are the next step's first
    // decoder group, requested a whole group of MFMAs ago.
    __builtin_amdgcn_s_waitcnt(DS_WAIT_VM0);
    if constexpr (ROWS) {
      // 64 token rows x 16 chunks of 8 channels
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = tid + 256 * u, tl = c >> 4, cc = c & 15;
        if (tl < nvalid)
          *reinterpret_cast<u32x4*>(out + (m0 + tl) * W + n0 + cc * 8) =
              *reinterpret_cast<const u32x4*>(sO + tl * OS + cc * 8);
      }
    } else {
      // 128 channel rows x 8 chunks of 8 tokens (ld % 8 == 0: aligned chunks)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = tid + 256 * u, cl = c >> 3, tc = (c & 7) * 8;
        uint16_t* dst = out + (int64_t)(n0 + cl) * ld + m0 + tc;
        const uint16_t* src = sO + cl * OS + tc;
        if (tc + 8 <= nvalid) {
          *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
        } else {
          for (int k = 0; k < 8 && tc + k < nvalid; ++k) dst[k] = src[k];
        }
      }
    }
    // the next step's centers: their latency runs under the barrier and the
    // first MFMA group
    ldmu(n0 + DS_CH);
  }
}

// ---------------------------------------------------------------------------
// Decoder stationary, both branches in one launch.  The unit of work is
// (branch, 128-channel block, 32-token group); each block (8 waves, one
// block per CU) takes an equal share of the units in that order.  For each
// run of its units with one (branch, channel block) it loads those 128
// decoder rows once into LDS (rows padded by 16 bytes, so the 16 rows one
// operand read touches fall on distinct banks); then every wave takes every
// eighth unit of the run: the 32 tokens' INT4 codes go straight into
// registers (16 bytes per lane per 64 coefficients, one unit ahead) and are
// dequantised there into the MFMA's B operand, against the decoder rows as A
// operand, so one dequantised fragment feeds four MFMAs (128 channels) and
// no decoder row is streamed per token.  The result plus the token's center
// is rounded to bf16 and leaves through a per-wave LDS tile as 16-byte
// stores: K rows [token][channel], V transposed [channel][token], whole
// groups of 32 (rows or columns up to the next multiple of 32 are written).
// Logical k order of MFMA step (j, s): lane half hl holds coefficients
// 64 j + 32 hl + 8 s .. + 7 in both operands, so a lane's codes for a group
// of 64 coefficients are 16 consecutive bytes (r % 64 == 0) under one scale
// (INT4 groups of 32 or more coefficients).
// ---------------------------------------------------------------------------
constexpr int DP_SK = 72, DP_SV = 40;  // staging strides (bf16): K [32][72], V [64][40]
constexpr int DP_STAGE = 64 * DP_SV;   // bf16 per wave (>= 32 * 72)

struct DecodePair {
  BranchArgs br[2];  // K, V
  uint16_t* kout;    // [total][W]
  uint16_t* vt;      // [W][ld]
  int64_t ld;
  RangeTable rows;
  int W, gshift, G;  // group = 1 << gshift; G = token groups of 32
  int64_t U;         // units = 2 (W / 128) G
};

template <int NJ>
__global__ __launch_bounds__(512, 1) void k_decode_pair(const DecodePair p) {
  extern __shared__ __attribute__((aligned(16))) char dsm[];
  constexpr int R = NJ * 64, RS = R + 8;
  uint16_t* sD = reinterpret_cast<uint16_t*>(dsm);
  const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5, n = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint16_t* sO = sD + 128 * RS + wave * DP_STAGE;
  const int W = p.W, ncb = W / 128;
  const int64_t total = p.rows.total;
  const int64_t u_beg = p.U * blockIdx.x / gridDim.x, u_end = p.U * (blockIdx.x + 1) / gridDim.x;
  // the row ranges in LDS: the token lookup then waits on LDS only, never
  // behind the stores of the unit before (global loads and stores share one
  // in-order counter)
  __shared__ int64_t sBeg[NKV_MAX_SEGMENTS], sPre[NKV_MAX_SEGMENTS + 1];
  const int nrange = p.rows.n;
  if (tid < nrange) sBeg[tid] = p.rows.begin[tid];
  if (tid <= nrange) sPre[tid] = p.rows.prefix[tid];
  auto token = [&](int64_t j) __attribute__((always_inline)) {
    int k = 0;
    while (k + 1 < nrange && sPre[k + 1] <= j) ++k;
    return sBeg[k] + (j - sPre[k]);
  };

  struct Pre {
    u32x4 c[NJ];
    uint16_t s[NJ];
    int32_t a;
  };
  for (int64_t s0 = u_beg; s0 < u_end;) {
    const int64_t seg = s0 / p.G;  // branch * ncb + channel block (block-uniform)
    const int64_t s1 = min(u_end, (seg + 1) * p.G);
    const int br = (int)(seg / ncb), cb = (int)(seg - (int64_t)br * ncb);
    const BranchArgs& b = p.br[br];
    // ---- the run's decoder rows cb*128 .. +127 into LDS ----------------------
    __syncthreads();  // every wave is done with the previous run's rows
    {
      const uint16_t* D = static_cast<const uint16_t*>(b.decoder) + (int64_t)cb * 128 * R;
      constexpr int NB = 128 * R / 8, PER = NB / 512;
      static_assert(NB % 512 == 0, "whole rounds of 16-byte pieces");
      // (the thread's slots from an opaque copy of its index: hoisted out of
      // the loops, their offsets would hold registers for the whole kernel)
      int ti = tid;
      asm volatile("" : "+v"(ti));
      // four 16-byte pieces per thread in flight at a time (once per run)
#pragma unroll
      for (int i0 = 0; i0 < PER; i0 += 4) {
        u32x4 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = ti + 512 * (i0 + i);
          if (i0 + i < PER) v[i] = ld_u32x4(D + 8 * c);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = ti + 512 * (i0 + i);
          if (i0 + i < PER) {
            const int row = c / (R / 8), blk = c - row * (R / 8);
            *reinterpret_cast<u32x4*>(sD + row * RS + 8 * blk) = v[i];
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
    // ---- this wave's units of the run -----------------------------------------
    const uint16_t* mu = static_cast<const uint16_t*>(b.centers);
    auto fetch = [&](int64_t u, Pre& f) __attribute__((always_inline)) {
      const int64_t g = u - seg * p.G;
      const int64_t m = min(g * 32 + n, total - 1);  // rows past the end repeat the last token
      const int64_t t = token(m);
      f.a = b.idx[t];
      const uint8_t* crow = b.codes + t * (R / 2) + 16 * hl;
#pragma unroll
      for (int j = 0; j < NJ; ++j) f.c[j] = ld_u32x4(crow + 32 * j);
      // the lane's scales: one per 32 coefficients (group >= 32); a token's
      // row holds R / group of them
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        f.s[j] = b.scales[t * (R >> p.gshift) + ((64 * j + 32 * hl) >> p.gshift)];
    };
    // the unit loop, compiled once per branch (the epilogue's layout differs)
    auto units = [&](auto brc) __attribute__((always_inline)) {
    constexpr int BR = decltype(brc)::value;
    // (every fetch is issued, a past-the-end unit clamped to the run's last:
    // the same memory operations on every path keep the waits exact)
    Pre nxt;
    auto one = [&](int64_t u) __attribute__((always_inline)) {
      const Pre cur = nxt;
      // The next unit's codes are requested halfway through this unit's
      // MFMAs (when half of this unit's codes are dead) and the centers of
      // this unit (the lane's 16 runs of 4 channels) two code groups before
      // the end: both land under MFMAs, without holding registers all along.
      uint2 mv[4][4];
      const uint16_t* mrow = mu + (int64_t)cur.a * W + cb * 128 + 4 * hl;
      auto load_mu = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq)
            mv[blk][gq] = *reinterpret_cast<const uint2*>(mrow + blk * 32 + gq * 8);
      };
      f32x16 acc[4];
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) acc[blk] = zero16();
      // the lane's decoder rows: two bases (rows n and 64 + n), each with
      // constant offsets inside the 16-bit LDS offset field; from an opaque
      // lane index, so they are formed here rather than held all along
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const uint16_t* arow0 = sD + (ln & 31) * RS + 32 * (ln >> 5);
      const uint16_t* arow1 = arow0 + 64 * RS;
      // decoder fragments of step k (k = 4 j + s): read one step ahead of
      // their MFMAs; the fences keep the scheduler from hoisting every read
      // of the unrolled loop (and its registers) to the top
      auto read_a = [&](int k, bf16x8 (&af)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
          af[blk] = as_bf16x8(*reinterpret_cast<const u32x4*>(
              (blk < 2 ? arow0 : arow1) + (blk & 1) * 32 * RS + 64 * (k >> 2) + 8 * (k & 3)));
      };
      bf16x8 a0[4], a1[4];
      read_a(0, a0);
#pragma unroll
      for (int k = 0; k < 4 * NJ; ++k) {
        bf16x8 (&ac)[4] = (k & 1) ? a1 : a0;
        bf16x8 (&an)[4] = (k & 1) ? a0 : a1;
        if (k + 1 < 4 * NJ) read_a(k + 1, an);
        if (k == 4 * (NJ / 2)) fetch(min(u + 8, s1 - 1), nxt);
        if (k == 4 * (NJ - 2)) load_mu();
        const int j = k >> 2, s = k & 3;
        const float sc = fp16_bits_to_f32(cur.s[j]);
        const float nb = -8.f * sc;
        // INT4 two's complement -> offset binary, nibbles spread to bytes:
        // (n' - 8) sc is exact in fp32 (fma), then one rounding to bf16
        const uint32_t w = cur.c[j][s] ^ 0x88888888u;
        const uint32_t lo = w & 0x0f0f0f0fu, hi = (w >> 4) & 0x0f0f0f0fu;
        u32x4 bv;
#pragma unroll
        for (int h = 0; h < 4; ++h)
          bv[h] = pack_bf16x2(fmaf((float)((lo >> (8 * h)) & 0xffu), sc, nb),
                              fmaf((float)((hi >> (8 * h)) & 0xffu), sc, nb));
        const bf16x8 bf = as_bf16x8(bv);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) acc[blk] = mfma_bf16(ac[blk], bf, acc[blk]);
        __builtin_amdgcn_sched_barrier(0);
      }
      // ---- epilogue: + center, bf16, through LDS as 16-byte stores -------------
      const int64_t g = u - seg * p.G, m0 = g * 32;
      // accumulators + centers -> bf16 pairs first (frees the accumulators)
      uint2 pk[4][4];
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const uint2 mq = mv[blk][gq];
          pk[blk][gq] = uint2{
              pack_bf16x2(acc[blk][4 * gq + 0] + bf16_bits_to_f32(uint16_t(mq.x & 0xffffu)),
                          acc[blk][4 * gq + 1] + bf16_bits_to_f32(uint16_t(mq.x >> 16))),
              pack_bf16x2(acc[blk][4 * gq + 2] + bf16_bits_to_f32(uint16_t(mq.y & 0xffffu)),
                          acc[blk][4 * gq + 3] + bf16_bits_to_f32(uint16_t(mq.y >> 16)))};
        }
      // one base per lane, every element at a constant offset from it
      int le = lane;
      asm volatile("" : "+v"(le));
      uint16_t* sw = BR == 0 ? sO + (le & 31) * DP_SK + 4 * (le >> 5)
                             : sO + 4 * (le >> 5) * DP_SV + (le & 31);
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
        for (int bl = 0; bl < 2; ++bl)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int cc = bl * 32 + gq * 8;  // + 4 hl, in the base
            const uint2 v = pk[2 * hb + bl][gq];
            if constexpr (BR == 0) {
              *reinterpret_cast<uint2*>(sw + cc) = v;
            } else {
              sw[(cc + 0) * DP_SV] = uint16_t(v.x & 0xffffu);
              sw[(cc + 1) * DP_SV] = uint16_t(v.x >> 16);
              sw[(cc + 2) * DP_SV] = uint16_t(v.y & 0xffffu);
              sw[(cc + 3) * DP_SV] = uint16_t(v.y >> 16);
            }
          }
        // the wave's own tile: LDS operations of a wave complete in order, so
        // only the compiler must keep the stores above the reads
        asm volatile("" ::: "memory");
        // whole groups of 32 rows (the caller's buffers hold them; the rows
        // past the end repeat the last token and are overwritten later)
        if constexpr (BR == 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int c = le + 64 * i, tk = c >> 3, c8 = c & 7;
            *reinterpret_cast<u32x4*>(p.kout + (m0 + tk) * W + cb * 128 + hb * 64 + 8 * c8) =
                *reinterpret_cast<const u32x4*>(sO + tk * DP_SK + 8 * c8);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int c = le + 64 * i, ch = c >> 2, t8 = 8 * (c & 3);
            *reinterpret_cast<u32x4*>(p.vt + (int64_t)(cb * 128 + hb * 64 + ch) * p.ld + m0 + t8) =
                *reinterpret_cast<const u32x4*>(sO + ch * DP_SV + t8);
          }
        }
        asm volatile("" ::: "memory");
      }
    };
    // The first unit is a copy of its own: the loop is then entered only
    // after a unit's memory operations, as on every later trip, and the
    // compiler's waits at its head count the previous unit's stores as
    // still in flight instead of waiting for them.
    const int64_t u0 = s0 + wave;
    fetch(min(u0, s1 - 1), nxt);
    if (u0 < s1) {
      one(u0);
      for (int64_t u = u0 + 8; u < s1; u += 8) one(u);
    }
    };
    if (br == 0) units(std::integral_constant<int, 0>{});
    else units(std::integral_constant<int, 1>{});
    s0 = s1;
  }
}

size_t decode_stationary_lds(int r) {
  const size_t o = std::max<size_t>((size_t)DS_TOK * (DS_CH + 8), (size_t)DS_CH * (DS_TOK + 8));
  return (size_t)DS_TOK * (r + 8) * 2 + o * 2;
}

nkv_status launch_decode_tuned(const BranchArgs& b, int W, int r, int group,
                               const RangeTable& rows, uint16_t* out, int64_t ld, bool transposed,
                               hipStream_t st) {
  if (rows.total == 0) return NKV_OK;
  if (r <= 512 && W % DS_CH == 0 && (transposed ? ld % 8 == 0 : true)) {
    const size_t lds = decode_stationary_lds(r);
    // about four blocks per CU: split the channel sweep when tokens are few
    const int64_t tb = ceil_div(rows.total, DS_TOK);
    const int ysplit = (int)std::min<int64_t>(W / DS_CH, std::max<int64_t>(1, 1024 / tb));
    const dim3 grid((unsigned)tb, (unsigned)ysplit);
    const int nks = r % 16 == 0 ? r / 16 : 0;
    auto go = [&](auto kern) -> nkv_status {
      if (lds > 64 * 1024)
        NKV_HIP_CHECK(hipFuncSetAttribute((const void*)kern,
                                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
      hipLaunchKernelGGL(kern, grid, dim3(256), lds, st, b, rows, W, r, group, out, ld);
      return NKV_OK;
    };
    nkv_status e;
    switch (nks) {
#define NKV_DECODE_NKS(n)                                                                    \
  case n:                                                                                   \
    e = transposed ? go(k_decode_stationary<false, n>) : go(k_decode_stationary<true, n>);  \
    break;
      NKV_DECODE_NKS(6)
      NKV_DECODE_NKS(8)
      NKV_DECODE_NKS(12)
      NKV_DECODE_NKS(16)
      NKV_DECODE_NKS(24)
      NKV_DECODE_NKS(32)
#undef NKV_DECODE_NKS
      default:
        e = transposed ? go(k_decode_stationary<false, 0>) : go(k_decode_stationary<true, 0>);
    }
    if (e) return e;
    NKV_LAUNCH_CHECK();
    return NKV_OK;
  }
  if (transposed) {
    DecodeTProblem p{W, (int)rows.total, r, group, b, rows, out, ld};
    return launch_gemm(p, 1, st);
  }
  DecodeProblem p{(int)rows.total, W, r, group, b, rows, out, ld, false};
  return launch_gemm(p, 1, st);
}

nkv_status launch_decode_pair_tuned(const BranchArgs& kb, const BranchArgs& vb, int W, int r,
                                    int group, const RangeTable& rows, uint16_t* kout,
                                    uint16_t* vt, int64_t ld, hipStream_t st) {
  if (rows.total == 0) return NKV_OK;
  auto al = [](const void* q, uintptr_t a) { return (reinterpret_cast<uintptr_t>(q) & (a - 1)) == 0; };
  const bool pow2 = group >= 32 && (group & (group - 1)) == 0 && r % group == 0;
  const bool fits = r % 64 == 0 && r >= 128 && r <= 448 && W % 128 == 0 && ld % 8 == 0 && pow2 &&
                    al(kb.codes, 16) && al(vb.codes, 16) && al(kb.decoder, 16) &&
                    al(vb.decoder, 16) && al(kb.centers, 8) && al(vb.centers, 8) &&
                    al(kout, 16) && al(vt, 16);
  if (!fits) {
    nkv_status e = launch_decode_tuned(kb, W, r, group, rows, kout, 0, false, st);
    if (e) return e;
    return launch_decode_tuned(vb, W, r, group, rows, vt, ld, true, st);
  }
  DecodePair p{};
  p.br[0] = kb;
  p.br[1] = vb;
  p.kout = kout;
  p.vt = vt;
  p.ld = ld;
  p.rows = rows;
  p.W = W;
  p.gshift = __builtin_ctz((unsigned)group);
  p.G = (int)ceil_div(rows.total, 32);
  p.U = 2 * (int64_t)(W / 128) * p.G;
  const int nblk = (int)std::min<int64_t>(device_cus(), ceil_div(p.U, 8));
  const size_t lds = ((size_t)128 * (r + 8) + 8 * DP_STAGE) * 2;
  auto go = [&](auto kern) -> nkv_status {
    NKV_HIP_CHECK(hipFuncSetAttribute((const void*)kern,
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
    hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(512), lds, st, p);
    NKV_LAUNCH_CHECK();
    return NKV_OK;
  };
  switch (r / 64) {
#define NKV_DP(nj) \
  case nj: return go(k_decode_pair<nj>);
    NKV_DP(2)
    NKV_DP(3)
    NKV_DP(4)
    NKV_DP(5)
    NKV_DP(6)
    NKV_DP(7)
#undef NKV_DP
    default: break;
  }
  return NKV_EUNSUPPORTED;  // not reached: r / 64 in 2..7 above
}

// ---------------------------------------------------------------------------
// current chunk -> attention workspace (K rows; V per-head transposed),
// plus zero padding of the key tail
// ---------------------------------------------------------------------------
__global__ void k_copy_rows(const uint16_t* __restrict__ src, int64_t n_rows, int W,
                            uint16_t* __restrict__ dst, int64_t pad_rows) {
  // 8 bf16 per thread; rows beyond n_rows up to pad_rows are zero-filled
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_row = W / 8;
  if (i >= pad_rows * per_row) return;
  const int64_t row = i / per_row;
  u32x4 v = u32x4{0u, 0u, 0u, 0u};
  if (row < n_rows) v = ld_u32x4(src + i * 8);
  *reinterpret_cast<u32x4*>(dst + i * 8) = v;
}

// V [n, W] -> V^T[h][dd][key0 + t] for t < n; zero for n <= t < n_pad
__global__ __launch_bounds__(256) void k_transpose_v(const uint16_t* __restrict__ src, int64_t n,
                                                     int64_t n_pad, int W, uint16_t* __restrict__ dst,
                                                     int64_t ld, int64_t key0) {
  __shared__ uint16_t tile[64][65];
  const int64_t t0 = (int64_t)blockIdx.x * 64;
  const int c0 = blockIdx.y * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int tt = i / 64, cc = i % 64;
    tile[tt][cc] = (t0 + tt < n) ? src[(t0 + tt) * W + c0 + cc] : uint16_t(0);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int cc = i / 64, tt = i % 64;
    const int c = c0 + cc;
    if (t0 + tt < n_pad) dst[((int64_t)(c >> 7) * 128 + (c & 127)) * ld + key0 + t0 + tt] = tile[tt][cc];
  }
}

// The same with 16-byte accesses (ld, key0 and n_pad multiples of 8): a
// 64-token x 64-channel tile is read as 8-channel chunks and written as
// 8-token chunks.
__global__ __launch_bounds__(256) void k_transpose_v16(const uint16_t* __restrict__ src, int64_t n,
                                                       int64_t n_pad, int W,
                                                       uint16_t* __restrict__ dst, int64_t ld,
                                                       int64_t key0) {
  __shared__ uint16_t tile[64][64 + 2];
  const int64_t t0 = (int64_t)blockIdx.x * 64;
  const int c0 = blockIdx.y * 64;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = threadIdx.x + 256 * k, tt = i >> 3, cc = (i & 7) * 8;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (t0 + tt < n) v = ld_u32x4(src + (t0 + tt) * W + c0 + cc);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      tile[tt][cc + 2 * q] = uint16_t(v[q] & 0xffffu);
      tile[tt][cc + 2 * q + 1] = uint16_t(v[q] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = threadIdx.x + 256 * k, cc = i >> 3, tt = (i & 7) * 8;
    if (t0 + tt >= n_pad) continue;  // n_pad % 8 == 0: a chunk is wholly in or out
    u32x4 v;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      v[q] = uint32_t(tile[tt + 2 * q][cc]) | (uint32_t(tile[tt + 2 * q + 1][cc]) << 16);
    const int c = c0 + cc;
    *reinterpret_cast<u32x4*>(dst + ((int64_t)(c >> 7) * 128 + (c & 127)) * ld + key0 + t0 + tt) = v;
  }
}

nkv_status launch_stage_current(const uint16_t* ck, const uint16_t* cv, int64_t n_cur,
                                int64_t n_pad_tail, int W, uint16_t* kall, uint16_t* vt,
                                int64_t ld, int64_t key0, hipStream_t st) {
  // rows key0 .. key0 + n_pad_tail of K_all: current chunk then zeros
  if (n_pad_tail <= 0) return NKV_OK;
  const int64_t nthreads = n_pad_tail * (W / 8);
  hipLaunchKernelGGL(k_copy_rows, dim3((unsigned)ceil_div(nthreads, 256)), dim3(256), 0, st, ck,
                     n_cur, W, kall + key0 * W, n_pad_tail);
  NKV_LAUNCH_CHECK();
  const bool wide = ld % 8 == 0 && key0 % 8 == 0 && n_pad_tail % 8 == 0 &&
                    ((reinterpret_cast<uintptr_t>(cv) | reinterpret_cast<uintptr_t>(vt)) & 15) == 0;
  if (wide)
    hipLaunchKernelGGL(k_transpose_v16, dim3((unsigned)ceil_div(n_pad_tail, 64), W / 64), dim3(256),
                       0, st, cv, n_cur, n_pad_tail, W, vt, ld, key0);
  else
    hipLaunchKernelGGL(k_transpose_v, dim3((unsigned)ceil_div(n_pad_tail, 64), W / 64), dim3(256), 0,
                       st, cv, n_cur, n_pad_tail, W, vt, ld, key0);
  NKV_LAUNCH_CHECK();
  return NKV_OK;
}

}  // namespace nkv
