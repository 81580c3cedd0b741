// Tuned encoder and decoder of libnanokv (bf16, MFMA).
//
// Encoder (NanoKV abstract; Figure 4(b)):
//   1. ||mu_a||^2 per center (fp32).
//   2. Distance GEMM  d(a, t) = ||mu_a||^2 - 2 mu_a . x_t  on bf16 MFMA (bf16
//      products are exact in fp32); the epilogue reduces each token's
//      column to (min distance, lowest index) and merges blocks with a
//      64-bit atomicMin on (order-preserving distance bits << 32 | a).
//   3. Projection GEMM z = E (x - mu_a): the fp32 residual (exact for bf16
//      inputs) is split into three bf16 terms hi + mid + lo = e, so three
//      exact-product MFMA passes with fp32 accumulation give the projection
//      at fp32 accuracy.
//   4. INT4 group quantisation of z.
// Decoder (Figure 4(b)): x_hat = mu_a + D (code * scale) as a GEMM whose A
// loader dequantises INT4 on the fly and whose epilogue adds the center and
// writes bf16 rows (K) or per-head transposed columns (V).
#include "prof.hpp"
#include "quant.hpp"
#include "tuned_internal.hpp"

namespace nkv {

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------
__global__ void k_center_norms(const uint16_t* __restrict__ mu, int A, int W, float* __restrict__ out) {
  const int a = blockIdx.x;
  const uint16_t* row = mu + (int64_t)a * W;
  float acc = 0.f;
  // lane l adds elements l, l + 64, ... in that order; eight loads are
  // issued before their FMAs (the same sums, without one round trip each)
  int w = threadIdx.x;
  for (; w + 7 * 64 < W; w += 8 * 64) {
    uint16_t b[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) b[u] = row[w + 64 * u];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float v = bf16_bits_to_f32(b[u]);
      acc = fmaf(v, v, acc);
    }
  }
  for (; w < W; w += 64) {
    const float v = bf16_bits_to_f32(row[w]);
    acc = fmaf(v, v, acc);
  }
  acc = wave_sum(acc);
  if (threadIdx.x == 0) out[a] = acc;
}

__global__ void k_fill_u64(uint64_t* p, int64_t n, uint64_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void k_unpack_idx(const uint64_t* __restrict__ keys, int64_t n, int32_t* __restrict__ idx) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) idx[i] = (int32_t)(keys[i] & 0xffffffffu);
}

__device__ __forceinline__ u32x4 load8_bf16(const uint16_t* base, int64_t row, int ld, int k,
                                            bool ok) {
  if (!ok) return u32x4{0u, 0u, 0u, 0u};
  return ld_u32x4(base + row * ld + k);
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
  uint64_t* keys;
  __device__ u32x4 load_a(int, int m, int k) const { return load8_bf16(mu, m, K, k, m < M && k < K); }
  __device__ u32x4 load_b(int, int n, int k) const { return load8_bf16(x, n, K, k, n < N && k < K); }
  __device__ void epilogue(int, int m0, int n0, int lane, const f32x16 (&acc)[2][2]) const {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float best = INFINITY;
      int besta = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int a = m0 + 32 * i + acc_row(e, lane);
          if (a < M) {
            const float dist = mu2[a] - 2.f * acc[i][j][e];
            if (dist < best || (dist == best && a < besta)) { best = dist; besta = a; }
          }
        }
      }
      const float ob = __shfl_xor(best, 32, 64);
      const int oa = __shfl_xor(besta, 32, 64);
      if (ob < best || (ob == best && oa < besta)) { best = ob; besta = oa; }
      const int n = n0 + 32 * j + (lane & 31);
      if (lane < 32 && n < N && besta != 0x7fffffff) {
        const uint64_t key = ((uint64_t)ordered_bits(best) << 32) | (uint32_t)besta;
        atomicMin(reinterpret_cast<unsigned long long*>(keys + n), (unsigned long long)key);
      }
    }
  }
};

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
    if (c + 1 < nchunk) put_res(rs ^ 1, xv[rs ^ 1], mv[rs ^ 1]);
    __syncthreads();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  for (int c = 0; c < nchunk; c += 6) {
    step(c, I0{}, I0{});
    if (c + 1 < nchunk) step(c + 1, I1{}, I1{});
    if (c + 2 < nchunk) step(c + 2, I0{}, I2{});
    if (c + 3 < nchunk) step(c + 3, I1{}, I0{});
    if (c + 4 < nchunk) step(c + 4, I0{}, I1{});
    if (c + 5 < nchunk) step(c + 5, I1{}, I2{});
  }
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

size_t tuned_assign_workspace(int64_t N, int32_t A) {
  return align_up(sizeof(float) * A, 256) + align_up(sizeof(uint64_t) * N, 256);
}

nkv_status tuned_assign(const nkv_shape* s, const void* x, int64_t N, const void* centers,
                        int32_t A, int32_t* idx, char* ws, hipStream_t st) {
  const int W = s->H * s->d;
  float* mu2 = reinterpret_cast<float*>(ws);
  uint64_t* keys = reinterpret_cast<uint64_t*>(ws + align_up(sizeof(float) * A, 256));
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* mub = static_cast<const uint16_t*>(centers);
  hipLaunchKernelGGL(k_center_norms, dim3(A), dim3(64), 0, st, mub, A, W, mu2);
  NKV_LAUNCH_CHECK();
  hipLaunchKernelGGL(k_fill_u64, dim3((unsigned)ceil_div(N, 256)), dim3(256), 0, st, keys, N,
                     ~0ull);
  NKV_LAUNCH_CHECK();
  DistProblem dp{A, (int)N, W, mub, xb, mu2, keys};
  nkv_status e;
  // (the register-staged GEMM with 64-wide k steps: measured faster here
  // than the direct-to-LDS one, whose 32-wide steps double the barriers)
  if ((e = launch_gemm(dp, 1, st))) return e;
  hipLaunchKernelGGL(k_unpack_idx, dim3((unsigned)ceil_div(N, 256)), dim3(256), 0, st, keys, N, idx);
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
