// NanoKV-Fast low-dimensional read on the tuned path (NanoKV pages,
// Figure 4(d): queries are reduced into coefficient space, scored and
// accumulated there, and the output dimension is restored before LSE
// merging; the abstract: the stored coefficients are reused).
//
// Per head h and low-routed token t (leading r_low coefficients c):
//   s = tau (q~_h . c^K_t + T_h[a^K_t]),   T_h[a] = q_h . mu^K_{a,h}
//   acc_h += p c^V_t,   M_h[a^V_t] += p,   O = (D_{V,h} acc_h + M_h mu^V_h) / sum p
//
// Design for CDNA4:
//  * The coefficients of a token are shared by every head (joint
//    head-channel coding), so one staged coefficient tile feeds 256 query
//    rows of a head through MFMA: scores as fp16 MFMA (q~ . c), the
//    coefficient accumulation as bf16 MFMA (P c^V).
//  * The per-row center tables T (read) and M (accumulate) have A entries per
//    row -- too large for LDS.  Low-routed tokens are therefore
//    counting-sorted into buckets by (a^V range, a^K range) of 64 centers
//    each (and within a bucket by the half of the a^V range); a block walks
//    the buckets in order, keeps the 64-entry slice of T in LDS (recomputed
//    per bucket by MFMA, q_h . mu^K exact-product bf16) and gathers it per
//    score with conflict-free LDS reads, and accumulates the 64 masses of the
//    current a^V range in registers through a one-hot MFMA (flushed to HBM
//    when the range is finished).
//  * Softmax uses a per-row upper bound B on every score instead of a
//    running maximum (B = tau (max over present centers of T + |q~| max|c^K|)),
//    so p = 2^(x - B) <= 1 needs no rescaling of the LDS tables and partial
//    sums from any split simply add.  Rows whose bound could be loose by
//    more than 2^60 are recomputed exactly by the generic kernel.
#include <algorithm>
#include <vector>

#include "lowdim.hpp"
#include "prof.hpp"

namespace nkv {

namespace {

constexpr int NT = 64;        // keys per tile (bucket padding unit)
constexpr int CR = 64;        // centers per range
constexpr int TS = 65;        // LDS row stride of the center tables (odd: rows spread over banks)
constexpr int CHUNK = 256;    // tokens per counting chunk
constexpr float BOUND_GAP_LIMIT = 60.f;  // log2 units

// Tile image: the exact LDS layout the main kernel consumes, so a tile moves
// from HBM/L2 to LDS with plain 1 KiB direct-to-LDS loads.  Both operand
// regions are fragment-major: every MFMA operand fragment is one 1 KiB chunk
// in which lane l's 16 bytes sit at l * 16 (one conflict-free ds_read_b128).
//   [0, ck_bytes)        K coefficients (fp16): chunk (kb, ks) holds key
//                        kb*32 + l%32, coefficients 16 ks + 8 (l/32) .. +7
//   [cv_off, +cv_bytes)  V coefficients, then the a^V one-hot over the 64
//                        centers of the range (bf16): chunk (kb, j, db) holds
//                        row db*32 + l%32 (a coefficient, or a center for
//                        db >= rp/32) for keys kb*32 + 16 j + 4 (l/32) + {0..3}
//                        and the same + 8 (the key order of P in registers)
//   [ko_off, +64)        per key: byte offset of its a^K slot in the T table row
//                        (one byte, 4 x the center's place in its range),
//                        ordered so that lane l's 16 keys of 32-key block kb
//                        (the keys of its score accumulator elements) are
//                        the 16 bytes at kb*32 + 16 (l/32): one 16-byte read
//   [hd_off, +16)        header: the facts of the FOLLOWING tile (its bucket,
//                        whether it opens that bucket, the a^K range of the
//                        bucket after it or -1; zero after the last tile), so
//                        a kernel learns them while it works on this tile;
//                        then this tile's step mask: bit 2s + u set when a
//                        real key of 16-key step s (keys 16 s .. 16 s + 15)
//                        has its V center in half u of the a^V range
struct TileGeom {
  int rlp, rp, nks, nvb, ck_bytes, cv_off, cv_bytes, ko_off, hd_off, bytes;
};
__host__ __device__ constexpr TileGeom tile_geom(int rlp) {
  const int rp = (rlp + 31) / 32 * 32;
  const int nks = rlp / 16, nvb = rp / 32 + CR / 32;  // K steps; V + one-hot row blocks
  const int ck_bytes = (NT / 32) * nks * 1024, cv_bytes = (NT / 32) * 2 * nvb * 1024;
  const int ko_off = ck_bytes + cv_bytes, hd_off = ko_off + NT;
  return TileGeom{rlp, rp, nks, nvb, ck_bytes, ck_bytes, cv_bytes, ko_off, hd_off,
                  (hd_off + 16 + 1023) / 1024 * 1024};
}

// Center-mass planes (bf16 hi | lo: 2 WS columns per (query m, head zb of
// the group) row) are stored in blocks of 128 rows x 32 columns (8 KiB):
// block (zb * nmt + m / 128) * (2 WS / 32) + col / 32, then row m % 128,
// then column col % 32 (nmt = ceil(Nq / 128)).  The restoration's K steps
// of 32 columns then read one contiguous block per 128 query rows, and a
// wave's flush of 32 rows writes contiguous 2 KiB pieces.
__host__ __device__ inline int64_t mass_pos(int64_t m, int zb, int col, int64_t nmt, int WS) {
  return ((((int64_t)zb * nmt + (m >> 7)) * (WS >> 4) + (col >> 5)) * 128 + (m & 127)) * 32 +
         (col & 31);
}

struct Plan {
  int64_t n_low = 0, nchunk = 0, max_tiles = 0, max_slots = 0, rows = 0;
  int GK = 0, GV = 0, NB = 0, rlp = 0, rp = 0, ra = 0, av = 0, avp = 0;
  TileGeom g;
  // byte offsets inside the low-path workspace
  size_t racc, rell;  // split coefficient sums reduced to bf16 hi/lo planes, and their ell
  size_t rmass;       // split center masses reduced to planes (one a^V range only), or 0
  size_t dkt, mvt, qt32, qt16, bound, tmax, present, misc, flags, cnt, base, tile_start, bcount,
      tile_bucket, perm, img, acc, wmass, ell, total;
};

Plan make_plan(const nkv_shape* s, int32_t A_k, int32_t A_v, const RangeTable& low, int32_t r_low,
               int64_t Nq, int64_t part_units) {
  Plan P;
  const int64_t W = (int64_t)s->H * s->d;
  P.n_low = low.total;
  P.rows = Nq * s->H;
  P.GK = (int)ceil_div(A_k, CR);
  P.GV = (int)ceil_div(A_v, CR);
  P.NB = P.GK * P.GV;
  P.nchunk = ceil_div(P.n_low, CHUNK);
  P.max_tiles = ceil_div(P.n_low, NT) + P.NB;
  P.max_slots = P.max_tiles * NT;
  P.rlp = (int)ceil_div(r_low, 16) * 16;
  P.rp = (int)ceil_div(r_low, 32) * 32;
  P.ra = P.rp;
  P.av = (int)ceil_div(A_v, 32) * 32;
  P.avp = P.av;
  P.g = tile_geom(P.rlp);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  P.dkt = take(sizeof(uint16_t) * r_low * W);
  P.mvt = take(sizeof(uint16_t) * W * P.avp);
  P.qt32 = take(sizeof(float) * P.rows * r_low);
  P.qt16 = take(sizeof(uint16_t) * P.rows * P.rlp);
  P.bound = take(sizeof(float) * P.rows);
  P.tmax = take(sizeof(uint32_t) * P.rows);
  P.present = take(sizeof(uint32_t) * ceil_div(A_k, 64) * 64);  // cleared to a whole 64-center block
  P.misc = take(sizeof(uint32_t) * 4);
  P.flags = take(sizeof(int32_t) * P.rows);
  // counting sort over sub-buckets: (bucket, which half of its a^V range)
  P.cnt = take(sizeof(int32_t) * P.nchunk * 2 * P.NB);
  P.base = take(sizeof(int32_t) * P.nchunk * 2 * P.NB);
  P.tile_start = take(sizeof(int32_t) * (P.NB + 1));
  P.bcount = take(sizeof(int32_t) * P.NB);
  P.tile_bucket = take(sizeof(int32_t) * P.max_tiles);
  P.perm = take(sizeof(int32_t) * P.max_slots);
  P.img = take((size_t)P.max_tiles * P.g.bytes);
  // partial sums of the main pass: (split, query, head of the group) rows
  const int64_t prows = Nq * part_units;
  // fp32 partials, or (one split) bf16 hi/lo planes of the same byte size:
  // acc rows of 2 x ra; mass rows of 2 x GV * 64 bf16, in 128-row blocks
  // (the rows of every head of the read, Nq rounded up to 128)
  P.acc = take(sizeof(float) * prows * P.ra);
  P.wmass = take(std::max(sizeof(float) * prows * P.GV * CR,
                          sizeof(uint16_t) * 2 * P.GV * CR * s->H * ceil_div(Nq, 128) * 128));
  P.ell = take(sizeof(float) * prows);
  P.racc = take(sizeof(float) * P.rows * P.ra);   // rows of 2 x ra bf16
  P.rell = take(sizeof(float) * P.rows);
  // with a single a^V range the key-range splits leave fp32 mass partials
  // (several ranges split at range boundaries and write planes directly)
  P.rmass = P.GV == 1 ? take(sizeof(uint16_t) * 2 * CR * s->H * ceil_div(Nq, 128) * 128) : 0;
  P.total = off;
  return P;
}

// ---------------------------------------------------------------------------
// preparation kernels
// ---------------------------------------------------------------------------
__global__ void k_zero_u32(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// dst[c][r] = src[r][c] for r < R, c < C (bf16); dst row stride ldd (zero pad
// for r in [R, ldd) when pad_zero).
__global__ __launch_bounds__(256) void k_transpose_bf16(const uint16_t* __restrict__ src, int R,
                                                        int C, int lds, uint16_t* __restrict__ dst,
                                                        int ldd) {
  __shared__ uint16_t tile[64][65];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int rr = i / 64, cc = i % 64;
    tile[rr][cc] = (r0 + rr < R && c0 + cc < C) ? src[(int64_t)(r0 + rr) * lds + c0 + cc] : 0;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int cc = i / 64, rr = i % 64;
    if (c0 + cc < C && r0 + rr < ldd) dst[(int64_t)(c0 + cc) * ldd + r0 + rr] = tile[rr][cc];
  }
}

// The same with 16-byte accesses, for lds % 8 == 0, ldd % 8 == 0 and 16-byte
// aligned arrays: a 64 x 64 tile is read as 8-column chunks (columns past C
// read as zero, C % 8 == 0) and written as 8-row chunks (rows past R zero).
__global__ __launch_bounds__(256) void k_transpose_bf16_16(const uint16_t* __restrict__ src, int R,
                                                           int C, int lds,
                                                           uint16_t* __restrict__ dst, int ldd) {
  __shared__ uint16_t tile[64][64 + 2];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = threadIdx.x + 256 * k, rr = i >> 3, cc = (i & 7) * 8;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (r0 + rr < R && c0 + cc < C) v = ld_u32x4(src + (int64_t)(r0 + rr) * lds + c0 + cc);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      tile[rr][cc + 2 * q] = uint16_t(v[q] & 0xffffu);
      tile[rr][cc + 2 * q + 1] = uint16_t(v[q] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = threadIdx.x + 256 * k, cc = i >> 3, rr = (i & 7) * 8;
    if (c0 + cc >= C || r0 + rr >= ldd) continue;  // ldd % 8 == 0: a chunk is wholly in or out
    u32x4 v;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      v[q] = uint32_t(tile[rr + 2 * q][cc]) | (uint32_t(tile[rr + 2 * q + 1][cc]) << 16);
    *reinterpret_cast<u32x4*>(dst + (int64_t)(c0 + cc) * ldd + r0 + rr) = v;
  }
}

// Sub-bucket of a token: its bucket (a^V range, a^K range) times two, plus
// which half of the a^V range its V center lies in.  Within a bucket the
// tokens of the lower half come first, so most 16-key steps of a tile touch
// one half of the range and need only one of the two one-hot MFMAs.
__device__ __forceinline__ int sub_bucket_of(const BranchArgs& kb, const BranchArgs& vb, int64_t t,
                                             int GK) {
  const int av = vb.idx[t];
  return ((av / CR) * GK + kb.idx[t] / CR) * 2 + ((av % CR) >= CR / 2 ? 1 : 0);
}

__global__ __launch_bounds__(256) void k_bucket_count(BranchArgs kb, BranchArgs vb, RangeTable low,
                                                      int GK, int NB, int32_t* __restrict__ cnt,
                                                      uint32_t* __restrict__ present) {
  extern __shared__ int lc[];  // per sub-bucket
  for (int b = threadIdx.x; b < 2 * NB; b += 256) lc[b] = 0;
  __syncthreads();
  const int64_t j0 = (int64_t)blockIdx.x * CHUNK;
  for (int i = threadIdx.x; i < CHUNK; i += 256) {
    const int64_t j = j0 + i;
    if (j < low.total) {
      const int64_t t = map_index(low, j);
      atomicAdd(&lc[sub_bucket_of(kb, vb, t, GK)], 1);
      present[kb.idx[t]] = 1u;
    }
  }
  __syncthreads();
  for (int b = threadIdx.x; b < 2 * NB; b += 256) cnt[(int64_t)blockIdx.x * 2 * NB + b] = lc[b];
}

// Bucket totals and tile counts: one block per bucket sums its two
// sub-buckets' per-chunk counts.
__global__ __launch_bounds__(256) void k_bucket_tot(const int32_t* __restrict__ cnt, int nchunk,
                                                    int NB, int32_t* __restrict__ bcount,
                                                    int32_t* __restrict__ ntile) {
  __shared__ int red[256];
  const int b = blockIdx.x;
  int t = 0;
  for (int c = threadIdx.x; c < nchunk; c += 256)
    t += cnt[(int64_t)c * 2 * NB + 2 * b] + cnt[(int64_t)c * 2 * NB + 2 * b + 1];
  red[threadIdx.x] = t;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (threadIdx.x < st) red[threadIdx.x] += red[threadIdx.x + st];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    bcount[b] = red[0];
    ntile[b] = (red[0] + NT - 1) / NT;
  }
}

// one block of 1024 threads: exclusive prefix sums of the tile counts
// (padded tile ranges of the buckets, total at tile_start[NB]) and the
// tile -> bucket table
__global__ __launch_bounds__(1024) void k_bucket_tiles(const int32_t* __restrict__ ntile, int NB,
                                                       int32_t* __restrict__ tile_start,
                                                       int32_t* __restrict__ tile_bucket) {
  __shared__ int part[1024];
  const int tid = threadIdx.x;
  const int per = (NB + 1023) / 1024;
  const int lo = tid * per, hi = min(NB, lo + per);
  int sum = 0;
  for (int b = lo; b < hi; ++b) sum += ntile[b];
  part[tid] = sum;
  __syncthreads();
  for (int st = 1; st < 1024; st <<= 1) {  // Hillis-Steele inclusive scan
    const int v = tid >= st ? part[tid - st] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - sum;
  for (int b = lo; b < hi; ++b) {
    const int nt = ntile[b];
    tile_start[b] = run;
    for (int k = 0; k < nt; ++k) tile_bucket[run + k] = b;
    run += nt;
  }
  if (tid == 1023) tile_start[NB] = part[1023];
}

// per-chunk bases of a bucket's sub-buckets (its lower-half tokens first,
// each in chunk order): one block per bucket, an exclusive scan over the
// 2 x nchunk counts in that order, offset by the bucket's first slot
__global__ __launch_bounds__(256) void k_bucket_base(const int32_t* __restrict__ cnt, int nchunk,
                                                     int NB, const int32_t* __restrict__ tile_start,
                                                     int32_t* __restrict__ base) {
  __shared__ int part[256];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int n = 2 * nchunk;  // entry e: half e / nchunk, chunk e % nchunk
  const int per = (n + 255) / 256;
  const int lo = tid * per, hi = min(n, lo + per);
  auto at = [&](int e) -> int64_t {
    const int half = e >= nchunk ? 1 : 0, c = e - half * nchunk;
    return (int64_t)c * 2 * NB + 2 * b + half;
  };
  int sum = 0;
  for (int e = lo; e < hi; ++e) sum += cnt[at(e)];
  part[tid] = sum;
  __syncthreads();
  for (int st = 1; st < 256; st <<= 1) {
    const int v = tid >= st ? part[tid - st] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = tile_start[b] * NT + part[tid] - sum;
  for (int e = lo; e < hi; ++e) {
    const int64_t k = at(e);
    const int v = cnt[k];
    base[k] = run;
    run += v;
  }
}

// stable scatter: slot = base[chunk][sub-bucket] + rank of the token among
// the chunk's earlier tokens of the same sub-bucket
__global__ __launch_bounds__(256) void k_bucket_scatter(BranchArgs kb, BranchArgs vb, RangeTable low,
                                                        int GK, int NB,
                                                        const int32_t* __restrict__ base,
                                                        int32_t* __restrict__ perm) {
  __shared__ int bid[CHUNK];
  const int64_t j0 = (int64_t)blockIdx.x * CHUNK;
  const int n = (int)min<int64_t>(CHUNK, low.total - j0);
  for (int i = threadIdx.x; i < n; i += 256) bid[i] = sub_bucket_of(kb, vb, map_index(low, j0 + i), GK);
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += 256) {
    const int b = bid[i];
    int rank = 0;
    for (int k = 0; k < i; ++k) rank += (bid[k] == b);
    perm[base[(int64_t)blockIdx.x * 2 * NB + b] + rank] = (int32_t)map_index(low, j0 + i);
  }
}

// One block per tile writes the tile image with coalesced stores: the keys'
// tokens, center indices and first r_low INT4 codes / fp16 scales are staged
// in LDS, then the fp16 K rows (16-byte chunks), the bf16 V and a^V one-hot
// rows (8-byte chunks), the T-table offsets and the header.  Also max |c^K[:r_low]|^2 over real keys.
constexpr int IMG_MAXB = 64;   // code bytes staged per key (r_low <= 128)
constexpr int IMG_MAXS = 16;   // scales staged per key (r_low / group, group >= 8)
__global__ __launch_bounds__(256) void k_build_images(
    BranchArgs kb, BranchArgs vb, int r, int group, int r_low, TileGeom g,
    const int32_t* __restrict__ tile_start, const int32_t* __restrict__ tile_bucket,
    const int32_t* __restrict__ bcount, int NB, int GK, const int32_t* __restrict__ perm,
    char* __restrict__ img, uint32_t* __restrict__ cmax2) {
  __shared__ int64_t stok[NT];
  __shared__ int sak[NT], sav[NT];
  __shared__ __attribute__((aligned(16))) uint8_t skc[NT][IMG_MAXB], svc[NT][IMG_MAXB];
  __shared__ uint16_t sks[NT][IMG_MAXS], svs[NT][IMG_MAXS];
  const int64_t tile = blockIdx.x;
  const int64_t ntl = tile_start[NB];
  if (tile >= ntl) return;
  const int tid = threadIdx.x;
  const int b = tile_bucket[tile];
  const int nreal = (int)max<int64_t>(0, min<int64_t>(NT, bcount[b] - (tile - tile_start[b]) * NT));
  const int nb = r_low / 2, ns = (r_low + group - 1) / group;
  if (tid < NT) {
    const bool real = tid < nreal;
    const int64_t t = real ? perm[tile * NT + tid] : -1;
    stok[tid] = t;
    sak[tid] = real ? kb.idx[t] : 0;
    sav[tid] = real ? vb.idx[t] : -1;
  }
  __syncthreads();
  // code bytes 4 at a time when the code arrays are word-aligned (rows and
  // runs are then whole words: r % 32 == 0, r_low % 16 == 0)
  const bool words = ((reinterpret_cast<uintptr_t>(kb.codes) | reinterpret_cast<uintptr_t>(vb.codes)) & 3) == 0;
  const int nw4 = words ? nb / 4 : 0;
  for (int i = tid; i < NT * nb && !words; i += 256) {
    const int k = i / nb, j = i - k * nb;
    const int64_t t = stok[k];
    skc[k][j] = t >= 0 ? kb.codes[t * (r / 2) + j] : uint8_t(0);
    svc[k][j] = t >= 0 ? vb.codes[t * (r / 2) + j] : uint8_t(0);
  }
  for (int i = tid; i < NT * nw4; i += 256) {
    const int k = i / nw4, j = i - k * nw4;
    const int64_t t = stok[k];
    const uint32_t* kc = reinterpret_cast<const uint32_t*>(kb.codes + (t >= 0 ? t : 0) * (r / 2));
    const uint32_t* vc = reinterpret_cast<const uint32_t*>(vb.codes + (t >= 0 ? t : 0) * (r / 2));
    reinterpret_cast<uint32_t*>(skc[k])[j] = t >= 0 ? kc[j] : 0u;
    reinterpret_cast<uint32_t*>(svc[k])[j] = t >= 0 ? vc[j] : 0u;
  }
  for (int i = tid; i < NT * ns; i += 256) {
    const int k = i / ns, j = i - k * ns;
    const int64_t t = stok[k];
    sks[k][j] = t >= 0 ? kb.scales[t * (r / group) + j] : uint16_t(0);
    svs[k][j] = t >= 0 ? vb.scales[t * (r / group) + j] : uint16_t(0);
  }
  __syncthreads();
  char* base = img + tile * g.bytes;
  // K fragments: chunk (kb, ks), lane l -> key kb*32 + l%32, coefficients
  // 16 ks + 8 (l/32) .. + 7 (zero past r_low and for dummies)
  for (int i = tid; i < (NT / 32) * g.nks * 64; i += 256) {
    const int ch = i >> 6, l = i & 63;
    const int kb = ch / g.nks, ks = ch - kb * g.nks;
    const int k = kb * 32 + (l & 31), j0 = 16 * ks + 8 * (l >> 5);
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u;
      v[u] = (j < r_low && k < nreal) ? (float)code_at(skc[k], j) * fp16_bits_to_f32(sks[k][j / group])
                                      : 0.f;
    }
    *reinterpret_cast<u32x4*>(base + ch * 1024 + l * 16) =
        u32x4{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3]), pack_f16x2(v[4], v[5]),
              pack_f16x2(v[6], v[7])};
  }
  // V fragments: chunk (kb, j, db), lane l -> row db*32 + l%32 (coefficient,
  // or center of the range for db >= rp/32), keys kb*32 + 16 j + 4 (l/32) +
  // {0..3} and + 8 + {0..3}
  for (int i = tid; i < (NT / 32) * 2 * g.nvb * 64; i += 256) {
    const int ch = i >> 6, l = i & 63;
    const int kbj = ch / g.nvb, db = ch - kbj * g.nvb;
    const int row = db * 32 + (l & 31);
    const int kq = (kbj >> 1) * 32 + 16 * (kbj & 1) + 4 * (l >> 5);
    uint16_t hv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = kq + (u & 3) + 8 * (u >> 2);
      uint16_t x = 0;
      if (k < nreal) {
        if (row < g.rp)
          x = row < r_low ? f32_to_bf16_bits((float)code_at(svc[k], row) *
                                             fp16_bits_to_f32(svs[k][row / group]))
                          : uint16_t(0);
        else
          x = (sav[k] % CR == row - g.rp) ? uint16_t(0x3F80) : uint16_t(0);
      }
      hv[u] = x;
    }
    *reinterpret_cast<u32x4*>(base + g.cv_off + ch * 1024 + l * 16) =
        u32x4{uint32_t(hv[0]) | (uint32_t(hv[1]) << 16), uint32_t(hv[2]) | (uint32_t(hv[3]) << 16),
              uint32_t(hv[4]) | (uint32_t(hv[5]) << 16), uint32_t(hv[6]) | (uint32_t(hv[7]) << 16)};
  }
  if (tid < NT) {
    // A dummy key takes the slot of key 0 (every tile has a real key 0):
    // its score is then that of a center present in the low set, which the
    // row bound covers, so p <= 1, and its zero V row and one-hot row make
    // the p irrelevant.  Byte place of key k: block kb = k / 32, then the
    // accumulator order (k % 32 = 8 g + 4 half + u -> 16 half + 4 g + u).
    const int k = tid, w = k & 31;
    const int place = (k >> 5) * 32 + ((w >> 2) & 1) * 16 + (w >> 3) * 4 + (w & 3);
    base[g.ko_off + place] = (uint8_t)((sak[k < nreal ? k : 0] % CR) * 4);
  }
  if (tid == 0) {
    u32x4 hd = {0u, 0u, 0u, 0u};
    if (tile + 1 < ntl) {
      const int bn = tile_bucket[tile + 1];
      const int tn = tile_start[bn + 1];
      hd = u32x4{(uint32_t)bn, tile + 1 == tile_start[bn] ? 1u : 0u,
                 (uint32_t)(tn < ntl ? tile_bucket[tn] % GK : -1), 0u};
    }
    uint32_t mask = 0u;
    for (int k = 0; k < nreal; ++k) mask |= 1u << (2 * (k / 16) + ((sav[k] % CR) >= CR / 2 ? 1 : 0));
    hd[3] = mask;
    *reinterpret_cast<u32x4*>(base + g.hd_off) = hd;
  }
  static_assert(NT == 64, "one wave holds the keys of a tile");
  if (tid < NT) {
    float n2 = 0.f;  // fixed order: deterministic bound
    for (int j = 0; j < r_low; ++j) {
      const float x = (float)code_at(skc[tid], j) * fp16_bits_to_f32(sks[tid][j / group]);
      n2 = fmaf(x, x, n2);
    }
    const float m = wave_max(tid < nreal ? n2 : 0.f);
    if (tid == 0 && nreal > 0) atomicMax(cmax2, ordered_bits(m));
  }
}

// q~ = per-head Q_h D_{K,h}[:, :r_low]  (rows = queries, cols = coefficients)
struct QtProblem {
  static constexpr int BK = 64;
  int M, N, K;  // Nq, r_low, 128
  int H;
  const uint16_t* q;
  const uint16_t* dkt;  // [r_low, W]
  float* qt32;          // [Nq*H, r_low]
  HeadSet hs;           // batch z serves head hs.h[z]
  __device__ u32x4 load_a(int z, int m, int k) const {
    if (m >= M) return u32x4{0u, 0u, 0u, 0u};
    return ld_u32x4(q + (int64_t)m * H * 128 + hs.h[z] * 128 + k);
  }
  __device__ u32x4 load_b(int z, int n, int k) const {
    if (n >= N) return u32x4{0u, 0u, 0u, 0u};
    return ld_u32x4(dkt + (int64_t)n * H * 128 + hs.h[z] * 128 + k);
  }
  __device__ const uint16_t* a_ptr(int z, int m, int k) const {
    return q + (int64_t)m * H * 128 + hs.h[z] * 128 + k;
  }
  __device__ const uint16_t* b_ptr(int z, int n, int k) const {
    return dkt + (int64_t)n * H * 128 + hs.h[z] * 128 + k;
  }
  bool dma_ok() const {
    return ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(dkt)) & 15) == 0;
  }
  __device__ void epilogue(int zb, int m0, int n0, int lane, const f32x16 (&acc)[2][2]) const {
    const int z = hs.h[zb];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = m0 + 32 * i + acc_row(e, lane), n = n0 + 32 * j + (lane & 31);
          if (m < M && n < N) qt32[((int64_t)m * H + z) * N + n] = acc[i][j][e];
        }
  }
};

// 16-byte block j of row r of 256-byte rows stored with block j of row r at
// block j ^ (r & 15) (conflict-free when 32 lanes read one block of 32 rows)
__device__ __forceinline__ u32x4 lds_row_block(const char* lds, int r, int j) {
  return *reinterpret_cast<const u32x4*>(lds + r * 256 + ((j ^ (r & 15)) << 4));
}

// max over centers present in the low set of q_h . mu^K_{a,h}, per row of
// the heads in hs.  One block = 128 queries of one head: 4 waves of 32
// queries keep their q fragments in registers while the head's center rows
// stream through LDS 64 at a time (double buffered, rows swizzled so that the
// MFMA operand reads are conflict-free); each lane folds its centers into a
// running max and one store per row replaces the atomics of a GEMM epilogue.
// Products are exact (bf16), sums fp32 in k order: the same values as a
// GEMM over k.  The presence flags (cleared to a whole 64-center block, so
// every load is unconditional) are requested one block ahead with the
// block's center rows, in two register sets: their latency runs under the
// MFMAs of the block before instead of after each block's own MFMAs.
constexpr int CM_Q = 128, CM_C = 64;
__global__ __launch_bounds__(256) void k_center_max(const uint16_t* __restrict__ q,
                                                    const uint16_t* __restrict__ muk,
                                                    const uint32_t* __restrict__ present,
                                                    int64_t Nq, int H, int A_k, HeadSet hs,
                                                    uint32_t* __restrict__ tmax) {
  __shared__ __attribute__((aligned(1024))) char sMu0[CM_C * 256];
  __shared__ __attribute__((aligned(1024))) char sMu1[CM_C * 256];
  const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = hs.h[blockIdx.y];
  const int64_t W = (int64_t)H * 128;
  const int64_t qrow = (int64_t)blockIdx.x * CM_Q + wave * 32 + (lane & 31);
  const bool rok = qrow < Nq;
  bf16x8 qv[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    qv[ks] = rok ? as_bf16x8(ld_u32x4(q + qrow * W + h * 128 + 16 * ks + 8 * hl))
                 : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  // 64 center rows (16 KiB): 16 direct-to-LDS loads of 1 KiB, 4 per wave;
  // row r's 16-byte block j lands at block j ^ (r & 15)
  auto load = [&](int blk, char* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < CM_C / 16; ++k) {
      const int c = wave + 4 * k;
      const int r = 4 * c + (lane >> 4), jp = lane & 15;
      const int j = jp ^ (r & 15);
      const int cen = min(blk * CM_C + r, A_k - 1);  // rows past A_k are masked below
      __builtin_amdgcn_global_load_lds(muk + (int64_t)cen * W + h * 128 + j * 8,
                                       (__attribute__((address_space(3))) void*)(dst + c * 1024),
                                       16, 0, 0);
    }
  };
  float best = -INFINITY;
  const int nblk = (A_k + CM_C - 1) / CM_C;
  // presence flags of the lane's 32 centers of block blk: (cb, g) -> the 4
  // consecutive centers blk*64 + 32 cb + 8 g + 4 hl .. + 3 (elements 4g..4g+3)
  auto ldpr = [&](int blk, u32x4 (&pr)[8]) __attribute__((always_inline)) {
    const int b = min(blk, nblk - 1);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      pr[i] = *reinterpret_cast<const u32x4*>(present + b * CM_C + (i >> 2) * 32 + (i & 3) * 8 +
                                               hl * 4);
  };
  auto block = [&](const char* cur, const u32x4 (&pr)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      f32x16 acc = zero16();
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        acc = mfma_bf16(as_bf16x8(lds_row_block(cur, cb * 32 + (lane & 31), 2 * ks + hl)),
                        qv[ks], acc);
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (pr[cb * 4 + g][u]) best = fmaxf(best, acc[4 * g + u]);
    }
  };
  u32x4 pr0[8], pr1[8];
  load(0, sMu0);
  ldpr(0, pr0);
  for (int blk = 0; blk < nblk; blk += 2) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (blk + 1 < nblk) load(blk + 1, sMu1);
    ldpr(blk + 1, pr1);
    block(sMu0, pr0);
    if (blk + 1 < nblk) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (blk + 2 < nblk) load(blk + 2, sMu0);
      ldpr(blk + 2, pr0);
      block(sMu1, pr1);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  best = fmaxf(best, __shfl_xor(best, 32, 64));
  // the encoding of "no present center" is the cleared value 0
  if (lane < 32 && rok) tmax[qrow * H + h] = best > -INFINITY ? ordered_bits(best) : 0u;
}

// per-row bound, fp16 c q~, and the list of rows needing the exact fallback;
// 16 lanes per row
__global__ __launch_bounds__(256) void k_row_bound(const float* __restrict__ qt32, int64_t Nq,
                                                   int H, HeadSet hs, int r_low, int rlp, float c,
                                                   const uint32_t* __restrict__ tmax,
                                                   const uint32_t* __restrict__ misc,
                                                   float* __restrict__ bound,
                                                   uint16_t* __restrict__ qt16,
                                                   int32_t* __restrict__ flags,
                                                   int32_t* __restrict__ nflag) {
  const int64_t rl = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 4;  // (query, head of the set)
  const int sub = threadIdx.x & 15;
  const bool ok = rl < Nq * hs.n;
  const int64_t row = ok ? (rl / hs.n) * H + hs.h[rl % hs.n] : 0;
  const float* qr = qt32 + (ok ? row : 0) * r_low;
  uint16_t* o = qt16 + (ok ? row : 0) * rlp;
  float n2 = 0.f, amax = 0.f;
  for (int j = 2 * sub; j < rlp; j += 32) {  // r_low even: a pair is wholly in or out
    float x0 = 0.f, x1 = 0.f;
    if (ok && j < r_low) {
      const f32x2 v = *reinterpret_cast<const f32x2*>(qr + j);
      x0 = v[0];
      x1 = v[1];
    }
    n2 = fmaf(x0, x0, fmaf(x1, x1, n2));
    amax = fmaxf(amax, fmaxf(fabsf(x0), fabsf(x1)));
    // fp16 c q~: the main kernel's score MFMA then yields c s directly
    if (ok) *reinterpret_cast<uint32_t*>(o + j) = pack_f16x2(c * x0, c * x1);
  }
#pragma unroll
  for (int m = 8; m > 0; m >>= 1) {
    n2 += __shfl_xor(n2, m, 16);
    amax = fmaxf(amax, __shfl_xor(amax, m, 16));
  }
  if (!ok || sub != 0) return;
  const float cmax = sqrtf(from_ordered_bits(misc[0]));
  const float qn = sqrtf(n2);
  const float T = from_ordered_bits(tmax[row]);
  const float B = c * (T + 1e-5f * fabsf(T) + 1.001f * qn * cmax) + 1e-3f;
  bound[row] = B;
  const bool bad = !(2.f * c * qn * cmax <= BOUND_GAP_LIMIT) || !(c * amax < 30000.f) ||
                   !(cmax < 30000.f) || !(fabsf(B) < 1e30f);
  if (bad) flags[atomicAdd(nflag, 1)] = (int32_t)row;
}

// ---------------------------------------------------------------------------
// the main low-dimensional kernel
// ---------------------------------------------------------------------------
struct MainArgs {
  const uint16_t* q;
  const uint16_t* muk;
  const uint16_t* qt16;
  const float* bound;
  const char* img;
  const int32_t* tile_start;
  const int32_t* tile_bucket;
  float* acc;
  float* wmass;
  float* ell;
  int64_t Nq;
  int H, A_k, A_v, GK, GV, NB, r_low, ra;
  int gvsplit;  // key-range splits at a^V-range boundaries
  int nqb, nsplit;  // query blocks and key-range splits (work unit = (query block, head, split))
  int ragged_last;  // the last query block holds fewer than 256 rows
  float c;
  HeadSet hs;  // heads of the group
};

constexpr int RBW = 256;                // query rows per block: 8 waves x 32 rows
constexpr int LDS_BYTES = 160 * 1024;

template <int RLP>
struct RowsGeo {
  static constexpr TileGeom G = tile_geom(RLP);
  static constexpr int NPB = G.rp / 32, CHUNKS = G.bytes / 1024;
  static constexpr int T_BYTES = RBW * TS * 4;
  static constexpr int M_BYTES = CR * 256;  // one 64-center slice of mu^K for one head (bf16)
  // the mu^K slice is staged in LDS when it fits next to two tile stages
  static constexpr bool SM = 2 * G.bytes + T_BYTES + M_BYTES <= LDS_BYTES;
  static_assert(2 * G.bytes + T_BYTES <= LDS_BYTES, "tile stages exceed LDS");
  static constexpr int DMA_PER_WAVE = (CHUNKS + 7) / 8;
};

// one wave's share of a tile: 1 KiB chunks w, w + 8, ... straight into LDS
template <int RLP>
__device__ __forceinline__ void load_tile(const char* __restrict__ src, char* lds, int wave,
                                          int lane) {
  constexpr int C = RowsGeo<RLP>::CHUNKS;
#pragma unroll
  for (int c = wave; c < C; c += 8)
    __builtin_amdgcn_global_load_lds(src + c * 1024 + lane * 16,
                                     (__attribute__((address_space(3))) void*)(lds + c * 1024), 16,
                                     0, 0);
}

// 256-byte bf16 rows (128 channels of one head) into LDS, four rows per 1 KiB
// load, with the 16-byte blocks of row r stored at block (j ^ (r & 15)) so
// that 32 lanes reading one block of 32 different rows hit distinct banks.
__device__ __forceinline__ void load_rows_swizzled(const uint16_t* __restrict__ base, int64_t ld,
                                                   int nrows, int valid, char* lds, int wave,
                                                   int lane) {
  for (int c = wave; c < nrows / 4; c += 8) {
    const int r = 4 * c + (lane >> 4), jp = lane & 15;
    const int j = jp ^ (r & 15);
    const int rr = r < valid ? r : 0;
    __builtin_amdgcn_global_load_lds(base + rr * ld + j * 8,
                                     (__attribute__((address_space(3))) void*)(lds + c * 1024), 16,
                                     0, 0);
  }
}


// ---------------------------------------------------------------------------
// Main kernel.  One block = 256 query rows of one head; wave w owns rows
// 32w..32w+31 and scores them against all 64 keys of every tile, so each
// tile brought into LDS feeds 8 waves' MFMAs and rows never meet across
// waves.
//   S^T[key][row] = T[row][a^K] + (c q~) . c^K       (T gathered into the
//                                                     accumulator, fp16 MFMA)
//   p = 2^S                                          (bound B already in T)
//   [acc^T ; M^T][coef|center][row] += [c^V ; onehot(a^V)]^T P^T   (bf16 MFMA)
// Tiles are double buffered with direct-to-LDS loads; each wave spreads its
// share of the next tile's loads over the first steps of its math, and the
// header of every tile already names the bucket facts of the next one.
// ---------------------------------------------------------------------------
template <int RLP>
__global__ __launch_bounds__(512, 1) void k_low_rows(const MainArgs a) {
  using Geo = RowsGeo<RLP>;
  constexpr TileGeom G = Geo::G;
  constexpr int NPB = Geo::NPB;
  constexpr bool SM = Geo::SM;
  // one array per pipeline stage: the stage of every LDS access is static,
  // so the compiler can see that reading one stage does not alias the
  // direct-to-LDS loads in flight into the other
  __shared__ __attribute__((aligned(1024))) char sB0[G.bytes];
  __shared__ __attribute__((aligned(1024))) char sB1[G.bytes];
  __shared__ __attribute__((aligned(1024))) char sM[SM ? Geo::M_BYTES : 16];
  __shared__ __attribute__((aligned(16))) float sT[RBW * TS];

  // wave index and tile count in scalar registers: tile addresses and the
  // LDS destinations of the tile loads are then computed on the scalar unit
  const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // XCD-aware order: the hardware deals consecutive block ids to the 8 XCDs
  // in turn (block L runs on XCD L % 8), so work unit u -- query block
  // fastest, then head, then key-range split -- is given to block
  // (u % per) * 8 + u / per: each XCD runs a contiguous run of units, which
  // read the same tiles (one split's tile range) at about the same time and
  // share them in that XCD's L2.
  const int nunits = a.nqb * a.hs.n * a.nsplit;
  const int per = (nunits + 7) / 8;
  const int u = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (u >= nunits) return;  // the whole block, before any barrier
  // Within a split, the ragged last query block of every head comes after
  // all full blocks: each XCD runs its units in order, and the few-row
  // blocks (fewer active waves, shorter) then fill the last round.
  const int split = u / (a.nqb * a.hs.n), nsplit = a.nsplit;
  const int rnk = u - split * a.nqb * a.hs.n;
  int bx, by;
  if (a.ragged_last && a.nqb > 1 && rnk >= (a.nqb - 1) * a.hs.n) {
    bx = a.nqb - 1;
    by = rnk - (a.nqb - 1) * a.hs.n;
  } else {
    const int nq = a.ragged_last && a.nqb > 1 ? a.nqb - 1 : a.nqb;
    bx = rnk % nq;
    by = rnk / nq;
  }
  const int h = a.hs.h[by];
  const int W = a.H * 128;
  const int64_t q0 = (int64_t)bx * RBW;
  const int rloc = wave * 32 + (lane & 31);
  const int64_t qrow = q0 + rloc;
  const bool rok = qrow < a.Nq;
  const bool active = q0 + wave * 32 < a.Nq;  // the wave owns at least one row
  const int64_t grow = (rok ? qrow : q0) * a.H + h;
  // partial-sum row of this (key-range split, query, head of the group)
  const int64_t prow = ((int64_t)split * a.Nq + (rok ? qrow : q0)) * a.hs.n + by;

  f16x8 qtf[RLP / 16];
#pragma unroll
  for (int ks = 0; ks < RLP / 16; ++ks)
    qtf[ks] = rok ? as_f16x8(ld_u32x4(a.qt16 + grow * RLP + 16 * ks + 8 * hl))
                  : as_f16x8(u32x4{0u, 0u, 0u, 0u});
  const float Bq = rok ? a.bound[grow] : 0.f;
  f32x16 accT[NPB], accW[2];
#pragma unroll
  for (int i = 0; i < NPB; ++i) accT[i] = zero16();
  accW[0] = zero16();
  accW[1] = zero16();
  float lsum = 0.f;

  // this split's tiles [ts, te) of the bucket-sorted sequence
  const int ntiles = __builtin_amdgcn_readfirstlane(a.tile_start[a.NB]);
  // Splits at a^V-range boundaries (gvsplit) own disjoint center-mass ranges
  // [g0, g1); otherwise a split is an equal share of the tile sequence
  const int g0 = a.gvsplit ? a.GV * split / nsplit : 0;
  const int g1 = a.gvsplit ? a.GV * (split + 1) / nsplit : a.GV;
  const int ts = __builtin_amdgcn_readfirstlane(
      a.gvsplit ? a.tile_start[g0 * a.GK] : (int)((int64_t)ntiles * split / nsplit));
  const int te = __builtin_amdgcn_readfirstlane(
      a.gvsplit ? a.tile_start[g1 * a.GK] : (int)((int64_t)ntiles * (split + 1) / nsplit));
  const char* sTrow = reinterpret_cast<const char*>(sT + rloc * TS);
  const uint16_t* qsrc = a.q + (rok ? qrow : q0) * W + h * 128 + 8 * hl;
  // the wave's q row fragments for the T slices: loaded once and kept in
  // registers up to r_low 96 (a bucket start then needs no q reload);
  // wider coefficient rows leave no room and reload them per bucket
  constexpr bool QRES = RLP <= 96;
  bf16x8 qres[QRES ? 8 : 1];
  if constexpr (QRES) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qres[ks] = as_bf16x8(ld_u32x4(qsrc + 16 * ks));
  }

  // mu^K rows of the 64-center slice gk for this head
  auto load_mu = [&](int gk) __attribute__((always_inline)) {
    const int valid = min(CR, a.A_k - gk * CR);
    load_rows_swizzled(a.muk + (int64_t)gk * CR * W + h * 128, W, CR, valid, sM, wave, lane);
  };

  // the k-th of this wave's 1 KiB chunks of tile tt into `dst`
  auto dma = [&](int tt, char* dst, int k) __attribute__((always_inline)) {
    const int c = wave + 8 * k;
    if (c < Geo::CHUNKS && tt < te) {
      const char* chunk = a.img + ((int64_t)tt * G.bytes + c * 1024);  // wave-uniform
      uint32_t lo = lane * 16;
      asm volatile("" : "+v"(lo));
      __builtin_amdgcn_global_load_lds(chunk + lo,
                                       (__attribute__((address_space(3))) void*)(dst + c * 1024),
                                       16, 0, 0);
    }
  };

  // masses of the a^V range gv from the accumulators
  // With one split the restoration reads the partials as bf16 hi/lo planes
  // (x = hi + lo to ~16 significant bits), written here once instead of being
  // split again for every use; rows [hi | lo] of 2 x GV * 64 (masses) and
  // 2 x ra (coefficient sums) bf16.
  // masses as planes when no other split writes the same rows; coefficient
  // sums as planes only without splits
  const bool planes = nsplit == 1 || a.gvsplit;
  const bool acc_planes = nsplit == 1;
  const int WS = a.GV * CR;
  auto put_hilo = [&](uint16_t* hi, uint16_t* lo, f32x4 v) __attribute__((always_inline)) {
    float l[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) l[u] = v[u] - (float)(__bf16)v[u];
    *reinterpret_cast<uint2*>(hi) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    *reinterpret_cast<uint2*>(lo) = uint2{pack_bf16x2(l[0], l[1]), pack_bf16x2(l[2], l[3])};
  };
  uint16_t* const mplane = reinterpret_cast<uint16_t*>(a.wmass);
  const int64_t nmt = (a.Nq + 127) / 128;
  auto put_mass = [&](int gv) __attribute__((always_inline)) {
    if (rok && planes) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int c = gv * CR + cb * 32 + e4 * 8 + hl * 4;
          put_hilo(mplane + mass_pos(qrow, by, c, nmt, WS),
                   mplane + mass_pos(qrow, by, WS + c, nmt, WS),
                   f32x4{accW[cb][4 * e4], accW[cb][4 * e4 + 1], accW[cb][4 * e4 + 2],
                         accW[cb][4 * e4 + 3]});
        }
    } else if (rok) {
      float* dst = a.wmass + prow * a.A_v + gv * CR;
      const int lim = a.A_v - gv * CR;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int c = cb * 32 + e4 * 8 + hl * 4;
          if ((a.A_v & 3) == 0 && c + 4 <= lim) {
            *reinterpret_cast<f32x4*>(dst + c) =
                f32x4{accW[cb][4 * e4], accW[cb][4 * e4 + 1], accW[cb][4 * e4 + 2],
                      accW[cb][4 * e4 + 3]};
          } else {
#pragma unroll
            for (int u = 0; u < 4; ++u)
              if (c + u < lim) dst[c + u] = accW[cb][4 * e4 + u];
          }
        }
    }
  };
  // zeros for the a^V ranges [g0, g1) this split never visits (the
  // restoration reads every range)
  auto zero_mass = [&](int g0, int g1) __attribute__((always_inline)) {
    if (!rok) return;
    if (planes) {
      for (int gv = g0; gv < g1; ++gv)
        for (int c = gv * CR + hl * 4; c < (gv + 1) * CR; c += 8) {
          *reinterpret_cast<uint2*>(mplane + mass_pos(qrow, by, c, nmt, WS)) = uint2{0u, 0u};
          *reinterpret_cast<uint2*>(mplane + mass_pos(qrow, by, WS + c, nmt, WS)) = uint2{0u, 0u};
        }
      return;
    }
    for (int gv = g0; gv < g1; ++gv) {
      float* dst = a.wmass + prow * a.A_v + gv * CR;
      const int lim = min(CR, a.A_v - gv * CR);
      for (int c = hl; c < lim; c += 2) dst[c] = 0.f;
    }
  };
  int zgv = g0;  // first a^V range of this split's rows not yet written
  auto flush = [&](int gv) __attribute__((always_inline)) {
    if (zgv < gv) zero_mass(zgv, gv);
    put_mass(gv);
    // the softmax denominator is the sum of the center masses: every key's
    // p lands in exactly one center (padding keys have p = 0)
#pragma unroll
    for (int e = 0; e < 16; ++e) lsum += accW[0][e] + accW[1][e];
    zgv = gv + 1;
    accW[0] = zero16();
    accW[1] = zero16();
  };

  // T[row][center] = c mu^K_{center,h} . q_h - B for the wave's rows
  // (exact bf16 products, fp32 sums) into the wave's own rows of sT
  auto t_slice = [&](int gk) __attribute__((always_inline)) {
    bf16x8 qv[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      if constexpr (QRES) qv[ks] = qres[ks];
      else qv[ks] = as_bf16x8(ld_u32x4(qsrc + 16 * ks));
    // two center blocks: independent accumulation chains, interleaved.  The
    // lane's LDS offsets are derived here from an opaque copy of the lane
    // index: hoisted out of the tile loop they would hold 64 registers for
    // the whole kernel.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    f32x16 tt[2] = {zero16(), zero16()};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        bf16x8 m;
        if constexpr (SM) {
          m = as_bf16x8(lds_row_block(sM, cb * 32 + (ln & 31), 2 * ks + (ln >> 5)));
        } else {
          const int cen = gk * CR + cb * 32 + (lane & 31);
          m = as_bf16x8(ld_u32x4(a.muk + (int64_t)(cen < a.A_k ? cen : 0) * W + h * 128 +
                                 8 * hl + 16 * ks));
        }
        tt[cb] = mfma_bf16(m, qv[ks], tt[cb]);
      }
    // element e of block cb is center cb*32 + acc_row(e, lane): one base
    // address per lane plus constant offsets
    float* trow = sT + (wave * 32 + (ln & 31)) * TS + (ln >> 5) * 4;
    if ((gk + 1) * CR <= a.A_k) {  // block-uniform: every center of the range exists
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          trow[cb * 32 + (e >> 2) * 8 + (e & 3)] = fmaf(tt[cb][e], a.c, -Bq);
    } else {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int cl = cb * 32 + acc_row(e, ln);
          trow[cb * 32 + (e >> 2) * 8 + (e & 3)] =
              (gk * CR + cl < a.A_k) ? fmaf(tt[cb][e], a.c, -Bq) : -INFINITY;
        }
    }
  };

  // bucket facts of the tile about to be processed: tile 0's from the tables,
  // every later tile's from the header of the tile before it
  int cur_b = 0, cur_first = 0, cur_ngk = -1;
  if (ts < te) {
    cur_b = a.tile_bucket[ts];
    cur_first = 1;  // a split may start inside a bucket: its T slice is still needed
    const int tn = a.tile_start[cur_b + 1];
    cur_ngk = tn < ntiles ? a.tile_bucket[tn] % a.GK : -1;
    if constexpr (SM) load_mu(cur_b % a.GK);
    load_tile<RLP>(a.img + (int64_t)ts * G.bytes, sB0, wave, lane);
  }

  int prev_gv = -1;
  // one tile: consume `cur`, load tile t + 1 into `nxt` while computing
  auto body = [&](int t, const char* cur, char* nxt) __attribute__((always_inline)) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (cur_first) {
      // ---- new bucket: (flush,) then the T slice of its a^K range -------------
      const int gv = cur_b / a.GK, gk = cur_b - gv * a.GK;
      if (gv != prev_gv && prev_gv >= 0) flush(prev_gv);
      prev_gv = gv;
      if (active) t_slice(gk);
      if constexpr (SM) {
        __syncthreads();  // sM is free once every wave has its T slice
        if (cur_ngk >= 0) load_mu(cur_ngk);
      }
    }
    // this tile's header: the bucket facts of tile t + 1
    uint32_t smask;  // this tile's step mask (which one-hot halves each step needs)
    {
      const u32x4 hd = *reinterpret_cast<const u32x4*>(cur + G.hd_off);
      cur_b = __builtin_amdgcn_readfirstlane((int)hd[0]);
      cur_first = __builtin_amdgcn_readfirstlane((int)hd[1]);
      cur_ngk = __builtin_amdgcn_readfirstlane((int)hd[2]);
      smask = __builtin_amdgcn_readfirstlane(hd[3]);
    }
    if (!active) {
#pragma unroll
      for (int k = 0; k < Geo::DMA_PER_WAVE; ++k) dma(t + 1, nxt, k);
      return;
    }
    // Operand batches are read into registers well ahead of their MFMAs;
    // sched_barrier keeps the scheduler from sinking each read next to its
    // use, which would expose a full LDS round trip per MFMA.
    auto gather = [&](int kb, f32x16& acc) __attribute__((always_inline)) {
      const u32x4 kov = *reinterpret_cast<const u32x4*>(cur + G.ko_off + kb * 32 + hl * 16);
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          acc[4 * g + u] = *reinterpret_cast<const float*>(sTrow + ((kov[g] >> (8 * u)) & 0xffu));
    };
    auto read_v = [&](int kb, int j, bf16x8 (&vo)[NPB + 2]) __attribute__((always_inline)) {
#pragma unroll
      for (int db = 0; db < NPB + 2; ++db)
        vo[db] = as_bf16x8(*reinterpret_cast<const u32x4*>(
            cur + G.cv_off + ((kb * 2 + j) * G.nvb + db) * 1024 + lane * 16));
    };
    // p = 2^S for the 16 keys of half hb of a 32-key block, packed to bf16 in
    // the key order of the B operand
    auto expo = [&](const f32x16& acc, int hb) __attribute__((always_inline)) {
      u32x4 pk;
#pragma unroll
      for (int g2 = 0; g2 < 2; ++g2) {
        const int g = 2 * hb + g2;
        float pv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) pv[u] = __builtin_amdgcn_exp2f(acc[4 * g + u]);
        pk[2 * g2] = pack_bf16x2(pv[0], pv[1]);
        pk[2 * g2 + 1] = pack_bf16x2(pv[2], pv[3]);
      }
      return as_bf16x8(pk);
    };
    // step s of the tile: MFMAs only for what its real keys touch (a step
    // of padding keys only has p = 0)
    auto pv = [&](const bf16x8 (&vo)[NPB + 2], bf16x8 p, int step) __attribute__((always_inline)) {
      const uint32_t m = (smask >> (2 * step)) & 3u;
      if (m == 0u) return;
#pragma unroll
      for (int db = 0; db < NPB; ++db) accT[db] = mfma_bf16(vo[db], p, accT[db]);
      if (m & 1u) accW[0] = mfma_bf16(vo[NPB], p, accW[0]);
      if (m & 2u) accW[1] = mfma_bf16(vo[NPB + 1], p, accW[1]);
    };
    // K operands in two batches of k-steps (both key halves each), the
    // second read while the first batch's MFMAs run
    constexpr int NKS = RLP / 16, HB = (NKS + 1) / 2;
    f32x16 s0, s1;
    f16x8 c0[HB], c1[HB];
    bf16x8 va[NPB + 2], vb[NPB + 2];
    auto read_kb = [&](int ks0, int n) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < HB; ++i)
        if (i < n) {
          c0[i] = as_f16x8(*reinterpret_cast<const u32x4*>(cur + (ks0 + i) * 1024 + lane * 16));
          c1[i] = as_f16x8(
              *reinterpret_cast<const u32x4*>(cur + (G.nks + ks0 + i) * 1024 + lane * 16));
        }
    };
    auto score_kb = [&](int ks0, int n) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < HB; ++i)
        if (i < n) {
          s0 = mfma_f16(c0[i], qtf[ks0 + i], s0);
          s1 = mfma_f16(c1[i], qtf[ks0 + i], s1);
        }
    };
    gather(0, s0);
    gather(1, s1);
    read_kb(0, HB);
    dma(t + 1, nxt, 0);
    __builtin_amdgcn_sched_barrier(0);
    // S^T = T + (c q~) . c^K for both key halves (fp16 MFMA): two independent
    // accumulation chains, interleaved
    score_kb(0, HB);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NKS > HB) {
      read_kb(HB, NKS - HB);
      __builtin_amdgcn_sched_barrier(0);
      score_kb(HB, NKS - HB);
    }
    read_v(0, 0, va);
    dma(t + 1, nxt, 1);
    __builtin_amdgcn_sched_barrier(0);
    // [acc^T ; M^T][coef|center][row] += [c^V ; onehot(a^V)]^T P^T, 16 keys
    // per step; each step's MFMAs overlap the exponentials of the next
    bf16x8 p = expo(s0, 0);
    read_v(0, 1, vb);
    dma(t + 1, nxt, 2);
    __builtin_amdgcn_sched_barrier(0);
    pv(va, p, 0);
    p = expo(s0, 1);
#pragma unroll
    for (int k = 3; k < Geo::DMA_PER_WAVE; ++k) dma(t + 1, nxt, k);
    __builtin_amdgcn_sched_barrier(0);
    read_v(1, 0, va);
    pv(vb, p, 1);
    p = expo(s1, 0);
    __builtin_amdgcn_sched_barrier(0);
    read_v(1, 1, vb);
    pv(va, p, 2);
    p = expo(s1, 1);
    __builtin_amdgcn_sched_barrier(0);
    pv(vb, p, 3);
  };
  for (int t = ts; t < te; t += 2) {
    body(t, sB0, sB1);
    if (t + 1 < te) body(t + 1, sB1, sB0);
  }
  // no row or tile load may still be in flight into LDS when the block ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (prev_gv >= 0) flush(prev_gv);
  if (zgv < g1) zero_mass(zgv, g1);
  lsum += __shfl_xor(lsum, 32, 64);
  if (rok) {
#pragma unroll
    for (int db = 0; db < NPB; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int dim = db * 32 + e4 * 8 + hl * 4;  // r_low % 16 == 0: whole f32x4 or none
        const f32x4 v{accT[db][4 * e4], accT[db][4 * e4 + 1], accT[db][4 * e4 + 2],
                      accT[db][4 * e4 + 3]};
        if (acc_planes) {
          // every dim < ra: past r_low the V rows are zero, and so are these
          // sums (the restoration reads whole planes)
          uint16_t* row = reinterpret_cast<uint16_t*>(a.acc) + prow * 2 * a.ra;
          put_hilo(row + dim, row + a.ra + dim, v);
        } else if (dim < a.r_low) {
          *reinterpret_cast<f32x4*>(a.acc + prow * a.r_low + dim) = v;
        }
      }
    if (hl == 0) a.ell[prow] = lsum;
  }
}

template <int RLP>
nkv_status launch_main(const MainArgs& m, hipStream_t st) {
  const int64_t units = (int64_t)m.nqb * m.hs.n * m.nsplit;
  hipLaunchKernelGGL(k_low_rows<RLP>, dim3((unsigned)(ceil_div(units, 8) * 8)), dim3(512), 0, st, m);
  NKV_LAUNCH_CHECK();
  return NKV_OK;
}

// ---------------------------------------------------------------------------
// Split center masses of a single a^V range (A_v <= 64) summed into the bf16
// hi/lo planes the restoration reads (the main kernel's plane layout, whole
// rows of WS = 64 columns: zero past A_v): thread i takes 4 centers of a row.
__device__ __forceinline__ void reduce_mass_one(int64_t i, const float* __restrict__ wmass,
                                                int64_t Nq, int nh, int nsplit, int A_v, int WS,
                                                uint16_t* __restrict__ planes) {
  const int per = WS / 4;
  if (i >= Nq * nh * per) return;
  const int64_t row = i / per;  // (query, head of the group)
  const int c = (int)(i - row * per) * 4;
  const int64_t m = row / nh;
  const int zb = (int)(row - m * nh);
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < nsplit; ++sp) {
    const float* src = wmass + ((int64_t)sp * Nq * nh + row) * A_v + c;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (c + u < A_v) v[u] += src[u];
  }
  float l[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) l[u] = v[u] - (float)(__bf16)v[u];
  const int64_t nmt = (Nq + 127) / 128;
  *reinterpret_cast<uint2*>(planes + mass_pos(m, zb, c, nmt, WS)) =
      uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  *reinterpret_cast<uint2*>(planes + mass_pos(m, zb, WS + c, nmt, WS)) =
      uint2{pack_bf16x2(l[0], l[1]), pack_bf16x2(l[2], l[3])};
}

// Split coefficient sums -> one bf16 hi/lo plane row each (and ell summed),
// in split order: rows = (query, head of the group); one thread per four
// plane columns of a row (r_low % 16 == 0; zeros in [r_low, ra)).
__global__ __launch_bounds__(256) void k_reduce_acc(const float* __restrict__ acc,
                                                    const float* __restrict__ ell, int64_t rows,
                                                    int nsplit, int r_low, int ra,
                                                    uint16_t* __restrict__ racc,
                                                    float* __restrict__ rell,
                                                    const float* __restrict__ wmass, int64_t Nq,
                                                    int nh, int A_v, int WS,
                                                    uint16_t* __restrict__ planes) {
  // threads [0, rows * ra / 4): coefficient sums; then, with `planes`, the
  // center masses of a single a^V range: [rows * ra / 4, + rows * WS / 4)
  const int per = ra / 4;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * per) {
    if (planes) reduce_mass_one(i - rows * per, wmass, Nq, nh, nsplit, A_v, WS, planes);
    return;
  }
  const int64_t row = i / per;
  const int c = (int)(i - row * per) * 4;
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  if (c < r_low) v = *reinterpret_cast<const f32x4*>(acc + row * r_low + c);
  for (int sp = 1; sp < nsplit && c < r_low; ++sp) {
    const f32x4 w = *reinterpret_cast<const f32x4*>(acc + ((int64_t)sp * rows + row) * r_low + c);
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] += w[u];
  }
  float l[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) l[u] = v[u] - (float)(__bf16)v[u];
  uint16_t* dst = racc + row * 2 * ra + c;
  *reinterpret_cast<uint2*>(dst) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  *reinterpret_cast<uint2*>(dst + ra) = uint2{pack_bf16x2(l[0], l[1]), pack_bf16x2(l[2], l[3])};
  if (c == 0) {
    float t = ell[row];
    for (int sp = 1; sp < nsplit; ++sp) t += ell[(int64_t)sp * rows + row];
    rell[row] = t;
  }
}

// ---------------------------------------------------------------------------
// restoration: O_low = (D_{V,h} acc + M mu^V_h) / ell,  LSE = (B + log2 ell) ln 2
// GEMM over K = [acc hi | acc lo | M hi | M lo] (fp32 split into bf16 pairs)
// ---------------------------------------------------------------------------
struct RestoreProblem {
  static constexpr int BK = 64;
  int M, N, K;  // Nq, 128, 2 ra + 2 av
  int H, ldv, r_low, ra, A_v, av;
  int nsplit;   // mass partials when !mass_planes (key-range splits: they add)
  int WS;       // bf16 hi/lo planes: mass rows [hi | lo] of 2 x WS
  int mass_planes;  // masses as planes (no split, or splits at a^V-range boundaries)
  // the coefficient sums are always planes [hi | lo] of 2 x ra and ell one
  // value per row (split partials are reduced before this GEMM)
  const float* acc;    // partials [nsplit][Nq][hs.n][r_low]
  const float* wmass;  // partials [nsplit][Nq][hs.n][A_v], or bf16 planes in 128-row blocks
  const uint16_t* dv;    // restoration map [W, ldv]
  const uint16_t* mvt;   // [W, av]
  const float* ell;     // partials [nsplit][Nq][hs.n]
  const float* bound;
  float* o_low;
  float* lse_low;
  HeadSet hs;  // batch z serves head hs.h[z]
  // partial row of split s for query m and group head zb
  __device__ int64_t prow(int s, int m, int zb) const {
    return ((int64_t)s * M + m) * hs.n + zb;
  }
  __device__ int64_t nmt() const { return (M + 127) / 128; }  // 128-row blocks of the mass planes
  __device__ u32x4 load_a(int zb, int m, int k) const {
    if (m >= M || k >= K) return u32x4{0u, 0u, 0u, 0u};
    if (k < 2 * ra || mass_planes != 0) {
      const int64_t pr = prow(0, m, zb);
      if (k < 2 * ra) {
        const int j = k >= ra ? k - ra : k;
        if (j >= r_low) return u32x4{0u, 0u, 0u, 0u};
        return ld_u32x4(reinterpret_cast<const uint16_t*>(acc) + pr * 2 * ra + k);
      }
      const int kk = k - 2 * ra;
      const int c = kk >= av ? kk - av + WS : kk;
      return ld_u32x4(reinterpret_cast<const uint16_t*>(wmass) + mass_pos(m, zb, c, nmt(), WS));
    }
    // masses as fp32 partials of key-range splits: summed and split here
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.f;
    bool lo;
    {
      const int kk = k - 2 * ra;
      lo = kk >= av;
      const int c = lo ? kk - av : kk;
      for (int s = 0; s < nsplit; ++s) {
        const float* src = wmass + prow(s, m, zb) * A_v + c;
        if ((A_v & 3) == 0 && c + 8 <= A_v) {
          const f32x4 x0 = *reinterpret_cast<const f32x4*>(src);
          const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) { v[i] += x0[i]; v[4 + i] += x1[i]; }
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] += (c + i < A_v) ? src[i] : 0.f;
        }
      }
    }
    u32x4 out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x0 = v[2 * i], x1 = v[2 * i + 1];
      if (lo) {
        x0 -= (float)(__bf16)x0;
        x1 -= (float)(__bf16)x1;
      }
      out[i] = pack_bf16x2(x0, x1);
    }
    return out;
  }
  __device__ u32x4 load_b(int zb, int n, int k) const {
    if (n >= N || k >= K) return u32x4{0u, 0u, 0u, 0u};
    const int64_t ch = (int64_t)hs.h[zb] * 128 + n;
    if (k < 2 * ra) {
      const int j = k >= ra ? k - ra : k;
      if (j >= r_low) return u32x4{0u, 0u, 0u, 0u};
      return ld_u32x4(dv + ch * ldv + j);
    }
    const int kk = k - 2 * ra;
    const int c = kk >= av ? kk - av : kk;
    return ld_u32x4(mvt + ch * av + c);
  }
  // direct-to-LDS operand rows (mass planes only): the same values as
  // load_a / load_b, except that past r_low the A planes hold zeros and B
  // any finite decoder value of the same row
  __device__ const uint16_t* a_ptr(int zb, int m, int k) const {
    const int64_t pr = prow(0, m, zb);
    if (k < 2 * ra) return reinterpret_cast<const uint16_t*>(acc) + pr * 2 * ra + k;
    const int kk = k - 2 * ra;
    return reinterpret_cast<const uint16_t*>(wmass) +
           mass_pos(m, zb, kk >= av ? kk - av + WS : kk, nmt(), WS);
  }
  __device__ const uint16_t* b_ptr(int zb, int n, int k) const {
    const int64_t ch = (int64_t)hs.h[zb] * 128 + n;
    if (k < 2 * ra) {
      const int j = k >= ra ? k - ra : k;
      return dv + ch * ldv + min(j, ldv - 8);
    }
    const int kk = k - 2 * ra;
    return mvt + ch * av + (kk >= av ? kk - av : kk);
  }
  bool dma_ok() const {
    const uintptr_t al = reinterpret_cast<uintptr_t>(acc) | reinterpret_cast<uintptr_t>(wmass) |
                         reinterpret_cast<uintptr_t>(dv) | reinterpret_cast<uintptr_t>(mvt);
    return mass_planes != 0 && (al & 15) == 0 && ldv % 8 == 0 && ldv >= 8 && ra % 8 == 0 &&
           WS % 8 == 0 && av % 8 == 0;
  }
  __device__ void epilogue(int zb, int m0, int n0, int lane, const f32x16 (&accv)[2][2]) const {
    const int z = hs.h[zb];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + 32 * i + acc_row(e, lane);
        if (m >= M) continue;
        const int64_t row = (int64_t)m * H + z;
        const float l = ell[prow(0, m, zb)];
        const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = n0 + 32 * j + (lane & 31);
          if (n < N) o_low[(int64_t)m * H * 128 + z * 128 + n] = accv[i][j][e] * inv;
          if (n == 0)
            lse_low[row] = l > 0.f ? (bound[row] + __log2f(l)) * 0.69314718055994531f : -INFINITY;
        }
      }
  }
};


}  // namespace

LowSplit low_split_plan(int64_t Nq, int n_heads, int64_t n_low, int A_v) {
  // One block per CU: choose the split count by how full the last round of
  // blocks is, less a small cost per split (partial sums, block set-up).
  // With several a^V ranges, split at range boundaries (powers of two, at
  // most one split per range) so that the center masses are not duplicated.
  const int GV = (int)ceil_div(A_v, CR);
  const int64_t blocks = std::max<int64_t>(1, ceil_div(Nq, RBW) * n_heads);
  const int64_t tiles = ceil_div(n_low, NT);
  auto score = [&](int S) {
    const double r = (double)(blocks * S) / 256.0;
    return r / std::ceil(r) - 0.004 * S;
  };
  LowSplit best{1, false};
  double bs = score(1);
  if (GV >= 2) {
    for (int S = 2; S <= 16 && S <= GV && tiles >= 8 * S; S *= 2)
      if (score(S) > bs + 1e-3) {
        bs = score(S);
        best = LowSplit{S, true};
      }
  } else {
    for (int S = 2; S <= 16 && tiles >= 8 * S; ++S)
      if (score(S) > bs + 1e-3) {
        bs = score(S);
        best = LowSplit{S, false};
      }
  }
  return best;
}

int64_t low_part_units(int64_t Nq, int H, int32_t r_low, const int32_t* r_low_h, int64_t n_low,
                       int A_v) {
  int64_t best = 0;
  std::vector<int> done(H, 0);
  for (int h0 = 0; h0 < H; ++h0) {
    if (done[h0]) continue;
    int n = 0;
    for (int h = h0; h < H; ++h) {
      const int w0 = r_low_h ? r_low_h[h0] : r_low, w = r_low_h ? r_low_h[h] : r_low;
      if (!done[h] && w == w0) {
        done[h] = 1;
        ++n;
      }
    }
    best = std::max<int64_t>(best, (int64_t)n * low_split_plan(Nq, n, n_low, A_v).S);
  }
  return best;
}

size_t low_workspace_bytes(const nkv_shape* s, int32_t A_k, int32_t A_v, const RangeTable& low,
                           int32_t r_low, const int32_t* r_low_h, int64_t Nq) {
  const int64_t units = low_part_units(Nq, s->H, r_low, r_low_h, low.total, A_v);
  return make_plan(s, A_k, A_v, low, r_low, Nq, units).total;
}

nkv_status launch_low(const nkv_shape* s, const BranchArgs& kb, const BranchArgs& vb,
                      const LowMaps& mp, const RangeTable& low, int32_t r_low, float tau,
                      const uint16_t* q,
                      int64_t Nq, float* o_low, float* lse_low, char* ws, int32_t r_low_max,
                      int64_t part_units, const HeadSet& hs, bool first, hipStream_t st) {
  // offsets from the widest group's plan, so that every group finds the
  // shared sort results in the same place; geometry from this group's width
  const Plan P = make_plan(s, kb.A, vb.A, low, r_low_max, Nq, part_units);
  const LowSplit split = low_split_plan(Nq, hs.n, low.total, vb.A);
  const int nsplit = split.S;
  const int rlp = (int)ceil_div(r_low, 16) * 16, ra = (int)ceil_div(r_low, 32) * 32;
  const TileGeom geom = tile_geom(rlp);
  const int H = s->H, W = H * s->d, r = s->r;
  const float c = tau * 1.4426950408889634f;
  auto at = [&](size_t off) { return ws + off; };
  uint16_t* dkt = reinterpret_cast<uint16_t*>(at(P.dkt));
  uint16_t* mvt = reinterpret_cast<uint16_t*>(at(P.mvt));
  float* qt32 = reinterpret_cast<float*>(at(P.qt32));
  uint16_t* qt16 = reinterpret_cast<uint16_t*>(at(P.qt16));
  float* bound = reinterpret_cast<float*>(at(P.bound));
  uint32_t* tmax = reinterpret_cast<uint32_t*>(at(P.tmax));
  uint32_t* present = reinterpret_cast<uint32_t*>(at(P.present));
  uint32_t* misc = reinterpret_cast<uint32_t*>(at(P.misc));
  int32_t* flags = reinterpret_cast<int32_t*>(at(P.flags));
  int32_t* cnt = reinterpret_cast<int32_t*>(at(P.cnt));
  int32_t* base = reinterpret_cast<int32_t*>(at(P.base));
  int32_t* tile_start = reinterpret_cast<int32_t*>(at(P.tile_start));
  int32_t* bcount = reinterpret_cast<int32_t*>(at(P.bcount));
  int32_t* tile_bucket = reinterpret_cast<int32_t*>(at(P.tile_bucket));
  int32_t* perm = reinterpret_cast<int32_t*>(at(P.perm));
  char* img = at(P.img);
  float* acc = reinterpret_cast<float*>(at(P.acc));
  float* wmass = reinterpret_cast<float*>(at(P.wmass));
  float* ell = reinterpret_cast<float*>(at(P.ell));
  nkv_status e;
  {
  ProfScope ps_prep("low_prep_tables", st);

  // zero the counters and row maxima (kernels: capturable)
  hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)ceil_div(P.rows, 256)), dim3(256), 0, st, tmax, P.rows);
  hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(64), 0, st, misc, (int64_t)4);
  NKV_LAUNCH_CHECK();
  // transposed query-reduction map (this width), transposed V centers
  auto transpose = [&](const void* src, int R, int C, int lds, uint16_t* dst, int ldd) {
    const dim3 grid((unsigned)ceil_div(ldd, 64), (unsigned)ceil_div(C, 64));
    const bool wide = lds % 8 == 0 && ldd % 8 == 0 && C % 8 == 0 &&
                      ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) == 0;
    if (wide)
      hipLaunchKernelGGL(k_transpose_bf16_16, grid, dim3(256), 0, st,
                         static_cast<const uint16_t*>(src), R, C, lds, dst, ldd);
    else
      hipLaunchKernelGGL(k_transpose_bf16, grid, dim3(256), 0, st, static_cast<const uint16_t*>(src),
                         R, C, lds, dst, ldd);
  };
  transpose(mp.qmap, W, r_low, mp.ld, dkt, W);
  if (first) transpose(vb.centers, vb.A, W, W, mvt, P.avp);
  NKV_LAUNCH_CHECK();
  }
  if (first) {
  ProfScope ps_sort("low_prep_sort", st);
  hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)ceil_div(kb.A, 256)), dim3(256), 0, st, present,
                     (int64_t)ceil_div(kb.A, 64) * 64);
  // bucket sort of the low-routed tokens
  const int nch = (int)P.nchunk;
  hipLaunchKernelGGL(k_bucket_count, dim3(nch), dim3(256), 2 * P.NB * sizeof(int), st, kb, vb, low,
                     P.GK, P.NB, cnt, present);
  // the tile counts go through `base` (rewritten right after)
  hipLaunchKernelGGL(k_bucket_tot, dim3(P.NB), dim3(256), 0, st, cnt, nch, P.NB, bcount, base);
  hipLaunchKernelGGL(k_bucket_tiles, dim3(1), dim3(1024), 0, st, base, P.NB, tile_start,
                     tile_bucket);
  hipLaunchKernelGGL(k_bucket_base, dim3(P.NB), dim3(256), 0, st, cnt, nch, P.NB, tile_start,
                     base);
  hipLaunchKernelGGL(k_bucket_scatter, dim3(nch), dim3(256), 0, st, kb, vb, low, P.GK, P.NB, base,
                     perm);
  }
  {
  ProfScope ps_img("low_prep_images", st);
  hipLaunchKernelGGL(k_build_images, dim3((unsigned)P.max_tiles), dim3(256), 0, st,
                     kb, vb, r, s->group, r_low, geom, tile_start, tile_bucket, bcount, P.NB, P.GK, perm,
                     img, misc);
  NKV_LAUNCH_CHECK();
  }
  {
  ProfScope ps_q("low_prep_query", st);
  // query reduction and per-row score bounds
  QtProblem qp{(int)Nq, r_low, 128, H, q, dkt, qt32, hs};
  if ((e = qp.dma_ok() ? launch_gemm_dma(qp, hs.n, st) : launch_gemm(qp, hs.n, st))) return e;
  hipLaunchKernelGGL(k_center_max, dim3((unsigned)ceil_div(Nq, CM_Q), (unsigned)hs.n), dim3(256),
                     0, st, q, static_cast<const uint16_t*>(kb.centers), present, Nq, H, kb.A, hs,
                     tmax);
  NKV_LAUNCH_CHECK();
  hipLaunchKernelGGL(k_row_bound, dim3((unsigned)ceil_div(Nq * hs.n * 16, 256)), dim3(256), 0, st,
                     qt32, Nq, H, hs, r_low, rlp, c, tmax, misc, bound, qt16, flags,
                     reinterpret_cast<int32_t*>(misc + 1));
  NKV_LAUNCH_CHECK();
  }
  // main pass
  {
  ProfScope ps_main("low_main", st);
  MainArgs m{q, static_cast<const uint16_t*>(kb.centers), qt16, bound, img, tile_start,
             tile_bucket, acc, wmass, ell, Nq, H, kb.A, vb.A, P.GK, P.GV, P.NB, r_low, ra,
             split.gv ? 1 : 0, (int)ceil_div(Nq, RBW), nsplit,
             Nq % RBW != 0 ? 1 : 0, c, hs};
  switch (rlp) {
    case 16: e = launch_main<16>(m, st); break;
    case 32: e = launch_main<32>(m, st); break;
    case 48: e = launch_main<48>(m, st); break;
    case 64: e = launch_main<64>(m, st); break;
    case 80: e = launch_main<80>(m, st); break;
    case 96: e = launch_main<96>(m, st); break;
    case 112: e = launch_main<112>(m, st); break;
    case 128: e = launch_main<128>(m, st); break;
    default: set_error("tuned low-dimensional read supports r_low <= 128"); return NKV_EUNSUPPORTED;
  }
  if (e) return e;
  }
  // restoration
  {
  ProfScope ps_restore("low_restore", st);
  const float* acc_r = acc;
  const float* ell_r = ell;
  const float* wmass_r = wmass;
  bool planes = nsplit == 1 || split.gv;
  if (nsplit > 1) {
    // split coefficient sums, and (a single a^V range: key-range splits)
    // the fp32 center-mass partials, reduced to planes in one launch
    const int64_t rows_g = Nq * hs.n;
    uint16_t* mplanes = !planes && P.rmass ? reinterpret_cast<uint16_t*>(at(P.rmass)) : nullptr;
    const int64_t n = rows_g * (ra / 4) + (mplanes ? rows_g * (P.GV * CR / 4) : 0);
    hipLaunchKernelGGL(k_reduce_acc, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, st, acc, ell,
                       rows_g, nsplit, r_low, ra, reinterpret_cast<uint16_t*>(at(P.racc)),
                       reinterpret_cast<float*>(at(P.rell)), wmass, Nq, hs.n, vb.A, P.GV * CR,
                       mplanes);
    NKV_LAUNCH_CHECK();
    acc_r = reinterpret_cast<const float*>(at(P.racc));
    ell_r = reinterpret_cast<const float*>(at(P.rell));
    if (mplanes) {
      wmass_r = reinterpret_cast<const float*>(mplanes);
      planes = true;
    }
  }
  RestoreProblem rp{(int)Nq, 128, 2 * ra + 2 * P.av, H, mp.ld, r_low, ra, vb.A, P.av, nsplit,
                    P.GV * CR, planes ? 1 : 0, acc_r, wmass_r,
                    static_cast<const uint16_t*>(mp.omap), mvt, ell_r, bound, o_low, lse_low, hs};
  if ((e = rp.dma_ok() ? launch_gemm_dma(rp, hs.n, st) : launch_gemm(rp, hs.n, st))) return e;
  }
  // rows whose bound may be loose: exact generic recomputation
  ProfScope ps_fallback("low_fallback", st);
  return launch_low_generic(NKV_BF16, q, Nq, H, s->d, r, s->group, r_low, tau, kb, vb, mp, low, flags,
                            reinterpret_cast<int32_t*>(misc + 1), P.rows, o_low, lse_low, st);
}

}  // namespace nkv
