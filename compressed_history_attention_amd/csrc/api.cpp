// C ABI of libnanokv: validation, workspace layout and dispatch.
//
// Every argument is checked on the host before anything is enqueued; the
// work itself runs in the HIP kernels of this library on the caller's stream.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "kernels.hpp"
#include "prof.hpp"
#include "tuned.hpp"

namespace nkv {

static thread_local char g_err[512];
static int g_force_generic = 0;

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

#define NKV_FAIL(code, ...)      \
  do {                           \
    ::nkv::set_error(__VA_ARGS__); \
    return code;                 \
  } while (0)

static nkv_status check_shape(const nkv_shape* s) {
  if (!s) NKV_FAIL(NKV_EINVAL, "shape is NULL");
  if (s->H < 1 || s->d < 1 || s->r < 1 || s->group < 1)
    NKV_FAIL(NKV_EINVAL, "H, d, r and group must be positive (H=%d d=%d r=%d group=%d)", s->H,
             s->d, s->r, s->group);
  if (s->dtype != NKV_F32 && s->dtype != NKV_BF16)
    NKV_FAIL(NKV_EINVAL, "dtype must be NKV_F32 or NKV_BF16 (got %d)", s->dtype);
  if (s->d != 16 && s->d != 32 && s->d != 64 && s->d != 128)
    NKV_FAIL(NKV_EUNSUPPORTED, "head dimension %d not in {16, 32, 64, 128}", s->d);
  if (s->group != 8 && s->group != 16 && s->group != 32 && s->group != 64)
    NKV_FAIL(NKV_EUNSUPPORTED, "group %d not in {8, 16, 32, 64}", s->group);
  if (s->r % 2 || s->r % s->group)
    NKV_FAIL(NKV_EUNSUPPORTED, "r=%d must be even and a multiple of group=%d", s->r, s->group);
  if ((int64_t)s->H * s->d > 8192) NKV_FAIL(NKV_EUNSUPPORTED, "H*d above 8192");
  if (s->r > 4096) NKV_FAIL(NKV_EUNSUPPORTED, "r above 4096");
  if (!(s->softmax_scale == s->softmax_scale) || isinf(s->softmax_scale))
    NKV_FAIL(NKV_EINVAL, "softmax_scale is not finite");
  return NKV_OK;
}

static float tau_of(const nkv_shape* s) {
  return s->softmax_scale > 0.f ? s->softmax_scale : 1.0f / sqrtf((float)s->d);
}

static bool tuned_applies(const nkv_shape* s, int32_t r_low) {
  if (g_force_generic) return false;
  return s->dtype == NKV_BF16 && s->d == 128 && s->r % 32 == 0 &&
         (r_low == 0 || (r_low % 16 == 0 && r_low <= 128));
}

// Build FULL / LOW range tables from a route; adjacent same-mode ranges are
// joined.  route == NULL means everything FULL.
static nkv_status build_routes(const nkv_segment* route, int32_t n_seg, int64_t N_hist,
                               RangeTable* full, RangeTable* low) {
  memset(full, 0, sizeof(*full));
  memset(low, 0, sizeof(*low));
  std::vector<nkv_segment> segs;
  if (!route || n_seg == 0) {
    if (n_seg != 0) NKV_FAIL(NKV_EINVAL, "route is NULL but n_seg=%d", n_seg);
    if (N_hist > 0) segs.push_back({0, N_hist, NKV_FULL});
  } else {
    if (n_seg < 0) NKV_FAIL(NKV_EINVAL, "n_seg negative");
    segs.assign(route, route + n_seg);
    for (auto& g : segs) {
      if (g.mode != NKV_FULL && g.mode != NKV_LOW)
        NKV_FAIL(NKV_EINVAL, "segment mode %d is neither NKV_FULL nor NKV_LOW", g.mode);
      if (g.begin < 0 || g.end < g.begin || g.end > N_hist)
        NKV_FAIL(NKV_EINVAL, "segment [%lld, %lld) outside [0, %lld)", (long long)g.begin,
                 (long long)g.end, (long long)N_hist);
    }
    std::sort(segs.begin(), segs.end(),
              [](const nkv_segment& a, const nkv_segment& b) { return a.begin < b.begin; });
    int64_t pos = 0;
    for (auto& g : segs) {
      if (g.begin != pos)
        NKV_FAIL(NKV_EINVAL, "segments must be disjoint and cover [0, N_hist) (gap/overlap at %lld)",
                 (long long)pos);
      pos = g.end;
    }
    if (pos != N_hist) NKV_FAIL(NKV_EINVAL, "segments cover [0, %lld) not [0, %lld)",
                                (long long)pos, (long long)N_hist);
  }
  for (auto& g : segs) {
    if (g.end == g.begin) continue;
    RangeTable* t = g.mode == NKV_FULL ? full : low;
    if (t->n > 0 && t->begin[t->n - 1] + (t->prefix[t->n] - t->prefix[t->n - 1]) == g.begin) {
      t->prefix[t->n] += g.end - g.begin;  // join with the previous adjacent range
    } else {
      if (t->n == NKV_MAX_SEGMENTS)
        NKV_FAIL(NKV_EUNSUPPORTED, "more than %d ranges of one mode", NKV_MAX_SEGMENTS);
      t->begin[t->n] = g.begin;
      t->prefix[t->n + 1] = t->prefix[t->n] + (g.end - g.begin);
      t->n += 1;
    }
    t->total = t->prefix[t->n];
  }
  return NKV_OK;
}

static nkv_status check_branch(const nkv_branch* b, const char* name, int64_t N_hist) {
  if (!b) NKV_FAIL(NKV_EINVAL, "%s branch is NULL", name);
  if (b->A < 1) NKV_FAIL(NKV_EINVAL, "%s branch: A=%d must be positive", name, b->A);
  if (b->A > 4096) NKV_FAIL(NKV_EUNSUPPORTED, "%s branch: A=%d above 4096", name, b->A);
  if (!b->centers || !b->decoder) NKV_FAIL(NKV_EINVAL, "%s branch: NULL centers/decoder", name);
  if (N_hist > 0 && (!b->idx || !b->codes || !b->scales))
    NKV_FAIL(NKV_EINVAL, "%s branch: NULL idx/codes/scales with N_hist>0", name);
  return NKV_OK;
}

static BranchArgs to_args(const nkv_branch* b) {
  return BranchArgs{b->idx, b->codes, b->scales, b->centers, b->decoder, b->A};
}

// --------------------------------------------------------------------------
// generic-path workspace
// --------------------------------------------------------------------------
struct GenericLayout {
  size_t k, v, o_full, lse_full, o_low, lse_low, rows, total;
};

static GenericLayout generic_layout(const nkv_shape* s, int64_t n_full, int64_t n_low, int64_t Nq,
                                    int64_t N_cur, bool per_head = false) {
  GenericLayout L{};
  const int64_t W = (int64_t)s->H * s->d;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  const int64_t nk = n_full + N_cur;
  L.k = take(sizeof(float) * nk * W);
  L.v = take(sizeof(float) * nk * W);
  if (n_low > 0) {
    L.o_full = take(sizeof(float) * Nq * W);
    L.lse_full = take(sizeof(float) * Nq * s->H);
    L.o_low = take(sizeof(float) * Nq * W);
    L.lse_low = take(sizeof(float) * Nq * s->H);
    if (per_head) L.rows = take(sizeof(int32_t) * (Nq * s->H + 1));  // row list + its length
  }
  L.total = off;
  return L;
}

// widths of a per-head call: each in [1, r]; returns the widest (0 on error)
static int32_t check_widths(const nkv_shape* s, const int32_t* r_low_h) {
  if (!r_low_h) {
    set_error("r_low_h is NULL");
    return 0;
  }
  if (s->H > NKV_MAX_HEADS) {
    set_error("per-head widths support H <= %d (H=%d)", NKV_MAX_HEADS, s->H);
    return 0;
  }
  int32_t mx = 0;
  for (int h = 0; h < s->H; ++h) {
    if (r_low_h[h] < 1 || r_low_h[h] > s->r) {
      set_error("r_low_h[%d]=%d must be in [1, r=%d]", h, r_low_h[h], s->r);
      return 0;
    }
    mx = std::max(mx, r_low_h[h]);
  }
  return mx;
}

// the tuned kernels serve a call when they serve every width in it
static bool tuned_applies_all(const nkv_shape* s, int32_t r_low, const int32_t* r_low_h) {
  if (!tuned_applies(s, r_low)) return false;
  if (r_low_h)
    for (int h = 0; h < s->H; ++h)
      if (!tuned_applies(s, r_low_h[h])) return false;
  return true;
}

static size_t workspace_common(const nkv_shape* shape, int32_t A_k, int32_t A_v, int64_t N_hist,
                               const nkv_segment* route, int32_t n_seg, int32_t r_low,
                               const int32_t* r_low_h, int64_t Nq, int64_t N_cur,
                               bool tuned_maps = true);

static nkv_status attend_common(const nkv_shape* shape, const nkv_branch* k, const nkv_branch* v,
                                int64_t N_hist, const nkv_segment* route, int32_t n_seg,
                                int32_t r_low, const int32_t* r_low_h, const nkv_low_maps* maps,
                                const void* q, int64_t Nq, const void* cur_k, const void* cur_v,
                                int64_t N_cur, void* out, float* lse, void* ws, size_t ws_bytes,
                                void* stream_, bool fast) {
  nkv_status st = check_shape(shape);
  if (st) return st;
  if ((st = check_branch(k, "K", N_hist)) || (st = check_branch(v, "V", N_hist))) return st;
  if (N_hist < 0 || Nq < 0 || N_cur < 0) NKV_FAIL(NKV_EINVAL, "negative size");
  if (Nq > (int64_t)1 << 31 || N_hist > (int64_t)1 << 31 || N_cur > (int64_t)1 << 31)
    NKV_FAIL(NKV_EUNSUPPORTED, "sizes above 2^31");
  if (Nq > 0 && (!q || !out || !lse)) NKV_FAIL(NKV_EINVAL, "NULL q/out/lse with Nq>0");
  if (N_cur > 0 && (!cur_k || !cur_v)) NKV_FAIL(NKV_EINVAL, "NULL current chunk with N_cur>0");
  RangeTable full, low;
  if (fast) {
    if (r_low_h && !(r_low = check_widths(shape, r_low_h))) return NKV_EUNSUPPORTED;
    if (r_low < 1 || r_low > shape->r)
      NKV_FAIL(NKV_EUNSUPPORTED, "r_low=%d must be in [1, r=%d]", r_low, shape->r);
    if ((st = build_routes(route, n_seg, N_hist, &full, &low))) return st;
  } else {
    if ((st = build_routes(nullptr, 0, N_hist, &full, &low))) return st;
  }
  // Nothing routed low: the widths play no part, exactly as in the size query
  // (workspace_common), so dispatch and workspace layout are the same
  if (low.total == 0) {
    r_low = 0;
    r_low_h = nullptr;
  }
  // query-reduction / restoration maps: the decoders unless the caller gives others
  LowMaps mp{k->decoder, v->decoder, shape->r};
  if (maps) {
    if (!maps->q_map || !maps->o_map) NKV_FAIL(NKV_EINVAL, "maps: NULL q_map/o_map");
    if (maps->ld < r_low)
      NKV_FAIL(NKV_EINVAL, "maps: ld=%d below the widest r_low=%d", maps->ld, r_low);
    mp = LowMaps{maps->q_map, maps->o_map, maps->ld};
  }
  const bool tuned_maps = mp.ld % 8 == 0 && (reinterpret_cast<uintptr_t>(mp.qmap) & 15) == 0 &&
                          (reinterpret_cast<uintptr_t>(mp.omap) & 15) == 0;
  const bool tuned = tuned_applies_all(shape, r_low, r_low_h) && (low.total == 0 || tuned_maps);
  if (low.total > 0 && r_low > 512 && !tuned)
    NKV_FAIL(NKV_EUNSUPPORTED, "generic low-dimensional read supports r_low <= 512");
  const size_t need = workspace_common(shape, k->A, v->A, N_hist, fast ? route : nullptr,
                                       fast ? n_seg : 0, r_low, r_low_h, Nq, N_cur, tuned_maps);
  if (need == SIZE_MAX) return NKV_EINVAL;
  if (Nq == 0) return NKV_OK;
  if (need > 0 && (!ws || ws_bytes < need))
    NKV_FAIL(NKV_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  hipStream_t s = static_cast<hipStream_t>(stream_);
  const float tau = tau_of(shape);
  const int dt = shape->dtype, H = shape->H, d = shape->d, r = shape->r, g = shape->group;
  const BranchArgs kb = to_args(k), vb = to_args(v);

  if (tuned) {
    return tuned_attend(shape, kb, vb, mp, full, low, r_low, r_low_h, tau, q, Nq, cur_k, cur_v,
                        N_cur, out, lse, static_cast<char*>(ws), ws_bytes, s);
  }

  const int64_t W = (int64_t)H * d;
  const GenericLayout L = generic_layout(shape, full.total, low.total, Nq, N_cur, r_low_h != nullptr);
  if (L.total > ws_bytes)  // the size query and this layout must agree
    NKV_FAIL(NKV_EWORKSPACE, "internal: generic layout of %zu bytes exceeds the %zu given", L.total,
             ws_bytes);
  char* base = static_cast<char*>(ws);
  float* kw = reinterpret_cast<float*>(base + L.k);
  float* vw = reinterpret_cast<float*>(base + L.v);
  if ((st = launch_decode_generic(dt, kb, (int)W, r, g, full, kw, s))) return st;
  if ((st = launch_decode_generic(dt, vb, (int)W, r, g, full, vw, s))) return st;
  if ((st = launch_rows_to_f32(dt, cur_k, N_cur * W, kw + full.total * W, s))) return st;
  if ((st = launch_rows_to_f32(dt, cur_v, N_cur * W, vw + full.total * W, s))) return st;
  const int64_t nk = full.total + N_cur;
  if (low.total == 0) {
    return launch_attention_generic(dt, false, q, Nq, H, d, tau, kw, vw, nk, out, lse, s);
  }
  float* of = reinterpret_cast<float*>(base + L.o_full);
  float* lf = reinterpret_cast<float*>(base + L.lse_full);
  float* ol = reinterpret_cast<float*>(base + L.o_low);
  float* ll = reinterpret_cast<float*>(base + L.lse_low);
  if ((st = launch_attention_generic(dt, true, q, Nq, H, d, tau, kw, vw, nk, of, lf, s))) return st;
  if (!r_low_h) {
    if ((st = launch_low_generic(dt, q, Nq, H, d, r, g, r_low, tau, kb, vb, mp, low, nullptr, nullptr,
                                 Nq * H, ol, ll, s)))
      return st;
  } else {
    // one generic launch per width over the rows of its heads
    int32_t* rows = reinterpret_cast<int32_t*>(base + L.rows);
    int32_t* nrows = rows + Nq * H;
    std::vector<int> done(H, 0);
    for (int h0 = 0; h0 < H; ++h0) {
      if (done[h0]) continue;
      HeadSet hs{};
      for (int h = h0; h < H; ++h)
        if (!done[h] && r_low_h[h] == r_low_h[h0]) {
          hs.h[hs.n++] = h;
          done[h] = 1;
        }
      if ((st = launch_head_rows(Nq, H, hs, rows, nrows, s))) return st;
      if ((st = launch_low_generic(dt, q, Nq, H, d, r, g, r_low_h[h0], tau, kb, vb, mp, low, rows,
                                   nrows, Nq * hs.n, ol, ll, s)))
        return st;
    }
  }
  return launch_lse_merge(Nq, H, d, of, lf, ol, ll, out, dt, lse, s);
}

static size_t workspace_common(const nkv_shape* shape, int32_t A_k, int32_t A_v, int64_t N_hist,
                               const nkv_segment* route, int32_t n_seg, int32_t r_low,
                               const int32_t* r_low_h, int64_t Nq, int64_t N_cur,
                               bool tuned_maps) {
  if (check_shape(shape) || A_k < 1 || A_v < 1 || N_hist < 0 || Nq < 0 || N_cur < 0)
    return SIZE_MAX;
  RangeTable full, low;
  if (build_routes(route, n_seg, N_hist, &full, &low)) return SIZE_MAX;
  if (low.total == 0) {
    r_low = 0;
    r_low_h = nullptr;
  }
  if (tuned_applies_all(shape, r_low, r_low_h) && (low.total == 0 || tuned_maps))
    return tuned_attend_workspace(shape, A_k, A_v, full, low, r_low, r_low_h, Nq, N_cur);
  return generic_layout(shape, full.total, low.total, Nq, N_cur, r_low_h != nullptr).total;
}

}  // namespace nkv

using namespace nkv;

extern "C" {

int nkv_version(void) { return NKV_VERSION; }

const char* nkv_last_error(void) { return g_err; }

void nkv_force_generic(int on) { g_force_generic = on ? 1 : 0; }

const char* nkv_status_string(nkv_status s) {
  switch (s) {
    case NKV_OK: return "ok";
    case NKV_EINVAL: return "invalid argument";
    case NKV_EUNSUPPORTED: return "unsupported shape";
    case NKV_EWORKSPACE: return "workspace too small";
    case NKV_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

size_t nkv_encode_workspace_size(const nkv_shape* shape, int64_t N, int32_t A) {
  g_err[0] = 0;
  if (check_shape(shape) || N < 0 || A < 1) return SIZE_MAX;
  if (tuned_applies(shape, 0)) return tuned_encode_workspace(shape, N, A);
  return 0;
}

nkv_status nkv_encode(const nkv_shape* shape, const void* x, int64_t N, const void* centers,
                      int32_t A, const void* encoder, int32_t* idx, uint8_t* codes,
                      uint16_t* scales, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  nkv_status st = check_shape(shape);
  if (st) return st;
  if (N < 0) NKV_FAIL(NKV_EINVAL, "N negative");
  if (N > (int64_t)1 << 31) NKV_FAIL(NKV_EUNSUPPORTED, "N above 2^31");
  if (A < 1) NKV_FAIL(NKV_EINVAL, "A=%d must be positive", A);
  if (A > 65536) NKV_FAIL(NKV_EUNSUPPORTED, "A above 65536");
  if (!centers || !encoder) NKV_FAIL(NKV_EINVAL, "NULL centers/encoder");
  if (N > 0 && (!x || !idx || !codes || !scales)) NKV_FAIL(NKV_EINVAL, "NULL x/idx/codes/scales with N>0");
  if (N == 0) return NKV_OK;
  const size_t need = nkv_encode_workspace_size(shape, N, A);
  if (need > 0 && (!ws || ws_bytes < need))
    NKV_FAIL(NKV_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int W = shape->H * shape->d;
  if (tuned_applies(shape, 0))
    return tuned_encode(shape, x, N, centers, A, encoder, idx, codes, scales,
                        static_cast<char*>(ws), ws_bytes, s);
  return launch_encode_generic(shape->dtype, x, N, W, centers, A, encoder, shape->r, shape->group,
                               idx, codes, scales, s);
}

size_t nkv_attend_workspace_size(const nkv_shape* shape, int32_t A_k, int32_t A_v, int64_t N_hist,
                                 const nkv_segment* route, int32_t n_seg, int32_t r_low,
                                 int64_t Nq, int64_t N_cur) {
  return workspace_common(shape, A_k, A_v, N_hist, route, n_seg, r_low, nullptr, Nq, N_cur);
}

size_t nkv_attend_heads_workspace_size(const nkv_shape* shape, int32_t A_k, int32_t A_v,
                                       int64_t N_hist, const nkv_segment* route, int32_t n_seg,
                                       const int32_t* r_low_h, int64_t Nq, int64_t N_cur) {
  if (check_shape(shape)) return SIZE_MAX;
  const int32_t mx = check_widths(shape, r_low_h);
  if (!mx) return SIZE_MAX;
  return workspace_common(shape, A_k, A_v, N_hist, route, n_seg, mx, r_low_h, Nq, N_cur);
}

nkv_status nkv_attend_fast_heads(const nkv_shape* shape, const nkv_branch* k,
                                 const nkv_branch* v, int64_t N_hist, const nkv_segment* route,
                                 int32_t n_seg, const int32_t* r_low_h, const void* q, int64_t Nq,
                                 const void* cur_k, const void* cur_v, int64_t N_cur, void* out,
                                 float* lse, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (!shape) NKV_FAIL(NKV_EINVAL, "shape is NULL");
  if (!r_low_h) NKV_FAIL(NKV_EINVAL, "r_low_h is NULL");
  return attend_common(shape, k, v, N_hist, route, n_seg, 0, r_low_h, nullptr, q, Nq, cur_k, cur_v,
                       N_cur, out, lse, ws, ws_bytes, stream, true);
}

nkv_status nkv_attend_fast_maps(const nkv_shape* shape, const nkv_branch* k,
                                const nkv_branch* v, int64_t N_hist, const nkv_segment* route,
                                int32_t n_seg, const int32_t* r_low_h, const nkv_low_maps* maps,
                                const void* q, int64_t Nq, const void* cur_k, const void* cur_v,
                                int64_t N_cur, void* out, float* lse, void* ws, size_t ws_bytes,
                                void* stream) {
  g_err[0] = 0;
  if (!shape) NKV_FAIL(NKV_EINVAL, "shape is NULL");
  if (!r_low_h) NKV_FAIL(NKV_EINVAL, "r_low_h is NULL");
  if (!maps) NKV_FAIL(NKV_EINVAL, "maps is NULL");
  return attend_common(shape, k, v, N_hist, route, n_seg, 0, r_low_h, maps, q, Nq, cur_k, cur_v,
                       N_cur, out, lse, ws, ws_bytes, stream, true);
}

size_t nkv_attend_maps_workspace_size(const nkv_shape* shape, int32_t A_k, int32_t A_v,
                                      int64_t N_hist, const nkv_segment* route, int32_t n_seg,
                                      const int32_t* r_low_h, const nkv_low_maps* maps,
                                      int64_t Nq, int64_t N_cur) {
  if (check_shape(shape) || !maps) return SIZE_MAX;
  const int32_t mx = check_widths(shape, r_low_h);
  if (!mx || maps->ld < mx) return SIZE_MAX;
  const bool tm = maps->ld % 8 == 0 && (reinterpret_cast<uintptr_t>(maps->q_map) & 15) == 0 &&
                  (reinterpret_cast<uintptr_t>(maps->o_map) & 15) == 0;
  return workspace_common(shape, A_k, A_v, N_hist, route, n_seg, mx, r_low_h, Nq, N_cur, tm);
}

nkv_status nkv_attend_full(const nkv_shape* shape, const nkv_branch* k, const nkv_branch* v,
                           int64_t N_hist, const void* q, int64_t Nq, const void* cur_k,
                           const void* cur_v, int64_t N_cur, void* out, float* lse, void* ws,
                           size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  return attend_common(shape, k, v, N_hist, nullptr, 0, 0, nullptr, nullptr, q, Nq, cur_k, cur_v,
                       N_cur, out, lse, ws, ws_bytes, stream, false);
}

nkv_status nkv_attend_fast(const nkv_shape* shape, const nkv_branch* k, const nkv_branch* v,
                           int64_t N_hist, const nkv_segment* route, int32_t n_seg, int32_t r_low,
                           const void* q, int64_t Nq, const void* cur_k, const void* cur_v,
                           int64_t N_cur, void* out, float* lse, void* ws, size_t ws_bytes,
                           void* stream) {
  g_err[0] = 0;
  return attend_common(shape, k, v, N_hist, route, n_seg, r_low, nullptr, nullptr, q, Nq, cur_k,
                       cur_v, N_cur, out, lse, ws, ws_bytes, stream, true);
}

size_t nkv_fit_workspace_size(const nkv_shape* shape, int64_t N, int32_t A) {
  g_err[0] = 0;
  if (check_shape(shape) || N < 0 || A < 1) return SIZE_MAX;
  const int64_t W = (int64_t)shape->H * shape->d;
  const bool tuned = tuned_applies(shape, 0);
  size_t off = tuned ? tuned_assign_workspace(N, A) : 0;
  if (tuned) off = align_up(off + sizeof(float) * (size_t)N, 256);  // ||x||^2 per row
  off = align_up(off + sizeof(int32_t) * (size_t)N, 256);        // assignment
  off = align_up(off + sizeof(int32_t) * (size_t)N, 256);        // rows sorted by center
  off = align_up(off + sizeof(int32_t) * (3 * (size_t)A + 1), 256);  // counts, offsets, cursor
  return off;
}

nkv_status nkv_fit_centers(const nkv_shape* shape, const void* x, int64_t N, void* centers,
                           int32_t A, int32_t iters, int32_t* idx, int32_t* counts, void* ws,
                           size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  nkv_status st = check_shape(shape);
  if (st) return st;
  if (N < 0 || iters < 0) NKV_FAIL(NKV_EINVAL, "N and iters must be non-negative");
  if (N > (int64_t)1 << 31) NKV_FAIL(NKV_EUNSUPPORTED, "N above 2^31");
  if (A < 1) NKV_FAIL(NKV_EINVAL, "A=%d must be positive", A);
  if (A > 65536) NKV_FAIL(NKV_EUNSUPPORTED, "A above 65536");
  if (!centers) NKV_FAIL(NKV_EINVAL, "centers is NULL");
  if (N > 0 && !x) NKV_FAIL(NKV_EINVAL, "x is NULL with N>0");
  if (reinterpret_cast<uintptr_t>(x) & 15) NKV_FAIL(NKV_EINVAL, "x must be 16-byte aligned");
  const size_t need = nkv_fit_workspace_size(shape, N, A);
  if (!ws || ws_bytes < need)
    NKV_FAIL(NKV_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int W = shape->H * shape->d;
  const bool tuned = tuned_applies(shape, 0);
  char* base = static_cast<char*>(ws);
  const size_t a_bytes = tuned ? tuned_assign_workspace(N, A) : 0;
  // ||x||^2 of the rows, summed once for every assignment below (tuned)
  float* xn = reinterpret_cast<float*>(base + a_bytes);
  const size_t l_off = tuned ? align_up(a_bytes + sizeof(float) * (size_t)N, 256) : a_bytes;
  int32_t* lab = reinterpret_cast<int32_t*>(base + l_off);
  size_t off = align_up(l_off + sizeof(int32_t) * (size_t)N, 256);
  int32_t* perm = reinterpret_cast<int32_t*>(base + off);
  off = align_up(off + sizeof(int32_t) * (size_t)N, 256);
  int32_t* cnt = reinterpret_cast<int32_t*>(base + off);
  int32_t* offs = cnt + A;
  int32_t* cursor = offs + A + 1;
  auto assign = [&](int32_t* out) -> nkv_status {
    if (N == 0) return NKV_OK;
    if (tuned) return tuned_assign(shape, x, N, centers, A, out, base, s, xn);
    return launch_assign_generic(shape->dtype, x, N, W, centers, A, out, s);
  };
  if (tuned && N > 0 && (iters > 0 || idx || counts)) {
    ProfScope ps("fit_rownorm", s);
    if ((st = tuned_row_sqnorm(shape, x, N, xn, s))) return st;
  }
  for (int it = 0; it < iters; ++it) {
    {
      ProfScope ps("fit_assign", s);
      if ((st = assign(lab))) return st;
    }
    ProfScope ps("fit_update", s);
    if ((st = launch_fit_update(shape->dtype, x, N, W, lab, A, cnt, offs, cursor, perm, centers, s)))
      return st;
  }
  if (idx || counts) {
    int32_t* out = idx ? idx : lab;
    if ((st = assign(out))) return st;
    if (counts && (st = launch_fit_counts(out, N, A, counts, s))) return st;
  }
  return NKV_OK;
}

nkv_status nkv_lse_merge(int64_t Nq, int32_t H, int32_t d, const float* o_a, const float* lse_a,
                         const float* o_b, const float* lse_b, void* out, int32_t out_dtype,
                         float* lse_out, void* stream) {
  g_err[0] = 0;
  if (Nq < 0 || H < 1 || d < 1) NKV_FAIL(NKV_EINVAL, "bad sizes Nq=%lld H=%d d=%d", (long long)Nq, H, d);
  if (out_dtype != NKV_F32 && out_dtype != NKV_BF16) NKV_FAIL(NKV_EINVAL, "bad out dtype %d", out_dtype);
  if (Nq > 0 && (!o_a || !lse_a || !o_b || !lse_b || !out || !lse_out))
    NKV_FAIL(NKV_EINVAL, "NULL pointer with Nq>0");
  if ((int64_t)H * d > 16384) NKV_FAIL(NKV_EUNSUPPORTED, "H*d above 16384");
  if (Nq > (int64_t)1 << 31) NKV_FAIL(NKV_EUNSUPPORTED, "Nq above 2^31");
  // Only exact aliasing is safe: an fp32 output equal to a part (each element
  // is read, then written, by one thread) and lse_out equal to a part's LSE.
  // Any other overlap, and a bf16 output over a part's bytes, races.
  const size_t ob = (size_t)Nq * H * d * (out_dtype == NKV_F32 ? 4 : 2);
  const size_t pb = (size_t)Nq * H * d * 4, lb = (size_t)Nq * H * 4;
  auto overlap = [](const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
  };
  for (const float* part : {o_a, o_b})
    if (overlap(out, ob, part, pb) && !(out_dtype == NKV_F32 && out == (const void*)part))
      NKV_FAIL(NKV_EINVAL, "out overlaps a part other than as the same fp32 array");
  for (const float* pl : {lse_a, lse_b})
    if (overlap(lse_out, lb, pl, lb) && lse_out != pl)
      NKV_FAIL(NKV_EINVAL, "lse_out partly overlaps a part's LSE");
  if (overlap(out, ob, lse_out, lb) || overlap(out, ob, lse_a, lb) || overlap(out, ob, lse_b, lb))
    NKV_FAIL(NKV_EINVAL, "out overlaps an LSE array");
  return launch_lse_merge(Nq, H, d, o_a, lse_a, o_b, lse_b, out, out_dtype, lse_out,
                          static_cast<hipStream_t>(stream));
}

}  // extern "C"
