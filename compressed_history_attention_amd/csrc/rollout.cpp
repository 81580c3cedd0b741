// Rollout support of libnanokv: the per-layer routing policy of the deployed
// Fast configurations (Table 7 of the NanoKV page), storage accounting
// (Figure 8 and Table 1) and the per-layer cache calls that a rollout loop
// makes for every chunk (attend over the history, then encode and append;
// Figure 4(a)/(b)).  Host logic only; the work runs in the library's kernels
// through nkv_attend_full / nkv_attend_fast_heads / nkv_encode.
#include <stdint.h>

#include <vector>

#include "nkv_common.hpp"

namespace nkv {

static nkv_status check_policy(const nkv_route_policy* p) {
  if (!p) { set_error("policy is NULL"); return NKV_EINVAL; }
  if (p->frame_tokens < 1 || p->recent_frames < 0 || p->sink_frames < 0 ||
      p->anchor_every < 0 || p->all_full_frames < 0) {
    set_error("policy: frame_tokens must be positive and frame counts non-negative");
    return NKV_EINVAL;
  }
  return NKV_OK;
}

// Route of frame f in a history of nf frames.
static int frame_mode(const nkv_route_policy* p, int64_t f, int64_t nf) {
  if (p->layer_full || nf <= p->all_full_frames) return NKV_FULL;
  if (f < p->sink_frames || f >= nf - p->recent_frames) return NKV_FULL;
  if (p->anchor_every > 0 && f % p->anchor_every == 0) return NKV_FULL;
  return NKV_LOW;
}

// Segments of the policy, one frame at a time, runs of one mode merged.
static void policy_segments(const nkv_route_policy* p, int64_t n_hist,
                            std::vector<nkv_segment>& out) {
  out.clear();
  if (n_hist <= 0) return;
  const int64_t T = p->frame_tokens;
  const int64_t nf = (n_hist + T - 1) / T;
  for (int64_t f = 0; f < nf; ++f) {
    const int mode = frame_mode(p, f, nf);
    const int64_t b = f * T, e = b + T < n_hist ? b + T : n_hist;
    if (!out.empty() && out.back().mode == mode) {
      out.back().end = e;
    } else {
      out.push_back(nkv_segment{b, e, mode});
    }
  }
}

}  // namespace nkv

using namespace nkv;

extern "C" {

nkv_status nkv_route_segments(const nkv_route_policy* policy, int64_t n_hist, nkv_segment* out,
                              int32_t max_out, int32_t* n_out) {
  if (!n_out) { set_error("n_out is NULL"); return NKV_EINVAL; }
  *n_out = 0;
  nkv_status st = check_policy(policy);
  if (st) return st;
  if (n_hist < 0) { set_error("n_hist negative"); return NKV_EINVAL; }
  std::vector<nkv_segment> segs;
  policy_segments(policy, n_hist, segs);
  if (segs.size() > (size_t)INT32_MAX) { set_error("too many segments"); return NKV_EINVAL; }
  *n_out = (int32_t)segs.size();
  if ((int64_t)segs.size() > (int64_t)max_out || (!out && !segs.empty())) {
    set_error("%zu segments needed, room for %d", segs.size(), max_out);
    return NKV_EINVAL;
  }
  for (size_t i = 0; i < segs.size(); ++i) out[i] = segs[i];
  return NKV_OK;
}

nkv_status nkv_storage_account(const nkv_shape* shape, int32_t A_k, int32_t A_v, int64_t n_hist,
                               nkv_storage* out) {
  if (!shape || !out) { set_error("NULL shape or out"); return NKV_EINVAL; }
  if (shape->H < 1 || shape->d < 1 || shape->r < 2 || shape->r % 2 || shape->group < 1 ||
      shape->r % shape->group || (shape->dtype != NKV_F32 && shape->dtype != NKV_BF16)) {
    set_error("invalid shape");
    return NKV_EINVAL;
  }
  if (A_k < 1 || A_v < 1 || n_hist < 0) {
    set_error("A_k, A_v must be positive and n_hist non-negative");
    return NKV_EINVAL;
  }
  const int64_t W = (int64_t)shape->H * shape->d, r = shape->r;
  const int64_t e = shape->dtype == NKV_BF16 ? 2 : 4;
  nkv_storage s{};
  s.idx = 2 * n_hist * 4;
  s.codes = 2 * n_hist * (r / 2);
  s.scales = 2 * n_hist * 2 * (r / shape->group);
  s.cached = s.idx + s.codes + s.scales;
  s.centers = ((int64_t)A_k + A_v) * W * e;
  s.encoders = 2 * r * W * e;
  s.decoders = 2 * W * r * e;
  s.resident = s.centers + s.encoders + s.decoders;
  s.total = s.cached + s.resident;
  s.original = 2 * n_hist * W * 2;
  s.cr_effective = s.total ? (double)s.original / (double)s.total : 0.0;
  s.cr_cached = s.cached ? (double)s.original / (double)s.cached : 0.0;
  s.cr_nominal = (double)(W * 16) / (double)(r * 4);
  *out = s;
  return NKV_OK;
}

}  // extern "C"

namespace nkv {

static nkv_status check_cache(const nkv_layer_cache* c) {
  if (!c) { set_error("cache is NULL"); return NKV_EINVAL; }
  if (c->n_hist < 0 || c->capacity < c->n_hist) {
    set_error("cache: need 0 <= n_hist <= capacity (n_hist=%lld capacity=%lld)",
              (long long)c->n_hist, (long long)c->capacity);
    return NKV_EINVAL;
  }
  return NKV_OK;
}

static nkv_branch view(const nkv_cache_branch& b) {
  return nkv_branch{b.idx, b.codes, b.scales, b.centers, b.decoder, b.A};
}

static bool all_full(const std::vector<nkv_segment>& segs) {
  for (auto& s : segs)
    if (s.mode != NKV_FULL) return false;
  return true;
}

}  // namespace nkv

extern "C" {

size_t nkv_layer_attend_workspace_size(const nkv_shape* shape, const nkv_layer_cache* cache,
                                       const nkv_route_policy* policy, const int32_t* r_low_h,
                                       int64_t Nq, int64_t N_cur) {
  if (check_cache(cache) || check_policy(policy)) return SIZE_MAX;
  std::vector<nkv_segment> segs;
  policy_segments(policy, cache->n_hist, segs);
  if (all_full(segs))
    return nkv_attend_workspace_size(shape, cache->k.A, cache->v.A, cache->n_hist, nullptr, 0, 0,
                                     Nq, N_cur);
  if (!r_low_h) return SIZE_MAX;
  return nkv_attend_heads_workspace_size(shape, cache->k.A, cache->v.A, cache->n_hist, segs.data(),
                                         (int32_t)segs.size(), r_low_h, Nq, N_cur);
}

nkv_status nkv_layer_attend(const nkv_shape* shape, const nkv_layer_cache* cache,
                            const nkv_route_policy* policy, const int32_t* r_low_h, const void* q,
                            int64_t Nq, const void* cur_k, const void* cur_v, int64_t N_cur,
                            void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  nkv_status st = check_cache(cache);
  if (st) return st;
  if ((st = check_policy(policy))) return st;
  std::vector<nkv_segment> segs;
  policy_segments(policy, cache->n_hist, segs);
  const nkv_branch kb = view(cache->k), vb = view(cache->v);
  if (all_full(segs))
    return nkv_attend_full(shape, &kb, &vb, cache->n_hist, q, Nq, cur_k, cur_v, N_cur, out, lse,
                           ws, ws_bytes, stream);
  if (!r_low_h) {
    set_error("r_low_h is NULL but the policy routes part of the history low");
    return NKV_EINVAL;
  }
  return nkv_attend_fast_heads(shape, &kb, &vb, cache->n_hist, segs.data(), (int32_t)segs.size(),
                               r_low_h, q, Nq, cur_k, cur_v, N_cur, out, lse, ws, ws_bytes,
                               stream);
}

size_t nkv_layer_append_workspace_size(const nkv_shape* shape, const nkv_layer_cache* cache,
                                       int64_t N) {
  if (check_cache(cache) || N < 0) return SIZE_MAX;
  const size_t a = nkv_encode_workspace_size(shape, N, cache->k.A);
  const size_t b = nkv_encode_workspace_size(shape, N, cache->v.A);
  if (a == SIZE_MAX || b == SIZE_MAX) return SIZE_MAX;
  return a > b ? a : b;
}

nkv_status nkv_layer_append(const nkv_shape* shape, nkv_layer_cache* cache, const void* k_new,
                            const void* v_new, int64_t N, void* ws, size_t ws_bytes,
                            void* stream) {
  nkv_status st = check_cache(cache);
  if (st) return st;
  if (!shape) { set_error("shape is NULL"); return NKV_EINVAL; }
  if (N < 0) { set_error("N negative"); return NKV_EINVAL; }
  if (N > cache->capacity - cache->n_hist) {
    set_error("cache full: n_hist=%lld + N=%lld exceeds capacity %lld", (long long)cache->n_hist,
              (long long)N, (long long)cache->capacity);
    return NKV_EINVAL;
  }
  if (N == 0) return NKV_OK;
  // validate both branches and the workspace before enqueuing anything
  const size_t need = nkv_layer_append_workspace_size(shape, cache, N);
  if (need == SIZE_MAX) {
    set_error("invalid shape or center count for the cache's codecs");
    return NKV_EINVAL;
  }
  if (need > 0 && (!ws || ws_bytes < need)) {
    set_error("workspace of %zu bytes needed, %zu given", need, ws_bytes);
    return NKV_EWORKSPACE;
  }
  nkv_cache_branch* br[2] = {&cache->k, &cache->v};
  const void* src[2] = {k_new, v_new};
  for (int b = 0; b < 2; ++b) {
    const nkv_cache_branch& c = *br[b];
    if (!src[b] || !c.idx || !c.codes || !c.scales || !c.centers || !c.encoder) {
      set_error("%s branch: NULL rows, history arrays or codec", b ? "V" : "K");
      return NKV_EINVAL;
    }
  }
  const int64_t n0 = cache->n_hist;
  const int64_t cb = shape->r / 2, sb = shape->r / shape->group;
  for (int b = 0; b < 2; ++b) {
    nkv_cache_branch& c = *br[b];
    st = nkv_encode(shape, src[b], N, c.centers, c.A, c.encoder, c.idx + n0, c.codes + n0 * cb,
                    c.scales + n0 * sb, ws, ws_bytes, stream);
    if (st) return st;
  }
  cache->n_hist = n0 + N;
  return NKV_OK;
}

}  // extern "C"
