// Host-side fuzz of libnanokv's C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (tests/test_host_sanitize.py).
//
// Every call here either fails validation (before any HIP call) or passes
// it and fails at its first kernel launch, there being no GPU: the fuzz runs
// only where no device is visible (exit 77 otherwise).  It drives argument
// validation, route building, workspace layout and dispatch, the rollout
// policies and storage account, and the merge's overlap checks with seeded
// random arguments, and checks the invariants that hold without a GPU:
//   * a call given exactly its queried workspace never fails with
//     NKV_EWORKSPACE, one byte less always does;
//   * route segments cover [0, n_hist) in order, alternate in mode and match
//     the policy frame by frame.
// Any memory error or undefined behaviour aborts the run (sanitizer report).
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <random>
#include <vector>

#include "nanokv.h"

static int g_fail = 0;
#define CHECK(cond, ...)                                          \
  do {                                                            \
    if (!(cond)) {                                                \
      fprintf(stderr, "CHECK failed (%s:%d): ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                               \
      fprintf(stderr, " [%s]\n", nkv_last_error());               \
      ++g_fail;                                                   \
    }                                                             \
  } while (0)

// pointers that validation accepts and nothing dereferences without a GPU
static void* const FAKE = reinterpret_cast<void*>(uintptr_t(0x10000));

static std::mt19937_64 rng(20261203);
static int64_t uni(int64_t lo, int64_t hi) {  // [lo, hi]
  return lo + (int64_t)(rng() % (uint64_t)(hi - lo + 1));
}

static nkv_shape random_shape() {
  static const int ds[] = {16, 32, 64, 128};
  static const int gs[] = {8, 16, 32, 64};
  nkv_shape s{};
  s.d = ds[uni(0, 3)];
  s.H = (int)uni(1, s.d == 128 ? 8 : 16);
  s.group = gs[uni(0, 3)];
  s.r = s.group * (int)uni(1, 8);
  s.dtype = uni(0, 3) == 0 ? NKV_F32 : NKV_BF16;
  s.softmax_scale = uni(0, 1) ? 0.f : 0.125f;
  if (uni(0, 20) == 0) s.d = 100;           // unsupported
  if (uni(0, 20) == 0) s.r += 1;            // odd r
  return s;
}

static std::vector<nkv_segment> random_route(int64_t n_hist) {
  std::vector<nkv_segment> segs;
  int64_t pos = 0;
  while (pos < n_hist) {
    const int64_t len = std::min<int64_t>(n_hist - pos, uni(1, std::max<int64_t>(1, n_hist / 3)));
    segs.push_back({pos, pos + len, (int32_t)uni(0, 1)});
    pos += len;
  }
  if (!segs.empty() && uni(0, 15) == 0) segs.back().end += 1;   // out of range
  if (segs.size() > 1 && uni(0, 15) == 0) segs[1].begin -= 1;   // overlap
  if (uni(0, 15) == 0) std::swap(segs.front(), segs.back());    // unsorted (valid)
  return segs;
}

static void fuzz_attend(int iters) {
  for (int it = 0; it < iters; ++it) {
    nkv_shape s = random_shape();
    const int32_t A_k = (int32_t)uni(1, 300), A_v = (int32_t)uni(1, 300);
    const int64_t n_hist = uni(0, 3000), Nq = uni(0, 300), N_cur = uni(0, 200);
    std::vector<nkv_segment> route = random_route(n_hist);
    const int32_t r_low = (int32_t)uni(1, std::max(1, s.r));
    nkv_branch kb{(const int32_t*)FAKE, (const uint8_t*)FAKE, (const uint16_t*)FAKE, FAKE, FAKE,
                  A_k};
    nkv_branch vb = kb;
    vb.A = A_v;
    const void* cur = N_cur ? FAKE : nullptr;
    const size_t need = nkv_attend_workspace_size(&s, A_k, A_v, n_hist, route.data(),
                                                  (int32_t)route.size(), r_low, Nq, N_cur);
    nkv_status st = nkv_attend_fast(&s, &kb, &vb, n_hist, route.data(), (int32_t)route.size(),
                                    r_low, FAKE, Nq, cur, cur, N_cur, FAKE, (float*)FAKE, FAKE,
                                    need == SIZE_MAX ? 0 : need, nullptr);
    if (need != SIZE_MAX) {
      CHECK(st != NKV_EWORKSPACE, "fast: workspace %zu refused (shape d=%d r=%d r_low=%d)", need,
            s.d, s.r, r_low);
      if (need > 0 && Nq > 0 && st == NKV_EHIP) {
        st = nkv_attend_fast(&s, &kb, &vb, n_hist, route.data(), (int32_t)route.size(), r_low,
                             FAKE, Nq, cur, cur, N_cur, FAKE, (float*)FAKE, FAKE, need - 1,
                             nullptr);
        CHECK(st == NKV_EWORKSPACE, "fast: workspace %zu - 1 accepted (status %d)", need, st);
      }
    }
    // per-head widths
    std::vector<int32_t> w(s.H > 0 ? s.H : 1);
    for (auto& x : w) x = (int32_t)uni(0, s.r + 1);  // includes invalid 0 and r + 1
    const size_t need_h = nkv_attend_heads_workspace_size(&s, A_k, A_v, n_hist, route.data(),
                                                          (int32_t)route.size(), w.data(), Nq,
                                                          N_cur);
    st = nkv_attend_fast_heads(&s, &kb, &vb, n_hist, route.data(), (int32_t)route.size(), w.data(),
                               FAKE, Nq, cur, cur, N_cur, FAKE, (float*)FAKE, FAKE,
                               need_h == SIZE_MAX ? 0 : need_h, nullptr);
    if (need_h != SIZE_MAX) CHECK(st != NKV_EWORKSPACE, "heads: workspace %zu refused", need_h);
    // caller-given maps
    nkv_low_maps mp{FAKE, FAKE, (int32_t)uni(1, s.r + 8)};
    const size_t need_m = nkv_attend_maps_workspace_size(&s, A_k, A_v, n_hist, route.data(),
                                                         (int32_t)route.size(), w.data(), &mp, Nq,
                                                         N_cur);
    st = nkv_attend_fast_maps(&s, &kb, &vb, n_hist, route.data(), (int32_t)route.size(), w.data(),
                              &mp, FAKE, Nq, cur, cur, N_cur, FAKE, (float*)FAKE, FAKE,
                              need_m == SIZE_MAX ? 0 : need_m, nullptr);
    if (need_m != SIZE_MAX) CHECK(st != NKV_EWORKSPACE, "maps: workspace %zu refused", need_m);
    // the full read
    const size_t need_f = nkv_attend_workspace_size(&s, A_k, A_v, n_hist, nullptr, 0, 0, Nq,
                                                    N_cur);
    st = nkv_attend_full(&s, &kb, &vb, n_hist, FAKE, Nq, cur, cur, N_cur, FAKE, (float*)FAKE, FAKE,
                         need_f == SIZE_MAX ? 0 : need_f, nullptr);
    if (need_f != SIZE_MAX) CHECK(st != NKV_EWORKSPACE, "full: workspace %zu refused", need_f);
  }
}

static void fuzz_encode_fit_merge(int iters) {
  for (int it = 0; it < iters; ++it) {
    nkv_shape s = random_shape();
    const int64_t N = uni(0, 5000);
    const int32_t A = (int32_t)uni(0, 2000);
    const size_t need = nkv_encode_workspace_size(&s, N, A);
    nkv_status st = nkv_encode(&s, FAKE, N, FAKE, A, FAKE, (int32_t*)FAKE, (uint8_t*)FAKE,
                               (uint16_t*)FAKE, FAKE, need == SIZE_MAX ? 0 : need, nullptr);
    if (need != SIZE_MAX) CHECK(st != NKV_EWORKSPACE, "encode: workspace %zu refused", need);
    st = nkv_encode_noalloc(&s, FAKE, N, FAKE, A, FAKE, (int32_t*)FAKE, (uint8_t*)FAKE,
                            (uint16_t*)FAKE, nullptr);
    if (need != SIZE_MAX && need > NKV_NOALLOC_SCRATCH_BYTES)
      CHECK(st == NKV_EUNSUPPORTED, "noalloc: %zu bytes accepted", need);
    const size_t need_fit = nkv_fit_workspace_size(&s, N, A);
    st = nkv_fit_centers(&s, FAKE, N, FAKE, A, (int32_t)uni(0, 3), nullptr, nullptr, FAKE,
                         need_fit == SIZE_MAX ? 0 : need_fit, nullptr);
    if (need_fit != SIZE_MAX) CHECK(st != NKV_EWORKSPACE, "fit: workspace %zu refused", need_fit);
    // merge: random overlaps of the six arrays inside one arena
    const int64_t Nq = uni(0, 50);
    const int32_t H = (int32_t)uni(0, 8), d = (int32_t)uni(0, 130);
    const uintptr_t base = 0x100000;
    auto p = [&]() { return reinterpret_cast<float*>(base + 16 * (uintptr_t)uni(0, 4096)); };
    st = nkv_lse_merge(Nq, H, d, p(), p(), p(), p(), p(), (int32_t)uni(0, 2), p(), nullptr);
    (void)st;
  }
}

static int mode_of(const nkv_route_policy& p, int64_t f, int64_t nf) {
  if (p.layer_full || nf <= p.all_full_frames || f < p.sink_frames || f >= nf - p.recent_frames ||
      (p.anchor_every > 0 && f % p.anchor_every == 0))
    return NKV_FULL;
  return NKV_LOW;
}

static void fuzz_rollout(int iters) {
  for (int it = 0; it < iters; ++it) {
    nkv_route_policy p{uni(0, 20) == 0 ? 0 : uni(1, 2000), (int32_t)uni(0, 6), (int32_t)uni(0, 3),
                       (int32_t)uni(0, 20), (int32_t)uni(0, 4), (int32_t)(uni(0, 9) == 0)};
    if (uni(0, 30) == 0) p.recent_frames = -1;  // malformed
    const int64_t n_hist = uni(0, 200000);
    const int32_t max_out = (int32_t)uni(0, 64);
    std::vector<nkv_segment> out(max_out + 1);
    int32_t n = -7;
    const nkv_status st = nkv_route_segments(&p, n_hist, out.data(), max_out, &n);
    if (st == NKV_OK) {
      CHECK(n >= 0 && n <= max_out, "route: %d segments for max %d", n, max_out);
      int64_t pos = 0;
      const int64_t nf = p.frame_tokens > 0 ? (n_hist + p.frame_tokens - 1) / p.frame_tokens : 0;
      for (int i = 0; i < n; ++i) {
        CHECK(out[i].begin == pos && out[i].end > out[i].begin, "route: segment %d not contiguous",
              i);
        if (i > 0) CHECK(out[i].mode != out[i - 1].mode, "route: adjacent equal modes");
        const int64_t f0 = out[i].begin / p.frame_tokens, f1 = (out[i].end - 1) / p.frame_tokens;
        CHECK(mode_of(p, f0, nf) == out[i].mode && mode_of(p, f1, nf) == out[i].mode,
              "route: mode of frames %lld..%lld", (long long)f0, (long long)f1);
        pos = out[i].end;
      }
      CHECK(pos == n_hist, "route: covers %lld of %lld", (long long)pos, (long long)n_hist);
    }
    nkv_shape s = random_shape();
    nkv_storage acc{};
    (void)nkv_storage_account(&s, (int32_t)uni(0, 300), (int32_t)uni(0, 300), uni(-1, 100000), &acc);
    // layer calls
    nkv_cache_branch cb{(int32_t*)FAKE, (uint8_t*)FAKE, (uint16_t*)FAKE, FAKE, FAKE, FAKE,
                        (int32_t)uni(1, 300)};
    nkv_layer_cache lc{cb, cb, uni(0, 5000), 0};
    lc.capacity = lc.n_hist + uni(-10, 5000);
    std::vector<int32_t> w(s.H > 0 ? s.H : 1);
    for (auto& x : w) x = (int32_t)uni(1, std::max(1, s.r));
    const int64_t Nq = uni(0, 100), N_cur = uni(0, 100);
    const void* cur = N_cur ? FAKE : nullptr;
    const size_t need = nkv_layer_attend_workspace_size(&s, &lc, &p, w.data(), Nq, N_cur);
    nkv_status s2 = nkv_layer_attend(&s, &lc, &p, w.data(), FAKE, Nq, cur, cur, N_cur, FAKE,
                                     (float*)FAKE, FAKE, need == SIZE_MAX ? 0 : need, nullptr);
    if (need != SIZE_MAX) CHECK(s2 != NKV_EWORKSPACE, "layer attend: workspace %zu refused", need);
    const int64_t Nn = uni(0, 3000);
    const size_t need_a = nkv_layer_append_workspace_size(&s, &lc, Nn);
    const int64_t before = lc.n_hist;
    s2 = nkv_layer_append(&s, &lc, FAKE, FAKE, Nn, FAKE, need_a == SIZE_MAX ? 0 : need_a, nullptr);
    if (s2 != NKV_OK) CHECK(lc.n_hist == before, "layer append: n_hist moved on failure");
  }
}

int main() {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0) {
    fprintf(stderr, "a GPU is visible: this fuzz launches with fake pointers; skipped\n");
    return 77;
  }
  nkv_profile_enable(1);  // scopes then try (and fail) to create events
  fuzz_attend(1500);
  fuzz_encode_fit_merge(1500);
  fuzz_rollout(3000);
  nkv_prof_entry pe[8];
  (void)nkv_profile_read(pe, 8);
  nkv_profile_enable(0);
  CHECK(strcmp(nkv_status_string(NKV_EWORKSPACE), "workspace too small") == 0, "status string");
  printf("abi_fuzz: %d failed checks\n", g_fail);
  return g_fail ? 1 : 0;
}
