// Orchestration of the tuned (MFMA) attention path: workspace layout and the
// sequence of kernels for the full-dimensional and the Fast reads.
#include "lowdim.hpp"
#include "prof.hpp"
#include "tuned_internal.hpp"

namespace nkv {

namespace {

struct Layout {
  int64_t nk = 0, nk_pad = 0;
  int fsplit = 1;  // key-range splits of the flash launch
  size_t kall = 0, vt = 0, o_full = 0, lse_full = 0, o_low = 0, lse_low = 0, low = 0;
  size_t total = 0;
};

Layout make_layout(const nkv_shape* s, int32_t A_k, int32_t A_v, const RangeTable& full,
                   const RangeTable& low, int32_t r_low, const int32_t* r_low_h, int64_t Nq,
                   int64_t N_cur) {
  Layout L;
  const int64_t W = (int64_t)s->H * s->d;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  L.nk = full.total + N_cur;
  L.nk_pad = ceil_div(L.nk, FA_KT) * FA_KT;
  L.kall = take(sizeof(uint16_t) * L.nk_pad * W);
  L.vt = take(sizeof(uint16_t) * L.nk_pad * W);
  L.fsplit = flash_splits(Nq, s->H, L.nk);
  if (low.total == 0 && L.fsplit > 1) {
    L.o_full = take(sizeof(float) * Nq * W * L.fsplit);
    L.lse_full = take(sizeof(float) * Nq * s->H * L.fsplit);
  }
  if (low.total > 0) {
    L.o_full = take(sizeof(float) * Nq * W * L.fsplit);
    L.lse_full = take(sizeof(float) * Nq * s->H * L.fsplit);
    L.o_low = take(sizeof(float) * Nq * W);
    L.lse_low = take(sizeof(float) * Nq * s->H);
    L.low = take(low_workspace_bytes(s, A_k, A_v, low, r_low, r_low_h, Nq));
  }
  L.total = off;
  return L;
}

}  // namespace

size_t tuned_attend_workspace(const nkv_shape* s, int32_t A_k, int32_t A_v, const RangeTable& full,
                              const RangeTable& low, int32_t r_low, const int32_t* r_low_h,
                              int64_t Nq, int64_t N_cur) {
  return make_layout(s, A_k, A_v, full, low, r_low, r_low_h, Nq, N_cur).total;
}

nkv_status tuned_attend(const nkv_shape* s, const BranchArgs& kb, const BranchArgs& vb,
                        const LowMaps& mp, const RangeTable& full, const RangeTable& low, int32_t r_low,
                        const int32_t* r_low_h, float tau, const void* q, int64_t Nq,
                        const void* cur_k, const void* cur_v, int64_t N_cur, void* out,
                        float* lse, char* ws, size_t ws_bytes, hipStream_t st) {
  const Layout L = make_layout(s, kb.A, vb.A, full, low, r_low, r_low_h, Nq, N_cur);
  if (L.total > ws_bytes) {  // the size query and this layout must agree
    set_error("internal: tuned layout of %zu bytes exceeds the %zu given", L.total, ws_bytes);
    return NKV_EWORKSPACE;
  }
  const int H = s->H, W = H * s->d;
  uint16_t* kall = reinterpret_cast<uint16_t*>(ws + L.kall);
  uint16_t* vt = reinterpret_cast<uint16_t*>(ws + L.vt);
  const uint16_t* qb = static_cast<const uint16_t*>(q);
  float* of = reinterpret_cast<float*>(ws + L.o_full);
  float* lf = reinterpret_cast<float*>(ws + L.lse_full);
  // decoded history + current chunk, then flash attention over them
  auto full_part = [&](bool to_out, hipStream_t fs) -> nkv_status {
    nkv_status e;
    {
      ProfScope ps("decode", fs);
      if ((e = launch_decode_pair_tuned(kb, vb, W, s->r, s->group, full, kall, vt, L.nk_pad, fs)))
        return e;
    }
    {
      ProfScope ps("stage_current", fs);
      if ((e = launch_stage_current(static_cast<const uint16_t*>(cur_k),
                                    static_cast<const uint16_t*>(cur_v), N_cur,
                                    L.nk_pad - full.total, W, kall, vt, L.nk_pad, full.total, fs)))
        return e;
    }
    ProfScope ps("flash", fs);
    if (to_out) return launch_flash(qb, Nq, H, tau, kall, vt, L.nk, L.nk_pad, false, out, lse, 1, fs);
    return launch_flash(qb, Nq, H, tau, kall, vt, L.nk, L.nk_pad, true, of, lf, L.fsplit, fs);
  };
  nkv_status e;
  if (low.total == 0) {
    if (L.fsplit == 1) return full_part(true, st);
    if ((e = full_part(false, st))) return e;
    ProfScope ps("merge", st);
    return launch_lse_merge_parts(Nq, H, s->d, L.fsplit, of, lf, nullptr, nullptr, out, NKV_BF16,
                                  lse, st);
  }
  float* ol = reinterpret_cast<float*>(ws + L.o_low);
  float* ll = reinterpret_cast<float*>(ws + L.lse_low);
  // heads grouped by width (one group when every head shares r_low), in the
  // order their widths first appear; r_low is the widest
  int widths[NKV_MAX_HEADS];
  HeadSet groups[NKV_MAX_HEADS];
  int ng = 0;
  for (int h = 0; h < H; ++h) {
    const int w = r_low_h ? r_low_h[h] : r_low;
    int g = 0;
    while (g < ng && widths[g] != w) ++g;
    if (g == ng) {
      widths[ng] = w;
      groups[ng].n = 0;
      ++ng;
    }
    groups[g].h[groups[g].n++] = h;
  }
  const int64_t units = low_part_units(Nq, H, r_low, r_low_h, low.total, vb.A);
  auto low_part = [&]() -> nkv_status {
    nkv_status e2;
    for (int g = 0; g < ng; ++g)
      if ((e2 = launch_low(s, kb, vb, mp, low, widths[g], tau, qb, Nq, ol, ll, ws + L.low, r_low,
                           units, groups[g], g == 0, st)))
        return e2;
    return NKV_OK;
  };
  // everything on the caller's stream: the library creates no streams or
  // events of its own
  if ((e = full_part(false, st)) || (e = low_part())) return e;
  ProfScope ps("merge", st);
  return launch_lse_merge_parts(Nq, H, s->d, L.fsplit, of, lf, ol, ll, out, NKV_BF16, lse, st);
}

}  // namespace nkv
