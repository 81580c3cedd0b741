// NanoKV-Fast low-dimensional read on the tuned path.
#pragma once

#include "tuned_internal.hpp"

namespace nkv {

// Key-range splits of one head group's main pass (more blocks when the group
// alone would leave CUs idle), and the partial-sum rows per query that the
// widest demand over the head groups of a call needs (groups as in
// tuned_attend: heads of equal width).
struct LowSplit {
  int S;    // splits of the tile sequence (grid z)
  bool gv;  // at a^V-range boundaries: each split owns its center-mass ranges
};
LowSplit low_split_plan(int64_t Nq, int n_heads, int64_t n_low, int A_v);
int64_t low_part_units(int64_t Nq, int H, int32_t r_low, const int32_t* r_low_h, int64_t n_low,
                       int A_v);
size_t low_workspace_bytes(const nkv_shape* s, int32_t A_k, int32_t A_v, const RangeTable& low,
                           int32_t r_low, const int32_t* r_low_h, int64_t Nq);
// Writes the columns of O_low fp32 [Nq, W] and LSE_low [Nq, H] of the heads
// in `hs` for the low-routed tokens, all read at width r_low; the workspace
// is laid out for the widest group, r_low_max.  `first` runs
// the width-independent preparation (bucket sort, transposed V centers);
// further calls on the same workspace for other head groups reuse it.
// `mp` holds the query-reduction and restoration maps (bf16, ld % 8 == 0).
nkv_status launch_low(const nkv_shape* s, const BranchArgs& kb, const BranchArgs& vb,
                      const LowMaps& mp, const RangeTable& low, int32_t r_low, float tau,
                      const uint16_t* q,
                      int64_t Nq, float* o_low, float* lse_low, char* ws, int32_t r_low_max,
                      int64_t part_units, const HeadSet& hs, bool first, hipStream_t st);

}  // namespace nkv
