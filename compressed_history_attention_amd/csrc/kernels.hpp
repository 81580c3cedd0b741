// Internal launcher declarations of libnanokv.
#pragma once

#include "nkv_common.hpp"

namespace nkv {

// Device view of one compressed branch (mirrors nkv_branch).
struct BranchArgs {
  const int32_t* idx;
  const uint8_t* codes;
  const uint16_t* scales;
  const void* centers;
  const void* decoder;
  int32_t A;
};

// Query-reduction and output-restoration maps of the low-dimensional read:
// head h reduces with rows h*d..h*d+d-1, columns 0..r_low-1 of qmap [W, ld]
// and restores with the same block of omap [W, ld].  The analytical maps are
// the decoders themselves (qmap = D_K, omap = D_V, ld = r).
struct LowMaps {
  const void* qmap;
  const void* omap;
  int32_t ld;
};

// generic kernels (generic.hip)
nkv_status launch_encode_generic(int dt, const void* x, int64_t N, int W, const void* centers,
                                 int A, const void* enc, int r, int group, int32_t* idx,
                                 uint8_t* codes, uint16_t* scales, hipStream_t s);
nkv_status launch_assign_generic(int dt, const void* x, int64_t N, int W, const void* centers,
                                 int A, int32_t* idx, hipStream_t s);
nkv_status launch_decode_generic(int dt, const BranchArgs& b, int W, int r, int group,
                                 const RangeTable& rows, float* out, hipStream_t s);
nkv_status launch_rows_to_f32(int dt, const void* src, int64_t n, float* dst, hipStream_t s);
nkv_status launch_attention_generic(int dt, bool out_f32, const void* q, int64_t Nq, int H,
                                    int d, float tau, const float* K, const float* V,
                                    int64_t Nk, void* out, float* lse, hipStream_t s);
size_t low_generic_lds_bytes(int A_k, int A_v, int r_low, int d);
nkv_status launch_low_generic(int dt, const void* q, int64_t Nq, int H, int d, int r, int group,
                              int r_low, float tau, const BranchArgs& kb, const BranchArgs& vb,
                              const LowMaps& mp, const RangeTable& low, const int32_t* rows,
                              const int32_t* nrows, int64_t max_rows, float* o_low,
                              float* lse_low, hipStream_t s);

// rows (query * H + head) of the heads in hs and their count, for a
// per-head generic low-dimensional read
nkv_status launch_head_rows(int64_t Nq, int H, const HeadSet& hs, int32_t* rows, int32_t* nrows,
                            hipStream_t s);

// center fitting (fit.hip): rows sorted by center (counts, offsets, cursor,
// perm), then per center the fp64 mean of its rows stored in the codec dtype
// (empty centers kept)
nkv_status launch_fit_update(int dt, const void* x, int64_t N, int W, const int32_t* idx, int A,
                             int32_t* counts, int32_t* offs, int32_t* cursor, int32_t* perm,
                             void* centers, hipStream_t s);
nkv_status launch_fit_counts(const int32_t* idx, int64_t N, int A, int32_t* counts,
                             hipStream_t s);

// LSE merge (merge.hip): n parts at slices of (o_parts, lse_parts) with
// strides Nq W / Nq H, plus an optional extra part (o_x, lse_x)
nkv_status launch_lse_merge_parts(int64_t Nq, int H, int d, int n, const float* o_parts,
                                  const float* lse_parts, const float* o_x, const float* lse_x,
                                  void* out, int out_dt, float* lse_out, hipStream_t s);
// LSE merge (merge.hip)
nkv_status launch_lse_merge(int64_t Nq, int H, int d, const float* o_a, const float* lse_a,
                            const float* o_b, const float* lse_b, void* out, int out_dt,
                            float* lse_out, hipStream_t s);

}  // namespace nkv
