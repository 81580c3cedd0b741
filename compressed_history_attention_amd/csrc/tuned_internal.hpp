// Internal interfaces between the tuned (MFMA) kernels of libnanokv.
#pragma once

#include "gemm.hpp"
#include "tuned.hpp"

namespace nkv {

constexpr int FA_KT = 64;     // keys per flash-attention tile (key padding unit)

nkv_status launch_decode_tuned(const BranchArgs& b, int W, int r, int group,
                               const RangeTable& rows, uint16_t* out, int64_t ld, bool transposed,
                               hipStream_t st);
// K rows and transposed V of the same routed rows in one launch (falls back
// to one launch_decode_tuned per branch where its kernel does not apply).
// Writes whole groups of 32: K rows and V^T columns [total, round_up(total,
// 32)) receive copies of the last row; the caller's buffers must hold them
// (the attention workspace pads keys to 64 and stages the current chunk over
// them afterwards).
nkv_status launch_decode_pair_tuned(const BranchArgs& kb, const BranchArgs& vb, int W, int r,
                                    int group, const RangeTable& rows, uint16_t* kout,
                                    uint16_t* vt, int64_t ld, hipStream_t st);
nkv_status launch_stage_current(const uint16_t* ck, const uint16_t* cv, int64_t n_cur,
                                int64_t n_pad_tail, int W, uint16_t* kall, uint16_t* vt,
                                int64_t ld, int64_t key0, hipStream_t st);
// Key-range splits for a flash launch (fill the last round of blocks).
int flash_splits(int64_t Nq, int H, int64_t Nk);
// out_f32: write fp32 O [Nq, W] (for merging) instead of bf16.  With
// nsplit > 1, split z writes its partial (normalised O, LSE) at slices
// out + z Nq W and lse + z Nq H (fp32 output only).
nkv_status launch_flash(const uint16_t* q, int64_t Nq, int H, float tau, const uint16_t* kall,
                        const uint16_t* vt, int64_t Nk, int64_t ld, bool out_f32, void* out,
                        float* lse, int nsplit, hipStream_t st);

}  // namespace nkv
