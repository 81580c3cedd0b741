// Tuned (MFMA) path of libnanokv: bf16 tensors, head dimension 128.
#pragma once

#include "kernels.hpp"

namespace nkv {

size_t tuned_encode_workspace(const nkv_shape* s, int64_t N, int32_t A);
// nearest center per token only (the encoder's first stage)
size_t tuned_assign_workspace(int64_t N, int32_t A);
// xnorm: NULL, or ||x_t||^2 per token from tuned_row_sqnorm (rows assigned
// more than once)
nkv_status tuned_assign(const nkv_shape* s, const void* x, int64_t N, const void* centers,
                        int32_t A, int32_t* idx, char* ws, hipStream_t st,
                        const float* xnorm = nullptr);
nkv_status tuned_row_sqnorm(const nkv_shape* s, const void* x, int64_t N, float* out,
                            hipStream_t st);
nkv_status tuned_encode(const nkv_shape* s, const void* x, int64_t N, const void* centers,
                        int32_t A, const void* enc, int32_t* idx, uint8_t* codes,
                        uint16_t* scales, char* ws, size_t ws_bytes, hipStream_t st);

size_t tuned_attend_workspace(const nkv_shape* s, int32_t A_k, int32_t A_v, const RangeTable& full,
                              const RangeTable& low, int32_t r_low, const int32_t* r_low_h,
                              int64_t Nq, int64_t N_cur);
// r_low_h: NULL, or one width per head (r_low is then the widest); mp: the
// low-dimensional maps
nkv_status tuned_attend(const nkv_shape* s, const BranchArgs& kb, const BranchArgs& vb,
                        const LowMaps& mp, const RangeTable& full, const RangeTable& low, int32_t r_low,
                        const int32_t* r_low_h, float tau, const void* q, int64_t Nq,
                        const void* cur_k, const void* cur_v, int64_t N_cur, void* out,
                        float* lse, char* ws, size_t ws_bytes, hipStream_t st);

}  // namespace nkv
