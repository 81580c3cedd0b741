// Low-dimensional read dispatch (interim: generic kernel).
#include "lowdim.hpp"

namespace nkv {

size_t low_workspace_bytes(const nkv_shape*, int32_t, int32_t, const RangeTable&, int32_t, int64_t) {
  return 0;
}

nkv_status launch_low(const nkv_shape* s, const BranchArgs& kb, const BranchArgs& vb,
                      const RangeTable& low, int32_t r_low, float tau, const uint16_t* q,
                      int64_t Nq, float* o_low, float* lse_low, char*, hipStream_t st) {
  return launch_low_generic(s->dtype, q, Nq, s->H, s->d, s->r, s->group, r_low, tau, kb, vb, low,
                            nullptr, nullptr, Nq * s->H, o_low, lse_low, st);
}

}  // namespace nkv
