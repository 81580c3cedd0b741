#include "tuned.hpp"
namespace nkv {
bool tuned_available() { return false; }
size_t tuned_encode_workspace(const nkv_shape*, int64_t, int32_t) { return 0; }
nkv_status tuned_encode(const nkv_shape*, const void*, int64_t, const void*, int32_t, const void*,
                        int32_t*, uint8_t*, uint16_t*, char*, size_t, hipStream_t) {
  set_error("tuned path not built");
  return NKV_EUNSUPPORTED;
}
size_t tuned_attend_workspace(const nkv_shape*, int32_t, int32_t, const RangeTable&,
                              const RangeTable&, int32_t, int64_t, int64_t) { return 0; }
nkv_status tuned_attend(const nkv_shape*, const BranchArgs&, const BranchArgs&, const RangeTable&,
                        const RangeTable&, int32_t, float, const void*, int64_t, const void*,
                        const void*, int64_t, void*, float*, char*, size_t, hipStream_t) {
  set_error("tuned path not built");
  return NKV_EUNSUPPORTED;
}
}  // namespace nkv
