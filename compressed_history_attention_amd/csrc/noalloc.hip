// Encoder entry point that allocates nothing and takes no workspace: for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// The encoder's scratch (center norms, per-slot nearest-center records,
// projection partial sums) lives in one fixed device
// array of this library, `scratch`, NKV_NOALLOC_SCRATCH_BYTES long.  Every
// GPU the library runs on holds its own copy until the process ends.  Its
// device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and kept; kernels receive that address, as they
// receive the caller's workspace in nkv_encode.  Every call on one GPU
// shares the array: calls that overlap on one GPU (two streams, two host
// threads) race, so callers serialise them.  The kernels clear every counter
// they rely on and overwrite every record before reading it, so nothing of
// an earlier call's contents is ever read.
#include <mutex>

#include "kernels.hpp"

static __device__ __attribute__((aligned(256))) char scratch[NKV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_ptr[MAX_DEVICES] = {};

}  // namespace

extern "C" nkv_status nkv_encode_noalloc(const nkv_shape* shape, const void* x, int64_t N,
                                         const void* centers, int32_t A, const void* encoder,
                                         int32_t* idx, uint8_t* codes, uint16_t* scales,
                                         void* stream) {
  // size check first: a call that cannot fit is refused before any device work
  const size_t need = nkv_encode_workspace_size(shape, N < 0 ? 0 : N, A);
  if (need == SIZE_MAX)
    return nkv_encode(shape, x, N, centers, A, encoder, idx, codes, scales, nullptr, 0, stream);
  if (need > (size_t)NKV_NOALLOC_SCRATCH_BYTES) {
    nkv::set_error("nkv_encode_noalloc: %zu bytes of scratch needed for N=%lld, A=%d, the fixed "
                   "array holds %zu (split the tokens into smaller calls)",
                   need, (long long)N, A, (size_t)NKV_NOALLOC_SCRATCH_BYTES);
    return NKV_EUNSUPPORTED;
  }
  if (N <= 0 || need == 0)
    return nkv_encode(shape, x, N, centers, A, encoder, idx, codes, scales, nullptr, 0, stream);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) {
    nkv::set_error("nkv_encode_noalloc: no current device (or device id above %d)", MAX_DEVICES);
    return NKV_EHIP;
  }
  void* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
      void* p = nullptr;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) {
        nkv::set_error("nkv_encode_noalloc: hipGetSymbolAddress(scratch) failed: %s",
                       hipGetErrorString(e));
        return NKV_EHIP;
      }
      g_ptr[dev] = p;
    }
    ptr = g_ptr[dev];
  }
  return nkv_encode(shape, x, N, centers, A, encoder, idx, codes, scales, ptr,
                    (size_t)NKV_NOALLOC_SCRATCH_BYTES, stream);
}
