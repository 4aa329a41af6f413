// kda_noalloc.hip -- the library's own prefill scratch, for callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).
//
// The prefill keeps its state-independent chunk operands in a scratch buffer
// between its launches.  kda_chunk_fwd takes that buffer from the caller;
// kda_chunk_fwd_noalloc takes it from the file-scope device array below, of a
// fixed size, which every GPU the library runs on holds until the process ends.
// The array's name is a host-side stand-in in host code: kernels are given the
// device address that hipGetSymbolAddress returns for it, looked up once per
// device with that device current.
#include <mutex>

#include "kda_common.h"

namespace kda {

namespace {

static __device__ __align__(256) uint8_t scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch`, per device

}  // namespace

// Device address of this device's scratch array (looked up on its first use).
kda_status_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "kda_chunk_fwd_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("kda_chunk_fwd_noalloc: device %d is beyond the %d devices the scratch table holds",
              dev, kMaxDevices);
    return KDA_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "kda_chunk_fwd_noalloc: hipGetSymbolAddress(scratch)");
    if (!p) {
      set_error("kda_chunk_fwd_noalloc: hipGetSymbolAddress(scratch) returned NULL");
      return KDA_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KDA_OK;
}

}  // namespace kda
