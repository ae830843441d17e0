// The fixed device array behind mla_kv_append_noalloc, for callers that cannot allocate:
// the fp32 partial sums of the new tokens' down-projection go here instead of to a caller's
// workspace.  Each GPU the library runs on holds its own copy of the array (at its own
// address) until the process ends.
//
// On the host, `scratch` names a host-side stand-in, not device memory: its device address
// is looked up once per device with hipGetSymbolAddress, with that device current, and only
// that address is ever handed to a kernel.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/mla_kv.h"

static __device__ __align__(256) unsigned char scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace mla {
namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_addr[kMaxDevices];
hipError_t g_lookup[kMaxDevices];

}  // namespace

// The array's device address on the current device, which must also be the device of
// `stream`.  The first call on a device looks the address up; later calls reuse it.
mla_status_t noalloc_scratch(hipStream_t stream, void** addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_LAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_DEVICE;
  hipDevice_t stream_dev = -1;
  if (hipStreamGetDevice(stream, &stream_dev) != hipSuccess) return MLA_ERR_LAUNCH;
  if (stream_dev != dev) return MLA_ERR_DEVICE;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_lookup[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_addr[dev] = p;
  });
  if (g_lookup[dev] != hipSuccess || g_addr[dev] == nullptr) return MLA_ERR_LAUNCH;
  *addr = g_addr[dev];
  return MLA_OK;
}

}  // namespace mla
