// m3_noalloc.hip -- the fixed device array behind m3_prefill_noalloc (the entry
// point is in m3_host.cpp): m3_prefill with the workspace taken from it instead
// of a caller buffer, for callers that cannot allocate device memory (code
// under stream capture, tight serving loops).
//
// The array is a file-scope __device__ variable: every GPU the library runs on
// holds its own copy (at its own address) until the process ends. In host code
// the variable's name is only a host-side stand-in, so its device address is
// looked up once per device (hipGetSymbolAddress, with that device current) and
// kept; only that address is ever handed to kernels.
#include <mutex>

#include "m3_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(M3_NOALLOC_SCRATCH_BYTES);
static_assert(kScratchBytes % 256 == 0, "scratch size");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

// device address of this device's copy of the scratch array (looked up once)
m3_status m3::noalloc_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return m3::set_error(M3_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return m3::set_error(M3_EUNSUPPORTED, "device index %d above %d", dev, kMaxDevices - 1);
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return m3::set_error(M3_EHIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                                 hipGetErrorString(e));
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return M3_OK;
}
