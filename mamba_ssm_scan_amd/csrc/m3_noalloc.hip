// m3_noalloc.hip -- m3_prefill_noalloc: m3_prefill with the workspace taken from
// a fixed device array instead of a caller buffer, for callers that cannot
// allocate device memory (code under stream capture, tight serving loops).
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

extern "C" size_t m3_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" m3_status m3_prefill_noalloc(const void* x, const float* dt, const float* A, const float* omega,
                                        const float* lambda, const void* B, const void* C, const float* D,
                                        int32_t R, int32_t chunk, const float* h0, void* y, float* h_out,
                                        const m3_dims* dims, m3_dtype io_dtype, const void* carry_B,
                                        const void* carry_x, void* stream) {
    m3_plan plan;
    m3_status s = m3_prefill_plan(dims, R, chunk, io_dtype, &plan);
    if (s != M3_OK) return s;
    if (plan.workspace_bytes > kScratchBytes)
        return m3::set_error(M3_EWORKSPACE,
                             "these sizes need %zu bytes of scratch, above the fixed %zu bytes of m3_prefill_noalloc",
                             plan.workspace_bytes, kScratchBytes);
    void* ws = nullptr;
    if (plan.workspace_bytes > 0 && dims->batch > 0 && dims->seqlen > 0) {
        if ((s = m3::noalloc_scratch(&ws)) != M3_OK) return s;
    }
    return m3_prefill(x, dt, A, omega, lambda, B, C, D, R, chunk, h0, y, h_out, dims, io_dtype, carry_B, carry_x,
                      ws, ws ? kScratchBytes : 0, stream);
}
