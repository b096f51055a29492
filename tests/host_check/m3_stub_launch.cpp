// m3_stub_launch.cpp -- the device side of libm3 replaced by stubs, for the
// host-only sanitizer build of the entry points (m3_host.cpp, m3_mixer.cpp,
// m3_paths.cpp). The argument checks these tests exercise all return before
// any launch, so reaching a stub is itself a failure: it reports and aborts.
#include <cstdio>
#include <cstdlib>

#include "m3_internal.h"

namespace m3 {
namespace {
[[noreturn]] void launched(const char* what) {
    std::fprintf(stderr, "host-only check build: %s reached a device launch\n", what);
    std::abort();
}
}  // namespace

hipError_t launch_prefill_mfma(const PrefillArgs&) { launched("launch_prefill_mfma"); }
hipError_t launch_prefill_scan(const PrefillArgs&) { launched("launch_prefill_scan"); }
hipError_t launch_prefill_generic(const PrefillArgs&) { launched("launch_prefill_generic"); }
hipError_t launch_decode(const DecodeArgs&) { launched("launch_decode"); }
hipError_t launch_backward(const BackwardArgs&) { launched("launch_backward"); }
hipError_t launch_prologue(const PrologueArgs&) { launched("launch_prologue"); }
hipError_t launch_carry_init(void*, const void*, int64_t, int, int, int64_t, hipStream_t) {
    launched("launch_carry_init");
}
hipError_t launch_copy_or_zero(uint32_t*, const uint32_t*, int64_t, hipStream_t) { launched("launch_copy_or_zero"); }
hipError_t launch_gate(void*, const void*, int64_t, hipStream_t) { launched("launch_gate"); }
m3_status noalloc_scratch(void**) { launched("noalloc_scratch"); }

}  // namespace m3
