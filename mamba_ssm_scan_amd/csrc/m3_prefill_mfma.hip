// m3_prefill_mfma.hip -- bf16 MFMA chunked prefill (placeholder until the kernel lands).
#include "m3_device.h"
#include "m3_internal.h"

namespace m3 {

bool mfma_path_supported(int32_t, int32_t, int32_t, int32_t, m3_dtype) { return false; }

hipError_t launch_prefill_mfma(const PrefillArgs&) { return hipErrorNotSupported; }

}  // namespace m3
