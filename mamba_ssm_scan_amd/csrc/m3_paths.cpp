// m3_paths.cpp -- which kernel family takes a problem, the chunk it walks and
// the workspace of the backward pass: host logic only, read by the planner
// (m3_host.cpp); the kernels that implement each family are in the .hip files.
#include "m3_internal.h"

namespace m3 {

bool mfma_path_supported(int32_t P_, int32_t N_, int32_t R, int32_t chunk, m3_dtype io) {
    // R 5 to 8 at the workloads' state (N 128, P 64): the R 8 wave-specialised kernel (zero ranks below 8)
    if (io == M3_BF16 && R >= 5 && R <= 8 && N_ == kMfmaN && P_ == kMfmaP && chunk >= 1) return true;
    return io == M3_BF16 && N_ >= 8 && N_ <= kMfmaMaxN && N_ % 8 == 0 && P_ >= 8 && P_ <= kMfmaMaxP &&
           P_ % 8 == 0 && R >= 1 && R <= 4 && chunk >= 1 && chunk <= 64;
}

// The chunk the MFMA kernels walk: the one asked for, except at R 5 to 8 (the
// R 8 kernel), whose chunks hold at most 32 tokens (256 (token, rank) rows). The
// chunk size only tiles the work: the recurrence's result does not depend on it.
int32_t mfma_kernel_chunk(int32_t R, int32_t chunk) { return R > 4 && chunk > 32 ? 32 : chunk; }

bool mfma_segments_supported(int32_t R, int32_t N_, int32_t P_) {
    return R != 1 && R <= 4 && N_ <= kMfmaN && P_ <= kMfmaP;
}

// the token walk: R 5 to 8 (the planner asks the chunked path first, which takes
// these ranks at N 128, P 64)
bool scan_path_supported(int32_t P, int32_t N, int32_t R, m3_dtype io) {
    return io == M3_BF16 && N % 16 == 0 && N <= 256 && P % 16 == 0 && P <= 64 && R >= 5 && R <= 8;
}

// one stored state per block of kBackwardCheckpoint tokens, plus the block's
// recomputed states (a per-(b, h) scratch)
size_t backward_workspace_bytes(int64_t b, int32_t H, int64_t L) {
    const int64_t nblk = (L + kBackwardCheckpoint - 1) / kBackwardCheckpoint;
    return size_t(b) * size_t(H) * size_t(nblk + kBackwardCheckpoint) * kBackwardStateFloats * sizeof(float);
}

bool backward_supported(int32_t P, int32_t N, int32_t R) { return N <= 128 && P <= 64 && R <= 4; }

}  // namespace m3
