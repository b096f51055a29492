// m3_internal.h -- what the host entry points (m3_host.cpp) hand to the kernel
// launchers (*.hip). Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/m3.h"

namespace m3 {

struct PrefillArgs {
    const void* x;
    const float* dt;
    const float* A;
    const float* omega;
    const float* lam;
    const void* B;
    const void* C;
    const float* D;
    const float* h0;       // nullable
    void* y;
    float* h_out;          // nullable
    const void* carry_B;   // nullable (both or neither)
    const void* carry_x;
    int64_t b, L;
    int32_t H, G, P, N, R, chunk;
    m3_dtype io;
    m3_plan plan;
    void* workspace;
    hipStream_t stream;
    // m3_prefill_fused: dt and lambda are raw projections (softplus with the
    // head's bias dt_bias[H] (NULL: 0), sigmoid), applied where the kernels load them
    const float* dt_bias;
    int raw_steps;
};

// The input prologue fused into a decode step (m3_decode_step_fused): the step
// reads raw B_t, C_t, dt_t, lambda_t and applies m3_prologue's reading itself.
struct DecodePrologue {
    const float* B_weight;  // [G][R][N] or NULL (1)
    const float* B_bias;    // [G][R][N] or NULL (0)
    const float* C_weight;
    const float* C_bias;
    const float* dt_bias;   // [H] or NULL (0)
    float eps;
};

struct DecodeArgs {
    float* h;
    void* carry_B;         // two slots [2][b][G][R][N] of the previous token's B rows, then parity words [b][H]
    void* carry_x;         // [b][H][R][P]
    const void* x;
    const float* dt;
    const float* A;
    const float* omega;
    const float* lam;
    const void* B;
    const void* C;
    const float* D;
    void* y;
    int64_t b;
    int32_t H, G, P, N, R;
    m3_dtype io;
    hipStream_t stream;
    int rev;               // walk the (b, h) workgroups backwards (a block-order hint: every other step)
    const DecodePrologue* pro;  // NULL: B, C, dt, lambda are the recurrence's inputs as given
};

// rows of R * N of the fused decode step's generic kernel held in LDS (B and C, fp32)
constexpr int64_t kDecodeFusedGenericRN = 8192;

// Bytes of the two B slots at the start of a decode carry_B buffer (16-byte
// aligned end; the per-head parity words follow).
inline size_t decode_carry_B_slots_bytes(int64_t b, int64_t G, int64_t R, int64_t N, size_t es) {
    return (size_t(2 * b * G * R * N) * es + 15) / 16 * 16;
}

struct PrologueArgs {
    const void* B_raw;     // [ntok][G][R][N] io dtype (with B, or both NULL)
    const void* C_raw;
    const float* B_weight; // [G][R][N] or NULL (1)
    const float* B_bias;   // [G][R][N] or NULL (0)
    const float* C_weight;
    const float* C_bias;
    float eps;
    const float* dt_raw;   // [ntok][H] (with dt, or both NULL)
    const float* dt_bias;  // [H] or NULL
    const float* lambda_raw;
    void* B;
    void* C;
    float* dt;
    float* lambda;
    int64_t ntok;
    int32_t H, GR, N;      // GR = G * R rows per token
    m3_dtype io;
    hipStream_t stream;
};

struct BackwardArgs {
    // the forward's inputs
    const void* x;
    const float* dt;
    const float* A;
    const float* omega;    // nullable (omega = 0)
    const float* lam;      // nullable (lambda = 1)
    const void* B;
    const void* C;
    const float* D;
    const float* h0;       // nullable
    const void* carry_B;   // nullable (both or neither)
    const void* carry_x;
    // incoming gradients
    const void* dy;        // [b][L][H][R][P] io dtype
    const float* dh_out;   // [b][H][N][P] or NULL
    // gradients (fp32); the accumulated ones are cleared by the launcher
    float* dx;             // [b][L][H][R][P]
    float* dB;             // [b][L][G][R][N] (summed over the heads of a group)
    float* dC;
    float* ddt;            // [b][L][H]
    float* dlam;           // [b][L][H] or NULL
    float* dA;             // [H] (summed over batch and tokens)
    float* domega;         // [H][N/2] or NULL
    float* dD;             // [H]
    float* dh0;            // [b][H][N][P] or NULL
    float* dcarry_B;       // [b][G][R][N] or NULL (with the carry)
    float* dcarry_x;       // [b][H][R][P] or NULL
    int64_t b, L;
    int32_t H, G, P, N, R;
    m3_dtype io;
    float* workspace;      // backward_workspace_floats(b, H, L) floats
    hipStream_t stream;
};

// Tokens between the backward's state checkpoints, and its workspace size.
constexpr int kBackwardCheckpoint = 16;
constexpr int kBackwardStateFloats = 128 * 64;  // floats of one stored backward state (N <= 128, P <= 64)
size_t backward_workspace_bytes(int64_t b, int32_t H, int64_t L);
bool backward_supported(int32_t P, int32_t N, int32_t R);

// Layout of the prefill workspace (byte offsets), shared by host and launchers.
struct PrefillWorkspace {
    size_t state_off;      // generic path: running state [b][H][N][P] fp32
    size_t ctrl_off;       // segmented path: ticket counter + flags
    size_t agg_off;        // segmented path: per-segment local end state [b*H*S][N][P] fp32
    size_t incl_off;       // segmented path: per-segment inclusive end state
    size_t tr_off;         // segmented path: per-segment total step (sum of dt) [b*H*S] fp64
    size_t ypart_off;      // chunked path, N above 128: fp32 outputs of the row passes [b][L][H][R][P]
    size_t total;
};

PrefillWorkspace prefill_workspace_layout(int64_t b, int64_t L, int32_t H, int32_t P, int32_t N, int32_t R,
                                          int32_t segments, int32_t path);

bool mfma_path_supported(int32_t P, int32_t N, int32_t R, int32_t chunk, m3_dtype io);
// polls of a look-back wait before it gives up (about a second; a wait normally ends in microseconds)
constexpr long kLookbackSpinLimit = 1L << 24;
// device address of m3_prefill_noalloc's scratch on the current device
m3_status noalloc_scratch(void** ptr);
// the MFMA path splits the sequence into segments (look-back) at these ranks
int32_t mfma_kernel_chunk(int32_t R, int32_t chunk);
bool mfma_segments_supported(int32_t R, int32_t N, int32_t P);
constexpr int32_t kMfmaMaxN = 512;   // largest N of the chunked path (passes of 128 rows)
constexpr int32_t kMfmaMaxP = 1024;  // largest P of the chunked path (passes of 64 columns)
constexpr int32_t kMfmaN = 128;      // state rows of one pass of the chunked kernels
constexpr int32_t kMfmaP = 64;       // state columns of one pass

// the token-walk path (bf16, N, P multiples of 16, N <= 256, P <= 64, R <= 8)
bool scan_path_supported(int32_t P, int32_t N, int32_t R, m3_dtype io);
hipError_t launch_prefill_scan(const PrefillArgs& a);
hipError_t launch_prefill_generic(const PrefillArgs& a);
// the mixer block's output gate: y <- bf16(y * silu(z)) over n bf16 entries, in place
hipError_t launch_gate(void* y, const void* z, int64_t n, hipStream_t s);
// set the thread's error detail (m3_last_error) and return s
m3_status set_error(m3_status s, const char* fmt, ...);
hipError_t launch_prefill_mfma(const PrefillArgs& a);
// the wave-specialised R 4 kernel for N 128, P 64 (m3_prefill_ws4.hip)
bool ws4_supported(const PrefillArgs& a);
hipError_t launch_prefill_ws4(const PrefillArgs& a);
hipError_t launch_decode(const DecodeArgs& a);
// carry[b][h] = src[b][h / (H / G)], rows of row_bytes (a multiple of 4), or zero when src is NULL
hipError_t launch_carry_init(void* carry, const void* src, int64_t b, int H, int G, int64_t row_bytes,
                             hipStream_t s);
hipError_t launch_prologue(const PrologueArgs& a);
hipError_t launch_backward(const BackwardArgs& a);
// dst[i] = src ? src[i] : 0 for n 32-bit words (a kernel, so it is safe under graph capture)
hipError_t launch_copy_or_zero(uint32_t* dst, const uint32_t* src, int64_t n_words, hipStream_t s);

}  // namespace m3
