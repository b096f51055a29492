// m3_gate.hip -- the output gate of the mixer block: y <- y * silu(z), elementwise
// over bf16 arrays of the same layout, in place on y (fp32 arithmetic, the
// result rounded to bf16, nearest even). silu(v) = v * sigmoid(v); the Mamba-2
// block the pages build on gates its SSM output this way.
#include "m3_device.h"
#include "m3_internal.h"

namespace m3 {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float silu(float v) { return v / (1.f + __expf(-v)); }

__device__ __forceinline__ unsigned gate2(unsigned y2, unsigned z2) {
    const float y0 = __uint_as_float(y2 << 16), y1 = __uint_as_float(y2 & 0xffff0000u);
    const float z0 = __uint_as_float(z2 << 16), z1 = __uint_as_float(z2 & 0xffff0000u);
    return unsigned(f32_to_bf16(y0 * silu(z0))) | (unsigned(f32_to_bf16(y1 * silu(z1))) << 16);
}

// 8 bf16 per thread and step (one 16-byte load of each operand)
__global__ void __launch_bounds__(256) gate_kernel(uint16_t* __restrict__ y, const uint16_t* __restrict__ z, int64_t n) {
    const int64_t n8 = n / 8;
    for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n8; i += int64_t(gridDim.x) * blockDim.x) {
        const u32x4 yv = reinterpret_cast<const u32x4*>(y)[i], zv = reinterpret_cast<const u32x4*>(z)[i];
        reinterpret_cast<u32x4*>(y)[i] = u32x4{gate2(yv[0], zv[0]), gate2(yv[1], zv[1]), gate2(yv[2], zv[2]),
                                               gate2(yv[3], zv[3])};
    }
    // the tail past the last multiple of 8
    const int64_t t = 8 * n8 + blockIdx.x * int64_t(blockDim.x) + threadIdx.x;
    if (t < n) {
        const float yv = bf16_to_f32(y[t]), zv = bf16_to_f32(z[t]);
        y[t] = f32_to_bf16(yv * silu(zv));
    }
}

}  // namespace

hipError_t launch_gate(void* y, const void* z, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n / 8 + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(gate_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, static_cast<uint16_t*>(y),
                       static_cast<const uint16_t*>(z), n);
    return hipGetLastError();
}

}  // namespace m3
