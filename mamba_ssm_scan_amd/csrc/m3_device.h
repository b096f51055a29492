// m3_device.h -- small device helpers shared by the HIP kernels of libm3.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace m3 {

// bf16 is carried as its raw 16 bits.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// A NULL lambda array means lambda = 1 for every token (the Euler / Mamba-2
// special case of the trapezoidal rule: no previous-input term); a NULL omega
// array means omega = 0 (real-valued state, no rotation).
__device__ __forceinline__ float lam_at(const float* lam, int64_t i) { return lam ? lam[i] : 1.f; }
__device__ __forceinline__ float om_at(const float* om, int64_t i) { return om ? om[i] : 0.f; }

// fp32 -> bf16, round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}

template <typename T>
struct Io;

template <>
struct Io<float> {
    __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
    __device__ __forceinline__ static void store(float* p, int64_t i, float v) { p[i] = v; }
};

template <>
struct Io<bf16_t> {
    __device__ __forceinline__ static float load(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i].bits); }
    __device__ __forceinline__ static void store(bf16_t* p, int64_t i, float v) { p[i].bits = f32_to_bf16(v); }
};

}  // namespace m3
