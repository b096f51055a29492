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

// The input prologue's scalar maps (m3_prologue's reading): softplus for the
// step and sigmoid for the trapezoid weight, through the hardware exp2 / log2 /
// rcp (a few ulp). softplus(x) = max(x, 0) + ln(1 + e^-|x|); below e^-|x| =
// 2^-24 the log term is taken as e^-|x| itself, where 1 + e^-|x| would round to 1.
__device__ __forceinline__ float softplus_f(float x) {
    constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;
    const float e = __builtin_amdgcn_exp2f(-fabsf(x) * kLog2e);
    const float l = e < 5.9604645e-8f ? e : __builtin_amdgcn_logf(1.f + e) * kLn2;
    return fmaxf(x, 0.f) + l;
}
__device__ __forceinline__ float sigmoid_f(float x) {
    constexpr float kLog2e = 1.4426950408889634f;
    const float e = __builtin_amdgcn_exp2f(-fabsf(x) * kLog2e);  // e^-|x| in (0, 1]
    const float r = __builtin_amdgcn_rcpf(1.f + e);
    return x >= 0.f ? r : e * r;
}

// The step inputs as a prefill kernel reads them: dt and lambda as given
// (raw = 0), or from their raw projections (raw = 1): dt = softplus(dt_raw +
// the head's bias), lambda = sigmoid(lambda_raw), applied where the kernel
// loads them. A NULL lambda array is lambda = 1 either way.
struct StepIn {
    float bias;  // the head's dt bias (raw only)
    int raw;
    __device__ __forceinline__ float dt(float v) const { return raw ? softplus_f(v + bias) : v; }
    __device__ __forceinline__ float lamv(float v) const { return raw ? sigmoid_f(v) : v; }
    __device__ __forceinline__ float lam(const float* l, int64_t i) const { return l ? lamv(l[i]) : 1.f; }
};
__device__ __forceinline__ StepIn step_in(const float* dt_bias, int raw, int h) {
    return StepIn{raw && dt_bias ? dt_bias[h] : 0.f, raw};
}

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
