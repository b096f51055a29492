// m3_prologue.hip -- the input prologue in front of the recurrence: a QK-norm
// with an elementwise weight and an additive bias on every (token, group, rank)
// row of B and C, softplus (with a per-head bias) on the step, sigmoid on the
// trapezoid weight ("复值SSM × 广义梯形离散 × MIMO，线性模型的全面重构", §2.4 and
// Fig. 4: QK-norm and learnable bias after the B/C projection).
//
// Memory-bound: every element is read once from HBM and written once. One
// launch covers all parts: blocks [0, nbB) normalise B rows, [nbB, nbB + nbC)
// C rows, the rest the per-(token, head) scalars (4 per thread). A row is
// handled by 16 lanes: each lane keeps 8 consecutive entries per 128 in
// registers, the sum of squares is reduced across the 16 lanes with DPP, and
// the lanes write their entries scaled, weighted and biased. At N <= 128 a
// 16-lane group takes 4 rows (a block 64), all loads issued first.
#include "m3_device.h"
#include "m3_internal.h"

namespace m3 {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Row8;  // 8 consecutive entries, 16-byte aligned

template <>
struct Row8<bf16_t> {
    __device__ __forceinline__ static void load(const bf16_t* p, float* v) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = __uint_as_float(w[j] << 16);
            v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
        }
    }
    __device__ __forceinline__ static void store(bf16_t* p, const float* v) {
        u32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = uint32_t(f32_to_bf16(v[2 * j])) | (uint32_t(f32_to_bf16(v[2 * j + 1])) << 16);
        *reinterpret_cast<u32x4*>(p) = w;
    }
};

template <>
struct Row8<float> {
    __device__ __forceinline__ static void load(const float* p, float* v) {
        const floatx4 a = *reinterpret_cast<const floatx4*>(p), b = *reinterpret_cast<const floatx4*>(p + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[j] = a[j];
            v[4 + j] = b[j];
        }
    }
    __device__ __forceinline__ static void store(float* p, const float* v) {
        *reinterpret_cast<floatx4*>(p) = floatx4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<floatx4*>(p + 4) = floatx4{v[4], v[5], v[6], v[7]};
    }
};

// log(1 + e^x) without overflow: max(x, 0) + log1p(e^-|x|)
__device__ __forceinline__ float softplus(float x) { return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))); }

// 1 / (1 + e^-x), with e^x / (1 + e^x) for x < 0 so e^-x never overflows
__device__ __forceinline__ float sigmoid(float x) {
    if (x >= 0.f) return 1.f / (1.f + expf(-x));
    const float e = expf(x);
    return e / (1.f + e);
}

// 8 consecutive fp32 parameters (weight or bias), 16-byte aligned
__device__ __forceinline__ void load_par8(const float* __restrict__ p, float* v) {
    const floatx4 a = *reinterpret_cast<const floatx4*>(p), b = *reinterpret_cast<const floatx4*>(p + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[j] = a[j];
        v[4 + j] = b[j];
    }
}

// Sum over the 16 lanes of a row, every lane getting the total: DPP swaps
// inside quads, then the mirror inside each 8-lane half and inside the 16-lane
// row (no LDS round trip). A row's 16 lanes are active or inactive together.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_sum16(float ss) {
    ss += dpp<0xb1>(ss);   // quad_perm [1, 0, 3, 2]
    ss += dpp<0x4e>(ss);   // quad_perm [2, 3, 0, 1]
    ss += dpp<0x141>(ss);  // row_half_mirror
    ss += dpp<0x140>(ss);  // row_mirror
    return ss;
}

// One (token, group, rank) row of N entries: raw / sqrt(mean square + eps) * w + bias.
// KP > 0: N % 8 == 0 and N <= 128 KP; lane l holds entries 8 l + 128 k .. + 7 of
// the row in registers (one read, one write). KP == 0: any N, one entry per
// lane and step, read twice (the second time from cache).
template <typename T, int KP>
__device__ __forceinline__ void norm_row(const T* __restrict__ src, T* dst, const float* __restrict__ w,
                                         const float* __restrict__ bias, int N, float eps, int l) {
    float ss = 0.f;
    if constexpr (KP > 0) {
        float v[KP][8];
#pragma unroll
        for (int k = 0; k < KP; ++k) {
            const int n0 = 8 * l + 128 * k;
            if (n0 < N) {
                Row8<T>::load(src + n0, v[k]);
#pragma unroll
                for (int e = 0; e < 8; ++e) ss += v[k][e] * v[k][e];
            }
        }
        const float scale = 1.f / sqrtf(row_sum16(ss) / float(N) + eps);
#pragma unroll
        for (int k = 0; k < KP; ++k) {
            const int n0 = 8 * l + 128 * k;
            if (n0 < N) {
                float wv[8], bv[8];
                if (w) load_par8(w + n0, wv);
                if (bias) load_par8(bias + n0, bv);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float o = v[k][e] * scale;
                    if (w) o *= wv[e];
                    if (bias) o += bv[e];
                    v[k][e] = o;
                }
                Row8<T>::store(dst + n0, v[k]);
            }
        }
    } else {
        for (int n = l; n < N; n += 16) {
            const float v = Io<T>::load(src, n);
            ss += v * v;
        }
        const float scale = 1.f / sqrtf(row_sum16(ss) / float(N) + eps);
        for (int n = l; n < N; n += 16) {
            float o = Io<T>::load(src, n) * scale;
            if (w) o *= w[n];
            if (bias) o += bias[n];
            Io<T>::store(dst, n, o);
        }
    }
}

// A block normalises 16 * RPG rows: the 16-lane group g takes rows
// 16 RPG blk + g + 16 j, j < RPG, with all their loads issued before the first
// reduction (more bytes in flight per lane).
template <typename T, int KP, int RPG>
__global__ void __launch_bounds__(256) prologue_kernel(PrologueArgs a, int64_t nbB, int64_t nbC) {
    const int64_t blk = blockIdx.x;
    const int tid = threadIdx.x, l = tid & 15;
    if (blk < nbB + nbC) {
        const bool isB = blk < nbB;
        const int64_t rows = a.ntok * a.GR;
        const int64_t row0 = (isB ? blk : blk - nbB) * (16 * RPG) + (tid >> 4);
        const float* w = isB ? a.B_weight : a.C_weight;
        const float* bias = isB ? a.B_bias : a.C_bias;
        const T* src = static_cast<const T*>(isB ? a.B_raw : a.C_raw);
        T* dst = static_cast<T*>(isB ? a.B : a.C);
        if constexpr (KP == 1) {
            float v[RPG][8];
#pragma unroll
            for (int j = 0; j < RPG; ++j) {
                const int64_t row = row0 + 16 * j;
                if (row < rows && 8 * l < a.N) Row8<T>::load(src + row * a.N + 8 * l, v[j]);
            }
#pragma unroll
            for (int j = 0; j < RPG; ++j) {
                const int64_t row = row0 + 16 * j;
                if (row >= rows) break;  // rows past the end: the group's lanes leave together
                float ss = 0.f;
                if (8 * l < a.N) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) ss += v[j][e] * v[j][e];
                }
                const float scale = 1.f / sqrtf(row_sum16(ss) / float(a.N) + a.eps);
                if (8 * l < a.N) {
                    const int64_t prow = (row % a.GR) * a.N + 8 * l;
                    float wv[8], bv[8];
                    if (w) load_par8(w + prow, wv);
                    if (bias) load_par8(bias + prow, bv);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float o = v[j][e] * scale;
                        if (w) o *= wv[e];
                        if (bias) o += bv[e];
                        v[j][e] = o;
                    }
                    Row8<T>::store(dst + row * a.N + 8 * l, v[j]);
                }
            }
        } else {
#pragma unroll 1
            for (int j = 0; j < RPG; ++j) {
                const int64_t row = row0 + 16 * j;
                if (row >= rows) break;
                const int64_t prow = (row % a.GR) * a.N;
                norm_row<T, KP>(src + row * a.N, dst + row * a.N, w ? w + prow : nullptr,
                                bias ? bias + prow : nullptr, a.N, a.eps, l);
            }
        }
        return;
    }
    // scalars: 4 consecutive (token, head) entries per thread
    const int64_t n = a.ntok * a.H;
    const int64_t i0 = (blk - nbB - nbC) * 1024 + 4 * int64_t(tid);
    if (i0 >= n) return;
    if (i0 + 4 <= n) {
        if (a.dt) {
            const floatx4 r = *reinterpret_cast<const floatx4*>(a.dt_raw + i0);
            floatx4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = softplus(r[e] + (a.dt_bias ? a.dt_bias[(i0 + e) % a.H] : 0.f));
            *reinterpret_cast<floatx4*>(a.dt + i0) = o;
        }
        if (a.lambda) {
            const floatx4 r = *reinterpret_cast<const floatx4*>(a.lambda_raw + i0);
            floatx4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = sigmoid(r[e]);
            *reinterpret_cast<floatx4*>(a.lambda + i0) = o;
        }
    } else {
        for (int64_t i = i0; i < n; ++i) {
            if (a.dt) a.dt[i] = softplus(a.dt_raw[i] + (a.dt_bias ? a.dt_bias[i % a.H] : 0.f));
            if (a.lambda) a.lambda[i] = sigmoid(a.lambda_raw[i]);
        }
    }
}

template <typename T>
hipError_t launch_t(const PrologueArgs& a) {
    const int64_t rows = a.ntok * a.GR;
    // rows per 16-lane group: 4 when a row's piece sits in registers, else 1
    const int kp = (a.N % 8 == 0 && a.N <= 128) ? 1 : (a.N % 8 == 0 && a.N <= 256) ? 2 : 0;
    const int rpg = kp == 1 ? 4 : 1;
    const int64_t nbB = a.B ? (rows + 16 * rpg - 1) / (16 * rpg) : 0, nbC = a.C ? (rows + 16 * rpg - 1) / (16 * rpg) : 0;
    const int64_t nbS = (a.dt || a.lambda) ? (a.ntok * a.H + 1023) / 1024 : 0;
    const int64_t nb = nbB + nbC + nbS;
    if (nb == 0) return hipSuccess;
    if (nb > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid{unsigned(nb)}, block{256u};
    if (kp == 1)
        hipLaunchKernelGGL((prologue_kernel<T, 1, 4>), grid, block, 0, a.stream, a, nbB, nbC);
    else if (kp == 2)
        hipLaunchKernelGGL((prologue_kernel<T, 2, 1>), grid, block, 0, a.stream, a, nbB, nbC);
    else
        hipLaunchKernelGGL((prologue_kernel<T, 0, 1>), grid, block, 0, a.stream, a, nbB, nbC);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prologue(const PrologueArgs& a) {
    return a.io == M3_BF16 ? launch_t<bf16_t>(a) : launch_t<float>(a);
}

}  // namespace m3
