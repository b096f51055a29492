// m3_decode.hip -- one recurrent step of the Mamba-3 SSM for every (batch, head).
//
// Per (b, h), with alpha = e^{dt A}, gamma = lambda dt, delta = (1 - lambda) dt
// (exponential-trapezoidal rule, "复值SSM × 广义梯形离散 × MIMO，线性模型的全面重构"
// §2.2) and the rotation of pair k by +dt*omega_k (complex state, same digest §2.1):
//
//   g   = h + delta * B_prev x_prev^T            (previous token, from the carry)
//   h'  = alpha * Rot(dt omega) g + gamma * B x^T   (rank-R: N x R times R x P, §2.3)
//   y   = h'^T C + D x
//
// The fp32 state is read and written once (the step is bound by that traffic:
// "Mamba-3架构技术解析：新一代语言建模的范式转移" §2.3 on decode being state-I/O
// bound). The previous token's rows: x per head (the workgroup of (b, h) reads
// its carry into LDS and, after a barrier, overwrites it with the current
// token's rows); B once per group, in two slots. Each head keeps a parity word:
// a step reads B_prev from the slot its parity names, the group's first head
// writes B_t into the other slot, and the head flips its parity. No slot is
// read and written in the same launch, and everything lives in device memory,
// so a captured graph of any number of steps replays correctly.
//
// Block order: `rev` (the host's step parity) walks the (b, h) workgroups
// backwards on every other step, so a step first reads the states the previous
// step wrote last, which the 256 MB memory-side cache (MALL) still holds when
// the state is about its size. A hint only: results do not depend on it.
#include <type_traits>

#include "m3_device.h"
#include "m3_internal.h"

namespace m3 {
namespace {

constexpr int kThreads = 256;  // generic kernel
constexpr float kInv2Pi = 0.15915494309189535f;

// (cos, sin) of theta = dt * omega through the hardware sine/cosine, which take
// revolutions: the per-step angle is a few radians at most, so after fract()
// the result is accurate to ~1e-6 absolute.
__device__ __forceinline__ void sincos_step(float theta, float* s, float* c) {
    const float r = __builtin_amdgcn_fractf(theta * kInv2Pi);
    *s = __builtin_amdgcn_sinf(r);
    *c = __builtin_amdgcn_cosf(r);
}

// The input prologue of m3_decode_step_fused (m3_prologue's reading, see
// m3_prologue.hip): softplus with the head's bias on the step, sigmoid on
// lambda (softplus_f, sigmoid_f of m3_device.h), and per (group, rank) row of B
// and C an RMS norm with weight and bias, the result rounded to the io dtype as
// m3_prologue stores it. The norm's reciprocal square root is the hardware one
// (v_rsq_f32, about 1 ulp; the row is rounded to bf16 after it): the precise
// square root and division cost 0.7 us per step at R 4, b 128, H 64.
template <typename T>
__device__ __forceinline__ float round_io(float v) {
    if constexpr (std::is_same<T, bf16_t>::value) return bf16_to_f32(f32_to_bf16(v));
    return v;
}
// The step's streaming rows in the merged-input MFMA kernel: x_t is read and
// y_t written once, by one workgroup. Non-temporal accesses keep them from
// displacing cached lines that are read again (the state between steps, B_t
// and C_t across a group's heads, the carries): b 128, H 64, R 4 91.4 -> 89.1 us
// per step. The other kernels keep cached accesses: with these hints the one
// with separate input sums ran slower (R 8 103.4 -> 111.4 us) and the row
// kernel gained at most 0.2 us at N 128, P 64 but lost 2.4 us at N 64, P 32.
__device__ __forceinline__ unsigned load_stream(const unsigned* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store_stream(bf16_t* p, int64_t i, float v) {
    __builtin_nontemporal_store(f32_to_bf16(v), &p[i].bits);
}
// the step's dt and lambda: as given, or through the prologue
template <bool PRO>
__device__ __forceinline__ void step_scalars(const float* dt, const float* lam, const DecodePrologue& pro, int64_t bh,
                                             int h, float* d, float* lm) {
    if constexpr (PRO) {
        *d = softplus_f(dt[bh] + (pro.dt_bias ? pro.dt_bias[h] : 0.f));
        *lm = lam ? sigmoid_f(lam[bh]) : 1.f;
    } else {
        *d = dt[bh];
        *lm = lam_at(lam, bh);
    }
}
// sum over aligned groups of GL lanes (32 or 64), off the LDS crossbar:
// inclusive prefix sums inside each 16-lane row by DPP row shifts, then the
// row totals (lanes 15, 31, 47, 63) read into scalar registers and added
template <int CTL>
__device__ __forceinline__ float dpp_shr(float u) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, u), CTL, 0xf, 0xf, false));
}
__device__ __forceinline__ float lane_of(float u, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, u), l));
}
template <int GL>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(GL == 32 || GL == 64, "lane group");
    v += dpp_shr<0x111>(v);
    v += dpp_shr<0x112>(v);
    v += dpp_shr<0x114>(v);
    v += dpp_shr<0x118>(v);
    const float r0 = lane_of(v, 15), r1 = lane_of(v, 31), r2 = lane_of(v, 47), r3 = lane_of(v, 63);
    if constexpr (GL == 64) return (r0 + r1) + (r2 + r3);
    return (threadIdx.x & 32) ? r2 + r3 : r0 + r1;
}
// io elements as loaded, in 32-bit words (two bf16, or one float), and the
// value of element i of them: loads kept in this form until their use need no
// wait where they are issued
template <typename T>
struct RawIo {
    static constexpr int per_word = 1;
    __device__ __forceinline__ static float val(const unsigned* w, int i) { return __uint_as_float(w[i]); }
};
template <>
struct RawIo<bf16_t> {
    static constexpr int per_word = 2;
    __device__ __forceinline__ static float val(const unsigned* w, int i) {
        return __uint_as_float((i & 1) ? w[i >> 1] & 0xffff0000u : w[i >> 1] << 16);
    }
};

// RMS-normalise the R rows of B (rb) and of C (rc), N fp32 values each in LDS,
// in place, with the weights and biases of group g; one wave per row. The
// caller synchronises before (rows staged) and after (rows read).
template <typename T>
__device__ void qk_norm_rows(float* rb, float* rc, int R, int N, int g, const DecodePrologue& pro, int tid,
                             int nthreads) {
    const int lane = tid & 63, nw = nthreads >> 6;
    for (int row = tid >> 6; row < 2 * R; row += nw) {
        const bool isC = row >= R;
        const int r = isC ? row - R : row;
        float* v = (isC ? rc : rb) + r * N;
        float ss = 0.f;
        for (int n = lane; n < N; n += 64) ss += v[n] * v[n];
#pragma unroll
        for (int sh = 32; sh >= 1; sh >>= 1) ss += __shfl_xor(ss, sh);
        const float scale = __builtin_amdgcn_rsqf(ss / float(N) + pro.eps);
        const float* w = isC ? pro.C_weight : pro.B_weight;
        const float* bb = isC ? pro.C_bias : pro.B_bias;
        const int64_t o = (int64_t(g) * R + r) * N;
        for (int n = lane; n < N; n += 64)
            v[n] = round_io<T>(v[n] * scale * (w ? w[o + n] : 1.f) + (bb ? bb[o + n] : 0.f));
    }
}

// Threads per workgroup of the N = 128, P = 64 kernel, per rank class.
#ifndef M3_DECODE_THREADS_R1
#define M3_DECODE_THREADS_R1 256
#endif
#ifndef M3_DECODE_THREADS_R4
#define M3_DECODE_THREADS_R4 1024
#endif

// N in {64, 128, 256}, P in {32, 64, 128}: with QP = P / 4 column quads per
// row, thread (kk, q), q = tid % QP, owns rows (2k, 2k+1), k = kk + (NTH/QP)*it,
// it < (N/2) / (NTH/QP), and columns 4q..4q+3, loaded and stored as float4 (a
// wave covers 64/QP row segments of P floats per access).
template <typename T, int R, int NTH, int N, int P, bool PRO>
__global__ void __launch_bounds__(NTH)
decode_rows_kernel(float* __restrict__ hstate, T* __restrict__ carry_B, T* __restrict__ carry_x,
                       unsigned* __restrict__ par, int rev, DecodePrologue pro,
                       const T* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
                       const float* __restrict__ omega, const float* __restrict__ lam, const T* __restrict__ B,
                       const T* __restrict__ C, const float* __restrict__ D, T* __restrict__ y, int64_t nb, int H,
                       int G) {
    constexpr int K = N / 2, QP = P / 4;
    constexpr int KS = NTH / QP;  // row-pair stride between a thread's iterations
    constexpr int IT = K / KS;    // row pairs per thread
    static_assert(NTH % QP == 0 && K % KS == 0 && IT >= 1 && QP <= 64 && NTH % 64 == 0, "decode tiling");
    __shared__ float sB[R][N], sBp[R][N], sC[R][N];
    __shared__ float sx[R][P], sxp[R][P];
    __shared__ float red[NTH / 64][R][P];

    const int tid = threadIdx.x;
    const int64_t bh = rev ? int64_t(gridDim.x) - 1 - blockIdx.x : int64_t(blockIdx.x);
    const int64_t b = bh / H;
    const int h = int(bh % H);
    const int g = h / (H / G);
    const int64_t bg = b * G + g;
    const unsigned pr = par[bh] & 1u;  // slot of B_prev
    float* hs = hstate + bh * (N * P);
    const int q = tid % QP, kk = tid / QP;

    // With the prologue, each rank row of B_t and C_t is normalised by the GL
    // lanes that load it (PE consecutive entries per lane): its sum of squares
    // never leaves them. Rows of B first, then of C, in whole lane groups (2 R GL
    // and NTH are multiples of GL). The rows and their weights are loaded first,
    // ahead of the state, so their latency hides under the state stream; the
    // rows stay raw until their use (a conversion here would wait for them
    // before the state loads are issued).
    constexpr int PE = N >= 256 ? N / 64 : 2, GL = N / PE;
    constexpr int NIT = PRO ? (2 * R * GL + NTH - 1) / NTH : 0;
    static_assert(GL <= 64 && (GL & (GL - 1)) == 0, "row lanes");
    constexpr int PW = PE / RawIo<T>::per_word;  // 32-bit words per item (rows start 16-byte aligned)
    unsigned pv[NIT > 0 ? NIT : 1][PW];
    float pw[NIT > 0 ? NIT : 1][PE], pb[NIT > 0 ? NIT : 1][PE];
    if constexpr (PRO) {
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int e = tid + it * NTH;
            if (e >= 2 * R * GL) continue;
            const bool isC = e >= R * GL;
            const int r = (isC ? e - R * GL : e) / GL, n0 = (e % GL) * PE;
            const T* src = (isC ? C : B) + bg * (R * N);
            const float* w = isC ? pro.C_weight : pro.B_weight;
            const float* bb = isC ? pro.C_bias : pro.B_bias;
            const int64_t o = (int64_t(g) * R + r) * N + n0;
            const unsigned* src32 = reinterpret_cast<const unsigned*>(src + r * N + n0);
#pragma unroll
            for (int i = 0; i < PW; ++i) pv[it][i] = src32[i];
#pragma unroll
            for (int i = 0; i < PE; ++i) {
                pw[it][i] = w ? w[o + i] : 1.f;
                pb[it][i] = bb ? bb[o + i] : 0.f;
            }
        }
    }

    // The step's other small rows (B_t and C_t unless the prologue loaded them,
    // B_prev, x_t, x_prev) as 32-bit words, also ahead of the state: staging
    // them then waits for them alone (completion counts are in order).
    constexpr int WPE = RawIo<T>::per_word;              // io elements per word
    constexpr int NWB = R * N / WPE, NWX = R * P / WPE;  // words per row set
    constexpr int IB = (NWB + NTH - 1) / NTH, IX = (NWX + NTH - 1) / NTH;
    const unsigned* Bt32 = reinterpret_cast<const unsigned*>(B + bg * (R * N));
    const unsigned* Ct32 = reinterpret_cast<const unsigned*>(C + bg * (R * N));
    const unsigned* Bp32 = reinterpret_cast<const unsigned*>(carry_B + (int64_t(pr) * nb * G + bg) * (R * N));
    const unsigned* xt32 = reinterpret_cast<const unsigned*>(x + bh * (R * P));
    const unsigned* xp32 = reinterpret_cast<const unsigned*>(carry_x + bh * (R * P));
    unsigned wb[PRO ? 1 : IB], wc[PRO ? 1 : IB], wbp[IB], wx[IX], wxp[IX];
#pragma unroll
    for (int it = 0; it < IB; ++it) {
        const int e = tid + it * NTH;
        if (e >= NWB) continue;
        if constexpr (!PRO) {
            wb[it] = Bt32[e];
            wc[it] = Ct32[e];
        }
        wbp[it] = Bp32[e];
    }
#pragma unroll
    for (int it = 0; it < IX; ++it) {
        const int e = tid + it * NTH;
        if (e >= NWX) continue;
        wx[it] = xt32[e];
        wxp[it] = xp32[e];
    }

    float4 v0[IT], v1[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int k = kk + KS * it;
        v0[it] = *reinterpret_cast<const float4*>(hs + (2 * k) * P + 4 * q);
        v1[it] = *reinterpret_cast<const float4*>(hs + (2 * k + 1) * P + 4 * q);
    }

#pragma unroll
    for (int it = 0; it < IB; ++it) {
        const int e = tid + it * NTH;
        if (e >= NWB) continue;
#pragma unroll
        for (int i = 0; i < WPE; ++i) {
            if constexpr (!PRO) {
                (&sB[0][0])[WPE * e + i] = RawIo<T>::val(&wb[it], i);
                (&sC[0][0])[WPE * e + i] = RawIo<T>::val(&wc[it], i);
            }
            (&sBp[0][0])[WPE * e + i] = RawIo<T>::val(&wbp[it], i);
        }
    }
    if constexpr (PRO) {
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int e = tid + it * NTH;
            if (e >= 2 * R * GL) continue;  // whole lane groups skip together
            const bool isC = e >= R * GL;
            const int r = (isC ? e - R * GL : e) / GL, n0 = (e % GL) * PE;
            float v[PE], ss = 0.f;
#pragma unroll
            for (int i = 0; i < PE; ++i) {
                v[i] = RawIo<T>::val(pv[it], i);
                ss += v[i] * v[i];
            }
            ss = group_sum<GL>(ss);
            const float k = __builtin_amdgcn_rsqf(ss * (1.f / float(N)) + pro.eps);
            float* dst = isC ? &sC[r][n0] : &sB[r][n0];
#pragma unroll
            for (int i = 0; i < PE; ++i) dst[i] = round_io<T>(v[i] * k * pw[it][i] + pb[it][i]);
        }
    }
#pragma unroll
    for (int it = 0; it < IX; ++it) {
        const int e = tid + it * NTH;
        if (e >= NWX) continue;
#pragma unroll
        for (int i = 0; i < WPE; ++i) {
            (&sx[0][0])[WPE * e + i] = RawIo<T>::val(&wx[it], i);
            (&sxp[0][0])[WPE * e + i] = RawIo<T>::val(&wxp[it], i);
        }
    }
    float d, lm;
    step_scalars<PRO>(dt, lam, pro, bh, h, &d, &lm);
    const float alpha = expf(d * A[h]);
    const float gamma = lm * d, delta = (1.f - lm) * d;
    __syncthreads();

    float yacc[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) yacc[r][c] = 0.f;

#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int k = kk + KS * it;
        float sn, cs;
        sincos_step(d * om_at(omega, int64_t(h) * K + k), &sn, &cs);
        sn *= alpha;  // alpha folded into the rotation
        cs *= alpha;
        float e0[4] = {v0[it].x, v0[it].y, v0[it].z, v0[it].w};
        float e1[4] = {v1[it].x, v1[it].y, v1[it].z, v1[it].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int p = 4 * q + c;
            float up0 = 0.f, up1 = 0.f, u0 = 0.f, u1 = 0.f;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                up0 += sBp[r][2 * k] * sxp[r][p];
                up1 += sBp[r][2 * k + 1] * sxp[r][p];
                u0 += sB[r][2 * k] * sx[r][p];
                u1 += sB[r][2 * k + 1] * sx[r][p];
            }
            const float g0 = e0[c] + delta * up0, g1 = e1[c] + delta * up1;
            const float n0 = (cs * g0 - sn * g1) + gamma * u0;
            const float n1 = (sn * g0 + cs * g1) + gamma * u1;
            e0[c] = n0;
            e1[c] = n1;
#pragma unroll
            for (int r = 0; r < R; ++r) yacc[r][c] += n0 * sC[r][2 * k] + n1 * sC[r][2 * k + 1];
        }
        *reinterpret_cast<float4*>(hs + (2 * k) * P + 4 * q) = make_float4(e0[0], e0[1], e0[2], e0[3]);
        *reinterpret_cast<float4*>(hs + (2 * k + 1) * P + 4 * q) = make_float4(e1[0], e1[1], e1[2], e1[3]);
    }

    // reduce over the row groups: 64/QP in a wave (lanes QP apart), then across waves
    const int wave = tid >> 6;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float v = yacc[r][c];
#pragma unroll
            for (int sh = QP; sh < 64; sh <<= 1) v += __shfl_xor(v, sh);
            if ((tid & 63) < QP) red[wave][r][4 * q + c] = v;
        }
    __syncthreads();
    const float Dh = D[h];
    for (int e = tid; e < R * P; e += NTH) {
        const int r = e / P, p = e % P;
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < NTH / 64; ++w) s += red[w][r][p];
        Io<T>::store(y, bh * (R * P) + e, s + Dh * sx[r][p]);
    }

    // this token becomes the carry of the next step, from the words it was
    // staged from (the carry was read before the barrier above)
#pragma unroll
    for (int it = 0; it < IX; ++it) {
        const int e = tid + it * NTH;
        if (e < NWX) reinterpret_cast<unsigned*>(carry_x + bh * (R * P))[e] = wx[it];
    }
    if (h % (H / G) == 0) {
        T* dst = carry_B + (int64_t(pr ^ 1u) * nb * G + bg) * (R * N);
        if constexpr (PRO) {
            for (int e = tid; e < R * N; e += NTH)
                Io<T>::store(dst, e, (&sB[0][0])[e]);  // the normalised row, already in the io dtype
        } else {
#pragma unroll
            for (int it = 0; it < IB; ++it) {
                const int e = tid + it * NTH;
                if (e < NWB) reinterpret_cast<unsigned*>(dst)[e] = wb[it];
            }
        }
    }
    if (tid == 0) par[bh] = pr ^ 1u;
}

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
// two floats -> packed bf16 (round to nearest even)
__device__ __forceinline__ unsigned pk_bf16(float lo, float hi) {
    bf16x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(unsigned, v);
}
__device__ __forceinline__ float bf_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

typedef float floatx16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ floatx16 mfma32_k16(u32x4 a, u32x4 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// bf16 I/O, N in {64, 128}, P = 64, R in {2, 3, 4, 8}: the step on 32 x 32 MFMA
// tiles (v_mfma_f32_32x32x16_bf16). With the exponential-trapezoidal step
//   h' = alpha Rot(h) + M,   M = gamma B^T x + alpha delta Rot(B_prev)^T x_prev,
// both input terms are one K = 16 contraction over k = (term, rank) at R <= 4
// and two at R 8: the A operand holds gamma B and alpha delta Rot(B_prev) per
// row n, each as a bf16 pair (hi, lo) whose sum is the fp32 value to 2^-16
// (R <= 4, four rank slots: k = 8 g2 + t, t < 4 the hi, t >= 4 the lo terms,
// g2 = 0 gamma B, g2 = 1 B_prev; R 8: the first MFMA takes the hi (g2 = 0) and
// lo (g2 = 1) terms of gamma B over the 8 ranks, the second those of B_prev),
// and the B operand holds x (against the gamma B terms) and x_prev (against
// the B_prev terms), exact in bf16. The rotation of B_prev's rows is
// the rotation the previous term takes in the state (it acts on the rows n
// only). Then y[r][p] = sum_n C[r][n] h'[n][p] takes one K = 16 MFMA per
// (tile, j): k = 8 g2 + t holds the hi (t < 4) and lo (t >= 4) bf16 terms of
// the lane's rows 8 j + 4 g2 + (t & 3), against C of those rows twice, which
// keeps y at fp32 accuracy with no cross-lane movement.
//
// One 256-thread workgroup per (b, h); wave w owns state columns
// 32 (w & 1) .. + 31 and the row tiles (32 rows each) of half (w >> 1) of the
// rows. In row tile nt, lane (l32, g2) holds column 32 (w & 1) + l32 of rows
// 32 nt + 8 j + 4 g2 + e (j, e = 0..3): the accumulator layout of the 32 x 32
// MFMA, with two whole rotation pairs per (j, lane). A state load or store of
// one wave covers two whole 128-byte row segments (32 consecutive floats of
// two rows); on 16 x 16 tiles (lane = 4 rows of one column) it moved 64-byte
// halves of four rows, and the step took 89.1 against 85.7 us (R 4, b 128,
// H 64) and 185.3 against 170.8 us at b 256; R 8, where an earlier kernel
// summed the two input terms in separate K = 16 MFMAs on 16 x 16 tiles:
// 103.2 against 92.9 us at b 128. The two waves of a column half
// add their partial y through LDS. The step's small rows (B_t, C_t, B_prev,
// x_t, x_prev) and the rotation frequencies are loaded before the state, so
// their staging runs while the state streams in.
template <int R, int N, bool PRO>
// Held to 4 waves per SIMD (no spills; without the bound the plain instances
// take 156 registers and run 3: 88.0 against 85.7 us per step at R 4, b 128;
// at 5 the plain ones gain nothing and the fused ones lose 1.2 us).
__global__ void __launch_bounds__(256, 4)
decode_mfma32_kernel(float* __restrict__ hstate, bf16_t* __restrict__ carry_B, bf16_t* __restrict__ carry_x,
                     unsigned* __restrict__ par, int rev, DecodePrologue pro,
                     const bf16_t* __restrict__ x, const float* __restrict__ dt,
                     const float* __restrict__ A, const float* __restrict__ omega, const float* __restrict__ lam,
                     const bf16_t* __restrict__ B, const bf16_t* __restrict__ C, const float* __restrict__ D,
                     bf16_t* __restrict__ y, int64_t nb, int H, int G) {
    static_assert((R >= 2 && R <= 4) || R == 8, "ranks 2-4 (R 3 with a zero rank slot) and 8");
    constexpr int NTH = 256, P = 64, K = N / 2, CS_ = N + 8, NT = N / 32, NTW = NT / 2;
    constexpr int RS = R <= 4 ? 4 : 8;           // rank slots
    constexpr int NBI = (RS * K + NTH - 1) / NTH;  // (rank slot, pair) items of B per thread
    constexpr int NCI = (R * K + NTH - 1) / NTH;  // (rank, pair) items of C per thread
    constexpr int AS = 4 * RS + 8;                // sA row stride (bf16): 4 RS used, 16-byte aligned rows
    // per row n, k = 0 .. 4 RS - 1: (gamma B)_hi, (gamma B)_lo, (alpha delta Rot B_prev)_hi, _lo; RS rank slots each
    __shared__ __attribute__((aligned(16))) uint16_t sA[N][AS];
    __shared__ __attribute__((aligned(16))) uint16_t sXt[P][RS];   // x^T, zero past R
    __shared__ __attribute__((aligned(16))) uint16_t sXpt[P][RS];  // x_prev^T
    __shared__ __attribute__((aligned(16))) uint16_t sC[R][CS_];  // C rows (padded)
    __shared__ __attribute__((aligned(16))) float sCS[K][2];      // alpha * (cos, sin) of pair k
    __shared__ float sY[2][RS][32];  // partial y of the second row half, per column half

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, g2 = lane >> 5;
    const int64_t bh = rev ? int64_t(gridDim.x) - 1 - blockIdx.x : int64_t(blockIdx.x);
    const int64_t b = bh / H;
    const int h = int(bh % H);
    const int gi = h / (H / G);
    const int64_t bg = b * G + gi;
    const unsigned pr = par[bh] & 1u;  // slot of B_prev
    float* hs = hstate + bh * (N * P);
    const int p = 32 * (w & 1) + l32;

    // The small rows first (raw with the prologue, with the norm weights).
    // Thread item e of B: rank slot r = e / K, pair j = e % K (rows 2 j, 2 j + 1).
    const unsigned* Bt32 = reinterpret_cast<const unsigned*>(B + bg * (R * N));
    const unsigned* Ct32 = reinterpret_cast<const unsigned*>(C + bg * (R * N));
    const unsigned* Bp32 = reinterpret_cast<const unsigned*>(carry_B + (int64_t(pr) * nb * G + bg) * (R * N));
    const unsigned* xt32 = reinterpret_cast<const unsigned*>(x + bh * (R * P));
    const unsigned* xp32 = reinterpret_cast<const unsigned*>(carry_x + bh * (R * P));
    auto wpair = [&](const float* v, int r, int j, float dflt) {
        if (!v) return float2{dflt, dflt};
        const int64_t o = (int64_t(gi) * R + r) * N + 2 * j;
        return float2{v[o], v[o + 1]};
    };
    unsigned rb[NBI], rbp[NBI], rc[NCI];
    float rom[NBI];
    float2 bw[PRO ? NBI : 1], bb2[PRO ? NBI : 1], cw[PRO ? NCI : 1], cb2[PRO ? NCI : 1];
#pragma unroll
    for (int it = 0; it < NBI; ++it) {
        const int e = tid + NTH * it, r = e / K, j = e % K;
        const bool in = e < RS * K && r < R;
        rb[it] = in ? Bt32[r * K + j] : 0u;
        rbp[it] = in ? Bp32[r * K + j] : 0u;
        rom[it] = e < RS * K ? om_at(omega, int64_t(h) * K + j) : 0.f;
        if constexpr (PRO) {
            bw[it] = in ? wpair(pro.B_weight, r, j, 1.f) : float2{1.f, 1.f};
            bb2[it] = in ? wpair(pro.B_bias, r, j, 0.f) : float2{0.f, 0.f};
        }
    }
#pragma unroll
    for (int it = 0; it < NCI; ++it) {
        const int e = tid + NTH * it;
        const bool in = e < R * K;
        rc[it] = in ? Ct32[e] : 0u;
        if constexpr (PRO) {
            cw[it] = in ? wpair(pro.C_weight, e / K, e % K, 1.f) : float2{1.f, 1.f};
            cb2[it] = in ? wpair(pro.C_bias, e / K, e % K, 0.f) : float2{0.f, 0.f};
        }
    }
    // x_t, x_prev: thread tid < RS P / 2 takes rank slot tid / (P / 2), column pair tid % (P / 2)
    const bool xin = tid < RS * (P / 2) && tid / (P / 2) < R;
    const unsigned rx = xin ? load_stream(&xt32[tid]) : 0u, rxp = xin ? xp32[tid] : 0u;

    const int nt0 = (w >> 1) * NTW;  // the wave's first row tile
    float st[NTW][16];
#pragma unroll
    for (int i = 0; i < NTW; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) st[i][v] = hs[(32 * (nt0 + i) + 8 * (v >> 2) + 4 * g2 + (v & 3)) * P + p];

    float d, lm;
    step_scalars<PRO>(dt, lam, pro, bh, h, &d, &lm);
    const float alpha = expf(d * A[h]);
    const float gamma = lm * d, ad = alpha * (1.f - lm) * d;

    // the normalised pair from a raw pair, its weights and biases; the K lanes
    // holding one rank row (a whole wave at N 128, half a wave at N 64) reduce its sum of squares
    auto norm_pair = [&](unsigned raw, int r, float2 wv, float2 bv) -> unsigned {
        const float v0 = bf_lo(raw), v1 = bf_hi(raw);
        const float ss = group_sum<K>(v0 * v0 + v1 * v1);
        if (r >= R) return 0u;
        const float k = __builtin_amdgcn_rsqf(ss * (1.f / float(N)) + pro.eps);
        return pk_bf16(v0 * k * wv.x + bv.x, v1 * k * wv.y + bv.y);
    };
#pragma unroll
    for (int it = 0; it < NBI; ++it) {
        const int e = tid + NTH * it;
        if (e >= RS * K) break;  // whole lane groups
        const int r = e / K, j = e % K;
        if constexpr (PRO) rb[it] = norm_pair(rb[it], r, bw[it], bb2[it]);  // kept for the carry
        float sn, cs;
        sincos_step(d * rom[it], &sn, &cs);
        if (r == 0) {
            sCS[j][0] = alpha * cs;
            sCS[j][1] = alpha * sn;
        }
        const float g0 = gamma * bf_lo(rb[it]), g1 = gamma * bf_hi(rb[it]);
        const float p0 = bf_lo(rbp[it]), p1 = bf_hi(rbp[it]);
        const float q0 = ad * (cs * p0 - sn * p1), q1 = ad * (sn * p0 + cs * p1);
        const unsigned gh = pk_bf16(g0, g1), qh = pk_bf16(q0, q1);
        const unsigned gl = pk_bf16(g0 - bf_lo(gh), g1 - bf_hi(gh)), ql = pk_bf16(q0 - bf_lo(qh), q1 - bf_hi(qh));
        sA[2 * j][r] = uint16_t(gh);
        sA[2 * j + 1][r] = uint16_t(gh >> 16);
        sA[2 * j][RS + r] = uint16_t(gl);
        sA[2 * j + 1][RS + r] = uint16_t(gl >> 16);
        sA[2 * j][2 * RS + r] = uint16_t(qh);
        sA[2 * j + 1][2 * RS + r] = uint16_t(qh >> 16);
        sA[2 * j][3 * RS + r] = uint16_t(ql);
        sA[2 * j + 1][3 * RS + r] = uint16_t(ql >> 16);
    }
    if (tid < RS * (P / 2)) {
        const int r = tid / (P / 2), j = tid % (P / 2);
        sXt[2 * j][r] = uint16_t(rx);
        sXt[2 * j + 1][r] = uint16_t(rx >> 16);
        sXpt[2 * j][r] = uint16_t(rxp);
        sXpt[2 * j + 1][r] = uint16_t(rxp >> 16);
    }
#pragma unroll
    for (int it = 0; it < NCI; ++it) {
        const int e = tid + NTH * it;
        if (e >= R * K) break;  // whole lane groups
        unsigned cv = rc[it];
        if constexpr (PRO) cv = norm_pair(cv, e / K, cw[it], cb2[it]);
        reinterpret_cast<unsigned*>(&sC[e / K][0])[e % K] = cv;
    }
    __syncthreads();

    // B operand of the input MFMA(s): k = 8 g2 .. 8 g2 + 7 -> RS 4: ranks 0..3 of x twice (g2 0) or of
    // x_prev twice (g2 1); RS 8: ranks 0..7 of x (against the gamma B terms) and of x_prev (second MFMA)
    u32x4 bx, bxp;
    if constexpr (RS == 4) {
        const u32x2 xr = *reinterpret_cast<const u32x2*>(g2 == 0 ? &sXt[p][0] : &sXpt[p][0]);
        bx = u32x4{xr[0], xr[1], xr[0], xr[1]};
        bxp = bx;
    } else {
        bx = *reinterpret_cast<const u32x4*>(&sXt[p][0]);
        bxp = *reinterpret_cast<const u32x4*>(&sXpt[p][0]);
    }
    const int rcl = l32 < R ? l32 : 0;
    const u32x2 zero = {0u, 0u};
    floatx16 yacc;
#pragma unroll
    for (int v = 0; v < 16; ++v) yacc[v] = 0.f;
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
        const int n0 = 32 * (nt0 + i);
        floatx16 M;
#pragma unroll
        for (int v = 0; v < 16; ++v) M[v] = 0.f;
        M = mfma32_k16(*reinterpret_cast<const u32x4*>(&sA[n0 + l32][8 * g2]), bx, M);
        if constexpr (RS == 8) M = mfma32_k16(*reinterpret_cast<const u32x4*>(&sA[n0 + l32][16 + 8 * g2]), bxp, M);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r0 = n0 + 8 * j + 4 * g2;  // the lane's rows r0 .. r0 + 3: pairs r0 / 2, r0 / 2 + 1
            // alpha (cos, sin) of those two pairs
            const floatx4 cs = *reinterpret_cast<const floatx4*>(&sCS[r0 >> 1][0]);
            float nv[4];
#pragma unroll
            for (int hp = 0; hp < 2; ++hp) {
                const float c = cs[2 * hp], sn = cs[2 * hp + 1];
                const float h0 = st[i][4 * j + 2 * hp], h1 = st[i][4 * j + 2 * hp + 1];
                nv[2 * hp] = (c * h0 - sn * h1) + M[4 * j + 2 * hp];
                nv[2 * hp + 1] = (sn * h0 + c * h1) + M[4 * j + 2 * hp + 1];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) hs[(r0 + e) * P + p] = nv[e];
            const unsigned h01 = pk_bf16(nv[0], nv[1]), h23 = pk_bf16(nv[2], nv[3]);
            const u32x4 hl = {h01, h23, pk_bf16(nv[0] - bf_lo(h01), nv[1] - bf_hi(h01)),
                              pk_bf16(nv[2] - bf_lo(h23), nv[3] - bf_hi(h23))};
            const u32x2 cv = l32 < R ? *reinterpret_cast<const u32x2*>(&sC[rcl][r0]) : zero;
            yacc = mfma32_k16(u32x4{cv[0], cv[1], cv[0], cv[1]}, hl, yacc);
        }
    }
    // lane (l32, g2) holds the partial y[r = 4 g2 + e][p] in yacc[e], e < 4
    if (w >= 2 && 4 * g2 < RS)
#pragma unroll
        for (int e = 0; e < 4; ++e) sY[w & 1][4 * g2 + e][l32] = yacc[e];
    __syncthreads();
    if (w < 2 && 4 * g2 < R) {
        const float Dh = D[h];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * g2 + e;
            if (r >= R) break;
            const float xv = __uint_as_float(unsigned(sXt[p][r]) << 16);
            store_stream(y, bh * (R * P) + r * P + p, (yacc[e] + sY[w][r][l32]) + Dh * xv);
        }
    }

    // this token becomes the carry of the next step, from the registers it was
    // staged from (the carry was read before the barrier above)
    if (tid < R * (P / 2)) reinterpret_cast<unsigned*>(carry_x + bh * (R * P))[tid] = rx;
    if (h % (H / G) == 0) {
        unsigned* cb32 = reinterpret_cast<unsigned*>(carry_B + (int64_t(pr ^ 1u) * nb * G + bg) * (R * N));
#pragma unroll
        for (int it = 0; it < NBI; ++it) {  // the normalised row with the prologue
            const int e = tid + NTH * it;
            if (e < R * K) cb32[e] = rb[it];
        }
    }
    if (tid == 0) par[bh] = pr ^ 1u;
}

// Any sizes: thread loops over (pair k, column p); y is a second pass over the new state.
template <typename T, bool PRO>
__global__ void __launch_bounds__(kThreads)
decode_generic_kernel(float* __restrict__ hstate, T* __restrict__ carry_B, T* __restrict__ carry_x,
                      unsigned* __restrict__ par, int rev, DecodePrologue pro,
                      const T* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
                      const float* __restrict__ omega, const float* __restrict__ lam, const T* __restrict__ B,
                      const T* __restrict__ C, const float* __restrict__ D, T* __restrict__ y, int64_t nb, int H,
                      int G, int P, int N, int R) {
    const int tid = threadIdx.x;
    const int64_t bh = rev ? int64_t(gridDim.x) - 1 - blockIdx.x : int64_t(blockIdx.x);
    const int64_t b = bh / H;
    const int h = int(bh % H);
    const int g = h / (H / G);
    const int64_t bg = b * G + g;
    const unsigned pr = par[bh] & 1u;  // slot of B_prev
    const int K = N / 2;
    float* hs = hstate + bh * int64_t(N) * P;
    const T* Bt = B + bg * int64_t(R) * N;
    const T* Ct = C + bg * int64_t(R) * N;
    const T* Bp = carry_B + (int64_t(pr) * nb * G + bg) * int64_t(R) * N;
    const T* xt = x + bh * int64_t(R) * P;
    const T* xp = carry_x + bh * int64_t(R) * P;
    float d, lm;
    step_scalars<PRO>(dt, lam, pro, bh, h, &d, &lm);
    const float alpha = expf(d * A[h]);
    const float gamma = lm * d, delta = (1.f - lm) * d;
    // with the prologue, B_t and C_t are read from their normalised copies in LDS
    extern __shared__ float sNorm[];  // [2][R][N] when PRO
    if constexpr (PRO) {
        for (int e = tid; e < R * N; e += kThreads) {
            sNorm[e] = Io<T>::load(Bt, e);
            sNorm[R * N + e] = Io<T>::load(Ct, e);
        }
        __syncthreads();
        qk_norm_rows<T>(sNorm, sNorm + R * N, R, N, g, pro, tid, kThreads);
        __syncthreads();
    }
    auto Bv = [&](int64_t i) { return PRO ? sNorm[i] : Io<T>::load(Bt, i); };
    auto Cv = [&](int64_t i) { return PRO ? sNorm[R * N + i] : Io<T>::load(Ct, i); };

    for (int e = tid; e < K * P; e += kThreads) {
        const int k = e / P, p = e % P;
        float up0 = 0.f, up1 = 0.f, u0 = 0.f, u1 = 0.f;
        for (int r = 0; r < R; ++r) {
            const float xpv = Io<T>::load(xp, int64_t(r) * P + p), xv = Io<T>::load(xt, int64_t(r) * P + p);
            up0 += Io<T>::load(Bp, int64_t(r) * N + 2 * k) * xpv;
            up1 += Io<T>::load(Bp, int64_t(r) * N + 2 * k + 1) * xpv;
            u0 += Bv(int64_t(r) * N + 2 * k) * xv;
            u1 += Bv(int64_t(r) * N + 2 * k + 1) * xv;
        }
        float sn, cs;
        sincos_step(d * om_at(omega, int64_t(h) * K + k), &sn, &cs);
        const float g0 = hs[int64_t(2 * k) * P + p] + delta * up0;
        const float g1 = hs[int64_t(2 * k + 1) * P + p] + delta * up1;
        hs[int64_t(2 * k) * P + p] = alpha * (cs * g0 - sn * g1) + gamma * u0;
        hs[int64_t(2 * k + 1) * P + p] = alpha * (sn * g0 + cs * g1) + gamma * u1;
    }
    __syncthreads();
    const float Dh = D[h];
    for (int e = tid; e < R * P; e += kThreads) {
        const int r = e / P, p = e % P;
        float s = 0.f;
        for (int n = 0; n < N; ++n) s += hs[int64_t(n) * P + p] * Cv(int64_t(r) * N + n);
        Io<T>::store(y, bh * int64_t(R) * P + e, s + Dh * Io<T>::load(xt, e));
    }
    // this token becomes the carry of the next step (every read of the carry
    // precedes the barrier above)
    for (int e = tid; e < R * P; e += kThreads) carry_x[bh * int64_t(R) * P + e] = xt[e];
    if (h % (H / G) == 0)
        for (int e = tid; e < R * N; e += kThreads) {
            T* dst = carry_B + (int64_t(pr ^ 1u) * nb * G + bg) * int64_t(R) * N;
            if constexpr (PRO)
                Io<T>::store(dst, e, sNorm[e]);
            else
                dst[e] = Bt[e];
        }
    if (tid == 0) par[bh] = pr ^ 1u;
}

// the per-head parity words behind the two B slots of the carry buffer
unsigned* parity_words(const DecodeArgs& a) {
    return reinterpret_cast<unsigned*>(static_cast<char*>(a.carry_B) +
                                       decode_carry_B_slots_bytes(a.b, a.G, a.R, a.N, a.io == M3_BF16 ? 2 : 4));
}

// (N, P, R) the row kernel is instantiated for (bf16 I/O) besides N 128, P 64 at R 1, 2, 4:
// R 8 only where its LDS (the rank rows and the per-wave y partials) fits
bool rows_kernel_sizes(int N, int P, int R) {
    const bool np = (N == 64 || N == 128 || N == 256) && (P == 32 || P == 64 || P == 128);
    return np && (R == 1 || R == 2 || R == 3 || R == 4 || (R == 8 && N * P <= 128 * 64));
}

// the step's prologue arguments (zeros when the step takes its inputs as given)
DecodePrologue pro_of(const DecodeArgs& a) { return a.pro ? *a.pro : DecodePrologue{}; }

// threads per workgroup: 2 row pairs per thread at R 1, one at R 2, 4 (as for
// N 128, P 64), at most 1024 (512 took 11% longer at N 256 and at P 128)
template <typename T, int R, int N, int P, bool PRO>
hipError_t launch_rows(const DecodeArgs& a, dim3 grid, T* cB, T* cx, const T* x, const T* B, const T* C, T* y) {
    constexpr int per = R == 1 ? 16 : 8;  // state floats per thread
    constexpr int want = N * P / per, cap = 1024;
    constexpr int NTH = want < cap ? want : cap;
    hipLaunchKernelGGL((decode_rows_kernel<T, R, NTH, N, P, PRO>), grid, dim3(NTH), 0, a.stream, a.h, cB, cx,
                       parity_words(a), a.rev, pro_of(a), x, a.dt, a.A, a.omega, a.lam, B, C, a.D, y, a.b, a.H, a.G);
    return hipGetLastError();
}

template <typename T, int N, int P, bool PRO>
hipError_t launch_rows_r(const DecodeArgs& a, dim3 grid, T* cB, T* cx, const T* x, const T* B, const T* C, T* y) {
    switch (a.R) {
        case 1: return launch_rows<T, 1, N, P, PRO>(a, grid, cB, cx, x, B, C, y);
        case 2: return launch_rows<T, 2, N, P, PRO>(a, grid, cB, cx, x, B, C, y);
        case 3: return launch_rows<T, 3, N, P, PRO>(a, grid, cB, cx, x, B, C, y);
        case 4: return launch_rows<T, 4, N, P, PRO>(a, grid, cB, cx, x, B, C, y);
        case 8:
            if constexpr (N * P <= 128 * 64) return launch_rows<T, 8, N, P, PRO>(a, grid, cB, cx, x, B, C, y);
            break;
    }
    return hipErrorInvalidValue;
}

template <typename T, bool PRO>
hipError_t launch_rows_sized(const DecodeArgs& a, dim3 grid, T* cB, T* cx, const T* x, const T* B, const T* C, T* y) {
#define M3_ROWS(NN, PP) \
    if (a.N == NN && a.P == PP) return launch_rows_r<T, NN, PP, PRO>(a, grid, cB, cx, x, B, C, y);
    M3_ROWS(64, 32) M3_ROWS(64, 64) M3_ROWS(64, 128)
    M3_ROWS(128, 32) M3_ROWS(128, 64) M3_ROWS(128, 128)
    M3_ROWS(256, 32) M3_ROWS(256, 64) M3_ROWS(256, 128)
#undef M3_ROWS
    return hipErrorInvalidValue;
}

template <bool PRO>
using MfmaKern = void (*)(float*, bf16_t*, bf16_t*, unsigned*, int, DecodePrologue, const bf16_t*, const float*,
                          const float*, const float*, const float*, const bf16_t*, const bf16_t*, const float*,
                          bf16_t*, int64_t, int, int);

// R 2-4 and 8 (fused step included) on the 32 x 32 kernel.
template <int N, bool PRO>
MfmaKern<PRO> mfma_kernel_for(int R) {
    return R == 2 ? decode_mfma32_kernel<2, N, PRO>
         : R == 3 ? decode_mfma32_kernel<3, N, PRO>
         : R == 4 ? decode_mfma32_kernel<4, N, PRO>
                  : decode_mfma32_kernel<8, N, PRO>;
}

template <typename T, bool PRO>
hipError_t launch_t(const DecodeArgs& a) {
    const dim3 grid(unsigned(a.b * a.H));
    T* cB = static_cast<T*>(a.carry_B);
    T* cx = static_cast<T*>(a.carry_x);
    const T* x = static_cast<const T*>(a.x);
    const T* B = static_cast<const T*>(a.B);
    const T* C = static_cast<const T*>(a.C);
    T* y = static_cast<T*>(a.y);
    if constexpr (std::is_same<T, bf16_t>::value) {
        if ((a.N == 64 || a.N == 128) && a.P == 64 && ((a.R >= 2 && a.R <= 4) || a.R == 8)) {
            // R 3 runs with a zero fourth rank slot (the staging zero-fills ranks past R); at
            // N 256 the 64 state values per lane spill (358 us against the row kernel's)
            const auto kern = a.N == 64 ? mfma_kernel_for<64, PRO>(a.R) : mfma_kernel_for<128, PRO>(a.R);
            hipLaunchKernelGGL(kern, grid, dim3(256), 0, a.stream, a.h, cB, cx, parity_words(a), a.rev, pro_of(a), x,
                               a.dt, a.A, a.omega, a.lam, B, C, a.D, y, a.b, a.H, a.G);
            return hipGetLastError();
        }
    }
    if (a.N == 128 && a.P == 64 && (a.R == 1 || a.R == 2 || a.R == 4)) {
        auto kern = a.R == 1 ? decode_rows_kernel<T, 1, M3_DECODE_THREADS_R1, 128, 64, PRO>
                  : a.R == 2 ? decode_rows_kernel<T, 2, M3_DECODE_THREADS_R4, 128, 64, PRO>
                             : decode_rows_kernel<T, 4, M3_DECODE_THREADS_R4, 128, 64, PRO>;
        const int nth = a.R == 1 ? M3_DECODE_THREADS_R1 : M3_DECODE_THREADS_R4;
        hipLaunchKernelGGL(kern, grid, dim3(nth), 0, a.stream, a.h, cB, cx, parity_words(a), a.rev, pro_of(a), x,
                           a.dt, a.A, a.omega, a.lam, B, C, a.D, y, a.b, a.H, a.G);
    } else {
        if constexpr (std::is_same<T, bf16_t>::value) {
            // other state sizes, head dims and ranks (bf16 I/O): the same kernel, instantiated per (N, P, R)
            if (rows_kernel_sizes(a.N, a.P, a.R))
                return launch_rows_sized<T, PRO>(a, grid, cB, cx, x, B, C, y);
        }
        // the fused step keeps B_t and C_t in LDS: [2][R][N] fp32
        const size_t lds = PRO ? size_t(2) * a.R * a.N * sizeof(float) : 0;
        if (PRO && int64_t(a.R) * a.N > kDecodeFusedGenericRN) return hipErrorInvalidValue;
        hipLaunchKernelGGL((decode_generic_kernel<T, PRO>), grid, dim3(kThreads), lds, a.stream, a.h, cB, cx,
                           parity_words(a), a.rev, pro_of(a), x, a.dt, a.A, a.omega, a.lam, B, C, a.D, y, a.b, a.H,
                           a.G, a.P, a.N, a.R);
    }
    return hipGetLastError();
}

// carry[b][h] = src[b][h / (H / G)] (rows of `words` 32-bit words), or zero
__global__ void carry_init_kernel(uint32_t* __restrict__ carry, const uint32_t* __restrict__ src, int64_t nb, int H,
                                  int G, int words) {
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / H;
    const int h = int(bh % H);
    const uint32_t* s = src ? src + (b * G + h / (H / G)) * int64_t(words) : nullptr;
    for (int e = threadIdx.x; e < words; e += blockDim.x) carry[bh * int64_t(words) + e] = s ? s[e] : 0u;
}

}  // namespace

hipError_t launch_carry_init(void* carry, const void* src, int64_t b, int H, int G, int64_t row_bytes,
                             hipStream_t s) {
    if (b * H == 0) return hipSuccess;
    if (b * H > 0x7fffffff || row_bytes % 4 || row_bytes / 4 > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(carry_init_kernel, dim3(unsigned(b * H)), dim3(256), 0, s, static_cast<uint32_t*>(carry),
                       static_cast<const uint32_t*>(src), b, H, G, int(row_bytes / 4));
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a) {
    if (a.b * a.H > 0x7fffffff) return hipErrorInvalidValue;
    if (a.pro) return a.io == M3_BF16 ? launch_t<bf16_t, true>(a) : launch_t<float, true>(a);
    return a.io == M3_BF16 ? launch_t<bf16_t, false>(a) : launch_t<float, false>(a);
}

}  // namespace m3
