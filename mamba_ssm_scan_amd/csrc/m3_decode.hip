// m3_decode.hip -- one recurrent step of the Mamba-3 SSM for every (batch, head).
//
// Per (b, h), with alpha = e^{dt A}, gamma = lambda dt, delta = (1 - lambda) dt
// (exponential-trapezoidal rule, "复值SSM × 广义梯形离散 × MIMO，线性模型的全面重构"
// §2.2) and the rotation of pair k by +dt*omega_k (complex state, same digest §2.1):
//
//   g   = h + delta * B_prev x_prev^T            (previous token, from the carry slot)
//   h'  = alpha * Rot(dt omega) g + gamma * B x^T   (rank-R: N x R times R x P, §2.3)
//   y   = h'^T C + D x
//
// The fp32 state is read and written once (the step is bound by that traffic:
// "Mamba-3架构技术解析：新一代语言建模的范式转移" §2.3 on decode being state-I/O
// bound). The current (B, x) is copied into the other carry slot for the next
// step; slots alternate, so no workgroup overwrites a value another one of the
// same launch still reads (B is shared by the H/G heads of a group).
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

// Threads per workgroup of the N = 128, P = 64 kernel, per rank class.
#ifndef M3_DECODE_THREADS_R1
#define M3_DECODE_THREADS_R1 512
#endif
#ifndef M3_DECODE_THREADS_R4
#define M3_DECODE_THREADS_R4 1024
#endif

// N in {64, 128, 256}, P in {32, 64, 128}: with QP = P / 4 column quads per
// row, thread (kk, q), q = tid % QP, owns rows (2k, 2k+1), k = kk + (NTH/QP)*it,
// it < (N/2) / (NTH/QP), and columns 4q..4q+3, loaded and stored as float4 (a
// wave covers 64/QP row segments of P floats per access).
template <typename T, int R, int NTH, int N, int P>
__global__ void __launch_bounds__(NTH)
decode_rows_kernel(float* __restrict__ hstate, T* __restrict__ carry_B, T* __restrict__ carry_x, int rd_slot,
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
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / H;
    const int h = int(bh % H);
    const int g = h / (H / G);
    const int64_t bg = b * G + g;
    float* hs = hstate + bh * (N * P);
    const int q = tid % QP, kk = tid / QP;

    float4 v0[IT], v1[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int k = kk + KS * it;
        v0[it] = *reinterpret_cast<const float4*>(hs + (2 * k) * P + 4 * q);
        v1[it] = *reinterpret_cast<const float4*>(hs + (2 * k + 1) * P + 4 * q);
    }

    const T* Bt = B + bg * (R * N);
    const T* Ct = C + bg * (R * N);
    const T* Bp = carry_B + (int64_t(rd_slot) * nb * G + bg) * (R * N);
    const T* xt = x + bh * (R * P);
    const T* xp = carry_x + (int64_t(rd_slot) * nb * H + bh) * (R * P);
    for (int e = tid; e < R * N; e += NTH) {
        (&sB[0][0])[e] = Io<T>::load(Bt, e);
        (&sBp[0][0])[e] = Io<T>::load(Bp, e);
        (&sC[0][0])[e] = Io<T>::load(Ct, e);
    }
    for (int e = tid; e < R * P; e += NTH) {
        (&sx[0][0])[e] = Io<T>::load(xt, e);
        (&sxp[0][0])[e] = Io<T>::load(xp, e);
    }
    const float d = dt[bh], lm = lam_at(lam, bh);
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

    // this token becomes the carry of the next step
    const int wr = rd_slot ^ 1;
    for (int e = tid; e < R * P; e += NTH) carry_x[(int64_t(wr) * nb * H + bh) * (R * P) + e] = xt[e];
    if (h % (H / G) == 0)
        for (int e = tid; e < R * N; e += NTH) carry_B[(int64_t(wr) * nb * G + bg) * (R * N) + e] = Bt[e];
}

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ floatx4 mfma_k16(u32x2 a, u32x2 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(shortx4, a), __builtin_bit_cast(shortx4, b), c,
                                                     0, 0, 0);
}
// two floats -> packed bf16 (round to nearest even)
__device__ __forceinline__ unsigned pk_bf16(float lo, float hi) {
    bf16x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(unsigned, v);
}
__device__ __forceinline__ float bf_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// bf16 I/O, N in {64, 128}, P = 64, R in {2, 3, 4, 8}: the rank-R contractions on MFMA
// (v_mfma_f32_16x16x16_bf16). One 256-thread workgroup per (b, h); wave w owns
// state columns 16 w .. 16 w + 15 and all 128 rows. In row tile nt, lane
// (l16, g4) holds rows 16 nt + 4 g4 .. + 3 of column 16 w + l16: two whole
// rotation pairs, and exactly the accumulator layout of the MFMA, so
//   U[n][p]  = sum_r B[r][n] x[r][p]      (A: B^T, rows n, k = r; B: x, k = r,
//   Up[n][p] = the same for the previous token   cols p; k = R..15 are zero)
// land in the lanes that own h[n][p], and
//   y[r][p] += sum_n C[r][n] h'[n][p]      (A: C, rows r (zero past R), k = n;
//                                           B: h', k = n, cols p)
// takes the lane's 4 new state values as its B operand. h' goes in as two bf16
// terms (hi + lo), which keeps y at fp32 accuracy; the products of bf16 inputs
// in U and Up are exact. No cross-lane reduction is left.
template <int R, int N>
__global__ void __launch_bounds__(256)
decode_mfma_kernel(float* __restrict__ hstate, bf16_t* __restrict__ carry_B, bf16_t* __restrict__ carry_x,
                   int rd_slot, const bf16_t* __restrict__ x, const float* __restrict__ dt,
                   const float* __restrict__ A, const float* __restrict__ omega, const float* __restrict__ lam,
                   const bf16_t* __restrict__ B, const bf16_t* __restrict__ C, const float* __restrict__ D,
                   bf16_t* __restrict__ y, int64_t nb, int H, int G) {
    constexpr int P = 64, K = N / 2, CS_ = N + 4, NT = N / 16;  // NT row tiles
    // rank slots: 4, or 8 at R above 4 (k = 4 g4 + 0..3 of the K = 16 MFMA, lanes g4 < RS / 4)
    constexpr int RS = R <= 4 ? 4 : 8;
    __shared__ __attribute__((aligned(16))) uint16_t sBt[N][RS];   // B^T: ranks contiguous, zero past R
    __shared__ __attribute__((aligned(16))) uint16_t sBpt[N][RS];  // B_prev^T
    __shared__ __attribute__((aligned(16))) uint16_t sXt[P][RS];   // x^T
    __shared__ __attribute__((aligned(16))) uint16_t sXpt[P][RS];  // x_prev^T
    __shared__ __attribute__((aligned(16))) uint16_t sC[R][CS_];  // C rows (padded: no bank conflicts)
    __shared__ __attribute__((aligned(16))) float sCS[K][2];      // alpha * (cos, sin) of pair k

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / H;
    const int h = int(bh % H);
    const int64_t bg = b * G + h / (H / G);
    float* hs = hstate + bh * (N * P);
    const int p = 16 * w + l16;

    float st[NT][4];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e) st[nt][e] = hs[(16 * nt + 4 * g4 + e) * P + p];

    const uint16_t* Bt = reinterpret_cast<const uint16_t*>(B) + bg * (R * N);
    const uint16_t* Ct = reinterpret_cast<const uint16_t*>(C) + bg * (R * N);
    const uint16_t* Bp = reinterpret_cast<const uint16_t*>(carry_B) + (int64_t(rd_slot) * nb * G + bg) * (R * N);
    const uint16_t* xt = reinterpret_cast<const uint16_t*>(x) + bh * (R * P);
    const uint16_t* xp = reinterpret_cast<const uint16_t*>(carry_x) + (int64_t(rd_slot) * nb * H + bh) * (R * P);
    for (int e = tid; e < RS * (N / 2); e += 256) {  // rank r, pair of rows (2 j, 2 j + 1): one 32-bit load
        const int r = e / (N / 2), j = e % (N / 2);
        const unsigned vb = r < R ? reinterpret_cast<const unsigned*>(Bt + r * N)[j] : 0u;
        const unsigned vp = r < R ? reinterpret_cast<const unsigned*>(Bp + r * N)[j] : 0u;
        sBt[2 * j][r] = uint16_t(vb);
        sBt[2 * j + 1][r] = uint16_t(vb >> 16);
        sBpt[2 * j][r] = uint16_t(vp);
        sBpt[2 * j + 1][r] = uint16_t(vp >> 16);
    }
    for (int e = tid; e < RS * (P / 2); e += 256) {  // rank r, pair of columns: one 32-bit load
        const int r = e / (P / 2), j = e % (P / 2);
        const unsigned vx = r < R ? reinterpret_cast<const unsigned*>(xt + r * P)[j] : 0u;
        const unsigned vp = r < R ? reinterpret_cast<const unsigned*>(xp + r * P)[j] : 0u;
        sXt[2 * j][r] = uint16_t(vx);
        sXt[2 * j + 1][r] = uint16_t(vx >> 16);
        sXpt[2 * j][r] = uint16_t(vp);
        sXpt[2 * j + 1][r] = uint16_t(vp >> 16);
    }
    for (int e = tid; e < R * (N / 2); e += 256)
        reinterpret_cast<unsigned*>(&sC[e / (N / 2)][0])[e % (N / 2)] = reinterpret_cast<const unsigned*>(Ct)[e];
    const float d = dt[bh], lm = lam_at(lam, bh);
    const float alpha = expf(d * A[h]);
    const float gamma = lm * d, delta = (1.f - lm) * d;
    if (tid < K) {
        float sn, cs;
        sincos_step(d * om_at(omega, int64_t(h) * K + tid), &sn, &cs);
        sCS[tid][0] = alpha * cs;
        sCS[tid][1] = alpha * sn;
    }
    __syncthreads();

    const u32x2 zero = {0u, 0u};
    const bool kin = g4 < RS / 4;  // this lane's k group holds ranks 4 g4 .. 4 g4 + 3
    const int ko = RS == 4 ? 0 : 4 * g4;
    const u32x2 xo = kin ? *reinterpret_cast<const u32x2*>(&sXt[p][ko]) : zero;
    const u32x2 xpo = kin ? *reinterpret_cast<const u32x2*>(&sXpt[p][ko]) : zero;
    const int rc = l16 < R ? l16 : 0;
    floatx4 yacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
    for (int nt = 0; nt < NT; ++nt) {
        const int n0 = 16 * nt;
        const u32x2 ab = *reinterpret_cast<const u32x2*>(&sBt[n0 + l16][ko]);
        const u32x2 abp = *reinterpret_cast<const u32x2*>(&sBpt[n0 + l16][ko]);
        const floatx4 U = mfma_k16(kin ? ab : zero, xo, floatx4{0.f, 0.f, 0.f, 0.f});
        const floatx4 Up = mfma_k16(kin ? abp : zero, xpo, floatx4{0.f, 0.f, 0.f, 0.f});
        // pairs 8 nt + 2 g4 (rows e = 0, 1) and 8 nt + 2 g4 + 1 (rows e = 2, 3)
        const floatx4 cs = *reinterpret_cast<const floatx4*>(&sCS[8 * nt + 2 * g4][0]);
        float nv[4];
#pragma unroll
        for (int hp = 0; hp < 2; ++hp) {
            const float c = cs[2 * hp], sn = cs[2 * hp + 1];
            const float g0 = st[nt][2 * hp] + delta * Up[2 * hp];
            const float g1 = st[nt][2 * hp + 1] + delta * Up[2 * hp + 1];
            nv[2 * hp] = (c * g0 - sn * g1) + gamma * U[2 * hp];
            nv[2 * hp + 1] = (sn * g0 + c * g1) + gamma * U[2 * hp + 1];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) hs[(n0 + 4 * g4 + e) * P + p] = nv[e];
        const unsigned h01 = pk_bf16(nv[0], nv[1]), h23 = pk_bf16(nv[2], nv[3]);
        const u32x2 hi = {h01, h23};
        const u32x2 lo = {pk_bf16(nv[0] - bf_lo(h01), nv[1] - bf_hi(h01)),
                          pk_bf16(nv[2] - bf_lo(h23), nv[3] - bf_hi(h23))};
        const u32x2 cv = *reinterpret_cast<const u32x2*>(&sC[rc][n0 + 4 * g4]);
        const u32x2 ac = l16 < R ? cv : zero;
        yacc = mfma_k16(ac, hi, yacc);
        yacc = mfma_k16(ac, lo, yacc);
    }
    // yacc lane (g4 = 0) holds y[r = e][p]
    if constexpr (RS == 4) {  // yacc lane (g4 = 0) holds y[r = e][p]
        if (g4 == 0) {
            const float Dh = D[h];
#pragma unroll
            for (int e = 0; e < R; ++e) {
                const float xv = __uint_as_float(unsigned(sXt[p][e]) << 16);
                Io<bf16_t>::store(y, bh * (R * P) + e * P + p, yacc[e] + Dh * xv);
            }
        }
    } else if (4 * g4 < R) {  // lane (l16, g4) holds y[r = 4 g4 + e][p]
        const float Dh = D[h];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * g4 + e;
            if (r >= R) continue;
            const float xv = __uint_as_float(unsigned(sXt[p][r]) << 16);
            Io<bf16_t>::store(y, bh * (R * P) + r * P + p, yacc[e] + Dh * xv);
        }
    }

    // this token becomes the carry of the next step
    const int wr = rd_slot ^ 1;
    for (int e = tid; e < R * P; e += 256) carry_x[(int64_t(wr) * nb * H + bh) * (R * P) + e] = x[bh * (R * P) + e];
    if (h % (H / G) == 0)
        for (int e = tid; e < R * N; e += 256)
            carry_B[(int64_t(wr) * nb * G + bg) * (R * N) + e] = B[bg * (R * N) + e];
}

// Any sizes: thread loops over (pair k, column p); y is a second pass over the new state.
template <typename T>
__global__ void __launch_bounds__(kThreads)
decode_generic_kernel(float* __restrict__ hstate, T* __restrict__ carry_B, T* __restrict__ carry_x, int rd_slot,
                      const T* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
                      const float* __restrict__ omega, const float* __restrict__ lam, const T* __restrict__ B,
                      const T* __restrict__ C, const float* __restrict__ D, T* __restrict__ y, int64_t nb, int H,
                      int G, int P, int N, int R) {
    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / H;
    const int h = int(bh % H);
    const int g = h / (H / G);
    const int64_t bg = b * G + g;
    const int K = N / 2;
    float* hs = hstate + bh * int64_t(N) * P;
    const T* Bt = B + bg * int64_t(R) * N;
    const T* Ct = C + bg * int64_t(R) * N;
    const T* Bp = carry_B + (int64_t(rd_slot) * nb * G + bg) * int64_t(R) * N;
    const T* xt = x + bh * int64_t(R) * P;
    const T* xp = carry_x + (int64_t(rd_slot) * nb * H + bh) * int64_t(R) * P;
    const float d = dt[bh], lm = lam_at(lam, bh);
    const float alpha = expf(d * A[h]);
    const float gamma = lm * d, delta = (1.f - lm) * d;

    for (int e = tid; e < K * P; e += kThreads) {
        const int k = e / P, p = e % P;
        float up0 = 0.f, up1 = 0.f, u0 = 0.f, u1 = 0.f;
        for (int r = 0; r < R; ++r) {
            const float xpv = Io<T>::load(xp, int64_t(r) * P + p), xv = Io<T>::load(xt, int64_t(r) * P + p);
            up0 += Io<T>::load(Bp, int64_t(r) * N + 2 * k) * xpv;
            up1 += Io<T>::load(Bp, int64_t(r) * N + 2 * k + 1) * xpv;
            u0 += Io<T>::load(Bt, int64_t(r) * N + 2 * k) * xv;
            u1 += Io<T>::load(Bt, int64_t(r) * N + 2 * k + 1) * xv;
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
        for (int n = 0; n < N; ++n) s += hs[int64_t(n) * P + p] * Io<T>::load(Ct, int64_t(r) * N + n);
        Io<T>::store(y, bh * int64_t(R) * P + e, s + Dh * Io<T>::load(xt, e));
    }
    const int wr = rd_slot ^ 1;
    for (int e = tid; e < R * P; e += kThreads) carry_x[(int64_t(wr) * nb * H + bh) * int64_t(R) * P + e] = xt[e];
    if (h % (H / G) == 0)
        for (int e = tid; e < R * N; e += kThreads)
            carry_B[(int64_t(wr) * nb * G + bg) * int64_t(R) * N + e] = Bt[e];
}

// (N, P, R) the row kernel is instantiated for (bf16 I/O) besides N 128, P 64 at R 1, 2, 4:
// R 8 only where its LDS (the rank rows and the per-wave y partials) fits
bool rows_kernel_sizes(int N, int P, int R) {
    const bool np = (N == 64 || N == 128 || N == 256) && (P == 32 || P == 64 || P == 128);
    return np && (R == 1 || R == 2 || R == 3 || R == 4 || (R == 8 && N * P <= 128 * 64));
}

// threads per workgroup: 2 row pairs per thread at R 1, one at R 2, 4 (as for
// N 128, P 64), at most 1024 (512 took 11% longer at N 256 and at P 128)
template <typename T, int R, int N, int P>
hipError_t launch_rows(const DecodeArgs& a, dim3 grid, T* cB, T* cx, const T* x, const T* B, const T* C, T* y) {
    constexpr int per = R == 1 ? 16 : 8;  // state floats per thread
    constexpr int want = N * P / per, cap = 1024;
    constexpr int NTH = want < cap ? want : cap;
    hipLaunchKernelGGL((decode_rows_kernel<T, R, NTH, N, P>), grid, dim3(NTH), 0, a.stream, a.h, cB, cx, a.rd_slot, x,
                       a.dt, a.A, a.omega, a.lam, B, C, a.D, y, a.b, a.H, a.G);
    return hipGetLastError();
}

template <typename T, int N, int P>
hipError_t launch_rows_r(const DecodeArgs& a, dim3 grid, T* cB, T* cx, const T* x, const T* B, const T* C, T* y) {
    switch (a.R) {
        case 1: return launch_rows<T, 1, N, P>(a, grid, cB, cx, x, B, C, y);
        case 2: return launch_rows<T, 2, N, P>(a, grid, cB, cx, x, B, C, y);
        case 3: return launch_rows<T, 3, N, P>(a, grid, cB, cx, x, B, C, y);
        case 4: return launch_rows<T, 4, N, P>(a, grid, cB, cx, x, B, C, y);
        case 8:
            if constexpr (N * P <= 128 * 64) return launch_rows<T, 8, N, P>(a, grid, cB, cx, x, B, C, y);
            break;
    }
    return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_rows_sized(const DecodeArgs& a, dim3 grid, T* cB, T* cx, const T* x, const T* B, const T* C, T* y) {
#define M3_ROWS(NN, PP) \
    if (a.N == NN && a.P == PP) return launch_rows_r<T, NN, PP>(a, grid, cB, cx, x, B, C, y);
    M3_ROWS(64, 32) M3_ROWS(64, 64) M3_ROWS(64, 128)
    M3_ROWS(128, 32) M3_ROWS(128, 64) M3_ROWS(128, 128)
    M3_ROWS(256, 32) M3_ROWS(256, 64) M3_ROWS(256, 128)
#undef M3_ROWS
    return hipErrorInvalidValue;
}

template <typename T>
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
            using K = void (*)(float*, bf16_t*, bf16_t*, int, const bf16_t*, const float*, const float*,
                               const float*, const float*, const bf16_t*, const bf16_t*, const float*, bf16_t*,
                               int64_t, int, int);
            K kern = a.N == 64 ? (a.R == 2   ? decode_mfma_kernel<2, 64>
                                  : a.R == 3 ? decode_mfma_kernel<3, 64>
                                  : a.R == 4 ? decode_mfma_kernel<4, 64>
                                             : decode_mfma_kernel<8, 64>)
                               : (a.R == 2   ? decode_mfma_kernel<2, 128>
                                  : a.R == 3 ? decode_mfma_kernel<3, 128>
                                  : a.R == 4 ? decode_mfma_kernel<4, 128>
                                             : decode_mfma_kernel<8, 128>);
            hipLaunchKernelGGL(kern, grid, dim3(256), 0, a.stream, a.h, cB, cx, a.rd_slot, x, a.dt, a.A, a.omega,
                               a.lam, B, C, a.D, y, a.b, a.H, a.G);
            return hipGetLastError();
        }
    }
    if (a.N == 128 && a.P == 64 && (a.R == 1 || a.R == 2 || a.R == 4)) {
        auto kern = a.R == 1 ? decode_rows_kernel<T, 1, M3_DECODE_THREADS_R1, 128, 64>
                  : a.R == 2 ? decode_rows_kernel<T, 2, M3_DECODE_THREADS_R4, 128, 64>
                             : decode_rows_kernel<T, 4, M3_DECODE_THREADS_R4, 128, 64>;
        const int nth = a.R == 1 ? M3_DECODE_THREADS_R1 : M3_DECODE_THREADS_R4;
        hipLaunchKernelGGL(kern, grid, dim3(nth), 0, a.stream, a.h, cB, cx, a.rd_slot, x, a.dt, a.A,
                           a.omega, a.lam, B, C, a.D, y, a.b, a.H, a.G);
    } else {
        if constexpr (std::is_same<T, bf16_t>::value) {
            // other state sizes, head dims and ranks (bf16 I/O): the same kernel, instantiated per (N, P, R)
            if (rows_kernel_sizes(a.N, a.P, a.R))
                return launch_rows_sized<T>(a, grid, cB, cx, x, B, C, y);
        }
        hipLaunchKernelGGL(decode_generic_kernel<T>, grid, dim3(kThreads), 0, a.stream, a.h, cB, cx, a.rd_slot, x,
                           a.dt, a.A, a.omega, a.lam, B, C, a.D, y, a.b, a.H, a.G, a.P, a.N, a.R);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a) {
    if (a.b * a.H > 0x7fffffff) return hipErrorInvalidValue;
    return a.io == M3_BF16 ? launch_t<bf16_t>(a) : launch_t<float>(a);
}

}  // namespace m3
