// m3_prefill_scan.hip -- prefill as a walk over the tokens with the state in
// registers, for bf16 I/O at the sizes the chunked MFMA kernels are not built
// for: N a multiple of 16 up to 256, P a multiple of 16 up to 64, R up to 8.
//
// Each step is the recurrence itself ("复值SSM × 广义梯形离散 × MIMO，线性模型的
// 全面重构" §2.1-§2.3; "Mamba-3架构技术解析" §2.1):
//   g = h + delta_t U_{t-1},  h = alpha_t Rot(dt_t omega) g + gamma_t U_t,
//   y_t = h^T C_t + D x_t,    U_t = B_t x_t^T (rank R),
// with alpha = e^{dt A}, gamma = lambda dt, delta = (1 - lambda) dt.
//
// One 256-thread workgroup per (b, h); wave w owns state columns 16 w .. 16 w + 15.
// In row tile nt, lane (l16, g4) holds rows 16 nt + 4 g4 .. + 3 of column
// 16 w + l16 (two whole rotation pairs), which is the accumulator layout of
// v_mfma_f32_16x16x16_bf16, so
//   U_t[n][p]  = sum_r B_t[r][n] x_t[r][p]   (A: B^T, k = rank; B: x)
// lands in the lanes that own h[n][p], and
//   y_t[r][p]  = sum_n C_t[r][n] h[n][p]     (A: C, k = n; B: the new state)
// takes the lane's four new state values as its B operand, as a bf16 hi + lo
// pair (y keeps fp32 accuracy; the products in U are exact). No cross-lane
// reduction is left. U_{t-1} is carried in registers from the previous step.
//
// A block of tokens is staged in LDS with one pass of global loads: B^T and
// x^T with the ranks of a row contiguous, C row-major, alpha (cos, sin) per
// (token, pair) and gamma, delta per token. Two barriers per block.
#include "m3_device.h"
#include "m3_internal.h"

namespace m3 {
namespace {

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int NT = 256;  // threads: 4 waves, 16 state columns each
constexpr float kInv2Pi = 0.15915494309189535f;

__device__ __forceinline__ floatx4 mfma16(u32x2 a, u32x2 b, floatx4 c) {
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

// sizes of one instance: NTL row tiles (N <= 16 NTL), RG groups of 4 ranks (R <= 4 RG)
template <int NTL, int RG>
struct ScanShape {
    static constexpr int NMAX = 16 * NTL, KMAX = NMAX / 2, RK = 4 * RG;
    static constexpr int BT = (NTL == 16 && RG == 2) ? 8 : 16;  // tokens per staged block
    static constexpr int NS = NMAX + 4;                         // C row stride (bf16)
};

template <int NTL, int RG>
struct ScanLds {
    typedef ScanShape<NTL, RG> S;
    uint16_t B[S::BT][S::NMAX][S::RK];  // B^T of the block's tokens (ranks past R zero)
    uint16_t X[S::BT][64][S::RK];       // x^T
    uint16_t C[S::BT][S::RK][S::NS];    // C rows
    float CS[S::BT][S::KMAX][2];        // alpha * (cos, sin) of each pair's step angle
    float GD[S::BT][2];                 // gamma, delta
};

template <int NTL, int RG>
__global__ void __launch_bounds__(NT) prefill_scan_kernel(PrefillArgs a) {
    typedef ScanShape<NTL, RG> S;
    constexpr int BT = S::BT;
    __shared__ __attribute__((aligned(16))) ScanLds<NTL, RG> s;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    // XCD-aware order: the 8 XCDs take workgroups round-robin; give each a
    // contiguous run of (b, h) so the heads sharing B, C meet in one L2
    const int64_t nbh = a.b * a.H;
    int64_t bh = blockIdx.x;
    if (nbh % 8 == 0) bh = (bh % 8) * (nbh / 8) + bh / 8;
    const int64_t b = bh / a.H;
    const int h = int(bh % a.H);
    const int g = h / (a.H / a.G);
    const int N = a.N, P = a.P, R = a.R, K = N / 2, ntl = N / 16;
    const int64_t L = a.L;
    const int p = 16 * w + l16;
    const bool active = 16 * w < P;  // uniform per wave
    const float Ah = a.A[h], Dh = a.D[h];
    const float* omh = a.omega ? a.omega + int64_t(h) * K : nullptr;
    const uint16_t* Bg = static_cast<const uint16_t*>(a.B);
    const uint16_t* Cg = static_cast<const uint16_t*>(a.C);
    const uint16_t* Xg = static_cast<const uint16_t*>(a.x);
    uint16_t* Yg = static_cast<uint16_t*>(a.y);

    // ranks past R stay zero in B^T and x^T for the whole walk
    for (int e = tid; e < int(sizeof(s.B) / 4); e += NT) reinterpret_cast<uint32_t*>(&s.B)[e] = 0u;
    for (int e = tid; e < int(sizeof(s.X) / 4); e += NT) reinterpret_cast<uint32_t*>(&s.X)[e] = 0u;

    // B rows of one token (rank r, rows 2i, 2i + 1 per 32-bit load) into slot j
    auto stage_bx = [&](int j, const uint16_t* brow, const uint16_t* xrow) {
        for (int e = tid; e < R * (N / 2); e += NT) {
            const int r = e / (N / 2), i = e % (N / 2);
            const unsigned v = reinterpret_cast<const unsigned*>(brow + r * N)[i];
            s.B[j][2 * i][r] = uint16_t(v);
            s.B[j][2 * i + 1][r] = uint16_t(v >> 16);
        }
        for (int e = tid; e < R * (P / 2); e += NT) {
            const int r = e / (P / 2), i = e % (P / 2);
            const unsigned v = reinterpret_cast<const unsigned*>(xrow + r * P)[i];
            s.X[j][2 * i][r] = uint16_t(v);
            s.X[j][2 * i + 1][r] = uint16_t(v >> 16);
        }
    };

    float st[NTL][4], up[NTL][4];
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int n = 16 * nt + 4 * g4 + e;
            st[nt][e] = (a.h0 && active && nt < ntl) ? a.h0[(bh * N + n) * int64_t(P) + p] : 0.f;
            up[nt][e] = 0.f;
        }
    const u32x2 zero = {0u, 0u};

    // U of the token before the first (the caller's carry), else zero
    if (a.carry_B) {
        __syncthreads();
        stage_bx(0, static_cast<const uint16_t*>(a.carry_B) + (b * a.G + g) * int64_t(R) * N,
                 static_cast<const uint16_t*>(a.carry_x) + bh * int64_t(R) * P);
        __syncthreads();
        if (active) {
            const int gc = g4 < RG ? g4 : 0;
            const u32x2 xo = g4 < RG ? *reinterpret_cast<const u32x2*>(&s.X[0][p][4 * gc]) : zero;
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt)
                if (nt < ntl) {
                    const u32x2 ab = g4 < RG ? *reinterpret_cast<const u32x2*>(&s.B[0][16 * nt + l16][4 * gc]) : zero;
                    const floatx4 U = mfma16(ab, xo, floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int e = 0; e < 4; ++e) up[nt][e] = U[e];
                }
        }
    }

    const int rc = l16 < R ? l16 : 0;
    const int gk = g4 < RG ? g4 : 0;  // in-range rank group for the lanes whose operand is zero
    for (int64_t t0 = 0; t0 < L; t0 += BT) {
        const int nt_ = int(L - t0 < BT ? L - t0 : BT);
        __syncthreads();  // the previous block's readers are done
        for (int j = 0; j < nt_; ++j)
            stage_bx(j, Bg + ((b * L + t0 + j) * a.G + g) * int64_t(R) * N,
                     Xg + ((b * L + t0 + j) * a.H + h) * int64_t(R) * P);
        for (int e = tid; e < nt_ * R * (N / 2); e += NT) {
            const int j = e / (R * (N / 2)), q = e % (R * (N / 2)), r = q / (N / 2), i = q % (N / 2);
            reinterpret_cast<unsigned*>(&s.C[j][r][0])[i] =
                reinterpret_cast<const unsigned*>(Cg + ((b * L + t0 + j) * a.G + g) * int64_t(R) * N + r * N)[i];
        }
        for (int e = tid; e < nt_ * K; e += NT) {
            const int j = e / K, k = e % K;
            const float d = a.dt[(b * L + t0 + j) * a.H + h];
            const float al = expf(d * Ah);
            const float rv = __builtin_amdgcn_fractf(d * om_at(omh, k) * kInv2Pi);
            s.CS[j][k][0] = al * __builtin_amdgcn_cosf(rv);
            s.CS[j][k][1] = al * __builtin_amdgcn_sinf(rv);
        }
        if (tid < nt_) {
            const int64_t i = (b * L + t0 + tid) * a.H + h;
            const float d = a.dt[i], lm = lam_at(a.lam, i);
            s.GD[tid][0] = lm * d;
            s.GD[tid][1] = (1.f - lm) * d;
        }
        __syncthreads();
        if (!active) continue;

        for (int j = 0; j < nt_; ++j) {
            const float gam = s.GD[j][0], del = s.GD[j][1];
            const u32x2 xo = g4 < RG ? *reinterpret_cast<const u32x2*>(&s.X[j][p][4 * gk]) : zero;
            floatx4 ya = {0.f, 0.f, 0.f, 0.f}, yb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                if (nt >= ntl) continue;
                const int n0 = 16 * nt;
                const u32x2 ab = g4 < RG ? *reinterpret_cast<const u32x2*>(&s.B[j][n0 + l16][4 * gk]) : zero;
                const floatx4 U = mfma16(ab, xo, floatx4{0.f, 0.f, 0.f, 0.f});
                // pairs 8 nt + 2 g4 (rows e = 0, 1) and 8 nt + 2 g4 + 1 (rows e = 2, 3)
                const floatx4 cs = *reinterpret_cast<const floatx4*>(&s.CS[j][(n0 >> 1) + 2 * g4][0]);
                float nv[4];
#pragma unroll
                for (int hp = 0; hp < 2; ++hp) {
                    const float c = cs[2 * hp], sn = cs[2 * hp + 1];
                    const float g0 = st[nt][2 * hp] + del * up[nt][2 * hp];
                    const float g1 = st[nt][2 * hp + 1] + del * up[nt][2 * hp + 1];
                    nv[2 * hp] = (c * g0 - sn * g1) + gam * U[2 * hp];
                    nv[2 * hp + 1] = (sn * g0 + c * g1) + gam * U[2 * hp + 1];
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    st[nt][e] = nv[e];
                    up[nt][e] = U[e];
                }
                const unsigned h01 = pk_bf16(nv[0], nv[1]), h23 = pk_bf16(nv[2], nv[3]);
                const u32x2 hi = {h01, h23};
                const u32x2 lo = {pk_bf16(nv[0] - bf_lo(h01), nv[1] - bf_hi(h01)),
                                  pk_bf16(nv[2] - bf_lo(h23), nv[3] - bf_hi(h23))};
                const u32x2 cv = *reinterpret_cast<const u32x2*>(&s.C[j][rc][n0 + 4 * g4]);
                const u32x2 ac = l16 < R ? cv : zero;
                if (nt & 1) {
                    yb = mfma16(ac, hi, yb);
                    yb = mfma16(ac, lo, yb);
                } else {
                    ya = mfma16(ac, hi, ya);
                    ya = mfma16(ac, lo, ya);
                }
            }
            // lane (l16, g4) holds y[r = 4 g4 + e][p]
            const int64_t yrow = ((b * L + t0 + j) * a.H + h) * int64_t(R) * P;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * g4 + e;
                if (r < R) {
                    const float xv = bf16_to_f32(s.X[j][p][r]);
                    Yg[yrow + r * P + p] = f32_to_bf16(ya[e] + yb[e] + Dh * xv);
                }
            }
        }
    }

    if (a.h_out && active)
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt)
            if (nt < ntl)
#pragma unroll
                for (int e = 0; e < 4; ++e) a.h_out[(bh * N + 16 * nt + 4 * g4 + e) * int64_t(P) + p] = st[nt][e];
}

template <int NTL, int RG>
hipError_t launch_ntl_rg(const PrefillArgs& a) {
    hipLaunchKernelGGL((prefill_scan_kernel<NTL, RG>), dim3(unsigned(a.b * a.H)), dim3(NT), 0, a.stream, a);
    return hipGetLastError();
}

}  // namespace

bool scan_path_supported(int32_t P, int32_t N, int32_t R, m3_dtype io) {
    return io == M3_BF16 && N % 16 == 0 && N <= 256 && P % 16 == 0 && P <= 64 && R >= 1 && R <= 8;
}

hipError_t launch_prefill_scan(const PrefillArgs& a) {
    if (a.b * a.H > 0x7fffffff) return hipErrorInvalidValue;
    if (!scan_path_supported(a.P, a.N, a.R, a.io)) return hipErrorInvalidValue;
    if (a.N <= 128) return a.R <= 4 ? launch_ntl_rg<8, 1>(a) : launch_ntl_rg<8, 2>(a);
    return a.R <= 4 ? launch_ntl_rg<16, 1>(a) : launch_ntl_rg<16, 2>(a);
}

}  // namespace m3
