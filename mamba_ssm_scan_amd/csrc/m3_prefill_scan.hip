// m3_prefill_scan.hip -- prefill as a walk over the tokens with the state in
// registers, for bf16 I/O at the ranks the chunked MFMA kernels are not built
// for (R 5 to 8): N a multiple of 16 up to 256, P a multiple of 16 up to 64.
//
// Each step is the recurrence itself ("复值SSM × 广义梯形离散 × MIMO，线性模型的
// 全面重构" §2.1-§2.3; "Mamba-3架构技术解析" §2.1):
//   g = h + delta_t U_{t-1},  h = alpha_t Rot(dt_t omega) g + gamma_t U_t,
//   y_t = h^T C_t + D x_t,    U_t = B_t x_t^T (rank R),
// with alpha = e^{dt A}, gamma = lambda dt, delta = (1 - lambda) dt.
//
// One workgroup per (b, h): wave w owns state columns 16 w .. + 15 and all the
// row tiles. In row tile nt, lane (l16, g4) holds rows
// 16 nt + 4 g4 .. + 3 of its column (two whole rotation pairs), which is the
// accumulator layout of
// v_mfma_f32_16x16x16_bf16, so
//   U_t[n][p]  = sum_r B_t[r][n] x_t[r][p]   (A: B^T, k = rank; B: x)
// lands in the lanes that own h[n][p], and
//   y_t[r][p]  = sum_n C_t[r][n] h[n][p]     (A: C, k = n; B: the new state)
// takes the lane's four new state values, rounded to bf16, as its B operand
// (as the chunked kernels feed the carried state to their inter-chunk term;
// the products in U are exact). No cross-lane reduction is left. Only one
// operand of each product needs its padding zeroed: x^T past rank R (so the
// A operand of U may hold any finite values there), and the output rows of y
// past R are not stored (so the A operand of y takes a clamped row).
//
// A block of tokens is staged in LDS with one pass of global loads (all of a
// thread's loads issued before its first LDS store): B, x and C as row-major
// copies of their rank rows, alpha (cos, sin) per (token, pair) and gamma,
// delta per token. The operands that need a rank-major layout (B^T, x^T) come
// out of row-major LDS through transposing reads (ds_read_b64_tr_b16: in each
// 16-lane group, lane t addresses 4 values of row t / 4 at column 4 (t % 4);
// lane j receives column j of those 4 rows). Two barriers per block.
#include "m3_device.h"
#include "m3_internal.h"

namespace m3 {
namespace {

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short shortx4_tr __attribute__((ext_vector_type(4)));


constexpr float kInv2Pi = 0.15915494309189535f;

__device__ __forceinline__ u32x2 load_tr(const uint16_t* p) {
    const shortx4_tr v =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) shortx4_tr*)(p));
    return __builtin_bit_cast(u32x2, v);
}
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

// sizes of one instance: NTL row tiles (N <= 16 NTL), RG groups of 4 ranks (R <= 4 RG)
template <int NTL, int RG>
struct ScanShape {
    static constexpr int NT = 256;                              // threads: 4 column groups
    static constexpr int NMAX = 16 * NTL, KMAX = NMAX / 2, RK = 4 * RG;
    static constexpr int NTW = NTL;                             // row tiles per wave
    static constexpr int BT = (NTL == 16 && RG == 2) ? 8 : 16;  // tokens per staged block
    static constexpr int NS = NMAX + 4;                         // B, C row stride (bf16)
    static constexpr int XS = 64 + 4;                           // x row stride (bf16)
    // staging: rows of N / 2 (B, C) or P / 2 (x) 32-bit words, several rows per pass
    static constexpr int WB = NMAX / 2, RPB = NT / WB, MAXB = BT * RK / RPB;
    static constexpr int RPX = NT / 32, MAXX = BT * RK / RPX;
    static constexpr int MAXCS = BT * KMAX / NT;
};

template <int NTL, int RG>
struct ScanLds {
    typedef ScanShape<NTL, RG> S;
    uint16_t B[S::BT][S::RK][S::NS];  // B rank rows of the block's tokens (rows past R zero)
    uint16_t X[S::BT][S::RK][S::XS];  // x rank rows (rows past R zero)
    uint16_t C[S::BT][S::RK][S::NS];  // C rank rows
    float CS[S::BT][S::KMAX][2];        // alpha * (cos, sin) of each pair's step angle
    float GD[S::BT][2];                 // gamma, delta
};

template <int NTL, int RG, bool FULL>
__global__ void __launch_bounds__(256) prefill_scan_kernel(PrefillArgs a) {
    typedef ScanShape<NTL, RG> S;
    constexpr int BT = S::BT, NT = S::NT;
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
    const int N = FULL ? S::NMAX : a.N, P = a.P, R = a.R, K = N / 2, ntl = FULL ? NTL : N / 16;
    const int64_t L = a.L;
    const int cw = w;  // column group
    const int p = 16 * cw + l16;
    const bool active = 16 * cw < P;    // uniform per wave
    const float Ah = a.A[h], Dh = a.D[h];
    const float* omh = a.omega ? a.omega + int64_t(h) * K : nullptr;
    const int64_t rowB = int64_t(a.G) * R * N, rowX = int64_t(a.H) * R * P;  // per-token strides
    const uint16_t* Bg = static_cast<const uint16_t*>(a.B) + (b * L * a.G + g) * int64_t(R) * N;
    const uint16_t* Cg = static_cast<const uint16_t*>(a.C) + (b * L * a.G + g) * int64_t(R) * N;
    const uint16_t* Xg = static_cast<const uint16_t*>(a.x) + (b * L * a.H + h) * int64_t(R) * P;
    uint16_t* Yg = static_cast<uint16_t*>(a.y) + (b * L * a.H + h) * int64_t(R) * P;
    const float* dtg = a.dt + b * L * a.H + h;
    const float* lmg = a.lam ? a.lam + b * L * a.H + h : nullptr;
    const StepIn si = step_in(a.dt_bias, a.raw_steps, h);  // dt and lambda as given, or from raw projections

    // ranks past R stay zero in B^T and x^T for the whole walk
    for (int e = tid; e < int(sizeof(s.B) / 4); e += NT) reinterpret_cast<uint32_t*>(&s.B)[e] = 0u;
    for (int e = tid; e < int(sizeof(s.X) / 4); e += NT) reinterpret_cast<uint32_t*>(&s.X)[e] = 0u;

    // (token j, rank r) of staging row q: j = q / R for q < 128, R <= 8 (exact)
    const unsigned invR = (65536u + unsigned(R) - 1u) / unsigned(R);
    auto delta_at = [&](int64_t t) {  // (1 - lambda) dt of token t, zero past the end
        return t < L ? (1.f - si.lam(lmg, t * a.H)) * si.dt(dtg[t * a.H]) : 0.f;
    };

    // The walk carries g_t = h_t + delta_{t+1} U_t, the state the next step turns:
    //   h_t = alpha_t Rot g_{t-1} + gamma_t U_t,  y_t = h_t^T C_t + D x_t,  g_t = h_t + delta_{t+1} U_t
    // so U_t is formed once. g_0 = h0 + delta_1 U_0 with U_0 from the caller's carry.
    // wave cw holds all row tiles of its 16 columns
    float st[S::NTW][4];
#pragma unroll
    for (int i = 0; i < S::NTW; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int nt = i, n = 16 * nt + 4 * g4 + e;
            st[i][e] = (a.h0 && active && nt < ntl) ? a.h0[(bh * N + n) * int64_t(P) + p] : 0.f;
        }
    const u32x2 zero = {0u, 0u};
    const int gk = g4 < RG ? g4 : 0;  // in-range rank group for the lanes whose operand is zero
    const int rc = l16 < R ? l16 : 0;

    if (a.carry_B) {
        __syncthreads();
        const uint16_t* cb = static_cast<const uint16_t*>(a.carry_B) + (b * a.G + g) * int64_t(R) * N;
        const uint16_t* cx = static_cast<const uint16_t*>(a.carry_x) + bh * int64_t(R) * P;
        for (int e = tid; e < R * (N / 2); e += NT)
            reinterpret_cast<unsigned*>(&s.B[0][e / (N / 2)][0])[e % (N / 2)] = reinterpret_cast<const unsigned*>(cb)[e];
        for (int e = tid; e < R * (P / 2); e += NT)
            reinterpret_cast<unsigned*>(&s.X[0][e / (P / 2)][0])[e % (P / 2)] = reinterpret_cast<const unsigned*>(cx)[e];
        __syncthreads();
        const float d1 = delta_at(0);
        if (active) {
            const u32x2 xv = load_tr(&s.X[0][4 * gk + (l16 >> 2)][16 * cw + 4 * (l16 & 3)]);
            const u32x2 xo = g4 < RG ? xv : zero;
#pragma unroll
            for (int i = 0; i < S::NTW; ++i) {
                const int nt = i;
                if (FULL || nt < ntl) {
                    const u32x2 ab = load_tr(&s.B[0][4 * gk + (l16 >> 2)][16 * nt + 4 * (l16 & 3)]);
                    const floatx4 U = mfma16(ab, xo, floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int e = 0; e < 4; ++e) st[i][e] += d1 * U[e];
                }
            }
        }
    }

    for (int64_t t0 = 0; t0 < L; t0 += BT) {
        const int nt_ = int(L - t0 < BT ? L - t0 : BT);
        // every load of the block first, then the barrier, then the LDS stores
        const int nrow = nt_ * R;
        // 32-bit word offsets from the block's first token (uniform bases)
        const unsigned* Bb = reinterpret_cast<const unsigned*>(Bg + t0 * rowB);
        const unsigned* Cb = reinterpret_cast<const unsigned*>(Cg + t0 * rowB);
        const unsigned* Xb = reinterpret_cast<const unsigned*>(Xg + t0 * rowX);
        const float* db = dtg + t0 * a.H;
        const unsigned wB = unsigned(rowB / 2), wX = unsigned(rowX / 2);
        unsigned vb[S::MAXB], vc[S::MAXB], vx[S::MAXX];
        float dcs[S::MAXCS];
        {
            const int wi = tid % S::WB, rs = tid / S::WB;
#pragma unroll
            for (int u = 0; u < S::MAXB; ++u) {
                const int q = u * S::RPB + rs;
                if (q < nrow && wi < N / 2) {
                    const unsigned j = (unsigned(q) * invR) >> 16, r = unsigned(q) - j * unsigned(R);
                    const unsigned o = j * wB + r * unsigned(N / 2) + unsigned(wi);
                    vb[u] = Bb[o];
                    vc[u] = Cb[o];
                }
            }
            const int xi = tid % 32, xs = tid / 32;
#pragma unroll
            for (int u = 0; u < S::MAXX; ++u) {
                const int q = u * S::RPX + xs;
                if (q < nrow && xi < P / 2) {
                    const unsigned j = (unsigned(q) * invR) >> 16, r = unsigned(q) - j * unsigned(R);
                    vx[u] = Xb[j * wX + r * unsigned(P / 2) + unsigned(xi)];
                }
            }
#pragma unroll
            for (int u = 0; u < S::MAXCS; ++u) {
                const int e = tid + u * NT, j = e / K;
                if (j < nt_) dcs[u] = si.dt(db[unsigned(j) * unsigned(a.H)]);
            }
            __syncthreads();  // every wave is done reading the previous block (its loads are in flight)
#pragma unroll
            for (int u = 0; u < S::MAXB; ++u) {
                const int q = u * S::RPB + rs;
                if (q < nrow && wi < N / 2) {
                    const int j = int((unsigned(q) * invR) >> 16), r = q - j * R;
                    reinterpret_cast<unsigned*>(&s.B[j][r][0])[wi] = vb[u];
                    reinterpret_cast<unsigned*>(&s.C[j][r][0])[wi] = vc[u];
                }
            }
#pragma unroll
            for (int u = 0; u < S::MAXX; ++u) {
                const int q = u * S::RPX + xs;
                if (q < nrow && xi < P / 2) {
                    const int j = int((unsigned(q) * invR) >> 16), r = q - j * R;
                    reinterpret_cast<unsigned*>(&s.X[j][r][0])[xi] = vx[u];
                }
            }
#pragma unroll
            for (int u = 0; u < S::MAXCS; ++u) {
                const int e = tid + u * NT, j = e / K, k = e - j * K;
                if (j < nt_) {
                    const float d = dcs[u];
                    const float al = expf(d * Ah);
                    const float rv = __builtin_amdgcn_fractf(d * om_at(omh, k) * kInv2Pi);
                    s.CS[j][k][0] = al * __builtin_amdgcn_cosf(rv);
                    s.CS[j][k][1] = al * __builtin_amdgcn_sinf(rv);
                }
            }
        }
        if (tid < nt_) {
            const int64_t t = t0 + tid;
            s.GD[tid][0] = si.lam(lmg, t * a.H) * si.dt(dtg[t * a.H]);
            s.GD[tid][1] = delta_at(t + 1);
        }
        __syncthreads();

        for (int j = 0; j < (active ? nt_ : 0); ++j) {
            const float gam = s.GD[j][0], dnx = s.GD[j][1];
            const u32x2 xv = load_tr(&s.X[j][4 * gk + (l16 >> 2)][16 * cw + 4 * (l16 & 3)]);
            const u32x2 xo = g4 < RG ? xv : zero;
            floatx4 yacc[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) yacc[q] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < S::NTW; ++i) {
                const int nt = i;
                if (!FULL && nt >= ntl) continue;
                const int n0 = 16 * nt;
                const u32x2 ab = load_tr(&s.B[j][4 * gk + (l16 >> 2)][n0 + 4 * (l16 & 3)]);
                const floatx4 U = mfma16(ab, xo, floatx4{0.f, 0.f, 0.f, 0.f});
                // pairs 8 nt + 2 g4 (rows e = 0, 1) and 8 nt + 2 g4 + 1 (rows e = 2, 3)
                const floatx4 cs = *reinterpret_cast<const floatx4*>(&s.CS[j][(n0 >> 1) + 2 * g4][0]);
                float nv[4];
#pragma unroll
                for (int hp = 0; hp < 2; ++hp) {
                    const float c = cs[2 * hp], sn = cs[2 * hp + 1];
                    const float g0 = st[i][2 * hp], g1 = st[i][2 * hp + 1];
                    nv[2 * hp] = (c * g0 - sn * g1) + gam * U[2 * hp];
                    nv[2 * hp + 1] = (sn * g0 + c * g1) + gam * U[2 * hp + 1];
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) st[i][e] = nv[e] + dnx * U[e];
                const u32x2 hb = {pk_bf16(nv[0], nv[1]), pk_bf16(nv[2], nv[3])};
                const u32x2 ac = *reinterpret_cast<const u32x2*>(&s.C[j][rc][n0 + 4 * g4]);
                yacc[i & 3] = mfma16(ac, hb, yacc[i & 3]);
            }
            // lane (l16, g4) holds this wave's part of y[r = 4 g4 + e][p]
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * g4 + e;
                if (r >= R) continue;
                const float v = (yacc[0][e] + yacc[1][e]) + (yacc[2][e] + yacc[3][e]);
                Yg[(t0 + j) * rowX + r * P + p] = f32_to_bf16(v + Dh * bf16_to_f32(s.X[j][r][p]));
            }
        }
    }

    // after the last token delta_{L+1} = 0, so the carried g is h_L
    if (a.h_out && active)
#pragma unroll
        for (int i = 0; i < S::NTW; ++i) {
            const int nt = i;
            if (FULL || nt < ntl)
#pragma unroll
                for (int e = 0; e < 4; ++e) a.h_out[(bh * N + 16 * nt + 4 * g4 + e) * int64_t(P) + p] = st[i][e];
        }
}

template <int NTL, int RG>
hipError_t launch_ntl_rg(const PrefillArgs& a) {
    const dim3 grid(unsigned(a.b * a.H)), block(256);
    if (a.N == 16 * NTL)
        hipLaunchKernelGGL((prefill_scan_kernel<NTL, RG, true>), grid, block, 0, a.stream, a);
    else
        hipLaunchKernelGGL((prefill_scan_kernel<NTL, RG, false>), grid, block, 0, a.stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_scan(const PrefillArgs& a) {
    if (a.b * a.H > 0x7fffffff) return hipErrorInvalidValue;
    if (!scan_path_supported(a.P, a.N, a.R, a.io)) return hipErrorInvalidValue;
    // one wave per 16 columns: 8 row tiles each up to N 128, 16 up to N 256
    return a.N <= 128 ? launch_ntl_rg<8, 2>(a) : launch_ntl_rg<16, 2>(a);
}

}  // namespace m3
