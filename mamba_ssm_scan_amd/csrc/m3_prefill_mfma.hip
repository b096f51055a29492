// m3_prefill_mfma.hip -- chunked prefill on bf16 MFMA (gfx950), N = 128, P = 64,
// rank R in {1, 2, 4}, chunk <= 64 tokens, bf16 I/O, fp32 state.
//
// One workgroup walks the chunks of one (batch, head). A chunk of Q tokens has
// Q*R rows rho = i*R + r (token i, rank r), padded to 64*R. With T_i the
// chunk-local cumulative step, S_i = A T_i and Phi_{i,k} = omega_k T_i:
//
//   y_rho = e^{S_i} C~_rho^T g  +  sum_{rho' : j <= i} M_ij (C~_rho . B~_rho') x_rho'  +  D x_rho
//   g'    = Rot(Phi_e) [ e^{S_e} g + sum_rho' w_j B~_rho' x_rho'^T ]
//
// with B~ = Rot(-Phi) B, C~ = Rot(-Phi) C (the complex transition folded into
// B and C as data-dependent RoPE: "复值SSM × 广义梯形离散 × MIMO，线性模型的全面重构",
// §2.1-§2.2), M_ij = e^{S_i-S_j} (gamma_j + [j<i] delta_{j+1}) the decay x
// width-2 convolution mask (same digest, Fig. 2), w_j = e^{S_e-S_j}(gamma_j +
// delta_{j+1}), e the chunk's last token and delta_{j+1} taken from the next
// token (zero past the sequence end). g is the state entering the chunk with
// the previous token's trapezoid term already added; it stays in registers
// (fp32) for the whole walk.
//
// The three contractions run on v_mfma_f32_16x16x32_bf16:
//   scores^T  [rho_j][rho_i] = B~ (A operand, LDS) x C~^T (B operand, registers), K = N
//   y         [rho_i][p]     = (M o scores) (A operand, straight from the score
//                              accumulators) x X (B operand, X^T in LDS), K = rho_j
//             [rho_i][p]    += C~ (A operand, the same registers) x g (g^T in LDS), K = N
//   state     [n][p]        += (w B~)^T (A operand, gathered from LDS) x X, K = rho
// An accumulator lane holds 4 consecutive rows of one column, which is exactly
// half of an A/B operand's 8 consecutive k values: two score tiles form one
// K = 32 operand (the k order inside an MFMA is free as long as A and B agree),
// so the masked scores never leave registers.
#include "m3_device.h"
#include "m3_internal.h"

namespace m3 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int N = 128;   // state rows
constexpr int P = 64;    // head dim
constexpr int K = 64;    // rotation pairs
constexpr int NS = N + 8;  // LDS row stride (bf16 elements) of B~ and g^T
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kInv2Pi = 0.15915494309189535f;

__device__ __forceinline__ floatx4 mfma32(u32x4 a, u32x4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16(u32x2 a, u32x2 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(shortx4, a), __builtin_bit_cast(shortx4, b),
                                                     c, 0, 0, 0);
}
// two floats -> packed bf16 (round to nearest even)
__device__ __forceinline__ unsigned pack2(float lo, float hi) {
    bf16x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(unsigned, v);
}
__device__ __forceinline__ float lo16(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi16(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// rotate the 4 pairs packed in w (8 bf16) by -Phi: (b0, b1) -> (c b0 + s b1, c b1 - s b0)
__device__ __forceinline__ u32x4 rot_neg(u32x4 w, const float2* cs) {
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float b0 = lo16(w[j]), b1 = hi16(w[j]);
        const float2 t = cs[j];
        o[j] = pack2(t.x * b0 + t.y * b1, t.x * b1 - t.y * b0);
    }
    return o;
}

template <int R, int NW>
struct Shape {
    static constexpr int QRP = 64 * R;       // padded rows per chunk
    static constexpr int NT = 64 * NW;       // threads
    static constexpr int XS = QRP + 8;       // LDS row stride (bf16) of X^T
    static constexpr int NSTRIP = QRP / 16;  // 16-row output strips
    static constexpr int SPW = NSTRIP / NW;  // strips per wave
    static constexpr int TPW = 32 / NW;      // 16x16 state tiles per wave
    static_assert(NSTRIP % NW == 0 && 32 % NW == 0 && TPW % 4 == 0, "tiling");
};

// strips are dealt to waves in snake order so every wave gets a similar share
// of the triangular score work
template <int NW>
__device__ __forceinline__ int strip_of(int wave, int si) {
    return si * NW + ((si & 1) ? (NW - 1 - wave) : wave);
}

template <int R, int NW>
__global__ void __launch_bounds__(64 * NW)
prefill_mfma_kernel(const uint16_t* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ Av,
                    const float* __restrict__ omega, const float* __restrict__ lam, const uint16_t* __restrict__ Bm,
                    const uint16_t* __restrict__ Cm, const float* __restrict__ Dv, const float* __restrict__ h0,
                    uint16_t* __restrict__ y, float* __restrict__ h_out, const uint16_t* __restrict__ carry_B,
                    const uint16_t* __restrict__ carry_x, int64_t L, int H, int G, int Q, int64_t n_chunks,
                    int64_t nbh) {
    using S = Shape<R, NW>;
    constexpr int QRP = S::QRP, NT = S::NT, XS = S::XS, SPW = S::SPW, TPW = S::TPW;

    __shared__ __attribute__((aligned(16))) uint16_t sBt[QRP * NS];  // B~ [rho][n]
    __shared__ __attribute__((aligned(16))) uint16_t sXT[P * XS];    // X^T [p][rho]
    __shared__ __attribute__((aligned(16))) uint16_t sGT[P * NS];    // g^T [p][n] (bf16 copy of the state)
    __shared__ __attribute__((aligned(16))) float2 sCS[64 * K];      // (cos, sin)(Phi_{i,k}) [i][k]
    __shared__ float sT[64], sS2[64], sGam[64], sDln[64], sExpS[64], sW[64];
    __shared__ float sOm[K];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;

    // XCD-aware order: the 8 XCDs take blocks round-robin; give each a
    // contiguous run of (b, h) so heads sharing B/C share an L2.
    int64_t bh;
    {
        const int64_t bid = blockIdx.x, q8 = nbh / 8, r8 = nbh % 8;
        const int64_t xcd = bid % 8, slot = bid / 8;
        bh = xcd * q8 + (xcd < r8 ? xcd : r8) + slot;
    }
    const int64_t b = bh / H;
    const int h = int(bh % H);
    const int grp = h / (H / G);
    const float A2 = Av[h] * kLog2e;
    const float Dh = Dv[h];
    for (int k = tid; k < K; k += NT) sOm[k] = omega[int64_t(h) * K + k] * kInv2Pi;

    // ---- initial state g = h0 + delta_0 carry_B^T carry_x, tiles (nt, pt) of this wave
    floatx4 gst[TPW];
    {
        const int64_t t0 = (b * L) * H + h;
        const float dl0 = (1.f - lam[t0]) * dt[t0];
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
            const int u = wave * TPW + m, nt = u >> 2, pt = u & 3;
            const int p = 16 * pt + l16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int n = 16 * nt + 4 * g4 + e;
                float v = h0 ? h0[(bh * N + n) * P + p] : 0.f;
                if (carry_B) {
                    float s = 0.f;
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        s += bf16_to_f32(carry_B[((b * G + grp) * R + r) * N + n]) *
                             bf16_to_f32(carry_x[(bh * R + r) * P + p]);
                    v += dl0 * s;
                }
                gst[m][e] = v;
            }
            *reinterpret_cast<u32x2*>(sGT + p * NS + 16 * nt + 4 * g4) =
                u32x2{pack2(gst[m][0], gst[m][1]), pack2(gst[m][2], gst[m][3])};
        }
    }
    __syncthreads();

    for (int64_t c = 0; c < n_chunks; ++c) {
        const int64_t c0 = c * Q;
        const int nq = int(L - c0 < Q ? L - c0 : Q);  // tokens in this chunk

        // ---- 1. per-token scalars (one wavefront, lane = token)
        if (wave == 0) {
            const int i = lane;
            float d = 0.f, lm = 0.f, dln = 0.f;
            if (i < nq) {
                const int64_t ti = (b * L + c0 + i) * H + h;
                d = dt[ti];
                lm = lam[ti];
                if (c0 + i + 1 < L) dln = (1.f - lam[ti + H]) * dt[ti + H];
            }
            float T = d;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float v = __shfl_up(T, off);
                if (lane >= off) T += v;
            }
            const float S2 = A2 * T;
            const float S2e = __shfl(S2, nq - 1);
            const float gam = lm * d;
            sT[i] = T;
            sS2[i] = S2;
            sGam[i] = gam;
            sDln[i] = dln;
            sExpS[i] = __builtin_amdgcn_exp2f(S2);
            sW[i] = __builtin_amdgcn_exp2f(S2e - S2) * (gam + dln);
        }
        __syncthreads();

        // ---- 2. rotation table (cos, sin)(omega_k T_i), angles in revolutions
        for (int e = tid; e < 64 * K; e += NT) {
            const int i = e / K, k = e % K;
            const float rev = __builtin_amdgcn_fractf(sOm[k] * sT[i]);
            sCS[e] = make_float2(__builtin_amdgcn_cosf(rev), __builtin_amdgcn_sinf(rev));
        }
        __syncthreads();

        // ---- 3. stage B~ and X^T in LDS, C~ strips in registers
        for (int u = tid; u < QRP * 16; u += NT) {
            const int rho = u >> 4, pc = u & 15;
            const int i = rho / R, r = rho % R;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (i < nq)
                v = *reinterpret_cast<const u32x4*>(Bm + (((b * L + c0 + i) * G + grp) * R + r) * N + 8 * pc);
            *reinterpret_cast<u32x4*>(sBt + rho * NS + 8 * pc) = rot_neg(v, sCS + i * K + 4 * pc);
        }
        for (int u = tid; u < QRP * 4; u += NT) {
            const int rp = u >> 3, pc = u & 7;
            const int rho0 = 2 * rp;
            u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
            {
                const int i = rho0 / R, r = rho0 % R;
                if (i < nq) v0 = *reinterpret_cast<const u32x4*>(x + (((b * L + c0 + i) * H + h) * R + r) * P + 8 * pc);
            }
            {
                const int i = (rho0 + 1) / R, r = (rho0 + 1) % R;
                if (i < nq) v1 = *reinterpret_cast<const u32x4*>(x + (((b * L + c0 + i) * H + h) * R + r) * P + 8 * pc);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int p = 8 * pc + 2 * j;
                *reinterpret_cast<unsigned*>(sXT + p * XS + rho0) = (v0[j] & 0xffffu) | (v1[j] << 16);
                *reinterpret_cast<unsigned*>(sXT + (p + 1) * XS + rho0) = (v0[j] >> 16) | (v1[j] & 0xffff0000u);
            }
        }
        u32x4 cr[SPW][4];  // C~ of this wave's strips: row 16s + l16, n = 32 ks + 8 g4 + 0..7
#pragma unroll
        for (int si = 0; si < SPW; ++si) {
            const int rho = 16 * strip_of<NW>(wave, si) + l16;
            const int i = rho / R, r = rho % R;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (i < nq)
                    v = *reinterpret_cast<const u32x4*>(Cm + (((b * L + c0 + i) * G + grp) * R + r) * N + 32 * ks +
                                                        8 * g4);
                cr[si][ks] = rot_neg(v, sCS + i * K + 16 * ks + 4 * g4);
            }
        }
        __syncthreads();

        // ---- 4. outputs of this wave's strips
#pragma unroll
        for (int si = 0; si < SPW; ++si) {
            const int s = strip_of<NW>(wave, si);
            floatx4 acc[4];
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                acc[pt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const u32x4 gb = *reinterpret_cast<const u32x4*>(sGT + (16 * pt + l16) * NS + 32 * ks + 8 * g4);
                    acc[pt] = mfma32(cr[si][ks], gb, acc[pt]);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float f = sExpS[(16 * s + 4 * g4 + e) / R];
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) acc[pt][e] *= f;
            }
            const int ti = (16 * s + l16) / R;  // token of this lane's score column
            const float S2i = sS2[ti];
            for (int jt = 0; jt <= s; jt += 2) {
                const bool two = jt + 1 <= s;
                floatx4 t0 = {0.f, 0.f, 0.f, 0.f}, t1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const u32x4 a0 = *reinterpret_cast<const u32x4*>(sBt + (16 * jt + l16) * NS + 32 * ks + 8 * g4);
                    t0 = mfma32(a0, cr[si][ks], t0);
                }
                if (two) {
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        const u32x4 a1 =
                            *reinterpret_cast<const u32x4*>(sBt + (16 * jt + 16 + l16) * NS + 32 * ks + 8 * g4);
                        t1 = mfma32(a1, cr[si][ks], t1);
                    }
                }
                float m0[4], m1[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int tj0 = (16 * jt + 4 * g4 + e) / R;
                    const float c0f = tj0 > ti ? 0.f
                                               : __builtin_amdgcn_exp2f(S2i - sS2[tj0]) *
                                                     (sGam[tj0] + (tj0 < ti ? sDln[tj0] : 0.f));
                    m0[e] = t0[e] * c0f;
                    const int tj1 = (16 * jt + 16 + 4 * g4 + e) / R;
                    const float c1f = (!two || tj1 > ti) ? 0.f
                                                         : __builtin_amdgcn_exp2f(S2i - sS2[tj1]) *
                                                               (sGam[tj1] + (tj1 < ti ? sDln[tj1] : 0.f));
                    m1[e] = t1[e] * c1f;
                }
                const unsigned p00 = pack2(m0[0], m0[1]), p01 = pack2(m0[2], m0[3]);
                if (two) {
                    const u32x4 pa = {p00, p01, pack2(m1[0], m1[1]), pack2(m1[2], m1[3])};
#pragma unroll
                    for (int pt = 0; pt < 4; ++pt) {
                        const uint16_t* xr = sXT + (16 * pt + l16) * XS + 16 * jt + 4 * g4;
                        const u32x2 xa = *reinterpret_cast<const u32x2*>(xr);
                        const u32x2 xb = *reinterpret_cast<const u32x2*>(xr + 16);
                        acc[pt] = mfma32(pa, u32x4{xa[0], xa[1], xb[0], xb[1]}, acc[pt]);
                    }
                } else {
                    const u32x2 pa = {p00, p01};
#pragma unroll
                    for (int pt = 0; pt < 4; ++pt) {
                        const u32x2 xa = *reinterpret_cast<const u32x2*>(sXT + (16 * pt + l16) * XS + 16 * jt + 4 * g4);
                        acc[pt] = mfma16(pa, xa, acc[pt]);
                    }
                }
            }
            // epilogue: + D x, store the valid rows
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rho = 16 * s + 4 * g4 + e;
                const int i = rho / R, r = rho % R;
                if (i < nq) {
                    uint16_t* yr = y + (((b * L + c0 + i) * H + h) * R + r) * P;
#pragma unroll
                    for (int pt = 0; pt < 4; ++pt) {
                        const int p = 16 * pt + l16;
                        const float xv = bf16_to_f32(sXT[p * XS + rho]);
                        yr[p] = f32_to_bf16(acc[pt][e] + Dh * xv);
                    }
                }
            }
        }
        __syncthreads();  // every wave is done reading g^T

        // ---- 5. state passed to the next chunk
        const int te = nq - 1;
        const float decE = sExpS[te];
#pragma unroll
        for (int m = 0; m < TPW; ++m) gst[m] *= decE;
#pragma unroll
        for (int mr = 0; mr < TPW / 4; ++mr) {
            const int nt = (wave * TPW) / 4 + mr;
            const int n = 16 * nt + l16;
#pragma unroll
            for (int ks = 0; ks < QRP / 32; ++ks) {
                const int rb = 32 * ks + 8 * g4;
                float wv[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) wv[j] = bf16_to_f32(sBt[(rb + j) * NS + n]) * sW[(rb + j) / R];
                const u32x4 a = {pack2(wv[0], wv[1]), pack2(wv[2], wv[3]), pack2(wv[4], wv[5]), pack2(wv[6], wv[7])};
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    const u32x4 xb = *reinterpret_cast<const u32x4*>(sXT + (16 * pt + l16) * XS + rb);
                    gst[mr * 4 + pt] = mfma32(a, xb, gst[mr * 4 + pt]);
                }
            }
        }
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
            const int u = wave * TPW + m, nt = u >> 2, pt = u & 3;
            const int k0 = 8 * nt + 2 * g4;
#pragma unroll
            for (int hp = 0; hp < 2; ++hp) {
                const float2 t = sCS[te * K + k0 + hp];
                const float a0 = gst[m][2 * hp], a1 = gst[m][2 * hp + 1];
                gst[m][2 * hp] = t.x * a0 - t.y * a1;
                gst[m][2 * hp + 1] = t.y * a0 + t.x * a1;
            }
            const int p = 16 * pt + l16;
            *reinterpret_cast<u32x2*>(sGT + p * NS + 16 * nt + 4 * g4) =
                u32x2{pack2(gst[m][0], gst[m][1]), pack2(gst[m][2], gst[m][3])};
        }
        __syncthreads();
    }

    if (h_out) {
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
            const int u = wave * TPW + m, nt = u >> 2, pt = u & 3;
            const int p = 16 * pt + l16;
#pragma unroll
            for (int e = 0; e < 4; ++e) h_out[(bh * N + 16 * nt + 4 * g4 + e) * P + p] = gst[m][e];
        }
    }
}

template <int R, int NW>
hipError_t launch_r(const PrefillArgs& a) {
    const int64_t nbh = a.b * a.H;
    hipLaunchKernelGGL((prefill_mfma_kernel<R, NW>), dim3(unsigned(nbh)), dim3(64 * NW), 0, a.stream,
                       static_cast<const uint16_t*>(a.x), a.dt, a.A, a.omega, a.lam,
                       static_cast<const uint16_t*>(a.B), static_cast<const uint16_t*>(a.C), a.D, a.h0,
                       static_cast<uint16_t*>(a.y), a.h_out, static_cast<const uint16_t*>(a.carry_B),
                       static_cast<const uint16_t*>(a.carry_x), a.L, a.H, a.G, a.chunk, a.plan.n_chunks, nbh);
    return hipGetLastError();
}

}  // namespace

bool mfma_path_supported(int32_t P_, int32_t N_, int32_t R, int32_t chunk, m3_dtype io) {
    return io == M3_BF16 && N_ == N && P_ == P && (R == 1 || R == 2 || R == 4) && chunk >= 1 && chunk <= 64;
}

hipError_t launch_prefill_mfma(const PrefillArgs& a) {
    if (a.b * a.H > 0x7fffffff || a.plan.segments != 1) return hipErrorInvalidValue;
    switch (a.R) {
        case 1: return launch_r<1, 4>(a);
        case 2: return launch_r<2, 4>(a);
        case 4: return launch_r<4, 4>(a);
    }
    return hipErrorInvalidValue;
}

}  // namespace m3
