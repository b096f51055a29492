// m3_prefill_mfma.hip -- chunked prefill on bf16 MFMA (gfx950), N = 128, P = 64,
// rank R in {1, 2, 4} (R 3 on the R 4 kernel with a zero fourth rank), chunk <= 64
// tokens, bf16 I/O, fp32 state. Other N and
// P (multiples of 8) run as passes of at most 128 state rows and 64 columns,
// zero-padded where a pass holds fewer: B/C rows past the pass's rows and x
// columns past its columns load as zero, so those state entries stay zero and
// add nothing to the scores or outputs (PassArgs below).
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
// The contractions run on v_mfma_f32_16x16x32_bf16:
//   scores^T  [rho_j][rho_i] = B~ (A operand, LDS) x C~^T (B operand, registers), K = N
//   y^T       [p][rho_i]     = X^T (A operand, LDS) x (M o scores^T) (B operand, straight
//                              from the score accumulators), K = rho_j
//             [p][rho_i]    += g^T (A operand, LDS) x C~^T (B operand, the same registers), K = N
//   state     [n][p]        += (w B~)^T (A operand, gathered from LDS) x X, K = rho
// An accumulator lane holds 4 consecutive rows of one column, which is exactly
// half of an A/B operand's 8 consecutive k values: two score tiles form one
// K = 32 operand (the k order inside an MFMA is free as long as A and B agree),
// so the masked scores never leave registers.
//
// The rotation angles are the same for B and C of a token and for all R ranks;
// each (token, pair) angle is evaluated once: the thread that stages a token's
// B rows also turns its C rows (into LDS when they fit, R <= 2), and at R = 4
// the four lanes holding one token's C rows share angles through DPP.
#include <cstdlib>
#include <type_traits>
#include "m3_device.h"
#include "m3_internal.h"
#include "m3_mfma_common.h"

namespace m3 {
namespace {

template <int R_, int NW_>
struct Shape {
    static constexpr int R = R_, NW = NW_;
    static constexpr int LR = R == 1 ? 0 : R == 2 ? 1 : 2;  // log2 R
    static constexpr int QRP = 64 * R;                     // padded rows per chunk
    static constexpr int NT = 64 * NW;                     // threads
    static constexpr int XS = QRP + 8;                     // LDS row stride (bf16) of X^T
    static constexpr int NSTRIP = QRP / 16;                // 16-row output strips
    static constexpr int PTG = NW > NSTRIP ? NW / NSTRIP : 1;  // p-tile groups per strip
    static constexpr int PTW = 4 / PTG;                    // 16-column p tiles per work item
    static constexpr int SPW = NSTRIP * PTG / NW;          // work items (strip, p group) per wave
    static constexpr int TPW = 32 / NW;                    // 16x16 state tiles per wave
    static constexpr bool C_LDS = R <= 2;                  // C~ staged in LDS (else built per strip)
    static constexpr int UPT = 64 * 16 / NT;               // (token, 8-column piece) staging units per thread
    static constexpr int XU = QRP * 4;                     // (row pair, 8 columns) units of X
    static constexpr int XPT = (XU + NT - 1) / NT;         // ... per thread
    static_assert((NSTRIP * PTG) % NW == 0 && 32 % NW == 0 && TPW % 4 == 0 && UPT >= 1, "tiling");
};

// strips are dealt to waves in snake order so every wave gets a similar share
// of the triangular score work
template <int NW>
__device__ __forceinline__ int strip_of(int wave, int si) {
    return si * NW + ((si & 1) ? (NW - 1 - wave) : wave);
}


// Global operands of one chunk, held in registers until they are staged.
template <class S>
struct ChunkRegs {
    float d, l, dn, ln;                    // lane = token: dt, lambda, and of the next token, as loaded
    unsigned ok;                           // bit 0: token in the chunk; bit 1: and a next token exists; bit 2: lambda given
    u32x4 b[S::UPT][S::R];                 // B rows (token, rank) of this thread's units
    u32x4 c[S::C_LDS ? S::UPT : 1][S::R];  // C rows, when staged in LDS
    u32x4 x0[S::XPT], x1[S::XPT];
};

template <class S>
__device__ __forceinline__ void load_chunk(ChunkRegs<S>& cr, const ChunkBase& cb, const float* __restrict__ dt,
                                           const float* __restrict__ lam, int64_t tok0, int64_t L, int64_t c0, int H,
                                           int G, int tid, int lane) {
    constexpr int R = S::R;
    const int nq = cb.nq;
    {
        const int ic = lane < nq ? lane : nq - 1;
        const int64_t ti = (tok0 + ic) * H;
        // kept as loaded and mapped at use (see the staging below); without
        // lambda, dt stands in as a valid address and the value is replaced at use
        const bool has_next = c0 + ic + 1 < L;
        const float* lp = lam ? lam : dt;
        cr.d = dt[ti];
        cr.l = lp[ti];
        cr.dn = dt[has_next ? ti + H : ti];
        cr.ln = lp[has_next ? ti + H : ti];
        cr.ok = (lane < nq ? 1u : 0u) | ((lane < nq && has_next) ? 2u : 0u) | (lam ? 4u : 0u);
    }
    const int pc = tid & 15;
#pragma unroll
    for (int m = 0; m < S::UPT; ++m) {
        const int i = (tid >> 4) + m * (S::NT / 16);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const bool in = 8 * pc < cb.nin && r < cb.rin;
            const int ts = G * cb.rin * cb.nrow;
            cr.b[m][r] = in ? load_tok(cb.B, i, nq, ts, r * cb.nrow + 8 * pc) : u32x4{0u, 0u, 0u, 0u};
            if constexpr (S::C_LDS)
                cr.c[m][r] = in ? load_tok(cb.C, i, nq, ts, r * cb.nrow + 8 * pc) : u32x4{0u, 0u, 0u, 0u};
        }
    }
    const bool xin = 8 * (tid & 7) < cb.pin;
#pragma unroll
    for (int m = 0; m < S::XPT; ++m) {
        if (S::XU % S::NT != 0 && tid + m * S::NT >= S::XU) break;
        const unsigned rho0 = 2u * ((tid >> 3) + m * (S::NT / 8));
        const int i0 = int(rho0 >> S::LR), r0 = int(rho0 & (R - 1));
        const int i1 = int((rho0 + 1) >> S::LR), r1 = int((rho0 + 1) & (R - 1));
        const int ts = H * cb.rin * cb.pcol;
        cr.x0[m] = (xin && r0 < cb.rin) ? load_tok(cb.x, i0, nq, ts, r0 * cb.pcol + 8 * (tid & 7)) : u32x4{0u, 0u, 0u, 0u};
        cr.x1[m] = (xin && r1 < cb.rin) ? load_tok(cb.x, i1, nq, ts, r1 * cb.pcol + 8 * (tid & 7)) : u32x4{0u, 0u, 0u, 0u};
    }
}

// C rows of one 16-row strip in the B-operand layout: row 16 s + l16, n = 32 ks + 8 g4 + 0..7
template <class S>
__device__ __forceinline__ void load_strip_c(u32x4 (&c)[4], const ChunkBase& cb, int s, int G, int lane) {
    const unsigned rho = 16u * s + (lane & 15);
    const int i = int(rho >> S::LR), r = int(rho & (S::R - 1));
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int n0 = 32 * ks + 8 * (lane >> 4);
        c[ks] = (n0 < cb.nin && r < cb.rin) ? load_tok(cb.C, i, cb.nq, G * cb.rin * cb.nrow, r * cb.nrow + n0)
                                            : u32x4{0u, 0u, 0u, 0u};
    }
}

// GEN: the pass described by pa (other sizes, row and column passes); without
// it the problem is exactly N = 128, P = 64 in one pass and pa is not read.
// YM is pa.ym and GP (columns other than 0..63 of P = 64) is part of GEN, both
// at compile time: as run-time values they cost the R 1 kernel 7% and 11%.
template <int R, int NW, bool GEN, int YM, bool GP>
__global__ void __launch_bounds__(64 * NW)
prefill_mfma_kernel(const uint16_t* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ Av,
                    const float* __restrict__ omega, const float* __restrict__ lam, const uint16_t* __restrict__ Bm,
                    const uint16_t* __restrict__ Cm, const float* __restrict__ Dv, const float* __restrict__ h0,
                    uint16_t* __restrict__ y, float* __restrict__ h_out, const uint16_t* __restrict__ carry_B,
                    const uint16_t* __restrict__ carry_x, int64_t L, int H, int G, int Q, int64_t n_chunks,
                    int64_t nbh, PassArgs pa, SegArgs sa, const float* __restrict__ dt_bias, int raw) {
    using S = Shape<R, NW>;
    const int Nin = GEN ? pa.nin : N, Nrow = GEN ? pa.nrow : N, n_off = GEN ? pa.n_off : 0;
    const int Pin = GP ? pa.pin : P, Pcol = GP ? pa.pcol : P, p_off = GP ? pa.p_off : 0;
    const int Rin = GEN ? pa.rin : R;  // the caller's rank (rows of rank Rin..R-1 are zero)
    constexpr int ym = YM;
    float* const ypart = pa.ypart;
    using CR = ChunkRegs<S>;
    constexpr int QRP = S::QRP, NT = S::NT, XS = S::XS, SPW = S::SPW, TPW = S::TPW, LR = S::LR;

    // One LDS block, carved with the arrays addressed through per-lane indices
    // plus constants first, so those constants fit the 16-bit offset field of
    // the LDS instructions (a separate array past 64 KiB costs an address add
    // per access):
    //   sW   per wave, per token: S2 (log2 decay), gamma, delta_next, e^{S}, state weight, T, tile weight
    //   sXT  X^T [p][rho]
    //   sGT  g^T [p][n], bf16, 2 buffers
    //   sBt  B~ [rho][n]
    //   sCt  C~ [rho][n] (R <= 2)
    constexpr int kW = NW * 7 * 64 * 4, kXT = P * XS * 2, kGT = 2 * P * NS * 2, kBT = QRP * NS * 2;
    constexpr int kCT = S::C_LDS ? QRP * NS * 2 : 0;
    static_assert(kW % 16 == 0 && kXT % 16 == 0 && kGT % 16 == 0 && kBT % 16 == 0, "LDS carve alignment");
    __shared__ __attribute__((aligned(16))) unsigned char smem[kW + kXT + kGT + kBT + kCT];
    auto* const sW = reinterpret_cast<float(*)[7 * 64]>(smem);
    uint16_t* const sXT = reinterpret_cast<uint16_t*>(smem + kW);
    auto* const sGT = reinterpret_cast<uint16_t(*)[P * NS]>(smem + kW + kXT);
    uint16_t* const sBt = reinterpret_cast<uint16_t*>(smem + kW + kXT + kGT);
    uint16_t* const sCt = reinterpret_cast<uint16_t*>(smem + kW + kXT + kGT + kBT);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
    const int l16 = lane & 15, g4 = lane >> 4;

    __shared__ unsigned sTicket;
    int64_t bh;
    int seg = 0;
    if (sa.nseg > 1) {
        // segments in ticket order, segment-major: a workgroup only ever waits
        // for lower tickets, which are already running
        if (tid == 0) sTicket = __hip_atomic_fetch_add(&sa.ctrl[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const int64_t t = sTicket;
        seg = int(t / nbh);
        bh = t % nbh;
    } else {
        // XCD-aware order: the 8 XCDs take blocks round-robin; give each a
        // contiguous run of (b, h) so heads sharing B/C share an L2.
        const int64_t bid = blockIdx.x, q8 = nbh / 8, r8 = nbh % 8;
        const int64_t xcd = bid % 8, slot = bid / 8;
        bh = xcd * q8 + (xcd < r8 ? xcd : r8) + slot;
    }
    const int64_t c_begin = int64_t(seg) * sa.cps;
    const int64_t c_end = c_begin + sa.cps < n_chunks ? c_begin + sa.cps : n_chunks;
    const int64_t b = bh / H;
    const int h = int(bh % H);
    const int grp = h / (H / G);
    const float A2 = Av[h] * kLog2e;
    const StepIn si = step_in(dt_bias, raw, h);  // dt and lambda as given, or from raw projections
    const float Dh = ym >= 2 ? 0.f : Dv[h];  // D x once, in the first row pass
    float* wsc = sW[wave];

    // rotation rates (revolutions per unit step) of the pairs this thread turns
    // (pairs past the caller's Nin / 2 hold zero rows: rate 0)
    const float* omh = omega ? omega + int64_t(h) * (Nrow / 2) + n_off / 2 : nullptr;
    auto omk = [&](int k) { return (omh && (!GEN || 2 * k < Nin)) ? omh[k] : 0.f; };
    float omB[4], omC[4], omS[TPW / 4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) omB[j] = omk(4 * (tid & 15) + j) * kInv2Pi;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) omC[ks] = omk(16 * ks + 4 * g4 + (l16 & 3)) * kInv2Pi;
#pragma unroll
    for (int mr = 0; mr < TPW / 4; ++mr)
#pragma unroll
        for (int hp = 0; hp < 2; ++hp) omS[mr][hp] = omk(8 * ((wave * TPW) / 4 + mr) + 2 * g4 + hp) * kInv2Pi;

    auto chunk_base = [&](int64_t cc) {
        const int64_t c0 = cc * Q, tok0 = b * L + c0;
        ChunkBase cb;
        cb.B = Bm + (tok0 * G + grp) * int64_t(Rin * Nrow) + n_off;
        cb.C = Cm + (tok0 * G + grp) * int64_t(Rin * Nrow) + n_off;
        cb.x = x + (tok0 * H + h) * int64_t(Rin * Pcol) + p_off;
        cb.nq = int(L - c0 < Q ? L - c0 : Q);
        cb.nin = Nin;
        cb.nrow = Nrow;
        cb.pin = Pin;
        cb.pcol = Pcol;
        cb.rin = Rin;
        return cb;
    };

    CR pre;
    {
        const ChunkBase cb = chunk_base(c_begin);
        load_chunk<S>(pre, cb, dt + h, lam ? lam + h : nullptr, b * L + c_begin * Q, L, c_begin * Q, H, G, tid, lane);
    }

    // ---- initial state g = h0 + delta_0 carry_B^T carry_x, tiles (nt, pt) of this wave
    //      (a later segment starts from zero: its incoming state is added afterwards)
    floatx4 gst[TPW];
    if (seg > 0) {
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
            const int u = wave * TPW + m, nt = u >> 2, pt = u & 3;
            gst[m] = floatx4{0.f, 0.f, 0.f, 0.f};
            *reinterpret_cast<u32x2*>(&sGT[0][(16 * pt + l16) * NS + 16 * nt + 4 * g4]) = u32x2{0u, 0u};
        }
    } else {
        const int64_t t0 = (b * L) * H + h;
        const float dl0 = (1.f - si.lam(lam, t0)) * si.dt(dt[t0]);
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
            const int u = wave * TPW + m, nt = u >> 2, pt = u & 3;
            const int p = 16 * pt + l16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int n = 16 * nt + 4 * g4 + e;
                const bool in = n < Nin && p < Pin;
                float v = (h0 && in) ? h0[(bh * Nrow + n_off + n) * Pcol + p_off + p] : 0.f;
                if (carry_B && in) {
                    float s = 0.f;
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        if (r < Rin)
                            s += bf16_to_f32(carry_B[((b * G + grp) * Rin + r) * Nrow + n_off + n]) *
                                 bf16_to_f32(carry_x[(bh * Rin + r) * Pcol + p_off + p]);
                    v += dl0 * s;
                }
                gst[m][e] = v;
            }
            *reinterpret_cast<u32x2*>(&sGT[0][p * NS + 16 * nt + 4 * g4]) =
                u32x2{pack2(gst[m][0], gst[m][1]), pack2(gst[m][2], gst[m][3])};
        }
    }

    double segT = 0.0;  // total step of this segment
#pragma unroll 1
    for (int64_t c = c_begin; c < c_end; ++c) {
        const ChunkBase cb = chunk_base(c);
        const int nq = cb.nq;
        const uint16_t* gT = sGT[(c - c_begin) & 1];
        uint16_t* gTn = sGT[(c - c_begin + 1) & 1];

        // ---- 1. per-token scalars, computed by every wave for itself (lane = token)
        const bool v0 = pre.ok & 1u, v1 = pre.ok & 2u, hl = pre.ok & 4u;
        const float d = v0 ? si.dt(pre.d) : 0.f, l = v0 ? (hl ? si.lamv(pre.l) : 1.f) : 0.f;
        const float dn = v1 ? si.dt(pre.dn) : 0.f, ln = v1 ? (hl ? si.lamv(pre.ln) : 1.f) : 0.f;
        const float T = wave_prefix_sum(d, lane);
        const float S2 = A2 * T;
        const float S2e = lane_read(S2, nq - 1);
        const float Te = lane_read(T, nq - 1);
        {
            const float gam = l * d, dln = (1.f - ln) * dn;
            wsc[lane] = S2;
            wsc[64 + lane] = gam;
            wsc[128 + lane] = dln;
            wsc[192 + lane] = __builtin_amdgcn_exp2f(S2);
            wsc[256 + lane] = __builtin_amdgcn_exp2f(S2e - S2) * (gam + dln);
            wsc[320 + lane] = T;
            // weight of row token j against the last token of its 16-row tile
            wsc[384 + lane] = __builtin_amdgcn_exp2f(tile_last<LR>(S2, lane) - S2) * (gam + dln);
        }

        // ---- 2. stage B~ (and C~ when it lives in LDS) and X^T; one angle per (token, pair)
#pragma unroll
        for (int m = 0; m < S::UPT; ++m) {
            const int i = (tid >> 4) + m * (NT / 16);
            const float Ti = wsc[320 + i];
            CS t[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) t[j] = cs_rev(omB[j], Ti);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int rho = i * R + r;
                const u32x4 vb = pre.b[m][r];
                *reinterpret_cast<u32x4*>(sBt + rho * NS + 8 * (tid & 15)) =
                    u32x4{rot_pair(vb[0], t[0]), rot_pair(vb[1], t[1]), rot_pair(vb[2], t[2]), rot_pair(vb[3], t[3])};
                if constexpr (S::C_LDS) {
                    const u32x4 vc = pre.c[m][r];
                    *reinterpret_cast<u32x4*>(sCt + rho * NS + 8 * (tid & 15)) = u32x4{
                        rot_pair(vc[0], t[0]), rot_pair(vc[1], t[1]), rot_pair(vc[2], t[2]), rot_pair(vc[3], t[3])};
                }
            }
        }
#pragma unroll
        for (int m = 0; m < S::XPT; ++m) {
            if (S::XU % NT != 0 && tid + m * NT >= S::XU) break;
            const int rho0 = 2 * ((tid >> 3) + m * (NT / 8));
            const int pc = tid & 7;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int p = 8 * pc + 2 * j;
                *reinterpret_cast<unsigned*>(sXT + p * XS + rho0) = (pre.x0[m][j] & 0xffffu) | (pre.x1[m][j] << 16);
                *reinterpret_cast<unsigned*>(sXT + (p + 1) * XS + rho0) =
                    (pre.x0[m][j] >> 16) | (pre.x1[m][j] & 0xffff0000u);
            }
        }
        // ---- 3. prefetch the next chunk's scalars, B, C and X (in flight through the compute below)
        const bool more = c + 1 < c_end;
        const ChunkBase cbn = chunk_base(more ? c + 1 : c);
        if (more) load_chunk<S>(pre, cbn, dt + h, lam ? lam + h : nullptr, b * L + (c + 1) * Q, L, (c + 1) * Q, H, G, tid, lane);
        segT += double(Te);
        lds_barrier();

        // This wave's output strips (16 rows each), ascending. The snake order deals
        // the triangle's score work evenly (strip s needs s + 1 score tiles), and
        // with an even wave count two strips that follow each other never share
        // a diagonal pair (when they differ by one row tile the first is odd).
        static_assert(S::PTG == 1 && S::PTW == 4, "a wave takes whole strips");
        static_assert(NW % 2 == 0, "snake order with an even wave count");
        int strip[SPW];
#pragma unroll
        for (int k = 0; k < SPW; ++k) strip[k] = strip_of<NW>(wave, k);

        // ---- 4. raw C rows of every strip of the wave (R = 4: not staged in LDS);
        //         their latency is covered by the state update below
        u32x4 craw[S::C_LDS ? 1 : SPW][4];
        if constexpr (!S::C_LDS) {
#pragma unroll
            for (int k = 0; k < SPW; ++k) load_strip_c<S>(craw[k], cb, strip[k], G, lane);
        }

        // ---- 5. state passed to the next chunk (written to the other g^T buffer)
        const int te = nq - 1;
        const float decE = wsc[192 + te];
#pragma unroll
        for (int m = 0; m < TPW; ++m) gst[m] *= decE;
        // A operand (w B~)^T: row n, k = 8 consecutive rho, read straight from the
        // row-major B~ with transposing LDS loads and scaled by the state weight
#pragma unroll 2
        for (int ks = 0; ks < QRP / 32; ++ks) {
            const unsigned rb = 32u * ks + 8u * g4;
            u32x4 xb[4];
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) xb[pt] = *reinterpret_cast<const u32x4*>(sXT + (16 * pt + l16) * XS + rb);
            float wr[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) wr[j] = wsc[256 + ((rb + j) >> LR)];
#pragma unroll
            for (int mr = 0; mr < TPW / 4; ++mr) {
                const int n0 = 16 * ((wave * TPW) / 4 + mr);
                const u32x2 lo = load_tr(sBt + (rb + (l16 >> 2)) * NS + n0 + 4 * (l16 & 3));
                const u32x2 hi = load_tr(sBt + (rb + 4 + (l16 >> 2)) * NS + n0 + 4 * (l16 & 3));
                const u32x4 a = {scale2(lo[0], wr[0], wr[1]), scale2(lo[1], wr[2], wr[3]), scale2(hi[0], wr[4], wr[5]),
                                 scale2(hi[1], wr[6], wr[7])};
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) gst[mr * 4 + pt] = mfma32(a, xb[pt], gst[mr * 4 + pt]);
            }
        }
#pragma unroll
        for (int mr = 0; mr < TPW / 4; ++mr) {
            const CS t0 = cs_rev(omS[mr][0], Te), t1 = cs_rev(omS[mr][1], Te);
            const int nt = (wave * TPW) / 4 + mr;
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                const int m = mr * 4 + pt;
                float a0 = gst[m][0], a1 = gst[m][1];
                gst[m][0] = t0.c * a0 - t0.s * a1;
                gst[m][1] = t0.s * a0 + t0.c * a1;
                a0 = gst[m][2];
                a1 = gst[m][3];
                gst[m][2] = t1.c * a0 - t1.s * a1;
                gst[m][3] = t1.s * a0 + t1.c * a1;
                const int p = 16 * pt + l16;
                *reinterpret_cast<u32x2*>(gTn + p * NS + 16 * nt + 4 * g4) =
                    u32x2{pack2(gst[m][0], gst[m][1]), pack2(gst[m][2], gst[m][3])};
            }
        }

        // ---- 6. C~ rows of the strips in the B-operand layout (col rho_i = 16 s + l16, k = n)
        u32x4 cr[SPW][4];
        float S2i[SPW], eSi[SPW];
        int tii[SPW];
#pragma unroll
        for (int k = 0; k < SPW; ++k) {
            const int s = strip[k];
            tii[k] = int((16u * s + l16) >> LR);
            S2i[k] = wsc[tii[k]];
            eSi[k] = wsc[192 + tii[k]];
            if constexpr (S::C_LDS) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    cr[k][ks] = *reinterpret_cast<const u32x4*>(sCt + (16 * s + l16) * NS + 32 * ks + 8 * g4);
            } else {
                // the 4 lanes of a DPP quad hold the 4 ranks of one token: each
                // evaluates one of the quad's 4 angles and shares it
                const float Ti = wsc[320 + tii[k]];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const CS own = cs_rev(omC[ks], Ti);
                    const CS t0{quad_bcast<0>(own.c), quad_bcast<0>(own.s)};
                    const CS t1{quad_bcast<1>(own.c), quad_bcast<1>(own.s)};
                    const CS t2{quad_bcast<2>(own.c), quad_bcast<2>(own.s)};
                    const CS t3{quad_bcast<3>(own.c), quad_bcast<3>(own.s)};
                    const u32x4 v = craw[k][ks];
                    cr[k][ks] = u32x4{rot_pair(v[0], t0), rot_pair(v[1], t1), rot_pair(v[2], t2), rot_pair(v[3], t3)};
                }
            }
        }

        // ---- 7. inter-chunk part y^T[p][rho_i] = e^{S_i} sum_n g^T[p][n] C~[rho_i][n]:
        //         each g^T operand serves every strip of the wave
        floatx4 acc[SPW][4];
#pragma unroll
        for (int k = 0; k < SPW; ++k)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[k][q] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            u32x4 ga[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) ga[q] = *reinterpret_cast<const u32x4*>(gT + (16 * q + l16) * NS + 32 * ks + 8 * g4);
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int k = 0; k < SPW; ++k) acc[k][q] = mfma32(ga[q], cr[k][ks], acc[k][q]);
        }
#pragma unroll
        for (int k = 0; k < SPW; ++k)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[k][q] *= eSi[k];

        // ---- 8. intra-chunk part, pair-major: the score tiles (jt, jt + 1) of every
        //         strip at or below the pair, masked (decay x width-2 convolution),
        //         then y^T[p][rho_i] += X^T[p][rho_j] (M o scores^T)[rho_j][rho_i].
        // Each pair's B~ operands (A operand of the scores, loaded one pair ahead),
        // its X^T operands and its mask scalars are loaded once for all strips.
        // Below the diagonal tile (every row token precedes every column token) the
        // decay splits at the tile's last token r: e^{S_i-S_j} = e^{S_i-S_r}
        // e^{S_r-S_j}, both factors <= 1, the second staged per token with the
        // width-2 weight, leaving one exp per lane and tile. The diagonal tile
        // takes the full mask, plus D on rho_j = rho_i (the skip term D x rides
        // in the same contraction).
        auto load_pair = [&](int jp, u32x4 (&a0)[4], u32x4 (&a1)[4]) {
            // operand rows past the chunk's padded rows (the prefetch after the last
            // pair) are clamped to valid rows; their products are never used
            const int r0 = 32 * jp + l16 < QRP ? 32 * jp + l16 : QRP - 1;
            const int r1 = r0 + 16 < QRP ? r0 + 16 : QRP - 1;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                a0[ks] = *reinterpret_cast<const u32x4*>(sBt + r0 * NS + 32 * ks + 8 * g4);
                a1[ks] = *reinterpret_cast<const u32x4*>(sBt + r1 * NS + 32 * ks + 8 * g4);
            }
        };
        auto read_below = [&](int jt, float& sr, float (&tw)[4]) {
            const unsigned rj = 16u * jt + 4u * g4;
            sr = wsc[(16 * jt + 15) >> LR];
#pragma unroll
            for (int e = 0; e < 4; ++e) tw[e] = wsc[384 + ((rj + e) >> LR)];
        };
        auto load_x = [&](int jp, u32x2 (&xa)[4], u32x2 (&xb)[4]) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint16_t* xr = sXT + (16 * q + l16) * XS + 32 * jp + 4 * g4;
                xa[q] = *reinterpret_cast<const u32x2*>(xr);
                xb[q] = *reinterpret_cast<const u32x2*>(xr + 16);
            }
        };
        auto score = [&](const u32x4 (&a)[4], const u32x4 (&c)[4]) {
            floatx4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) t = mfma32(a[ks], c[ks], t);
            return t;
        };
        auto mask_below = [&](const floatx4& t, float sr, const float (&tw)[4], float S2, float* m) {
            const float a = __builtin_amdgcn_exp2f(S2 - sr);
#pragma unroll
            for (int e = 0; e < 4; ++e) m[e] = t[e] * (tw[e] * a);
        };
        auto mask_diag = [&](const floatx4& t, int jt, int k, float* m) {
            const unsigned rj = 16u * jt + 4u * g4;
            const int rho_i = 16 * strip[k] + l16;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                m[e] = t[e] * mask_coef(int((rj + e) >> LR), tii[k], S2i[k], wsc) + (int(rj + e) == rho_i ? Dh : 0.f);
        };
        auto y_pair = [&](floatx4 (&ac)[4], const u32x2 (&xa)[4], const u32x2 (&xb)[4], const float* m0,
                          const float* m1) {
            const u32x4 pb = {pack2(m0[0], m0[1]), pack2(m0[2], m0[3]), pack2(m1[0], m1[1]), pack2(m1[2], m1[3])};
#pragma unroll
            for (int q = 0; q < 4; ++q) ac[q] = mfma32(u32x4{xa[q][0], xa[q][1], xb[q][0], xb[q][1]}, pb, ac[q]);
        };
        // pair jp for strips k0 .. SPW-1; strip k0 holds its diagonal tile in this
        // pair when DIAG (its last pair), every other strip lies wholly below it
        auto pair_step = [&](auto k0c, auto diagc, int jp, const u32x4 (&a0)[4], const u32x4 (&a1)[4]) {
            constexpr int K0 = decltype(k0c)::value;
            constexpr bool DIAG = decltype(diagc)::value;
            float sr0, sr1, tw0[4], tw1[4];
            read_below(2 * jp, sr0, tw0);
            read_below(2 * jp + 1, sr1, tw1);
            u32x2 xa[4], xb[4];
            load_x(jp, xa, xb);
            floatx4 t0[SPW], t1[SPW];
#pragma unroll
            for (int k = K0; k < SPW; ++k) {
                t0[k] = score(a0, cr[k]);
                t1[k] = score(a1, cr[k]);
            }
#pragma unroll
            for (int k = K0; k < SPW; ++k) {
                float m0[4], m1[4];
                if (DIAG && k == K0) {
                    if (strip[k] & 1) {
                        mask_below(t0[k], sr0, tw0, S2i[k], m0);
                        mask_diag(t1[k], 2 * jp + 1, k, m1);
                    } else {
                        mask_diag(t0[k], 2 * jp, k, m0);
#pragma unroll
                        for (int e = 0; e < 4; ++e) m1[e] = 0.f;
                    }
                } else {
                    mask_below(t0[k], sr0, tw0, S2i[k], m0);
                    mask_below(t1[k], sr1, tw1, S2i[k], m1);
                }
                y_pair(acc[k], xa, xb, m0, m1);
            }
        };
        {
            u32x4 pa0[4], pa1[4];
            load_pair(0, pa0, pa1);
            int jp = 0;
            auto run_strip = [&](auto k0c) {
                constexpr int K0 = decltype(k0c)::value;
                const int jd = strip[K0] >> 1;  // the pair holding strip K0's diagonal tile
#pragma unroll 1
                for (; jp < jd; ++jp) {
                    u32x4 a0[4], a1[4];
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        a0[ks] = pa0[ks];
                        a1[ks] = pa1[ks];
                    }
                    load_pair(jp + 1, pa0, pa1);
                    pair_step(k0c, std::false_type{}, jp, a0, a1);
                }
                u32x4 a0[4], a1[4];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    a0[ks] = pa0[ks];
                    a1[ks] = pa1[ks];
                }
                if (K0 + 1 < SPW) load_pair(jp + 1, pa0, pa1);
                pair_step(k0c, std::true_type{}, jp, a0, a1);
                ++jp;
            };
            run_strip(std::integral_constant<int, 0>{});
            if constexpr (SPW > 1) run_strip(std::integral_constant<int, 1>{});
            if constexpr (SPW > 2) run_strip(std::integral_constant<int, 2>{});
            if constexpr (SPW > 3) run_strip(std::integral_constant<int, 3>{});
            static_assert(SPW <= 4, "at most four strips per wave");
        }

        // ---- 9. epilogue: 4 consecutive p of row rho_i per lane (D x is already in)
#pragma unroll
        for (int k = 0; k < SPW; ++k) {
            const int rho_i = 16 * strip[k] + l16;
            if ((rho_i >> LR) < nq && (rho_i & (R - 1)) < Rin) {
                const int i = rho_i >> LR, r = rho_i & (R - 1);
                const int64_t yo =
                    ((b * L + c * Q) * H + h) * int64_t(Rin * Pcol) + int64_t(i * H * Rin + r) * Pcol + p_off;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int p = 16 * q + 4 * g4;
                    if (GP && p >= Pin) continue;  // Pin is a multiple of 8
                    floatx4 v = acc[k][q];
                    if (ym >= 2) v += *reinterpret_cast<const floatx4*>(ypart + yo + p);
                    if (ym == 1 || ym == 3)
                        *reinterpret_cast<floatx4*>(ypart + yo + p) = v;
                    else
                        *reinterpret_cast<u32x2*>(y + yo + p) = u32x2{pack2(v[0], v[1]), pack2(v[2], v[3])};
                }
            }
        }
        lds_barrier();
    }

    if (ym == 0 && sa.nseg > 1) {
        // ================= sequence segments: look-back and correction
        __shared__ unsigned sFlag;
        const int64_t bs = bh * sa.nseg + seg;
        auto tile_ptr = [&](float* base, int m) {  // this lane's first element of state tile m
            const int u = wave * TPW + m, nt = u >> 2, pt = u & 3;
            return base + (16 * nt + 4 * g4) * P + 16 * pt + l16;
        };
        auto publish = [&](float* dst, const floatx4* v, unsigned flag, bool with_total) {
#pragma unroll
            for (int m = 0; m < TPW; ++m) {
                float* q = tile_ptr(dst + bs * (N * P), m);
#pragma unroll
                for (int e = 0; e < 4; ++e) q[e * P] = v[m][e];
            }
            __syncthreads();
            if (tid == 0) {
                if (with_total) sa.tr[bs] = segT;
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                __hip_atomic_store(&sa.ctrl[2 + bs], flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        };
        floatx4 gin[TPW];  // state entering this segment (g form)
#pragma unroll
        for (int m = 0; m < TPW; ++m) gin[m] = floatx4{0.f, 0.f, 0.f, 0.f};
        if (seg == 0) {
            publish(sa.incl, gst, 2u, false);
        } else {
            publish(sa.agg, gst, 1u, true);
            double Tacc = 0.0;  // total step between predecessor j's end and this segment's start
            for (int j = seg - 1; j >= 0; --j) {
                const int64_t bj = bh * sa.nseg + j;
                if (tid == 0) {
                    // A predecessor holds a lower ticket, so it is running or done and
                    // this wait ends; the bound guards against a hang all the same.
                    // Giving up sets the workspace's error flag (m3_prefill_check
                    // reports it); the outputs of this call are then not valid.
                    unsigned f = 0u;
                    long spins = 0;
                    while (sa.spin_limit > 0 && (f = __hip_atomic_load(&sa.ctrl[2 + bj], __ATOMIC_RELAXED,
                                                                        __HIP_MEMORY_SCOPE_AGENT)) == 0u) {
                        __builtin_amdgcn_s_sleep(2);
                        if (++spins > sa.spin_limit) break;
                    }
                    if (f == 0u) {
                        __hip_atomic_store(&sa.ctrl[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        f = 2u;
                    }
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                    sFlag = f;
                }
                __syncthreads();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                const unsigned f = sFlag;
                const float* src = (f == 2u ? sa.incl : sa.agg) + bj * (N * P);
#pragma unroll
                for (int m = 0; m < TPW; ++m) {
                    const float* q = tile_ptr(const_cast<float*>(src), m);
                    const floatx4 v = {q[0], q[P], q[2 * P], q[3 * P]};
                    gin[m] += transfer(v, A2, omS[m >> 2], Tacc);
                }
                if (f == 2u) break;
                Tacc += sa.tr[bj];
                __syncthreads();
            }
            // inclusive end state = transfer(segment) g_in + local end state
            floatx4 inc[TPW];
#pragma unroll
            for (int m = 0; m < TPW; ++m) inc[m] = transfer(gin[m], A2, omS[m >> 2], segT) + gst[m];
            publish(sa.incl, inc, 2u, false);
#pragma unroll
            for (int m = 0; m < TPW; ++m) gst[m] = inc[m];

            // correction: y_t += e^{S_t} C~_t^T g_c for the part g_c of the chunk-entry
            // state that comes from g_in, chunk by chunk until its decay is exactly 0
#pragma unroll
            for (int m = 0; m < TPW; ++m) {
                const int u = wave * TPW + m, nt = u >> 2, pt = u & 3;
                *reinterpret_cast<u32x2*>(&sGT[0][(16 * pt + l16) * NS + 16 * nt + 4 * g4]) =
                    u32x2{pack2(gin[m][0], gin[m][1]), pack2(gin[m][2], gin[m][3])};
            }
            __syncthreads();
            double Tcum = 0.0;
#pragma unroll 1
            for (int64_t c = c_begin; c < c_end; ++c) {
                if (__builtin_amdgcn_exp2f(float(double(A2) * Tcum)) == 0.f) break;
                const int64_t c0 = c * Q;
                const int nq = int(L - c0 < Q ? L - c0 : Q);
                float T = 0.f;
                if (lane < nq) T = si.dt(dt[(b * L + c0 + lane) * H + h]);
                T = wave_prefix_sum(T, lane);
                const float Te = lane_read(T, nq - 1);
                wsc[192 + lane] = __builtin_amdgcn_exp2f(A2 * T);
                wsc[320 + lane] = T;
                const ChunkBase cbc = chunk_base(c);
                const uint16_t* gT = sGT[(c - c_begin) & 1];
#pragma unroll 1
                for (int si = 0; si < SPW; ++si) {
                    const int item = strip_of<NW>(wave, si);
                    const int s = item / S::PTG, pt0 = (item % S::PTG) * S::PTW;
                    const unsigned rho = 16u * s + l16;
                    const int ti = int(rho >> LR);
                    const float Ti = wsc[320 + ti];
                    u32x4 craw2[4], cr[4];
                    load_strip_c<S>(craw2, cbc, s, G, lane);
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        CS t[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            t[j] = cs_rev(omk(16 * ks + 4 * g4 + j) * kInv2Pi, Ti);
                        cr[ks] = u32x4{rot_pair(craw2[ks][0], t[0]), rot_pair(craw2[ks][1], t[1]),
                                       rot_pair(craw2[ks][2], t[2]), rot_pair(craw2[ks][3], t[3])};
                    }
                    floatx4 a[S::PTW];
#pragma unroll
                    for (int q = 0; q < S::PTW; ++q) {
                        a[q] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < 4; ++ks) {
                            const u32x4 ga = *reinterpret_cast<const u32x4*>(gT + (16 * (pt0 + q) + l16) * NS +
                                                                             32 * ks + 8 * g4);
                            a[q] = mfma32(ga, cr[ks], a[q]);
                        }
                    }
                    if (ti < nq && int(rho & (R - 1)) < Rin) {
                        uint16_t* yr = y + ((b * L + c0) * H + h) * int64_t(Rin * Pcol) +
                                       int64_t(ti * H * Rin + int(rho & (R - 1))) * Pcol + p_off;
                        const float f = wsc[192 + ti];
#pragma unroll
                        for (int q = 0; q < S::PTW; ++q) {
                            const int pp = 16 * (pt0 + q) + 4 * g4;
                            if (GP && pp >= Pin) continue;
                            const u32x2 old = *reinterpret_cast<const u32x2*>(yr + pp);
                            *reinterpret_cast<u32x2*>(yr + pp) =
                                u32x2{pack2(lo16(old[0]) + f * a[q][0], hi16(old[0]) + f * a[q][1]),
                                      pack2(lo16(old[1]) + f * a[q][2], hi16(old[1]) + f * a[q][3])};
                        }
                    }
                }
                // g_{c+1} = e^{S_e} Rot(Phi_e) g_c (no input)
                uint16_t* gTn = sGT[(c - c_begin + 1) & 1];
#pragma unroll
                for (int m = 0; m < TPW; ++m) {
                    const int u = wave * TPW + m, nt = u >> 2, pt = u & 3;
                    gin[m] = transfer(gin[m], A2, omS[m >> 2], double(Te));
                    *reinterpret_cast<u32x2*>(gTn + (16 * pt + l16) * NS + 16 * nt + 4 * g4) =
                        u32x2{pack2(gin[m][0], gin[m][1]), pack2(gin[m][2], gin[m][3])};
                }
                Tcum += double(Te);
                __syncthreads();
            }
        }
        if (seg != sa.nseg - 1) return;
    }
    if (h_out) {
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
            const int u = wave * TPW + m, nt = u >> 2, pt = u & 3;
            const int p = 16 * pt + l16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int n = 16 * nt + 4 * g4 + e;
                if (n < Nin && p < Pin) h_out[(bh * Nrow + n_off + n) * Pcol + p_off + p] = gst[m][e];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// R = 1 with wave specialisation: 8 waves, waves 0-3 compute chunk c (scores,
// masked product, inter-chunk term, state update) while waves 4-7 load, rotate
// and stage chunk c+1 into the other half of double-buffered LDS and prefetch
// chunk c+2 into registers. One barrier per chunk hands the buffers over. The
// rotation and staging VALU work of one chunk thus runs next to the MFMA and
// masking work of the previous one on every SIMD.
namespace ws1 {

constexpr int QRP = 64;             // rows per chunk (R = 1)
// LDS row strides (bf16) and the X^T column swizzle, chosen with the device's
// bank-conflict counter (32 banks of 4 bytes): rows of 144 make the 16-byte
// reads of B~ and C~ rows by 16 lanes conflict-free (136 costs 4 cycles per
// read) and leave the staging writes and the transposing loads as they were.
// X^T rows of 80 with the 16-byte column blocks of row p XORed with
// (p / 8) mod 8 make the staging waves' transposed writes conflict-free (8
// lanes on one bank at 72 unswizzled) and keep the 8-byte y-operand reads so.
constexpr int NSB = N + 16;         // B~, C~ row stride
constexpr int XS = QRP + 16;        // X^T row stride
// column c of X^T row p is stored at c ^ xsw(p)
__device__ __forceinline__ int xsw(int p) { return 8 * ((p >> 3) & 7); }
constexpr int NCW = 4;              // compute waves
constexpr int NSW = 8;              // staging waves
constexpr int NST = 64 * NSW;       // staging threads
constexpr int TSTEP = NST / 16;     // token step between a staging thread's rows
constexpr int MT = QRP / TSTEP;     // B/C rows (8 columns each) per staging thread
constexpr int NXT = 256;            // staging threads that move X (32 row pairs x 8 pieces)
constexpr int MRW = 3;  // most state row tiles (of 16 rows) a compute wave holds (split 3, 3, 1, 1)
static_assert(MT >= 1 && QRP % TSTEP == 0 && NST >= NXT && NCW == 4, "staging split");

struct StageRegs {
    float d, l, dn, ln;  // lane = token, as loaded; l, dn, ln only in the scalar wave
    unsigned ok;         // bit 0: token inside the chunk, bit 1: and a next token exists
    u32x4 b[MT], c[MT];  // token (stid >> 4) + TSTEP m, 8 columns at 8 (stid & 15)
    u32x4 x0, x1;        // X rows 2 (stid >> 3), +1, 8 columns at 8 (stid & 7), stid < NXT
};

__device__ __forceinline__ void stage_load(StageRegs& r, const ChunkBase& cb, const float* __restrict__ dt,
                                           const float* __restrict__ lam, int64_t tok0, int64_t L, int64_t c0, int H,
                                           int G, int stid, int lane, bool scal) {
    const int nq = cb.nq;
    {
        const int ic = lane < nq ? lane : nq - 1;
        const int64_t ti = (tok0 + ic) * H;
        // Kept as loaded: masking them here would wait for these loads, and
        // with them for the other register set's (the counter is in order).
        // Without lambda (lambda = 1) dt stands in as a valid address and the
        // value is replaced at use.
        r.d = dt[ti];
        const bool has_next = c0 + ic + 1 < L;
        r.ok = (lane < nq ? 1u : 0u) | ((lane < nq && has_next) ? 2u : 0u) | (lam ? 4u : 0u);
        if (scal) {
            const float* lp = lam ? lam : dt;
            r.l = lp[ti];
            r.dn = dt[has_next ? ti + H : ti];
            r.ln = lp[has_next ? ti + H : ti];
        }
    }
    const int pc = stid & 15;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int i = (stid >> 4) + TSTEP * m;
        const bool in = 8 * pc < cb.nin;
        r.b[m] = in ? load_tok(cb.B, i, nq, G * cb.nrow, 8 * pc) : u32x4{0u, 0u, 0u, 0u};
        r.c[m] = in ? load_tok(cb.C, i, nq, G * cb.nrow, 8 * pc) : u32x4{0u, 0u, 0u, 0u};
    }
    if (stid < NXT) {
        const int rho0 = 2 * (stid >> 3);
        const bool xin = 8 * (stid & 7) < cb.pin;
        r.x0 = xin ? load_tok(cb.x, rho0, nq, H * cb.pcol, 8 * (stid & 7)) : u32x4{0u, 0u, 0u, 0u};
        r.x1 = xin ? load_tok(cb.x, rho0 + 1, nq, H * cb.pcol, 8 * (stid & 7)) : u32x4{0u, 0u, 0u, 0u};
    }
}

// rotate and write one chunk into one LDS buffer; the scalar wave also writes
// the per-token scalars
// Returns the chunk's total step (sum of dt). base[j] = frac(omega_j T0 / 2 pi)
// for the thread's four pairs, T0 the total step before the chunk: B and C are
// turned by the absolute angle omega (T0 + T_i), so the carried state needs
// no rotation of its own. ROT = false: omega = 0, B and C are staged as given.
template <bool ROT>
__device__ __forceinline__ float stage_write(const StageRegs& r, int nq, float A2, const float* omB, const float* base,
                                             uint16_t* sBt, uint16_t* sCt, uint16_t* sXT, float* sSc, int stid,
                                             int lane, bool scal, const StepIn& si) {
    const float rd = (r.ok & 1u) ? si.dt(r.d) : 0.f;
    const float T = wave_prefix_sum(rd, lane);
    if (scal) {
        const float S2 = A2 * T;
        const float S2e = lane_read(S2, nq - 1);
        const float rdn = (r.ok & 2u) ? si.dt(r.dn) : 0.f;
        const float rl = (r.ok & 1u) ? ((r.ok & 4u) ? si.lamv(r.l) : 1.f) : 0.f;
        const float rln = (r.ok & 2u) ? ((r.ok & 4u) ? si.lamv(r.ln) : 1.f) : 0.f;
        const float gam = rl * rd, dln = (1.f - rln) * rdn;
        sSc[lane] = S2;
        sSc[64 + lane] = gam;
        sSc[128 + lane] = dln;
        sSc[192 + lane] = __builtin_amdgcn_exp2f(S2);
        sSc[256 + lane] = __builtin_amdgcn_exp2f(S2e - S2) * (gam + dln);
        sSc[320 + lane] = T;
        // weight of row token j against the last token of its 16-token tile
        const float S2r = row_last(S2, lane);
        sSc[384 + lane] = __builtin_amdgcn_exp2f(S2r - S2) * (gam + dln);
    }
    const int pc = stid & 15;
    // a staging wave's lanes cover tokens tb + row + TSTEP m (row = lane / 16)
    const int tb = __builtin_amdgcn_readfirstlane(stid >> 4) & ~3;
    const int row = lane >> 4;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int i = (stid >> 4) + TSTEP * m;
        if constexpr (!ROT) {
            *reinterpret_cast<u32x4*>(sBt + i * NSB + 8 * pc) = r.b[m];
            *reinterpret_cast<u32x4*>(sCt + i * NSB + 8 * pc) = r.c[m];
            continue;
        }
        const float t0 = lane_read(T, tb + TSTEP * m), t1 = lane_read(T, tb + TSTEP * m + 1);
        const float t2 = lane_read(T, tb + TSTEP * m + 2), t3 = lane_read(T, tb + TSTEP * m + 3);
        const float Ti = row == 0 ? t0 : row == 1 ? t1 : row == 2 ? t2 : t3;
        CS t[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float rv = __builtin_amdgcn_fractf(base[j] + omB[j] * Ti);
            t[j] = CS{__builtin_amdgcn_cosf(rv), __builtin_amdgcn_sinf(rv)};
        }
        const u32x4 vb = r.b[m], vc = r.c[m];
        *reinterpret_cast<u32x4*>(sBt + i * NSB + 8 * pc) =
            u32x4{rot_pair(vb[0], t[0]), rot_pair(vb[1], t[1]), rot_pair(vb[2], t[2]), rot_pair(vb[3], t[3])};
        *reinterpret_cast<u32x4*>(sCt + i * NSB + 8 * pc) =
            u32x4{rot_pair(vc[0], t[0]), rot_pair(vc[1], t[1]), rot_pair(vc[2], t[2]), rot_pair(vc[3], t[3])};
    }
    if (stid < NXT) {
        const int rho0 = 2 * (stid >> 3);
        const int pcx = stid & 7;
        // the thread's rows 8 pcx .. 8 pcx + 7 share one swizzle
        uint16_t* xw = sXT + 8 * pcx * XS + (rho0 ^ xsw(8 * pcx));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            *reinterpret_cast<unsigned*>(xw + 2 * j * XS) = (r.x0[j] & 0xffffu) | (r.x1[j] << 16);
            *reinterpret_cast<unsigned*>(xw + (2 * j + 1) * XS) = (r.x0[j] >> 16) | (r.x1[j] & 0xffff0000u);
        }
    }
    return lane_read(T, 63);  // tokens past the chunk's end carry dt = 0
}

}  // namespace ws1

// GEN, YM, GP as for prefill_mfma_kernel
template <bool ROT, bool GEN, int YM, bool GP>
__global__ void __launch_bounds__(64 * (ws1::NCW + ws1::NSW))
prefill_ws_r1_kernel(const uint16_t* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ Av,
                     const float* __restrict__ omega, const float* __restrict__ lam, const uint16_t* __restrict__ Bm,
                     const uint16_t* __restrict__ Cm, const float* __restrict__ Dv, const float* __restrict__ h0,
                     uint16_t* __restrict__ y, float* __restrict__ h_out, const uint16_t* __restrict__ carry_B,
                     const uint16_t* __restrict__ carry_x, int64_t L, int H, int G, int Q, int64_t n_chunks,
                     int64_t nbh, PassArgs pa, const float* __restrict__ dt_bias, int raw) {
    using namespace ws1;
    const int Nin = GEN ? pa.nin : N, Nrow = GEN ? pa.nrow : N, n_off = GEN ? pa.n_off : 0;
    const int Pin = GP ? pa.pin : P, Pcol = GP ? pa.pcol : P, p_off = GP ? pa.p_off : 0;
    constexpr int ym = YM;
    float* const ypart = pa.ypart;
    __shared__ __attribute__((aligned(16))) uint16_t sBt[2][QRP * NSB];  // B~ [rho][n]
    __shared__ __attribute__((aligned(16))) uint16_t sCt[2][QRP * NSB];  // C~ [rho][n]
    __shared__ __attribute__((aligned(16))) uint16_t sXT[2][P * XS];     // X^T [p][rho], swizzled (xsw)
    __shared__ __attribute__((aligned(16))) uint16_t sGT[2][P * NS];    // g^T [p][n], bf16
    // per token: S2 (log2 decay), gamma, delta_next, e^{S}, state weight, T, tile weight
    __shared__ float sSc[2][7 * 64];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
    const int l16 = lane & 15, g4 = lane >> 4;
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
    const StepIn si = step_in(dt_bias, raw, h);  // dt and lambda as given, or from raw projections
    const float Dh = ym >= 2 ? 0.f : Dv[h];  // D x once, in the first row pass
    // pairs past the caller's Nin / 2 hold zero rows: rate 0
    const float* omh = omega ? omega + int64_t(h) * (Nrow / 2) + n_off / 2 : nullptr;
    auto omk = [&](int k) { return (omh && (!GEN || 2 * k < Nin)) ? omh[k] : 0.f; };
    auto chunk_base = [&](int64_t cc) {
        const int64_t c0 = cc * Q, tok0 = b * L + c0;
        ChunkBase cb;
        cb.B = Bm + (tok0 * G + grp) * int64_t(Nrow) + n_off;
        cb.C = Cm + (tok0 * G + grp) * int64_t(Nrow) + n_off;
        cb.x = x + (tok0 * H + h) * int64_t(Pcol) + p_off;
        cb.nq = int(L - c0 < Q ? L - c0 : Q);
        cb.nin = Nin;
        cb.nrow = Nrow;
        cb.pin = Pin;
        cb.pcol = Pcol;
        cb.rin = 1;
        return cb;
    };

    if (wave >= NCW) {
        // ===================== staging waves. Two register sets: chunk k lives in
        // set k & 1, and its loads are issued two chunks ahead of its rotation.
        const int stid = tid - 64 * NCW;
        const bool scal = wave == NCW + NSW - 1;  // the wave that also stages the per-token scalars
        float omB[4];
        double omD[4];  // omega / 2 pi of the thread's four pairs, for the chunk base angles
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            omB[j] = omk(4 * (stid & 15) + j) * kInv2Pi;
            omD[j] = double(omk(4 * (stid & 15) + j)) * kInv2PiD;
        }
        double Tacc = 0.0;  // total step before the chunk being written
        StageRegs ra, rb;
        auto load = [&](StageRegs& r, int64_t cc) {
            stage_load(r, chunk_base(cc), dt + h, lam ? lam + h : nullptr, b * L + cc * Q, L, cc * Q, H, G, stid, lane, scal);
        };
        auto write = [&](const StageRegs& r, int64_t cc) {
            const int bn = int(cc & 1);
            float base[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const double rv = omD[j] * Tacc;
                base[j] = float(rv - floor(rv));
            }
            Tacc += stage_write<ROT>(r, chunk_base(cc).nq, A2, omB, base, sBt[bn], sCt[bn], sXT[bn], sSc[bn], stid,
                                     lane, scal, si);
        };
        load(ra, 0);
        if (n_chunks > 1) load(rb, 1);
        write(ra, 0);
        if (n_chunks > 2) load(ra, 2);
        lds_barrier();
        // during chunk c: write chunk c + 1, then issue the loads of chunk c + 3 into the freed set
        auto step = [&](StageRegs& r, int64_t c) {
            if (c + 1 < n_chunks) {
                write(r, c + 1);
                if (c + 3 < n_chunks) load(r, c + 3);
            }
            lds_barrier();
        };
#pragma unroll 1
        for (int64_t c = 0; c < n_chunks; c += 2) {
            step(rb, c);
            if (c + 1 < n_chunks) step(ra, c + 1);
        }
        return;
    }

    // ========================= compute waves: output strip `wave`; state row tiles
    // nt0 .. nt0 + ntc - 1 (all 4 column tiles each). The strips' score work
    // grows with the strip index, so the state rows are dealt unevenly
    // (3, 3, 1, 1 row tiles) to even out the waves' time per chunk.
    const int nt0 = wave == 0 ? 0 : wave == 1 ? 3 : wave == 2 ? 6 : 7;
    const int ntc = wave < 2 ? 3 : 1;
    double Tacc = 0.0;  // total step so far: the angle that turns the state back at the end
    floatx4 gst[MRW * 4];
    {
        const int64_t t0 = (b * L) * H + h;
        const float dl0 = (1.f - si.lam(lam, t0)) * si.dt(dt[t0]);
#pragma unroll
        for (int m = 0; m < MRW * 4; ++m) {
            gst[m] = floatx4{0.f, 0.f, 0.f, 0.f};
            if ((m >> 2) >= ntc) continue;
            const int nt = nt0 + (m >> 2), pt = m & 3;
            const int p = 16 * pt + l16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int n = 16 * nt + 4 * g4 + e;
                const bool in = n < Nin && p < Pin;
                float v = (h0 && in) ? h0[(bh * Nrow + n_off + n) * Pcol + p_off + p] : 0.f;
                if (carry_B && in)
                    v += dl0 * bf16_to_f32(carry_B[(b * G + grp) * Nrow + n_off + n]) *
                         bf16_to_f32(carry_x[bh * Pcol + p_off + p]);
                gst[m][e] = v;
            }
            *reinterpret_cast<u32x2*>(&sGT[0][p * NS + 16 * nt + 4 * g4]) =
                u32x2{pack2(gst[m][0], gst[m][1]), pack2(gst[m][2], gst[m][3])};
        }
    }
    lds_barrier();

    const int s = wave;
    const int ti = 16 * s + l16;  // token of this lane's column
    // X^T reads: row 16 q + l16 swizzles by 16 q + 8 (l16 / 8), so column
    // 16 jt + 4 g4 sits at 16 (jt ^ q) + (4 g4 ^ 8 (l16 / 8)) (disjoint bits),
    // and column 32 ks + 8 g4 of row 16 pt + l16 at xs[pt & 1] + 32 (ks ^ (pt / 2))
    const int xy = (4 * g4) ^ (8 * (l16 >> 3));
    const int xs[2] = {(8 * g4) ^ (8 * (l16 >> 3)), ((8 * g4) ^ (8 * (l16 >> 3))) ^ 16};
#pragma unroll 1
    for (int64_t c = 0; c < n_chunks; ++c) {
        const int buf = int(c & 1);
        const int nq = int(L - c * Q < Q ? L - c * Q : Q);
        const uint16_t* Bt = sBt[buf];
        const uint16_t* Ct = sCt[buf];
        const uint16_t* XT = sXT[buf];
        const float* sc = sSc[buf];
        const uint16_t* gT = sGT[buf];
        uint16_t* gTn = sGT[buf ^ 1];

        u32x4 cr[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) cr[ks] = *reinterpret_cast<const u32x4*>(Ct + ti * NSB + 32 * ks + 8 * g4);
        const float S2i = sc[ti];
        floatx4 acc[4];  // the p tiles' accumulation chains interleaved
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x4 ga = *reinterpret_cast<const u32x4*>(gT + (16 * q + l16) * NS + 32 * ks + 8 * g4);
                acc[q] = mfma32(ga, cr[ks], acc[q]);
            }
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] *= sc[192 + ti];
        // M o scores for row tile jt. Below the diagonal tile (jt < s, every
        // j < i) the decay splits at the tile's last token r = 16 jt + 15:
        // e^{S_i-S_j} = e^{S_i-S_r} e^{S_r-S_j}, both factors <= 1, the second
        // staged per token with the width-2 weight; one exp per lane and tile.
        // The diagonal tile takes the full mask, plus D on i = j (the skip term
        // D x_i rides along in the same contraction).
        auto mask_tile = [&](const floatx4& t, int jt, float* m) {
            if (jt < s) {
                const float a = __builtin_amdgcn_exp2f(S2i - sc[16 * jt + 15]);
                const floatx4 bw = *reinterpret_cast<const floatx4*>(sc + 384 + 16 * jt + 4 * g4);
#pragma unroll
                for (int e = 0; e < 4; ++e) m[e] = t[e] * (bw[e] * a);
            } else {
                const int rj = 16 * jt + 4 * g4;
#pragma unroll
                for (int e = 0; e < 4; ++e) m[e] = t[e] * mask_coef(rj + e, ti, S2i, sc) + (rj + e == ti ? Dh : 0.f);
            }
        };
        auto scores = [&](int jt, floatx4& t0, floatx4& t1) {
            t0 = floatx4{0.f, 0.f, 0.f, 0.f};
            t1 = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const u32x4 a0 = *reinterpret_cast<const u32x4*>(Bt + (16 * jt + l16) * NSB + 32 * ks + 8 * g4);
                t0 = mfma32(a0, cr[ks], t0);
            }
            if (jt + 1 <= s) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const u32x4 a1 =
                        *reinterpret_cast<const u32x4*>(Bt + (16 * jt + 16 + l16) * NSB + 32 * ks + 8 * g4);
                    t1 = mfma32(a1, cr[ks], t1);
                }
            }
        };
        floatx4 c0t, c1t;
        scores(0, c0t, c1t);
#pragma unroll 1
        for (int jt = 0; jt <= s; jt += 2) {
            floatx4 n0t, n1t;
            if (jt + 2 <= s) scores(jt + 2, n0t, n1t);
            const bool two = jt + 1 <= s;
            float m0[4], m1[4];
            mask_tile(c0t, jt, m0);
            if (two) mask_tile(c1t, jt + 1, m1);
            const unsigned p00 = pack2(m0[0], m0[1]), p01 = pack2(m0[2], m0[3]);
            if (two) {
                const u32x4 pb = {p00, p01, pack2(m1[0], m1[1]), pack2(m1[2], m1[3])};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint16_t* xr = XT + (16 * q + l16) * XS + xy;
                    const u32x2 xa = *reinterpret_cast<const u32x2*>(xr + 16 * (jt ^ q));
                    const u32x2 xb = *reinterpret_cast<const u32x2*>(xr + 16 * ((jt + 1) ^ q));
                    acc[q] = mfma32(u32x4{xa[0], xa[1], xb[0], xb[1]}, pb, acc[q]);
                }
            } else {
                const u32x2 pb = {p00, p01};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const u32x2 xa = *reinterpret_cast<const u32x2*>(XT + (16 * q + l16) * XS + xy + 16 * (jt ^ q));
                    acc[q] = mfma16(xa, pb, acc[q]);
                }
            }
            c0t = n0t;
            c1t = n1t;
        }
        if (ti < nq) {
            const int64_t yo = ((b * L + c * Q + ti) * H + h) * int64_t(Pcol) + p_off;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int p = 16 * q + 4 * g4;
                if (GP && p >= Pin) continue;  // Pin is a multiple of 8
                floatx4 v = acc[q];
                if (ym >= 2) v += *reinterpret_cast<const floatx4*>(ypart + yo + p);
                if (ym == 1 || ym == 3)
                    *reinterpret_cast<floatx4*>(ypart + yo + p) = v;
                else
                    *reinterpret_cast<u32x2*>(y + yo + p) = u32x2{pack2(v[0], v[1]), pack2(v[2], v[3])};
            }
        }

        // state update (decay and the chunk's inputs; no rotation in the absolute frame)
        const int te = nq - 1;
        const float decE = sc[192 + te];
        Tacc += sc[320 + te];
#pragma unroll
        for (int m = 0; m < MRW * 4; ++m) gst[m] *= decE;
        // A operand (w B~)^T: row n, k = 8 consecutive rho, from the row-major B~
        // through transposing LDS loads, scaled by the state weight
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int rb = 32 * ks + 8 * g4;
            u32x4 xb[4];
#pragma unroll
            for (int pt = 0; pt < 4; ++pt)
                xb[pt] = *reinterpret_cast<const u32x4*>(XT + (16 * pt + l16) * XS + xs[pt & 1] + 32 * (ks ^ (pt >> 1)));
            const floatx4 w0 = *reinterpret_cast<const floatx4*>(sc + 256 + rb);
            const floatx4 w1 = *reinterpret_cast<const floatx4*>(sc + 260 + rb);
#pragma unroll
            for (int mr = 0; mr < MRW; ++mr) {
                if (mr >= ntc) continue;
                const int n0 = 16 * (nt0 + mr);
                const u32x2 lo = load_tr(Bt + (rb + (l16 >> 2)) * NSB + n0 + 4 * (l16 & 3));
                const u32x2 hi = load_tr(Bt + (rb + 4 + (l16 >> 2)) * NSB + n0 + 4 * (l16 & 3));
                const u32x4 a = {scale2(lo[0], w0[0], w0[1]), scale2(lo[1], w0[2], w0[3]), scale2(hi[0], w1[0], w1[1]),
                                 scale2(hi[1], w1[2], w1[3])};
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) gst[mr * 4 + pt] = mfma32(a, xb[pt], gst[mr * 4 + pt]);
            }
        }
#pragma unroll
        for (int mr = 0; mr < MRW; ++mr) {
            if (mr >= ntc) continue;
            const int nt = nt0 + mr;
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                const int m = mr * 4 + pt;
                const int p = 16 * pt + l16;
                *reinterpret_cast<u32x2*>(gTn + p * NS + 16 * nt + 4 * g4) =
                    u32x2{pack2(gst[m][0], gst[m][1]), pack2(gst[m][2], gst[m][3])};
            }
        }
        lds_barrier();
    }
    if (h_out) {
        // back from the absolute frame: pair k turned by omega_k times the total step
#pragma unroll
        for (int mr = 0; mr < MRW; ++mr) {
            if (mr >= ntc) continue;
            CS t[2];
#pragma unroll
            for (int hp = 0; hp < 2; ++hp) {
                const double rv = double(omk(8 * (nt0 + mr) + 2 * g4 + hp)) * kInv2PiD * Tacc;
                const float r = float(rv - floor(rv));
                t[hp] = CS{__builtin_amdgcn_cosf(r), __builtin_amdgcn_sinf(r)};
            }
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                const int m = mr * 4 + pt, nt = nt0 + mr;
                const int p = 16 * pt + l16;
                float v[4];
#pragma unroll
                for (int hp = 0; hp < 2; ++hp) {
                    const float a0 = gst[m][2 * hp], a1 = gst[m][2 * hp + 1];
                    v[2 * hp] = t[hp].c * a0 - t[hp].s * a1;
                    v[2 * hp + 1] = t[hp].s * a0 + t[hp].c * a1;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int n = 16 * nt + 4 * g4 + e;
                    if (n < Nin && p < Pin) h_out[(bh * Nrow + n_off + n) * Pcol + p_off + p] = v[e];
                }
            }
        }
    }
}

// Calls f(GEN, YM, GP) with the instance for a pass: the exact N = 128, P = 64
// problem, or a general pass of the given kind.
template <class F>
hipError_t dispatch_pass(bool gen, const PassArgs& pa, F&& f) {
    using std::integral_constant;
    if (!gen) return f(integral_constant<bool, false>{}, integral_constant<int, 0>{}, integral_constant<bool, false>{});
    const bool gp = pa.pcol != P;
    auto with_ym = [&](auto g) {
        switch (pa.ym) {
            case 0: return f(integral_constant<bool, true>{}, integral_constant<int, 0>{}, g);
            case 1: return f(integral_constant<bool, true>{}, integral_constant<int, 1>{}, g);
            case 2: return f(integral_constant<bool, true>{}, integral_constant<int, 2>{}, g);
            case 3: return f(integral_constant<bool, true>{}, integral_constant<int, 3>{}, g);
        }
        return hipErrorInvalidValue;
    };
    return gp ? with_ym(integral_constant<bool, true>{}) : with_ym(integral_constant<bool, false>{});
}

hipError_t launch_ws_r1(const PrefillArgs& a, const PassArgs& pa, bool gen) {
    const int64_t nbh = a.b * a.H;
    return dispatch_pass(gen, pa, [&](auto g, auto ym, auto gp) {
        constexpr bool GEN = decltype(g)::value, GP = decltype(gp)::value;
        constexpr int YM = decltype(ym)::value;
        auto kern = a.omega ? prefill_ws_r1_kernel<true, GEN, YM, GP> : prefill_ws_r1_kernel<false, GEN, YM, GP>;
        hipLaunchKernelGGL(kern, dim3(unsigned(nbh)), dim3(64 * (ws1::NCW + ws1::NSW)), 0, a.stream,
                           static_cast<const uint16_t*>(a.x), a.dt, a.A, a.omega, a.lam,
                           static_cast<const uint16_t*>(a.B), static_cast<const uint16_t*>(a.C), a.D, a.h0,
                           static_cast<uint16_t*>(a.y), a.h_out, static_cast<const uint16_t*>(a.carry_B),
                           static_cast<const uint16_t*>(a.carry_x), a.L, a.H, a.G, a.chunk, a.plan.n_chunks, nbh, pa,
                           a.dt_bias, a.raw_steps);
        return hipGetLastError();
    });
}

template <int R, int NW>
hipError_t launch_r(const PrefillArgs& a, const PassArgs& pa, bool gen) {
    const int64_t nbh = a.b * a.H;
    SegArgs sa{a.plan.segments, a.plan.chunks_per_segment, nullptr, nullptr, nullptr, nullptr, kLookbackSpinLimit};
    // M3_LOOKBACK_SPIN_LIMIT (polls, >= 0) overrides the bound: 0 makes every wait
    // give up at once, which exercises the error report
    if (const char* env = getenv("M3_LOOKBACK_SPIN_LIMIT")) sa.spin_limit = atol(env) > 0 ? atol(env) : 0;
    if (sa.nseg > 1) {
        if (pa.ym != 0) return hipErrorInvalidValue;  // segments only in a single row pass
        const PrefillWorkspace w =
            prefill_workspace_layout(a.b, a.L, a.H, a.P, a.N, a.R, a.plan.segments, a.plan.path);
        char* base = static_cast<char*>(a.workspace);
        sa.ctrl = reinterpret_cast<unsigned*>(base + w.ctrl_off);
        sa.agg = reinterpret_cast<float*>(base + w.agg_off);
        sa.incl = reinterpret_cast<float*>(base + w.incl_off);
        sa.tr = reinterpret_cast<double*>(base + w.tr_off);
        // ticket, error flag and per-segment flags start at zero (a kernel, so
        // the call stays capturable in a graph)
        const hipError_t e = launch_copy_or_zero(sa.ctrl, nullptr, 2 + nbh * sa.nseg, a.stream);
        if (e != hipSuccess) return e;
    }
    return dispatch_pass(gen, pa, [&](auto g, auto ym, auto gp) {
        constexpr bool GEN = decltype(g)::value, GP = decltype(gp)::value;
        constexpr int YM = decltype(ym)::value;
        hipLaunchKernelGGL((prefill_mfma_kernel<R, NW, GEN, YM, GP>), dim3(unsigned(nbh * sa.nseg)), dim3(64 * NW),
                           0, a.stream, static_cast<const uint16_t*>(a.x), a.dt, a.A, a.omega, a.lam,
                           static_cast<const uint16_t*>(a.B), static_cast<const uint16_t*>(a.C), a.D, a.h0,
                           static_cast<uint16_t*>(a.y), a.h_out, static_cast<const uint16_t*>(a.carry_B),
                           static_cast<const uint16_t*>(a.carry_x), a.L, a.H, a.G, a.chunk, a.plan.n_chunks, nbh, pa,
                           sa, a.dt_bias, a.raw_steps);
        return hipGetLastError();
    });
}

}  // namespace

// N and P multiples of 8: up to 128 rows and 64 columns in one pass (zero-padded
// below: the loads of B, C and x rows stop at the caller's sizes); beyond, in
// passes of 128 rows (outputs summed in fp32 in the workspace) and 64 columns
static_assert(N == kMfmaN && P == kMfmaP, "one pass of the chunked kernels");

hipError_t launch_prefill_mfma(const PrefillArgs& a) {
    if (ws4_supported(a)) return launch_prefill_ws4(a);
    if (a.b * a.H * a.plan.segments > 0x7fffffff) return hipErrorInvalidValue;
    if (a.R == 1 && a.plan.segments != 1) return hipErrorInvalidValue;
    const int row_passes = (a.N + N - 1) / N, col_passes = (a.P + P - 1) / P;
    const bool gen = a.N != N || a.P != P || a.R == 3;
    float* ypart = nullptr;
    if (row_passes > 1) {
        const PrefillWorkspace w =
            prefill_workspace_layout(a.b, a.L, a.H, a.P, a.N, a.R, a.plan.segments, a.plan.path);
        ypart = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + w.ypart_off);
    }
    for (int j = 0; j < col_passes; ++j)
        for (int k = 0; k < row_passes; ++k) {
            PassArgs pa;
            pa.nin = a.N - k * N < N ? a.N - k * N : N;
            pa.nrow = a.N;
            pa.n_off = k * N;
            pa.pin = a.P - j * P < P ? a.P - j * P : P;
            pa.pcol = a.P;
            pa.p_off = j * P;
            pa.rin = a.R;
            pa.ym = row_passes == 1 ? 0 : k == 0 ? 1 : k == row_passes - 1 ? 2 : 3;
            pa.ypart = ypart;
            hipError_t e;
            switch (a.R) {
                case 1: e = launch_ws_r1(a, pa, gen); break;
                case 2: e = launch_r<2, 4>(a, pa, gen); break;
                case 3:  // the R 4 kernel with a zero fourth rank
                case 4: e = launch_r<4, 4>(a, pa, gen); break;
                default: e = hipErrorInvalidValue;
            }
            if (e != hipSuccess) return e;
        }
    return hipSuccess;
}

}  // namespace m3
