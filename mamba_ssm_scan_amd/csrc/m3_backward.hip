// m3_backward.hip -- gradients of a prefill: reverse-mode through the recurrence,
// fp32 arithmetic, for N <= 128 (N even), P <= 64, R <= 4.
//
// Forward (per (batch b, head h), token t; "复值SSM × 广义梯形离散 × MIMO，线性模型的
// 全面重构" §2.1-§2.3, "Mamba-3架构技术解析" §2.1):
//   u_t = B_t x_t^T,  g_t = h_{t-1} + delta_t u_{t-1},
//   h_t = alpha_t Rot(dt_t omega) g_t + gamma_t u_t,  y_t = h_t^T C_t + D x_t
// with alpha = e^{dt A}, gamma = lambda dt, delta = (1 - lambda) dt.
//
// Backward, step by step in reverse with the adjoint a of h_t (a starts at the
// gradient of h_L) and e_t = delta_{t+1} dg_{t+1} (the next step's share of du_t):
//   a += C_t dy_t^T;  dC_t = h_t dy_t;  dx_t = D dy_t + du_t^T B_t;  dD += <dy_t, x_t>
//   w = h_t - gamma u_t (= alpha Rot g_t): <w, a> -> dt (times A) and A (times dt);
//     per pair k, <J w, a> (J: a quarter turn) -> dt (times omega_k) and omega_k (times dt)
//   dg = alpha Rot^T a;  du_t = gamma a + e_t;  <u_t, a> -> gamma;  <u_{t-1}, dg> -> delta
//   dB_t = du_t x_t;  a <- dg;  e_{t-1} = delta_t dg
// and gamma = lambda dt, delta = (1 - lambda) dt give d lambda and the rest of d dt.
//
// One workgroup of 1024 threads per (b, h). Thread (k, c) = (tid / 16, tid % 16)
// holds state rows 2k, 2k+1 (one rotation pair) at columns c + 16 j, j < 4:
// reductions over the columns (dC, dB, the pair's angle) stay inside a 16-lane
// DPP row; the one over rows (dx) goes through LDS. The token's B, C, x, dy
// (and the previous token's B, x) are staged in LDS as fp32, [row][4 ranks].
//
// h_t is needed in reverse order: a first pass stores the state every 32
// tokens in the workspace; each 32-token block is then run forward again from
// its checkpoint, keeping its states in a per-(b, h) scratch, and walked back.
// Gradients summed over several workgroups (dB and dC over the heads of a
// group, dA, domega, dD over batch and tokens, dcarry_B) are added with device
// atomics into arrays the launcher clears first; their summation order is not
// fixed. Everything else is written once.
#include "m3_device.h"
#include "m3_internal.h"

namespace m3 {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int NT = 1024;         // threads per workgroup
constexpr int KMAX = 64;         // rotation pairs (N <= 128)
constexpr int PMAX = 64;         // columns (P <= 64)
constexpr int SV = 8;            // state entries per thread
constexpr int CK = kBackwardCheckpoint;
constexpr int STATE = NT * SV;   // floats per stored state (covers 128 x 64)

// staged token inputs, fp32, 4 ranks per row (ranks past R are zero)
struct Stage {
    floatx4 B[2 * KMAX], C[2 * KMAX], Bp[2 * KMAX];  // [n][r]
    floatx4 X[PMAX], DY[PMAX], Xp[PMAX];            // [p][r]
    float dt, lam;
};

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
// sum over the 16 lanes of a DPP row (every lane gets it)
__device__ __forceinline__ float row_sum16(float v) {
    v += dpp<0xb1>(v);   // quad_perm [1, 0, 3, 2]
    v += dpp<0x4e>(v);   // quad_perm [2, 3, 0, 1]
    v += dpp<0x141>(v);  // row_half_mirror
    v += dpp<0x140>(v);  // row_mirror
    return v;
}
// sum over the 4 lanes of a quad
__device__ __forceinline__ float quad_sum(float v) {
    v += dpp<0xb1>(v);
    v += dpp<0x4e>(v);
    return v;
}
__device__ __forceinline__ float lane_read(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ float wave_sum(float v) {
    v = row_sum16(v);
    return lane_read(v, 0) + lane_read(v, 16) + lane_read(v, 32) + lane_read(v, 48);
}

template <typename T>
struct Bw {
    const BackwardArgs& a;
    int64_t b;
    int h, g, K;
    int tid, k, c;
    __device__ Bw(const BackwardArgs& a_, int64_t bh) : a(a_) {
        b = bh / a.H;
        h = int(bh % a.H);
        g = h / (a.H / a.G);
        K = a.N / 2;
        tid = threadIdx.x;
        k = tid >> 4;
        c = tid & 15;
    }
    __device__ const T* brow(int64_t t) const {  // B of token t (t = -1: the carry)
        return t >= 0 ? static_cast<const T*>(a.B) + ((b * a.L + t) * a.G + g) * int64_t(a.R * a.N)
                      : (a.carry_B ? static_cast<const T*>(a.carry_B) + (b * a.G + g) * int64_t(a.R * a.N) : nullptr);
    }
    __device__ const T* xrow(int64_t t) const {
        return t >= 0 ? static_cast<const T*>(a.x) + ((b * a.L + t) * a.H + h) * int64_t(a.R * a.P)
                      : (a.carry_x ? static_cast<const T*>(a.carry_x) + (b * a.H + h) * int64_t(a.R * a.P) : nullptr);
    }
    // rows [n][r] of an [R][rows] source (NULL: zeros) into dst[rows][4]
    __device__ void put_rows(floatx4* dst, const T* src, int rows) const {
        for (int e = tid; e < rows * a.R; e += NT) {
            const int n = e % rows, r = e / rows;
            reinterpret_cast<float*>(dst)[4 * n + r] = src ? Io<T>::load(src, int64_t(r) * rows + n) : 0.f;
        }
    }
    __device__ void stage_bx(Stage& s, int64_t t) const {  // B_t, x_t only
        put_rows(s.B, brow(t), a.N);
        put_rows(s.X, xrow(t), a.P);
        if (tid == 0 && t >= 0) {
            const int64_t i = (b * a.L + t) * a.H + h;
            s.dt = a.dt[i];
            s.lam = lam_at(a.lam, i);
        }
    }
    __device__ void stage_full(Stage& s, int64_t t) const {
        stage_bx(s, t);
        put_rows(s.C, static_cast<const T*>(a.C) + ((b * a.L + t) * a.G + g) * int64_t(a.R * a.N), a.N);
        put_rows(s.DY, static_cast<const T*>(a.dy) + ((b * a.L + t) * a.H + h) * int64_t(a.R * a.P), a.P);
        put_rows(s.Bp, brow(t - 1), a.N);
        put_rows(s.Xp, xrow(t - 1), a.P);
    }
    __device__ float om_k() const { return k < K ? om_at(a.omega ? a.omega + int64_t(h) * K : nullptr, k) : 0.f; }
    // u = B x^T at this thread's entries, from staged rows
    __device__ void outer(const floatx4* Bs, const floatx4* Xs, float (&u)[2][4]) const {
        const floatx4 b0 = Bs[2 * k], b1 = Bs[2 * k + 1];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const floatx4 xv = Xs[c + 16 * j];
            u[0][j] = b0[0] * xv[0] + b0[1] * xv[1] + b0[2] * xv[2] + b0[3] * xv[3];
            u[1][j] = b1[0] * xv[0] + b1[1] * xv[1] + b1[2] * xv[2] + b1[3] * xv[3];
        }
    }
    // one forward step on this thread's entries
    __device__ void fwd_step(const Stage& s, float (&hs)[2][4], float (&up)[2][4], float A, float om) const {
        float u[2][4];
        outer(s.B, s.X, u);
        const float d = s.dt, l = s.lam;
        const float al = expf(d * A), gam = l * d, del = (1.f - l) * d;
        float sn, cs;
        sincosf(d * om, &sn, &cs);
        const float ca = al * cs, sa = al * sn;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float g0 = hs[0][j] + del * up[0][j], g1 = hs[1][j] + del * up[1][j];
            hs[0][j] = ca * g0 - sa * g1 + gam * u[0][j];
            hs[1][j] = sa * g0 + ca * g1 + gam * u[1][j];
            up[0][j] = u[0][j];
            up[1][j] = u[1][j];
        }
    }
};

__device__ __forceinline__ void store8(float* p, const float (&v)[2][4]) {
    reinterpret_cast<floatx4*>(p)[0] = floatx4{v[0][0], v[0][1], v[0][2], v[0][3]};
    reinterpret_cast<floatx4*>(p)[1] = floatx4{v[1][0], v[1][1], v[1][2], v[1][3]};
}
__device__ __forceinline__ void load8(const float* p, float (&v)[2][4]) {
    const floatx4 a0 = reinterpret_cast<const floatx4*>(p)[0], a1 = reinterpret_cast<const floatx4*>(p)[1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[0][j] = a0[j];
        v[1][j] = a1[j];
    }
}

template <typename T>
__global__ void __launch_bounds__(NT) backward_kernel(BackwardArgs a) {
    __shared__ Stage sIn[2];
    __shared__ floatx4 sRed[KMAX * PMAX];  // dx partials [k][p][r]
    __shared__ float sScal[NT / 64][4];

    const int64_t bh = blockIdx.x;
    Bw<T> w(a, bh);
    const int tid = w.tid, k = w.k, c = w.c, K = w.K;
    const int64_t L = a.L;
    const float A = a.A[w.h], Dh = a.D[w.h];
    const float om = w.om_k();
    const int64_t nblk = (L + CK - 1) / CK;
    float* ck = a.workspace + bh * nblk * int64_t(STATE);                           // checkpoints
    float* scr = a.workspace + (a.b * a.H) * nblk * int64_t(STATE) + bh * int64_t(CK) * STATE;  // block states

    // zero both staging buffers once: ranks past R, rows past N and columns past P stay zero
    for (int e = tid; e < int(2 * sizeof(Stage) / 4); e += NT) reinterpret_cast<float*>(sIn)[e] = 0.f;
    __syncthreads();

    // ---- 1. forward over the sequence, the state stored before every block of CK tokens
    float hs[2][4], up[2][4];
    {
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = 2 * k + r, p = c + 16 * j;
                hs[r][j] = (a.h0 && k < K && p < a.P) ? a.h0[(bh * a.N + n) * int64_t(a.P) + p] : 0.f;
            }
        w.stage_bx(sIn[1], -1);  // the carry (zeros without one)
        __syncthreads();
        w.outer(sIn[1].B, sIn[1].X, up);
        if (L > 0) w.stage_bx(sIn[0], 0);
        __syncthreads();
    }
    for (int64_t t = 0; t < L; ++t) {
        if (t % CK == 0) store8(ck + (t / CK) * int64_t(STATE) + tid * SV, hs);
        if (t + 1 < L) w.stage_bx(sIn[(t + 1) & 1], t + 1);
        w.fwd_step(sIn[t & 1], hs, up, A, om);
        __syncthreads();
    }

    // ---- 2. backward, block by block from the end
    float ad[2][4], e[2][4];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = 2 * k + r, p = c + 16 * j;
            ad[r][j] = (a.dh_out && k < K && p < a.P) ? a.dh_out[(bh * a.N + n) * int64_t(a.P) + p] : 0.f;
            e[r][j] = 0.f;
        }
    float dA_acc = 0.f, dom_acc = 0.f, dD_acc = 0.f;
    const int ro = tid >> 2, part = tid & 3;  // reducer: output (p, r) = (ro / 4, ro % 4), k quarter
    const int rp = ro >> 2, rr = ro & 3;
    const bool red_ok = rp < a.P && rr < a.R;

    for (int64_t blk = nblk - 1; blk >= 0; --blk) {
        const int64_t t0 = blk * CK, t1 = t0 + CK < L ? t0 + CK : L;
        // 2a. this block's states, from its checkpoint
        load8(ck + blk * int64_t(STATE) + tid * SV, hs);
        w.stage_bx(sIn[1], t0 - 1);
        __syncthreads();
        w.outer(sIn[1].B, sIn[1].X, up);
        w.stage_bx(sIn[0], t0);
        __syncthreads();
        for (int64_t t = t0; t < t1; ++t) {
            if (t + 1 < t1) w.stage_bx(sIn[(t + 1 - t0) & 1], t + 1);
            w.fwd_step(sIn[(t - t0) & 1], hs, up, A, om);
            store8(scr + (t - t0) * int64_t(STATE) + tid * SV, hs);
            __syncthreads();
        }
        // 2b. walk the block back
        w.stage_full(sIn[(t1 - 1) & 1], t1 - 1);
        __syncthreads();
        for (int64_t t = t1 - 1; t >= t0; --t) {
            const Stage& s = sIn[t & 1];
            float ht[2][4], u[2][4], uq[2][4];
            load8(scr + (t - t0) * int64_t(STATE) + tid * SV, ht);
            w.outer(s.B, s.X, u);
            w.outer(s.Bp, s.Xp, uq);
            const float d = s.dt, l = s.lam;
            const float al = expf(d * A), gam = l * d, del = (1.f - l) * d;
            float sn, cs;
            sincosf(d * om, &sn, &cs);
            const floatx4 c0 = s.C[2 * k], c1 = s.C[2 * k + 1];
            const floatx4 b0 = s.B[2 * k], b1 = s.B[2 * k + 1];
            float dc0[4] = {0.f, 0.f, 0.f, 0.f}, dc1[4] = {0.f, 0.f, 0.f, 0.f};
            float db0[4] = {0.f, 0.f, 0.f, 0.f}, db1[4] = {0.f, 0.f, 0.f, 0.f};
            float s_al = 0.f, s_ga = 0.f, s_de = 0.f, dth = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int p = c + 16 * j;
                const floatx4 dy = s.DY[p], xv = s.X[p];
                // a += C dy^T
                ad[0][j] += c0[0] * dy[0] + c0[1] * dy[1] + c0[2] * dy[2] + c0[3] * dy[3];
                ad[1][j] += c1[0] * dy[0] + c1[1] * dy[1] + c1[2] * dy[2] + c1[3] * dy[3];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    dc0[r] += ht[0][j] * dy[r];
                    dc1[r] += ht[1][j] * dy[r];
                }
                const float w0 = ht[0][j] - gam * u[0][j], w1 = ht[1][j] - gam * u[1][j];
                s_al += w0 * ad[0][j] + w1 * ad[1][j];
                dth += w0 * ad[1][j] - w1 * ad[0][j];
                s_ga += u[0][j] * ad[0][j] + u[1][j] * ad[1][j];
                // dg = alpha Rot^T a
                const float g0 = al * (cs * ad[0][j] + sn * ad[1][j]);
                const float g1 = al * (cs * ad[1][j] - sn * ad[0][j]);
                const float du0 = gam * ad[0][j] + e[0][j], du1 = gam * ad[1][j] + e[1][j];
                s_de += uq[0][j] * g0 + uq[1][j] * g1;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    db0[r] += du0 * xv[r];
                    db1[r] += du1 * xv[r];
                }
                // dx partial over this thread's two rows
                sRed[k * PMAX + p] = floatx4{du0 * b0[0] + du1 * b1[0], du0 * b0[1] + du1 * b1[1],
                                             du0 * b0[2] + du1 * b1[2], du0 * b0[3] + du1 * b1[3]};
                ad[0][j] = g0;
                ad[1][j] = g1;
                e[0][j] = del * g0;
                e[1][j] = del * g1;
            }
            // column reductions inside the 16-lane row: dC, dB, the pair's angle
            dth = row_sum16(dth);
            if (k < K) {
                const int64_t rowb = ((w.b * L + t) * a.G + w.g) * int64_t(a.R * a.N);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float v0 = row_sum16(dc0[r]), v1 = row_sum16(dc1[r]);
                    const float u0 = row_sum16(db0[r]), u1 = row_sum16(db1[r]);
                    if (c == 0 && r < a.R) {
                        atomicAdd(a.dC + rowb + r * a.N + 2 * k, v0);
                        atomicAdd(a.dC + rowb + r * a.N + 2 * k + 1, v1);
                        atomicAdd(a.dB + rowb + r * a.N + 2 * k, u0);
                        atomicAdd(a.dB + rowb + r * a.N + 2 * k + 1, u1);
                    }
                }
            }
            if (c == 0) dom_acc += d * dth;
            const float s_om = (c == 0) ? om * dth : 0.f;
            {
                const float v0 = wave_sum(s_al), v1 = wave_sum(s_ga), v2 = wave_sum(s_de), v3 = wave_sum(s_om);
                if ((tid & 63) == 0) {
                    sScal[tid >> 6][0] = v0;
                    sScal[tid >> 6][1] = v1;
                    sScal[tid >> 6][2] = v2;
                    sScal[tid >> 6][3] = v3;
                }
            }
            __syncthreads();
            // row reduction of dx through LDS: 4 lanes per (p, r), 16 pairs each
            {
                float v = 0.f;
                if (red_ok) {
                    const int kb = 16 * part, ke = kb + 16 < K ? kb + 16 : K;
                    for (int kk = kb; kk < ke; ++kk) v += sRed[kk * PMAX + rp][rr];
                }
                v = quad_sum(v);
                if (red_ok && part == 0) {
                    const float dyv = s.DY[rp][rr], xv = s.X[rp][rr];
                    a.dx[((w.b * L + t) * a.H + w.h) * int64_t(a.R * a.P) + rr * a.P + rp] = v + Dh * dyv;
                    dD_acc += dyv * xv;
                }
            }
            if (tid == 0) {
                float sa = 0.f, sg = 0.f, sd = 0.f, so = 0.f;
                for (int q = 0; q < NT / 64; ++q) {
                    sa += sScal[q][0];
                    sg += sScal[q][1];
                    sd += sScal[q][2];
                    so += sScal[q][3];
                }
                const int64_t i = (w.b * L + t) * a.H + w.h;
                a.ddt[i] = A * sa + so + l * sg + (1.f - l) * sd;
                if (a.dlam) a.dlam[i] = d * (sg - sd);
                dA_acc += d * sa;
            }
            if (t > t0) w.stage_full(sIn[(t - 1) & 1], t - 1);
            __syncthreads();
        }
    }

    // ---- 3. what is left: dh0, the carry, and the summed parameter gradients
    if (a.dh0 && k < K)
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int p = c + 16 * j;
                if (p < a.P) a.dh0[(bh * a.N + 2 * k + r) * int64_t(a.P) + p] = ad[r][j];
            }
    if (a.dcarry_B) {
        // du_0 = e; the carry's B and x are in the staging buffer of token 0 (Bp, Xp)
        const Stage& s = sIn[0];
        const floatx4 b0 = s.Bp[2 * k], b1 = s.Bp[2 * k + 1];
        float db0[4] = {0.f, 0.f, 0.f, 0.f}, db1[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int p = c + 16 * j;
            const floatx4 xv = s.Xp[p];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                db0[r] += e[0][j] * xv[r];
                db1[r] += e[1][j] * xv[r];
            }
            sRed[k * PMAX + p] = floatx4{e[0][j] * b0[0] + e[1][j] * b1[0], e[0][j] * b0[1] + e[1][j] * b1[1],
                                         e[0][j] * b0[2] + e[1][j] * b1[2], e[0][j] * b0[3] + e[1][j] * b1[3]};
        }
        if (k < K) {
            const int64_t rowb = (w.b * a.G + w.g) * int64_t(a.R * a.N);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float v0 = row_sum16(db0[r]), v1 = row_sum16(db1[r]);
                if (c == 0 && r < a.R) {
                    atomicAdd(a.dcarry_B + rowb + r * a.N + 2 * k, v0);
                    atomicAdd(a.dcarry_B + rowb + r * a.N + 2 * k + 1, v1);
                }
            }
        }
        __syncthreads();
        float v = 0.f;
        if (red_ok) {
            const int kb = 16 * part, ke = kb + 16 < K ? kb + 16 : K;
            for (int kk = kb; kk < ke; ++kk) v += sRed[kk * PMAX + rp][rr];
        }
        v = quad_sum(v);
        if (red_ok && part == 0) a.dcarry_x[(w.b * a.H + w.h) * int64_t(a.R * a.P) + rr * a.P + rp] = v;
    }
    if (tid == 0) atomicAdd(a.dA + w.h, dA_acc);
    if (a.domega && c == 0 && k < K) atomicAdd(a.domega + int64_t(w.h) * K + k, dom_acc);
    if (red_ok && part == 0) atomicAdd(a.dD + w.h, dD_acc);
}

template <typename T>
hipError_t launch_t(const BackwardArgs& a) {
    const int64_t nbh = a.b * a.H;
    hipLaunchKernelGGL(backward_kernel<T>, dim3(unsigned(nbh)), dim3(NT), 0, a.stream, a);
    return hipGetLastError();
}

}  // namespace

struct Z0 {
    float* p;
    int64_t n;
    const float* src;
};

size_t backward_workspace_bytes(int64_t b, int32_t H, int64_t L) {
    const int64_t nblk = (L + CK - 1) / CK;
    return size_t(b) * size_t(H) * size_t(nblk + CK) * STATE * sizeof(float);
}

bool backward_supported(int32_t P, int32_t N, int32_t R) { return N <= 2 * KMAX && P <= PMAX && R <= 4; }

hipError_t launch_backward(const BackwardArgs& a) {
    if (a.b * a.H == 0) return hipSuccess;
    if (a.b * a.H > 0x7fffffff) return hipErrorInvalidValue;
    if (a.L == 0) {
        // no tokens: h_out = h0, so dh0 = dh_out, and nothing else depends on the loss
        const Z0 z0[] = {{a.dA, a.H, nullptr}, {a.dD, a.H, nullptr},
                         {a.domega, a.domega ? int64_t(a.H) * (a.N / 2) : 0, nullptr},
                         {a.dcarry_B, a.dcarry_B ? a.b * a.G * int64_t(a.R) * a.N : 0, nullptr},
                         {a.dcarry_x, a.dcarry_x ? a.b * a.H * int64_t(a.R) * a.P : 0, nullptr},
                         {a.dh0, a.dh0 ? a.b * a.H * int64_t(a.N) * a.P : 0, a.dh_out}};
        for (const Z0& q : z0) {
            if (!q.p || q.n == 0) continue;
            const hipError_t e = launch_copy_or_zero(reinterpret_cast<uint32_t*>(q.p),
                                                     reinterpret_cast<const uint32_t*>(q.src), q.n, a.stream);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    // clear the accumulated gradients (a kernel, so the call stays capturable)
    const int64_t rowsBC = a.b * a.L * a.G * int64_t(a.R) * a.N;
    struct Z { float* p; int64_t n; };
    const Z z[] = {{a.dB, rowsBC}, {a.dC, rowsBC}, {a.dA, a.H}, {a.dD, a.H},
                   {a.domega, a.domega ? int64_t(a.H) * (a.N / 2) : 0},
                   {a.dcarry_B, a.dcarry_B ? a.b * a.G * int64_t(a.R) * a.N : 0}};
    for (const Z& q : z) {
        if (!q.p || q.n == 0) continue;
        const hipError_t e = launch_copy_or_zero(reinterpret_cast<uint32_t*>(q.p), nullptr, q.n, a.stream);
        if (e != hipSuccess) return e;
    }
    return a.io == M3_BF16 ? launch_t<bf16_t>(a) : launch_t<float>(a);
}

}  // namespace m3
