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
// DPP row; the one over rows (dx) goes through LDS. A block of tokens' B, C,
// x, dy (and the previous token's B, x) is staged in LDS in the I/O type, one
// LDS word per row holding its RK ranks (RK = R rounded up to 1, 2 or 4, a
// compile-time count, so the rank loops do no padded work).
//
// h_t is needed in reverse order: a first pass stores the state before every
// block of kBackwardCheckpoint tokens in the workspace; each block is then run
// forward again from its checkpoint, keeping its states in a per-(b, h)
// scratch, and walked back.
// Gradients summed over several workgroups (dB and dC over the heads of a
// group, dA, domega, dD over batch and tokens, dcarry_B) are added with device
// atomics into arrays the launcher clears first; their summation order is not
// fixed. Everything else is written once.
#include "m3_device.h"
#include "m3_internal.h"

namespace m3 {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int NT = 1024;          // threads per workgroup
constexpr int NW = NT / 64;       // waves
constexpr int KMAX = 64;          // rotation pairs (N <= 128)
constexpr int PMAX = 64;          // columns (P <= 64)
constexpr int SV = 8;             // state entries per thread
constexpr int BT = kBackwardCheckpoint;  // tokens per block: staged in LDS at once, one checkpoint each
constexpr int STATE = NT * SV;    // floats per stored state (covers 128 x 64)
static_assert(STATE == kBackwardStateFloats && 2 * KMAX == 128 && PMAX == 64, "sizes the planner assumes");

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// an LDS word of 2 .. 16 bytes, read and written as one access
template <int BYTES>
struct Word;
template <>
struct Word<2> {
    typedef uint16_t type;
};
template <>
struct Word<4> {
    typedef uint32_t type;
};
template <>
struct Word<8> {
    typedef u32x2 type;
};
template <>
struct Word<16> {
    typedef u32x4 type;
};

template <int RK>
struct Vr {
    float f[RK];
};

// the RK ranks of one row (ranks past R are zero) in the I/O type
template <typename T, int RK>
struct Row {
    typedef typename Word<int(sizeof(T)) * RK>::type W;
    W w;
    __device__ Vr<RK> get() const {
        const W x = w;
        Vr<RK> out;
        if constexpr (sizeof(T) == 4) {
            __builtin_memcpy(out.f, &x, sizeof(x));
        } else {
            uint16_t u[RK];
            __builtin_memcpy(u, &x, sizeof(x));
#pragma unroll
            for (int r = 0; r < RK; ++r) out.f[r] = __uint_as_float(uint32_t(u[r]) << 16);
        }
        return out;
    }
};

// LDS image of one block: B and x of tokens t0 - 1 .. t1 - 1, C and dy of t0 .. t1 - 1
template <typename T, int RK>
struct Block {
    Row<T, RK> B[BT + 1][2 * KMAX];
    Row<T, RK> X[BT + 1][PMAX];
    Row<T, RK> C[BT][2 * KMAX];
    Row<T, RK> DY[BT][PMAX];
    float dt[BT], lam[BT];
};

constexpr float kInv2Pi = 0.15915494309189535f;

// e^{dt A} and (sin, cos)(dt omega) of one step: the hardware exp2 and the
// hardware sine / cosine, which take revolutions (the per-step angle is a few
// radians at most, so after fract() the result is good to ~1e-6 absolute)
__device__ __forceinline__ float step_decay(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
__device__ __forceinline__ void step_sincos(float theta, float* s, float* c) {
    const float r = __builtin_amdgcn_fractf(theta * kInv2Pi);
    *s = __builtin_amdgcn_sinf(r);
    *c = __builtin_amdgcn_cosf(r);
}

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
// sum over the 4 DPP rows of the wave (lanes l, l ^ 16, l ^ 32, l ^ 48)
__device__ __forceinline__ float rows_sum4(float v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

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

template <typename T, int RK>
struct Bw {
    const BackwardArgs& a;
    Block<T, RK>& s;
    int64_t b;
    int h, g, K;
    int tid, k, c;
    __device__ Bw(const BackwardArgs& a_, Block<T, RK>& s_, int64_t bh) : a(a_), s(s_) {
        b = bh / a.H;
        h = int(bh % a.H);
        g = h / (a.H / a.G);
        K = a.N / 2;
        tid = threadIdx.x;
        k = tid >> 4;
        c = tid & 15;
    }
    __device__ const T* brow(int64_t t) const {  // B of token t (t = -1: the carry; NULL: zeros)
        return t >= 0 ? static_cast<const T*>(a.B) + ((b * a.L + t) * a.G + g) * int64_t(a.R * a.N)
                      : (a.carry_B ? static_cast<const T*>(a.carry_B) + (b * a.G + g) * int64_t(a.R * a.N) : nullptr);
    }
    __device__ const T* xrow(int64_t t) const {
        return t >= 0 ? static_cast<const T*>(a.x) + ((b * a.L + t) * a.H + h) * int64_t(a.R * a.P)
                      : (a.carry_x ? static_cast<const T*>(a.carry_x) + (b * a.H + h) * int64_t(a.R * a.P) : nullptr);
    }
    __device__ static void put(Row<T, RK>& dst, int r, const T* src, int64_t i) {
        if constexpr (sizeof(T) == 4) {
            reinterpret_cast<float*>(&dst.w)[r] = src ? Io<T>::load(src, i) : 0.f;
        } else {
            reinterpret_cast<uint16_t*>(&dst.w)[r] = src ? reinterpret_cast<const uint16_t*>(src)[i] : uint16_t(0);
        }
    }
    // Stage tokens [t0, t1): B, x also of t0 - 1; C, dy only when full. Every global
    // load of the block is issued before the first LDS store (its latency is paid
    // once per block). Rows are copied a 32-bit word at a time: a row is the N (or P)
    // entries of one (token, rank), word i holds entries EPW i .. EPW i + EPW - 1, and
    // they land in the LDS rows' rank slot r (the ranks of an LDS row are contiguous).
    static constexpr int EPW = 4 / int(sizeof(T));          // entries per 32-bit word
    static constexpr int WN = 2 * KMAX / EPW, WP = PMAX / EPW;  // most words per B/C, x/dy row
    static constexpr int PB = NT / WN, PX = NT / WP;           // rows per pass
    static constexpr int MB = ((BT + 1) * RK + PB - 1) / PB, MC = (BT * RK + PB - 1) / PB;
    static constexpr int MX = ((BT + 1) * RK + PX - 1) / PX, MY = (BT * RK + PX - 1) / PX;
    __device__ static void put_word(Row<T, RK>* row, int r, uint32_t v) {  // entries EPW i .. of rows row[0..]
        if constexpr (sizeof(T) == 4) {
            reinterpret_cast<float*>(&row[0].w)[r] = __uint_as_float(v);
        } else {
            reinterpret_cast<uint16_t*>(&row[0].w)[r] = uint16_t(v);
            reinterpret_cast<uint16_t*>(&row[1].w)[r] = uint16_t(v >> 16);
        }
    }
    __device__ void load_block(int64_t t0, int64_t t1, bool full) {
        const int nt = int(t1 - t0), R = a.R, N = a.N, P = a.P;
        const int wn = N / EPW, wp = P / EPW;  // N even; P even for bf16 (checked by the host)
        const unsigned invR = (65536u + unsigned(R) - 1u) / unsigned(R);  // q / R exact for q < 16384
        const int bi = tid % WN, bq = tid / WN, xi = tid % WP, xq = tid / WP;
        uint32_t vb[MB], vc[MC], vx[MX], vy[MY];
        const int nbr = (nt + 1) * R, ncr = full ? nt * R : 0;
#pragma unroll
        for (int u = 0; u < MB; ++u) {
            const int q = bq + u * PB;
            if (q < nbr && bi < wn) {
                const int j = int((unsigned(q) * invR) >> 16), r = q - j * R;
                const T* src = brow(t0 - 1 + j);
                vb[u] = src ? reinterpret_cast<const uint32_t*>(src + int64_t(r) * N)[bi] : 0u;
            }
        }
#pragma unroll
        for (int u = 0; u < MC; ++u) {
            const int q = bq + u * PB;
            if (q < ncr && bi < wn) {
                const int j = int((unsigned(q) * invR) >> 16), r = q - j * R;
                const T* src = static_cast<const T*>(a.C) + ((b * a.L + t0 + j) * a.G + g) * int64_t(R * N);
                vc[u] = reinterpret_cast<const uint32_t*>(src + int64_t(r) * N)[bi];
            }
        }
#pragma unroll
        for (int u = 0; u < MX; ++u) {
            const int q = xq + u * PX;
            if (q < nbr && xi < wp) {
                const int j = int((unsigned(q) * invR) >> 16), r = q - j * R;
                const T* src = xrow(t0 - 1 + j);
                vx[u] = src ? reinterpret_cast<const uint32_t*>(src + int64_t(r) * P)[xi] : 0u;
            }
        }
#pragma unroll
        for (int u = 0; u < MY; ++u) {
            const int q = xq + u * PX;
            if (q < ncr && xi < wp) {
                const int j = int((unsigned(q) * invR) >> 16), r = q - j * R;
                const T* src = static_cast<const T*>(a.dy) + ((b * a.L + t0 + j) * a.H + h) * int64_t(R * P);
                vy[u] = reinterpret_cast<const uint32_t*>(src + int64_t(r) * P)[xi];
            }
        }
        float dtv = 0.f, lmv = 0.f;
        if (tid < nt) {
            const int64_t i = (b * a.L + t0 + tid) * a.H + h;
            dtv = a.dt[i];
            lmv = lam_at(a.lam, i);
        }
#pragma unroll
        for (int u = 0; u < MB; ++u) {
            const int q = bq + u * PB;
            if (q < nbr && bi < wn) {
                const int j = int((unsigned(q) * invR) >> 16), r = q - j * R;
                put_word(&s.B[j][EPW * bi], r, vb[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < MC; ++u) {
            const int q = bq + u * PB;
            if (q < ncr && bi < wn) {
                const int j = int((unsigned(q) * invR) >> 16), r = q - j * R;
                put_word(&s.C[j][EPW * bi], r, vc[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < MX; ++u) {
            const int q = xq + u * PX;
            if (q < nbr && xi < wp) {
                const int j = int((unsigned(q) * invR) >> 16), r = q - j * R;
                put_word(&s.X[j][EPW * xi], r, vx[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < MY; ++u) {
            const int q = xq + u * PX;
            if (q < ncr && xi < wp) {
                const int j = int((unsigned(q) * invR) >> 16), r = q - j * R;
                put_word(&s.DY[j][EPW * xi], r, vy[u]);
            }
        }
        if (tid < nt) {
            s.dt[tid] = dtv;
            s.lam[tid] = lmv;
        }
    }
    __device__ float om_k() const { return k < K ? om_at(a.omega ? a.omega + int64_t(h) * K : nullptr, k) : 0.f; }
    // u = B x^T at this thread's entries, from block token slot j
    __device__ void outer(int j, float (&u)[2][4]) const {
        const Vr<RK> b0 = s.B[j][2 * k].get(), b1 = s.B[j][2 * k + 1].get();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const Vr<RK> xv = s.X[j][c + 16 * q].get();
            float s0 = b0.f[0] * xv.f[0], s1 = b1.f[0] * xv.f[0];
#pragma unroll
            for (int r = 1; r < RK; ++r) {
                s0 += b0.f[r] * xv.f[r];
                s1 += b1.f[r] * xv.f[r];
            }
            u[0][q] = s0;
            u[1][q] = s1;
        }
    }
    // forward step of block slot j (token t0 + j) on this thread's entries
    __device__ void fwd_step(int j, float (&hs)[2][4], float (&up)[2][4], float A, float om) const {
        float u[2][4];
        outer(j + 1, u);
        const float d = s.dt[j], l = s.lam[j];
        const float al = step_decay(d * A), gam = l * d, del = (1.f - l) * d;
        float sn, cs;
        step_sincos(d * om, &sn, &cs);
        const float ca = al * cs, sa = al * sn;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float g0 = hs[0][q] + del * up[0][q], g1 = hs[1][q] + del * up[1][q];
            hs[0][q] = ca * g0 - sa * g1 + gam * u[0][q];
            hs[1][q] = sa * g0 + ca * g1 + gam * u[1][q];
            up[0][q] = u[0][q];
            up[1][q] = u[1][q];
        }
    }
};

template <typename T, int RK>
__global__ void __launch_bounds__(NT) backward_kernel(BackwardArgs a) {
    static_assert(sizeof(Block<T, RK>) % 4 == 0, "the block image is cleared in 4-byte words");
    __shared__ Block<T, RK> sBlk;
    __shared__ floatx4 sRed[2][NW][PMAX];  // dx partials: rows of each wave summed, double-buffered
    __shared__ float sScal[2][NW][4];

    const int64_t bh = blockIdx.x;
    Bw<T, RK> w(a, sBlk, bh);
    const int tid = w.tid, k = w.k, c = w.c, K = w.K, wave = tid >> 6;
    const int64_t L = a.L;
    const float A = a.A[w.h], Dh = a.D[w.h];
    const float om = w.om_k();
    const int64_t nblk = (L + BT - 1) / BT;
    float* ck = a.workspace + bh * nblk * int64_t(STATE);                                      // checkpoints
    float* scr = a.workspace + (a.b * a.H) * nblk * int64_t(STATE) + bh * int64_t(BT) * STATE;  // block states

    // zero the block image once: ranks past R, rows past N, columns past P stay zero
    for (int e = tid; e < int(sizeof(Block<T, RK>) / 4); e += NT) reinterpret_cast<float*>(&sBlk)[e] = 0.f;
    __syncthreads();

    // ---- 1. forward over the sequence, the state stored before every block
    float hs[2][4], up[2][4];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int n = 2 * k + r, p = c + 16 * q;
            hs[r][q] = (a.h0 && k < K && p < a.P) ? a.h0[(bh * a.N + n) * int64_t(a.P) + p] : 0.f;
        }
    for (int64_t blk = 0; blk < nblk; ++blk) {
        const int64_t t0 = blk * BT, t1 = t0 + BT < L ? t0 + BT : L;
        store8(ck + blk * int64_t(STATE) + tid * SV, hs);
        w.load_block(t0, t1, false);
        __syncthreads();
        w.outer(0, up);
        for (int j = 0; j < int(t1 - t0); ++j) w.fwd_step(j, hs, up, A, om);
        __syncthreads();
    }

    // ---- 2. backward, block by block from the end
    float ad[2][4], e[2][4];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int n = 2 * k + r, p = c + 16 * q;
            ad[r][q] = (a.dh_out && k < K && p < a.P) ? a.dh_out[(bh * a.N + n) * int64_t(a.P) + p] : 0.f;
            e[r][q] = 0.f;
        }
    float dA_acc = 0.f, dom_acc = 0.f, dD_acc = 0.f;
    const int ro = tid >> 2, part = tid & 3;  // reducer: output (p, r) = (ro / 4, ro % 4), waves part*4 .. +3
    const int rp = ro >> 2, rr = ro & 3;
    const bool red_ok = rp < a.P && rr < a.R;

    for (int64_t blk = nblk - 1; blk >= 0; --blk) {
        const int64_t t0 = blk * BT, t1 = t0 + BT < L ? t0 + BT : L;
        const int nt = int(t1 - t0);
        // 2a. this block's inputs, and its states from the checkpoint
        w.load_block(t0, t1, true);
        load8(ck + blk * int64_t(STATE) + tid * SV, hs);
        __syncthreads();
        w.outer(0, up);
        for (int j = 0; j < nt; ++j) {
            w.fwd_step(j, hs, up, A, om);
            store8(scr + j * int64_t(STATE) + tid * SV, hs);  // read back by this thread only
        }
        // 2b. walk the block back (one barrier per token: partials double-buffered);
        // u of token t - 1 is u of the next (earlier) step
        float u[2][4];
        w.outer(nt, u);
        for (int j = nt - 1; j >= 0; --j) {
            const int64_t t = t0 + j;
            const int par = j & 1;
            float ht[2][4], uq[2][4];
            load8(scr + j * int64_t(STATE) + tid * SV, ht);
            w.outer(j, uq);
            const float d = sBlk.dt[j], l = sBlk.lam[j];
            const float al = step_decay(d * A), gam = l * d, del = (1.f - l) * d;
            float sn, cs;
            step_sincos(d * om, &sn, &cs);
            const Vr<RK> c0 = sBlk.C[j][2 * k].get(), c1 = sBlk.C[j][2 * k + 1].get();
            const Vr<RK> b0 = sBlk.B[j + 1][2 * k].get(), b1 = sBlk.B[j + 1][2 * k + 1].get();
            float dc0[RK], dc1[RK], db0[RK], db1[RK];
#pragma unroll
            for (int r = 0; r < RK; ++r) dc0[r] = dc1[r] = db0[r] = db1[r] = 0.f;
            float dxp[4][RK];
            float s_al = 0.f, s_ga = 0.f, s_de = 0.f, dth = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int p = c + 16 * q;
                const Vr<RK> dy = sBlk.DY[j][p].get(), xv = sBlk.X[j + 1][p].get();
                // a += C dy^T
#pragma unroll
                for (int r = 0; r < RK; ++r) {
                    ad[0][q] += c0.f[r] * dy.f[r];
                    ad[1][q] += c1.f[r] * dy.f[r];
                }
#pragma unroll
                for (int r = 0; r < RK; ++r) {
                    dc0[r] += ht[0][q] * dy.f[r];
                    dc1[r] += ht[1][q] * dy.f[r];
                }
                const float w0 = ht[0][q] - gam * u[0][q], w1 = ht[1][q] - gam * u[1][q];
                s_al += w0 * ad[0][q] + w1 * ad[1][q];
                dth += w0 * ad[1][q] - w1 * ad[0][q];
                s_ga += u[0][q] * ad[0][q] + u[1][q] * ad[1][q];
                // dg = alpha Rot^T a
                const float g0 = al * (cs * ad[0][q] + sn * ad[1][q]);
                const float g1 = al * (cs * ad[1][q] - sn * ad[0][q]);
                const float du0 = gam * ad[0][q] + e[0][q], du1 = gam * ad[1][q] + e[1][q];
                s_de += uq[0][q] * g0 + uq[1][q] * g1;
#pragma unroll
                for (int r = 0; r < RK; ++r) {
                    db0[r] += du0 * xv.f[r];
                    db1[r] += du1 * xv.f[r];
                    dxp[q][r] = du0 * b0.f[r] + du1 * b1.f[r];  // dx over this thread's two rows
                }
                ad[0][q] = g0;
                ad[1][q] = g1;
                e[0][q] = del * g0;
                e[1][q] = del * g1;
                u[0][q] = uq[0][q];
                u[1][q] = uq[1][q];
            }
            // column reductions inside the 16-lane row: dC, dB, the pair's angle
            dth = row_sum16(dth);
            if (k < K) {
                const int64_t rowb = ((w.b * L + t) * a.G + w.g) * int64_t(a.R * a.N);
#pragma unroll
                for (int r = 0; r < RK; ++r) {
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
            // dx: the wave's four row pairs summed, one partial per wave and column
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                floatx4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int r = 0; r < RK; ++r) v[r] = rows_sum4(dxp[q][r]);
                if ((tid & 63) < 16) sRed[par][wave][c + 16 * q] = v;
            }
            {
                const float v0 = wave_sum(s_al), v1 = wave_sum(s_ga), v2 = wave_sum(s_de), v3 = wave_sum(s_om);
                if ((tid & 63) == 0) {
                    sScal[par][wave][0] = v0;
                    sScal[par][wave][1] = v1;
                    sScal[par][wave][2] = v2;
                    sScal[par][wave][3] = v3;
                }
            }
            __syncthreads();
            {
                float v = 0.f;
                if (red_ok) {
#pragma unroll
                    for (int q = 0; q < NW / 4; ++q) v += sRed[par][part * (NW / 4) + q][rp][rr];
                }
                v = quad_sum(v);
                if (red_ok && part == 0) {
                    const float dyv = sBlk.DY[j][rp].get().f[rr], xv = sBlk.X[j + 1][rp].get().f[rr];
                    a.dx[((w.b * L + t) * a.H + w.h) * int64_t(a.R * a.P) + rr * a.P + rp] = v + Dh * dyv;
                    dD_acc += dyv * xv;
                }
            }
            if (tid == 0) {
                float sa = 0.f, sg = 0.f, sd = 0.f, so = 0.f;
                for (int q = 0; q < NW; ++q) {
                    sa += sScal[par][q][0];
                    sg += sScal[par][q][1];
                    sd += sScal[par][q][2];
                    so += sScal[par][q][3];
                }
                const int64_t i = (w.b * L + t) * a.H + w.h;
                a.ddt[i] = A * sa + so + l * sg + (1.f - l) * sd;
                if (a.dlam) a.dlam[i] = d * (sg - sd);
                dA_acc += d * sa;
            }
        }
        __syncthreads();  // the reducers are done with this block's image before the next load
    }

    // ---- 3. what is left: dh0, the carry, and the summed parameter gradients
    if (a.dh0 && k < K)
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int p = c + 16 * q;
                if (p < a.P) a.dh0[(bh * a.N + 2 * k + r) * int64_t(a.P) + p] = ad[r][q];
            }
    if (a.dcarry_B) {
        // du_0 = e; the carry's B and x are in block slot 0 of the first block (still staged)
        const Vr<RK> b0 = sBlk.B[0][2 * k].get(), b1 = sBlk.B[0][2 * k + 1].get();
        float db0[RK], db1[RK];
#pragma unroll
        for (int r = 0; r < RK; ++r) db0[r] = db1[r] = 0.f;
        float dxp[4][RK];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const Vr<RK> xv = sBlk.X[0][c + 16 * q].get();
#pragma unroll
            for (int r = 0; r < RK; ++r) {
                db0[r] += e[0][q] * xv.f[r];
                db1[r] += e[1][q] * xv.f[r];
                dxp[q][r] = e[0][q] * b0.f[r] + e[1][q] * b1.f[r];
            }
        }
        if (k < K) {
            const int64_t rowb = (w.b * a.G + w.g) * int64_t(a.R * a.N);
#pragma unroll
            for (int r = 0; r < RK; ++r) {
                const float v0 = row_sum16(db0[r]), v1 = row_sum16(db1[r]);
                if (c == 0 && r < a.R) {
                    atomicAdd(a.dcarry_B + rowb + r * a.N + 2 * k, v0);
                    atomicAdd(a.dcarry_B + rowb + r * a.N + 2 * k + 1, v1);
                }
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            floatx4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < RK; ++r) v[r] = rows_sum4(dxp[q][r]);
            if ((tid & 63) < 16) sRed[0][wave][c + 16 * q] = v;
        }
        __syncthreads();
        float v = 0.f;
        if (red_ok) {
#pragma unroll
            for (int q = 0; q < NW / 4; ++q) v += sRed[0][part * (NW / 4) + q][rp][rr];
        }
        v = quad_sum(v);
        if (red_ok && part == 0) a.dcarry_x[(w.b * a.H + w.h) * int64_t(a.R * a.P) + rr * a.P + rp] = v;
    }
    if (tid == 0) atomicAdd(a.dA + w.h, dA_acc);
    if (a.domega && c == 0 && k < K) atomicAdd(a.domega + int64_t(w.h) * K + k, dom_acc);
    if (red_ok && part == 0) atomicAdd(a.dD + w.h, dD_acc);
}

template <typename T, int RK>
hipError_t launch_rk(const BackwardArgs& a) {
    const int64_t nbh = a.b * a.H;
    hipLaunchKernelGGL((backward_kernel<T, RK>), dim3(unsigned(nbh)), dim3(NT), 0, a.stream, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const BackwardArgs& a) {
    return a.R == 1 ? launch_rk<T, 1>(a) : a.R == 2 ? launch_rk<T, 2>(a) : launch_rk<T, 4>(a);
}

}  // namespace

struct Z0 {
    float* p;
    int64_t n;
    const float* src;
};

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
