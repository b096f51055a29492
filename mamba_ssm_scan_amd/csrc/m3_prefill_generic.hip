// m3_prefill_generic.hip -- chunked prefill for any sizes, fp32 arithmetic.
//
// This is the path for fp32 I/O and for shapes the MFMA kernel does not
// cover. One workgroup walks the chunks of one (batch, head); the running state
// lives in the workspace. Within a chunk of n tokens (local index i, j), with
// T_i the chunk-local cumulative step, S_i = A*T_i and Phi_i = omega*T_i:
//
//   y_i  = e^{S_i} C~_i^T g + sum_{j<=i} e^{S_i-S_j} (gamma_j + [j<i] delta_{j+1}) (C~_i . B~_j) x_j + D x_i
//   g'   = Rot(Phi_e) [ e^{S_e} g + sum_j e^{S_e-S_j} (gamma_j + delta_{j+1}) B~_j x_j^T ]
//
// where B~_j = Rot(-Phi_j) B_j, C~_i = Rot(-Phi_i) C_i (data-dependent RoPE,
// "复值SSM × 广义梯形离散 × MIMO，线性模型的全面重构" §2.2), the weights are the
// rows of the decay x width-2 convolution mask (same digest, Fig. 2), e is
// the chunk's last token and delta_{j+1} is the next token's (zero past the
// end). g is the state entering the chunk with the previous token's trapezoid
// term already added, so chunks couple only through g. C~_i . B~_j is C_i^T
// Rot(Phi_i - Phi_j) B_j, the relative turn. When the chunk's B~ and C~ fit
// in LDS next to the token scalars (2 Q R N floats, up to kRotCacheBytes),
// they are formed once per chunk and every contraction is a plain dot
// product; when the chunk's masked scores fit as well (Q^2 R^2 more floats),
// they are formed once per chunk too (cached = 2); otherwise the turns are
// recomputed where they are used.
#include "m3_device.h"
#include "m3_internal.h"

namespace m3 {
namespace {

constexpr int kThreads = 256;
constexpr size_t kRotCacheBytes = 128 * 1024;  // dynamic LDS limit of the cached forms

template <typename T>
__global__ void __launch_bounds__(kThreads)
prefill_generic_kernel(const T* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
                       const float* __restrict__ omega, const float* __restrict__ lam,
                       const T* __restrict__ B, const T* __restrict__ C, const float* __restrict__ D,
                       const float* __restrict__ h0, T* __restrict__ y, float* __restrict__ h_out,
                       const T* __restrict__ carry_B, const T* __restrict__ carry_x, float* __restrict__ state,
                       int64_t L, int H, int G, int P, int N, int R, int Q, const float* __restrict__ dt_bias,
                       int raw, int cached) {
    extern __shared__ float sm[];
    float* Tc = sm;          // [Q] chunk-local cumulative dt
    float* gam = sm + Q;     // [Q] lambda*dt
    float* dln = sm + 2 * Q; // [Q] (1-lambda)*dt of the following token
    float* Bt = sm + 3 * Q;                    // cached: [Q][R][N] B~ of the chunk
    float* Ct = Bt + int64_t(Q) * R * N;       // cached: [Q][R][N] C~
    float* Wm = Ct + int64_t(Q) * R * N;       // cached 2: [Q][R][Q][R] masked scores M_ij (C~_i . B~_j)

    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / H;
    const int h = int(bh % H);
    const int g = h / (H / G);
    const int K = N / 2;
    const float Ah = A[h], Dh = D[h];
    const float* om = omega ? omega + int64_t(h) * K : nullptr;
    float* st = state + bh * int64_t(N) * P;
    const StepIn si = step_in(dt_bias, raw, h);  // dt and lambda as given, or from raw projections

    // g = h0 + delta_0 * carry_B^T carry_x
    const float d0 = (1.f - si.lam(lam, (b * L) * H + h)) * si.dt(dt[(b * L) * H + h]);
    for (int e = tid; e < N * P; e += kThreads) {
        const int n = e / P, p = e % P;
        float v = h0 ? h0[bh * int64_t(N) * P + e] : 0.f;
        if (carry_B) {
            float u = 0.f;
            for (int r = 0; r < R; ++r)
                u += Io<T>::load(carry_B, ((b * G + g) * R + r) * int64_t(N) + n) *
                     Io<T>::load(carry_x, ((b * H + h) * R + r) * int64_t(P) + p);
            v += d0 * u;
        }
        st[e] = v;
    }
    __syncthreads();

    for (int64_t c0 = 0; c0 < L; c0 += Q) {
        const int nt = int(L - c0 < Q ? L - c0 : Q);
        if (tid == 0) {
            float acc = 0.f;
            for (int i = 0; i < nt; ++i) {
                const int64_t ti = (b * L + c0 + i) * H + h;
                const float d = si.dt(dt[ti]);
                acc += d;
                Tc[i] = acc;
                gam[i] = si.lam(lam, ti) * d;
                const int64_t tn = c0 + i + 1;
                dln[i] = tn < L ? (1.f - si.lam(lam, (b * L + tn) * H + h)) * si.dt(dt[(b * L + tn) * H + h]) : 0.f;
            }
        }
        __syncthreads();
        if (cached) {  // B~_j = Rot(-Phi_j) B_j and C~_j for every (token, rank, pair) of the chunk
            for (int e = tid; e < nt * R * K; e += kThreads) {
                const int j = e / (R * K), r = (e / K) % R, k = e % K;
                float s, c;
                sincosf(om_at(om, k) * Tc[j], &s, &c);
                const int64_t src = ((b * L + c0 + j) * G + g) * int64_t(R) * N + int64_t(r) * N + 2 * k;
                const float b0 = Io<T>::load(B, src), b1 = Io<T>::load(B, src + 1);
                const float c0v = Io<T>::load(C, src), c1v = Io<T>::load(C, src + 1);
                const int64_t o = (int64_t(j) * R + r) * N + 2 * k;
                Bt[o] = c * b0 + s * b1;
                Bt[o + 1] = c * b1 - s * b0;
                Ct[o] = c * c0v + s * c1v;
                Ct[o + 1] = c * c1v - s * c0v;
            }
            __syncthreads();
        }
        if (cached == 2) {  // the masked scores of the chunk's causal (i, j) pairs, rank by rank
            const int QR = Q * R;
            for (int e = tid; e < nt * R * nt * R; e += kThreads) {
                const int ir = e / (nt * R), jr = e % (nt * R);
                const int i = ir / R, j = jr / R;
                float v = 0.f;
                if (j <= i) {
                    const float* Ci = Ct + int64_t(ir) * N;
                    const float* Bj = Bt + int64_t(jr) * N;
                    for (int n = 0; n < N; ++n) v += Ci[n] * Bj[n];
                    v *= expf(Ah * (Tc[i] - Tc[j])) * (gam[j] + (j < i ? dln[j] : 0.f));
                }
                Wm[int64_t(ir) * QR + jr] = v;
            }
            __syncthreads();
        }

        // outputs of the chunk
        for (int e = tid; cached && e < nt * R * P; e += kThreads) {
            const int i = e / (R * P), r = (e / P) % R, p = e % P;
            const float* Cti = Ct + (int64_t(i) * R + r) * N;
            const float Ti = Tc[i];
            float inter = 0.f;
            for (int n = 0; n < N; ++n) inter += Cti[n] * st[n * P + p];
            float acc = expf(Ah * Ti) * inter;
            if (cached == 2) {
                const float* Wi = Wm + (int64_t(i) * R + r) * (int64_t(Q) * R);
                for (int j = 0; j <= i; ++j) {
                    const T* xj = x + ((b * L + c0 + j) * H + h) * int64_t(R) * P;
                    for (int rr = 0; rr < R; ++rr) acc += Wi[j * R + rr] * Io<T>::load(xj, int64_t(rr) * P + p);
                }
            }
            for (int j = 0; cached == 1 && j <= i; ++j) {
                const float m = expf(Ah * (Ti - Tc[j])) * (gam[j] + (j < i ? dln[j] : 0.f));
                const T* xj = x + ((b * L + c0 + j) * H + h) * int64_t(R) * P;
                for (int rr = 0; rr < R; ++rr) {
                    const float* Btj = Bt + (int64_t(j) * R + rr) * N;
                    float sc = 0.f;
                    for (int n = 0; n < N; ++n) sc += Cti[n] * Btj[n];
                    acc += m * sc * Io<T>::load(xj, int64_t(rr) * P + p);
                }
            }
            const int64_t yi = ((b * L + c0 + i) * H + h) * int64_t(R) * P + int64_t(r) * P + p;
            Io<T>::store(y, yi, acc + Dh * Io<T>::load(x, yi));
        }
        for (int e = tid; !cached && e < nt * R * P; e += kThreads) {
            const int i = e / (R * P), r = (e / P) % R, p = e % P;
            const T* Ci = C + ((b * L + c0 + i) * G + g) * int64_t(R) * N + int64_t(r) * N;
            const float Ti = Tc[i];
            float inter = 0.f;
            for (int k = 0; k < K; ++k) {
                float s, c;
                sincosf(om_at(om, k) * Ti, &s, &c);
                const float c0v = Io<T>::load(Ci, 2 * k), c1v = Io<T>::load(Ci, 2 * k + 1);
                inter += (c * c0v + s * c1v) * st[(2 * k) * P + p] + (c * c1v - s * c0v) * st[(2 * k + 1) * P + p];
            }
            float acc = expf(Ah * Ti) * inter;
            for (int j = 0; j <= i; ++j) {
                const float dT = Ti - Tc[j];
                const float m = expf(Ah * dT) * (gam[j] + (j < i ? dln[j] : 0.f));
                const T* Bj = B + ((b * L + c0 + j) * G + g) * int64_t(R) * N;
                const T* xj = x + ((b * L + c0 + j) * H + h) * int64_t(R) * P;
                for (int rr = 0; rr < R; ++rr) {
                    float sc = 0.f;
                    for (int k = 0; k < K; ++k) {
                        float s, c;
                        sincosf(om_at(om, k) * dT, &s, &c);
                        const float b0 = Io<T>::load(Bj, int64_t(rr) * N + 2 * k);
                        const float b1 = Io<T>::load(Bj, int64_t(rr) * N + 2 * k + 1);
                        const float c0v = Io<T>::load(Ci, 2 * k), c1v = Io<T>::load(Ci, 2 * k + 1);
                        sc += c0v * (c * b0 - s * b1) + c1v * (s * b0 + c * b1);
                    }
                    acc += m * sc * Io<T>::load(xj, int64_t(rr) * P + p);
                }
            }
            const int64_t yi = ((b * L + c0 + i) * H + h) * int64_t(R) * P + int64_t(r) * P + p;
            Io<T>::store(y, yi, acc + Dh * Io<T>::load(x, yi));
        }
        __syncthreads();

        // state passed to the next chunk
        const float Te = Tc[nt - 1];
        const float dec = expf(Ah * Te);
        for (int e = tid; e < K * P; e += kThreads) {
            const int k = e / P, p = e % P;
            float a0 = dec * st[(2 * k) * P + p], a1 = dec * st[(2 * k + 1) * P + p];
            for (int j = 0; j < nt; ++j) {
                const float w = expf(Ah * (Te - Tc[j])) * (gam[j] + dln[j]);
                const T* xj = x + ((b * L + c0 + j) * H + h) * int64_t(R) * P;
                if (cached) {
                    for (int r = 0; r < R; ++r) {
                        const float* Btj = Bt + (int64_t(j) * R + r) * N + 2 * k;
                        const float xv = w * Io<T>::load(xj, int64_t(r) * P + p);
                        a0 += Btj[0] * xv;
                        a1 += Btj[1] * xv;
                    }
                    continue;
                }
                float s, c;
                sincosf(om_at(om, k) * Tc[j], &s, &c);
                const T* Bj = B + ((b * L + c0 + j) * G + g) * int64_t(R) * N;
                for (int r = 0; r < R; ++r) {
                    const float b0 = Io<T>::load(Bj, int64_t(r) * N + 2 * k);
                    const float b1 = Io<T>::load(Bj, int64_t(r) * N + 2 * k + 1);
                    const float xv = w * Io<T>::load(xj, int64_t(r) * P + p);
                    a0 += (c * b0 + s * b1) * xv;
                    a1 += (c * b1 - s * b0) * xv;
                }
            }
            float s, c;
            sincosf(om_at(om, k) * Te, &s, &c);
            st[(2 * k) * P + p] = c * a0 - s * a1;
            st[(2 * k + 1) * P + p] = s * a0 + c * a1;
        }
        __syncthreads();
    }
    if (h_out)
        for (int e = tid; e < N * P; e += kThreads) h_out[bh * int64_t(N) * P + e] = st[e];
}

__global__ void copy_or_zero_kernel(uint32_t* __restrict__ dst, const uint32_t* __restrict__ src, int64_t n) {
    for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
        dst[i] = src ? src[i] : 0u;
}

template <typename T>
hipError_t launch_generic_t(const PrefillArgs& a) {
    const PrefillWorkspace ws = prefill_workspace_layout(a.b, a.L, a.H, a.P, a.N, a.R, a.plan.segments, a.plan.path);
    float* state = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + ws.state_off);
    // the chunk's B~ and C~ in LDS when they fit (chunk <= L does not change the need)
    const size_t base = size_t(3) * a.chunk * sizeof(float);
    const size_t rot = size_t(2) * a.chunk * a.R * a.N * sizeof(float);
    const size_t scores = size_t(a.chunk) * a.R * a.chunk * a.R * sizeof(float);
    const int cached = base + rot + scores <= kRotCacheBytes ? 2 : base + rot <= kRotCacheBytes ? 1 : 0;
    const size_t shmem = cached == 2 ? base + rot + scores : cached ? base + rot : base;
    const dim3 grid(unsigned(a.b * a.H));
    hipLaunchKernelGGL(prefill_generic_kernel<T>, grid, dim3(kThreads), shmem, a.stream,
                       static_cast<const T*>(a.x), a.dt, a.A, a.omega, a.lam, static_cast<const T*>(a.B),
                       static_cast<const T*>(a.C), a.D, a.h0, static_cast<T*>(a.y), a.h_out,
                       static_cast<const T*>(a.carry_B), static_cast<const T*>(a.carry_x), state, a.L, a.H, a.G,
                       a.P, a.N, a.R, a.chunk, a.dt_bias, a.raw_steps, cached);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_generic(const PrefillArgs& a) {
    if (a.b * a.H > 0x7fffffff) return hipErrorInvalidValue;
    return a.io == M3_BF16 ? launch_generic_t<bf16_t>(a) : launch_generic_t<float>(a);
}

hipError_t launch_copy_or_zero(uint32_t* dst, const uint32_t* src, int64_t n_words, hipStream_t s) {
    if (n_words <= 0) return hipSuccess;
    int64_t blocks = (n_words + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(copy_or_zero_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, dst, src, n_words);
    return hipGetLastError();
}

}  // namespace m3
