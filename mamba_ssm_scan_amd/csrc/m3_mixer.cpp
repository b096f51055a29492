// m3_mixer.cpp -- the mixer block around the recurrence: input projections,
// the input prologue, the recurrence (prefill or one decode step), the silu
// gate and the output projection, as one call.
//
// The PaperWeekly digest ("复值SSM × 广义梯形离散 × MIMO，线性模型的全面重构",
// §2.4 and Fig. 4) lists what one Mamba-3 block holds (the rotating state with
// the trapezoid rule, MIMO inputs, QK-norm plus bias after the B/C projection,
// no short convolution) without a block formula; the block here is the Mamba-2
// layout with those changes:
//   x = u W_x^T, z = u W_z^T, B_raw = u W_B^T, C_raw = u W_C^T, dt_raw = u W_dt^T, lambda_raw = u W_lambda^T
//   (B, C, dt, lambda) = prologue(...);  y = recurrence(x, dt, A, omega, lambda, B, C, D)
//   out = (y * silu(z)) W_out^T          (weights [out][in], as a linear layer stores them)
// The projections are plain library GEMMs (hipBLASLt, bf16 operands, fp32
// accumulation; dt_raw and lambda_raw are written in fp32, the rest in bf16);
// every other step is one of this library's kernels. Intermediates live in the
// caller's workspace; the mixer object holds the hipBLASLt handle and the
// chosen GEMM algorithms (per shape), so it must not be shared between threads.
// The first call for a GEMM shape times the library's candidate algorithms on
// the call's own operands and synchronises the stream once; calls captured in
// a graph should therefore follow one eager call of the same sizes. For few
// tokens (a decode step) the input projections fan out to three side streams of
// the mixer object (fork and join events on the caller's stream, so a captured
// call captures them too); the object must then not be used from two streams
// at once.
#include <hipblaslt/hipblaslt.h>

#include <cstdio>
#include <cstring>
#include <map>
#include <tuple>

#include "m3_internal.h"

namespace {

constexpr size_t kGemmWorkspace = size_t(32) << 20;  // hipBLASLt scratch per stream, in the caller's workspace
constexpr int kSide = 3;                              // side streams the decode-step projections fan out to
constexpr int64_t kFanOutMaxTokens = 1024;            // fan out only GEMMs this short (they cannot fill the chip)
constexpr int kCandidates = 64;                       // algorithms timed per GEMM shape at first use

size_t up256(size_t v) { return (v + 255) & ~size_t(255); }

struct Gemm {
    hipblasLtMatmulDesc_t op = nullptr;
    hipblasLtMatrixLayout_t a = nullptr, b = nullptr, d = nullptr;
    hipblasLtMatmulAlgo_t algo{};
    size_t ws = 0;
};

// offsets of the block's intermediates in the workspace (tokens T)
struct MixerLayout {
    size_t x, z, B, C, dt, lam, y, Blast, xlast, pre, gemm, total;
};

MixerLayout layout(const m3_dims* d, int32_t R, int32_t chunk, size_t* pre_bytes) {
    const size_t T = size_t(d->batch) * size_t(d->seqlen);
    const size_t HRP = size_t(d->heads) * R * d->headdim, GRN = size_t(d->groups) * R * d->dstate;
    MixerLayout L{};
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o += up256(bytes);
        return at;
    };
    L.x = take(T * HRP * 2);
    L.z = take(T * HRP * 2);
    L.B = take(T * GRN * 2);
    L.C = take(T * GRN * 2);
    L.dt = take(T * d->heads * 4);
    L.lam = take(T * d->heads * 4);
    L.y = take(T * HRP * 2);
    L.Blast = take(size_t(d->batch) * GRN * 2);
    L.xlast = take(size_t(d->batch) * HRP * 2);
    *pre_bytes = m3_prefill_workspace_size(d, R, chunk, M3_BF16);
    L.pre = take(*pre_bytes);
    L.gemm = take(kGemmWorkspace * (1 + kSide));
    L.total = o;
    return L;
}

}  // namespace

struct m3_mixer {
    hipblasLtHandle_t lt = nullptr;
    std::map<std::tuple<int64_t, int64_t, int64_t, int>, Gemm> gemms;
    // short input projections run concurrently: forked from the caller's stream to
    // these (default priority) and joined back with events
    hipStream_t side[kSide] = {};
    hipEvent_t fork = nullptr, join[kSide] = {};

    ~m3_mixer() {
        for (int i = 0; i < kSide; ++i) {
            if (side[i]) (void)hipStreamDestroy(side[i]);
            if (join[i]) (void)hipEventDestroy(join[i]);
        }
        if (fork) (void)hipEventDestroy(fork);
        for (auto& kv : gemms) {
            Gemm& g = kv.second;
            if (g.a) hipblasLtMatrixLayoutDestroy(g.a);
            if (g.b) hipblasLtMatrixLayoutDestroy(g.b);
            if (g.d) hipblasLtMatrixLayoutDestroy(g.d);
            if (g.op) hipblasLtMatmulDescDestroy(g.op);
        }
        if (lt) hipblasLtDestroy(lt);
    }

    // D[M][N] = U[M][K] W[N][K]^T, all row-major (W as a linear layer stores it, [out][in]);
    // U, W bf16, D bf16 (f32out = 0) or fp32. In hipBLASLt's column-major terms
    // D^T (N x M) = op(W') U^T with W' the K x N matrix of W's bytes and op a transpose.
    m3_status gemm(int64_t M, int64_t N, int64_t K, const void* U, const void* W, void* D, bool f32out, void* ws,
                   hipStream_t s) {
        if (M == 0 || N == 0) return M3_OK;
        const auto key = std::make_tuple(M, N, K, int(f32out));
        auto it = gemms.find(key);
        if (it == gemms.end()) {
            Gemm g;
            const hipDataType dtD = f32out ? HIP_R_32F : HIP_R_16BF;
            const int32_t opT = HIPBLAS_OP_T;
            bool ok = hipblasLtMatmulDescCreate(&g.op, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS &&
                      hipblasLtMatmulDescSetAttribute(g.op, HIPBLASLT_MATMUL_DESC_TRANSA, &opT, sizeof opT) ==
                          HIPBLAS_STATUS_SUCCESS &&
                      hipblasLtMatrixLayoutCreate(&g.a, HIP_R_16BF, uint64_t(K), uint64_t(N), K) ==
                          HIPBLAS_STATUS_SUCCESS &&
                      hipblasLtMatrixLayoutCreate(&g.b, HIP_R_16BF, uint64_t(K), uint64_t(M), K) ==
                          HIPBLAS_STATUS_SUCCESS &&
                      hipblasLtMatrixLayoutCreate(&g.d, dtD, uint64_t(N), uint64_t(M), N) == HIPBLAS_STATUS_SUCCESS;
            hipblasLtMatmulPreference_t pref = nullptr;
            int found = 0;
            hipblasLtMatmulHeuristicResult_t res[kCandidates];
            if (ok) {
                uint64_t cap = kGemmWorkspace;
                ok = hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS &&
                     hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &cap,
                                                           sizeof cap) == HIPBLAS_STATUS_SUCCESS &&
                     hipblasLtMatmulAlgoGetHeuristic(lt, g.op, g.a, g.b, g.d, g.d, pref, kCandidates, res, &found) ==
                         HIPBLAS_STATUS_SUCCESS &&
                     found > 0;
            }
            if (pref) hipblasLtMatmulPreferenceDestroy(pref);
            if (!ok) {
                if (g.a) hipblasLtMatrixLayoutDestroy(g.a);
                if (g.b) hipblasLtMatrixLayoutDestroy(g.b);
                if (g.d) hipblasLtMatrixLayoutDestroy(g.d);
                if (g.op) hipblasLtMatmulDescDestroy(g.op);
                return m3::set_error(M3_EHIP, "no hipBLASLt algorithm for a %lld x %lld x %lld bf16 GEMM (%s out)",
                                     (long long)M, (long long)N, (long long)K, f32out ? "fp32" : "bf16");
            }
            // the heuristic's first choice can leave most of the chip idle on skinny
            // shapes (few output tiles): time its candidates once on the real operands
            // and keep the fastest (not while the stream is being captured)
            int best = 0;
            hipStreamCaptureStatus cap_st = hipStreamCaptureStatusNone;
            if (found > 1 && hipStreamIsCapturing(s, &cap_st) == hipSuccess && cap_st == hipStreamCaptureStatusNone)
                best = fastest(g, res, found, U, W, D, ws, s);
            g.algo = res[best].algo;
            g.ws = res[best].workspaceSize;
            it = gemms.emplace(key, g).first;
        }
        const Gemm& g = it->second;
        return run(g, g.algo, U, W, D, ws, s);
    }

    m3_status run(const Gemm& g, const hipblasLtMatmulAlgo_t& algo, const void* U, const void* W, void* D, void* ws,
                  hipStream_t s) {
        const float one = 1.f, zero = 0.f;
        const hipblasStatus_t st = hipblasLtMatmul(lt, g.op, &one, W, g.a, U, g.b, &zero, D, g.d, D, g.d, &algo, ws,
                                                   kGemmWorkspace, s);
        if (st != HIPBLAS_STATUS_SUCCESS) return m3::set_error(M3_EHIP, "hipblasLtMatmul failed (%d)", int(st));
        return M3_OK;
    }

    // index of the fastest candidate: one warm-up call, then the best of 3 rounds of 3
    // timed calls each (HIP events on s; a single round let noise pick slower kernels)
    int fastest(const Gemm& g, const hipblasLtMatmulHeuristicResult_t* res, int n, const void* U, const void* W,
                void* D, void* ws, hipStream_t s) {
        hipEvent_t e0 = nullptr, e1 = nullptr;
        if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
            if (e0) (void)hipEventDestroy(e0);
            return 0;
        }
        int best = 0;
        float best_ms = 3.0e38f;
        for (int i = 0; i < n; ++i) {
            if (res[i].state != HIPBLAS_STATUS_SUCCESS || res[i].workspaceSize > kGemmWorkspace) continue;
            if (run(g, res[i].algo, U, W, D, ws, s) != M3_OK) continue;
            for (int round = 0; round < 3; ++round) {
                if (hipEventRecord(e0, s) != hipSuccess) break;
                for (int k = 0; k < 3; ++k) run(g, res[i].algo, U, W, D, ws, s);
                if (hipEventRecord(e1, s) != hipSuccess) break;
                float ms = 0.f;
                if (hipEventSynchronize(e1) == hipSuccess && hipEventElapsedTime(&ms, e0, e1) == hipSuccess &&
                    ms < best_ms) {
                    best_ms = ms;
                    best = i;
                }
            }
        }
        (void)hipEventDestroy(e0);
        (void)hipEventDestroy(e1);
        return best;
    }
};

namespace {

m3_status check_weights(const m3_mixer_weights* w) {
    if (!w) return m3::set_error(M3_EINVAL, "weights is NULL");
    if (w->d_model < 1) return m3::set_error(M3_EINVAL, "d_model %d < 1", w->d_model);
    const void* req[] = {w->W_x, w->W_z, w->W_B, w->W_C, w->W_dt, w->W_lambda, w->W_out, w->A, w->D};
    const char* names[] = {"W_x", "W_z", "W_B", "W_C", "W_dt", "W_lambda", "W_out", "A", "D"};
    for (int i = 0; i < 9; ++i)
        if (!req[i]) return m3::set_error(M3_EINVAL, "%s is NULL", names[i]);
    if (!(w->eps >= 0.f) || w->eps > 3.0e38f) return m3::set_error(M3_EINVAL, "eps must be finite and >= 0");
    return M3_OK;
}

// the four projections of ntok tokens into the workspace, the prologue in place
m3_status project_in(m3_mixer* m, const m3_mixer_weights* w, const m3_dims* d, int32_t R, int64_t ntok,
                     const void* u, char* ws, const MixerLayout& L, hipStream_t s) {
    const int64_t K = w->d_model, HRP = int64_t(d->heads) * R * d->headdim, GRN = int64_t(d->groups) * R * d->dstate;
    // Few tokens (a decode step): x on the caller's stream, z, (B, C) and (dt, lambda)
    // on the side streams, each with its own GEMM scratch, joined before the
    // prologue. Many tokens: all on the caller's stream (each GEMM fills the chip).
    const bool fan = ntok <= kFanOutMaxTokens;
    auto gws = [&](int i) { return static_cast<void*>(ws + L.gemm + size_t(fan ? i : 0) * kGemmWorkspace); };
    auto on = [&](int i) { return fan && i > 0 ? m->side[i - 1] : s; };
    if (fan) {
        if (hipEventRecord(m->fork, s) != hipSuccess) return m3::set_error(M3_EHIP, "event record failed");
        for (int i = 0; i < kSide; ++i)
            if (hipStreamWaitEvent(m->side[i], m->fork, 0) != hipSuccess)
                return m3::set_error(M3_EHIP, "stream wait failed");
    }
    m3_status st;
    if ((st = m->gemm(ntok, HRP, K, u, w->W_x, ws + L.x, false, gws(0), on(0))) != M3_OK) return st;
    if ((st = m->gemm(ntok, HRP, K, u, w->W_z, ws + L.z, false, gws(1), on(1))) != M3_OK) return st;
    if ((st = m->gemm(ntok, GRN, K, u, w->W_B, ws + L.B, false, gws(2), on(2))) != M3_OK) return st;
    if ((st = m->gemm(ntok, GRN, K, u, w->W_C, ws + L.C, false, gws(2), on(2))) != M3_OK) return st;
    if ((st = m->gemm(ntok, d->heads, K, u, w->W_dt, ws + L.dt, true, gws(3), on(3))) != M3_OK) return st;
    if ((st = m->gemm(ntok, d->heads, K, u, w->W_lambda, ws + L.lam, true, gws(3), on(3))) != M3_OK) return st;
    if (fan)
        for (int i = 0; i < kSide; ++i)
            if (hipEventRecord(m->join[i], m->side[i]) != hipSuccess || hipStreamWaitEvent(s, m->join[i], 0) != hipSuccess)
                return m3::set_error(M3_EHIP, "stream join failed");
    float* dt = reinterpret_cast<float*>(ws + L.dt);
    float* lam = reinterpret_cast<float*>(ws + L.lam);
    return m3_prologue(d, R, M3_BF16, ntok, ws + L.B, ws + L.C, w->B_weight, w->B_bias, w->C_weight, w->C_bias, w->eps,
                       dt, w->dt_bias, lam, ws + L.B, ws + L.C, dt, lam, s);
}

// y *= silu(z) in place, then out = y W_out
m3_status project_out(m3_mixer* m, const m3_mixer_weights* w, const m3_dims* d, int32_t R, int64_t ntok, void* out,
                      char* ws, const MixerLayout& L, hipStream_t s) {
    const int64_t HRP = int64_t(d->heads) * R * d->headdim;
    hipError_t e = m3::launch_gate(ws + L.y, ws + L.z, ntok * HRP, s);
    if (e != hipSuccess) return m3::set_error(M3_EHIP, "gate launch failed: %s", hipGetErrorString(e));
    return m->gemm(ntok, w->d_model, HRP, ws + L.y, w->W_out, out, false, ws + L.gemm, s);
}

}  // namespace

extern "C" {

m3_status m3_mixer_create(m3_mixer** out) {
    if (!out) return m3::set_error(M3_EINVAL, "out is NULL");
    *out = nullptr;
    m3_mixer* m = new (std::nothrow) m3_mixer();
    if (!m) return m3::set_error(M3_EINVAL, "out of host memory");
    if (hipblasLtCreate(&m->lt) != HIPBLAS_STATUS_SUCCESS) {
        m->lt = nullptr;
        delete m;
        return m3::set_error(M3_EHIP, "hipblasLtCreate failed");
    }
    bool ok = hipEventCreateWithFlags(&m->fork, hipEventDisableTiming) == hipSuccess;
    for (int i = 0; i < kSide && ok; ++i)
        ok = hipStreamCreateWithFlags(&m->side[i], hipStreamNonBlocking) == hipSuccess &&
             hipEventCreateWithFlags(&m->join[i], hipEventDisableTiming) == hipSuccess;
    if (!ok) {
        delete m;
        return m3::set_error(M3_EHIP, "stream / event creation failed");
    }
    *out = m;
    return M3_OK;
}

void m3_mixer_destroy(m3_mixer* m) { delete m; }

size_t m3_mixer_workspace_size(const m3_dims* dims, int32_t R, int32_t chunk, int32_t d_model) {
    if (!dims || d_model < 1 || chunk < 1) return 0;
    m3_plan plan;
    if (m3_prefill_plan(dims, R, chunk, M3_BF16, &plan) != M3_OK) return 0;
    size_t pre = 0;
    return layout(dims, R, chunk, &pre).total;
}

m3_status m3_mixer_prefill(m3_mixer* m, const m3_mixer_weights* w, const m3_dims* dims, int32_t R, int32_t chunk,
                           const void* u, void* out, const float* h0, float* h_out, m3_decode_state* st,
                           void* workspace, size_t workspace_bytes, void* stream) {
    m3_status s = check_weights(w);
    if (s != M3_OK) return s;
    if (!dims) return m3::set_error(M3_EINVAL, "dims is NULL");
    m3_plan plan;
    if ((s = m3_prefill_plan(dims, R, chunk, M3_BF16, &plan)) != M3_OK) return s;
    size_t pre = 0;
    const MixerLayout L = layout(dims, R, chunk, &pre);
    const int64_t T = dims->batch * dims->seqlen;
    if (T > 0 && (!u || !out)) return m3::set_error(M3_EINVAL, "u and out must not be NULL");
    if (!workspace || workspace_bytes < L.total)
        return m3::set_error(M3_EWORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, L.total);
    if (st) {
        if (st->R != R || st->io_dtype != M3_BF16 || st->dims.batch != dims->batch || st->dims.heads != dims->heads ||
            st->dims.groups != dims->groups || st->dims.headdim != dims->headdim || st->dims.dstate != dims->dstate)
            return m3::set_error(M3_EINVAL, "decode state does not match the block's sizes");
        if (dims->batch > 0 && (!st->h || !st->carry_B || !st->carry_x))
            return m3::set_error(M3_EINVAL, "decode state buffers are not bound");
    }
    if (!m) return m3::set_error(M3_EINVAL, "mixer is NULL");
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    float* hfin = st ? st->h : h_out;
    if (T > 0) {
        if ((s = project_in(m, w, dims, R, T, u, ws, L, hs)) != M3_OK) return s;
        if ((s = m3_prefill(ws + L.x, reinterpret_cast<float*>(ws + L.dt), w->A, w->omega,
                            reinterpret_cast<float*>(ws + L.lam), ws + L.B, ws + L.C, w->D, R, chunk, h0, ws + L.y,
                            hfin, dims, M3_BF16, nullptr, nullptr, ws + L.pre, pre, stream)) != M3_OK)
            return s;
        if ((s = project_out(m, w, dims, R, T, out, ws, L, hs)) != M3_OK) return s;
    } else if (hfin && dims->batch > 0 && hfin != h0) {  // no tokens: h_L = h0
        const int64_t words = dims->batch * int64_t(dims->heads) * dims->dstate * dims->headdim;
        if (m3::launch_copy_or_zero(reinterpret_cast<uint32_t*>(hfin), reinterpret_cast<const uint32_t*>(h0), words,
                                    hs) != hipSuccess)
            return m3::set_error(M3_EHIP, "state copy failed");
    }
    if (st) {
        if (h_out && h_out != st->h && dims->batch > 0) {
            const size_t hb = size_t(dims->batch) * dims->heads * dims->dstate * dims->headdim * 4;
            if (hipMemcpyAsync(h_out, st->h, hb, hipMemcpyDeviceToDevice, hs) != hipSuccess)
                return m3::set_error(M3_EHIP, "copy of the final state failed");
        }
        const int64_t Lq = dims->seqlen;
        const void* Bl = nullptr;
        const void* xl = nullptr;
        if (Lq > 0 && dims->batch > 0) {  // the last token's B and x, one row per batch
            const size_t grn = size_t(dims->groups) * R * dims->dstate * 2, hrp = size_t(dims->heads) * R * dims->headdim * 2;
            if (hipMemcpy2DAsync(ws + L.Blast, grn, ws + L.B + (Lq - 1) * grn, Lq * grn, grn, dims->batch,
                                 hipMemcpyDeviceToDevice, hs) != hipSuccess ||
                hipMemcpy2DAsync(ws + L.xlast, hrp, ws + L.x + (Lq - 1) * hrp, Lq * hrp, hrp, dims->batch,
                                 hipMemcpyDeviceToDevice, hs) != hipSuccess)
                return m3::set_error(M3_EHIP, "copy of the last token failed");
            Bl = ws + L.Blast;
            xl = ws + L.xlast;
        }
        if ((s = m3_decode_state_init(st, dims, R, M3_BF16, st->h, st->carry_B, st->carry_x, st->h, Bl, xl, Lq,
                                      stream)) != M3_OK)
            return s;
    }
    return M3_OK;
}

m3_status m3_mixer_decode_step(m3_mixer* m, const m3_mixer_weights* w, m3_decode_state* st, const void* u_t,
                               void* out_t, void* workspace, size_t workspace_bytes, void* stream) {
    m3_status s = check_weights(w);
    if (s != M3_OK) return s;
    if (!st) return m3::set_error(M3_EINVAL, "state is NULL");
    if (st->io_dtype != M3_BF16) return m3::set_error(M3_EDTYPE, "the block runs in bf16");
    m3_dims d = st->dims;
    d.seqlen = 1;
    const int32_t R = st->R;
    size_t pre = 0;
    const MixerLayout L = layout(&d, R, 64, &pre);
    if (!workspace || workspace_bytes < L.total)
        return m3::set_error(M3_EWORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, L.total);
    const int64_t b = d.batch;
    if (b > 0 && (!u_t || !out_t)) return m3::set_error(M3_EINVAL, "u_t and out_t must not be NULL");
    if (!m) return m3::set_error(M3_EINVAL, "mixer is NULL");
    if (b == 0) return M3_OK;
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    if ((s = project_in(m, w, &d, R, b, u_t, ws, L, hs)) != M3_OK) return s;
    if ((s = m3_decode_step(st, ws + L.x, reinterpret_cast<float*>(ws + L.dt), w->A, w->omega,
                            reinterpret_cast<float*>(ws + L.lam), ws + L.B, ws + L.C, w->D, R, ws + L.y, stream)) !=
        M3_OK)
        return s;
    return project_out(m, w, &d, R, b, out_t, ws, L, hs);
}

}  // extern "C"
