// m3_host.cpp -- the C entry points of libm3.so: argument checks, planning and
// dispatch. Host code only: every check runs before the first HIP call, so the
// error paths can be exercised on a machine without a GPU.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "m3_internal.h"

namespace {

thread_local char g_err[512] = "";

m3_status fail(m3_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

size_t io_size(m3_dtype t) { return t == M3_BF16 ? 2 : 4; }

}  // namespace

m3_status m3::set_error(m3_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
    const char* name;
    uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(const Range& a, const Range& b) {
    return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

Range rng(const char* name, const void* p, size_t bytes) {
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{name, lo, p ? lo + bytes : lo};
}

m3_status check_dims(const m3_dims* d, int32_t R) {
    if (!d) return fail(M3_EINVAL, "dims is NULL");
    if (d->batch < 0) return fail(M3_EINVAL, "batch %lld < 0", (long long)d->batch);
    if (d->seqlen < 0) return fail(M3_EINVAL, "seqlen %lld < 0", (long long)d->seqlen);
    if (d->heads < 1) return fail(M3_EINVAL, "heads %d < 1", d->heads);
    if (d->groups < 1) return fail(M3_EINVAL, "groups %d < 1", d->groups);
    if (d->heads % d->groups != 0)
        return fail(M3_EINVAL, "groups %d does not divide heads %d", d->groups, d->heads);
    if (d->headdim < 1) return fail(M3_EINVAL, "headdim %d < 1", d->headdim);
    if (d->dstate < 2 || d->dstate % 2 != 0)
        return fail(M3_EINVAL, "dstate %d must be even and >= 2 (rotation pairs)", d->dstate);
    if (R < 1) return fail(M3_EINVAL, "rank R %d < 1", R);
    if (d->headdim > 65536 || d->dstate > 65536 || R > 1024 || d->heads > (1 << 24))
        return fail(M3_EUNSUPPORTED, "sizes beyond the supported range");
    return M3_OK;
}

m3_status check_dtype(m3_dtype t) {
    if (t != M3_F32 && t != M3_BF16) return fail(M3_EDTYPE, "unknown io dtype %d", (int)t);
    return M3_OK;
}

int32_t choose_segments(int64_t bh, int64_t n_chunks) {
    // Enough (b, h, segment) walks to give every compute unit one, with at
    // least 8 chunks per segment so the look-back stays a small fraction.
    const char* env = getenv("M3_PREFILL_SEGMENTS");
    int64_t s;
    if (env && atoi(env) > 0) {
        s = atoi(env);
    } else {
        const int64_t target = 256;
        s = bh >= target ? 1 : (target + bh - 1) / bh;
        s = std::min<int64_t>(s, std::max<int64_t>(1, n_chunks / 8));
    }
    s = std::max<int64_t>(1, std::min<int64_t>(s, std::max<int64_t>(1, n_chunks)));
    return (int32_t)std::min<int64_t>(s, 4096);
}

m3_status make_plan(const m3_dims* d, int32_t R, int32_t chunk, m3_dtype io, m3_plan* p) {
    m3_status s = check_dims(d, R);
    if (s != M3_OK) return s;
    if ((s = check_dtype(io)) != M3_OK) return s;
    if (chunk < 1) return fail(M3_EINVAL, "chunk %d < 1", chunk);
    if (chunk > 4096) return fail(M3_EUNSUPPORTED, "chunk %d above 4096", chunk);
    std::memset(p, 0, sizeof *p);
    const int64_t L = d->seqlen;
    const bool mfma = m3::mfma_path_supported(d->headdim, d->dstate, R, chunk, io);
    if (mfma) chunk = m3::mfma_kernel_chunk(R, chunk);
    p->n_chunks = (L + chunk - 1) / chunk;
    p->last_chunk_len = L == 0 ? 0 : L - (p->n_chunks - 1) * chunk;
    p->path = mfma ? M3_PATH_MFMA
                   : m3::scan_path_supported(d->headdim, d->dstate, R, io) ? M3_PATH_SCAN : M3_PATH_GENERIC;
    p->segments = (mfma && m3::mfma_segments_supported(R, d->dstate, d->headdim))
                      ? choose_segments(d->batch * d->heads, p->n_chunks) : 1;
    p->chunks_per_segment = p->segments > 0 ? (p->n_chunks + p->segments - 1) / p->segments : 0;
    if (mfma && p->chunks_per_segment > 0)  // no empty trailing segment
        p->segments = (int32_t)((p->n_chunks + p->chunks_per_segment - 1) / p->chunks_per_segment);
    if (p->segments < 1) p->segments = 1;
    p->workspace_bytes = m3::prefill_workspace_layout(d->batch, d->seqlen, d->heads, d->headdim, d->dstate, R,
                                                      p->segments, p->path).total;
    return M3_OK;
}

}  // namespace

namespace m3 {

static size_t up256(size_t v) { return (v + 255) & ~size_t(255); }

PrefillWorkspace prefill_workspace_layout(int64_t b, int64_t L, int32_t H, int32_t P, int32_t N, int32_t R,
                                          int32_t segments, int32_t path) {
    PrefillWorkspace w{};
    const size_t bh = size_t(b) * size_t(H);
    size_t off = 0;
    if (path == M3_PATH_GENERIC) {
        w.state_off = off;
        off += up256(bh * size_t(N) * size_t(P) * 4);
    } else if (segments > 1) {
        // segment states of the chunked kernels, which hold N below 128 zero-padded to 128 rows
        N = path == M3_PATH_MFMA ? 128 : N;
        const size_t nseg = bh * size_t(segments);
        w.ctrl_off = off;
        off += up256(256 + nseg * 4);
        w.agg_off = off;
        off += up256(nseg * size_t(N) * size_t(P) * 4);
        w.incl_off = off;
        off += up256(nseg * size_t(N) * size_t(P) * 4);
        w.tr_off = off;
        off += up256(nseg * 8);
    } else if (path == M3_PATH_MFMA && N > 128) {
        w.ypart_off = off;
        off += up256(bh * size_t(L) * size_t(R) * size_t(P) * 4);
    }
    w.total = off;
    return w;
}

}  // namespace m3

extern "C" {

int32_t m3_abi_version(void) { return M3_ABI_VERSION; }

const char* m3_last_error(void) { return g_err; }

const char* m3_status_string(m3_status s) {
    switch (s) {
        case M3_OK: return "ok";
        case M3_EINVAL: return "invalid argument";
        case M3_ESHAPE: return "inconsistent shapes";
        case M3_EDTYPE: return "unsupported dtype";
        case M3_EALIGN: return "pointer not 16-byte aligned";
        case M3_EUNSUPPORTED: return "unsupported configuration";
        case M3_EHIP: return "HIP runtime error";
        case M3_EWORKSPACE: return "workspace missing or too small";
        case M3_ELOOKBACK: return "a sequence-segment look-back gave up; outputs not valid";
    }
    return "unknown status";
}

m3_status m3_prefill_plan(const m3_dims* dims, int32_t R, int32_t chunk, m3_dtype io_dtype, m3_plan* plan) {
    g_err[0] = 0;
    if (!plan) return fail(M3_EINVAL, "plan is NULL");
    return make_plan(dims, R, chunk, io_dtype, plan);
}

size_t m3_prefill_workspace_size(const m3_dims* dims, int32_t R, int32_t chunk, m3_dtype io_dtype) {
    m3_plan p;
    if (make_plan(dims, R, chunk, io_dtype, &p) != M3_OK) return 0;
    return p.workspace_bytes;
}

m3_status m3_prefill_check(const m3_dims* dims, int32_t R, int32_t chunk, m3_dtype io_dtype,
                           const void* workspace, size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    m3_plan plan;
    m3_status s = make_plan(dims, R, chunk, io_dtype, &plan);
    if (s != M3_OK) return s;
    if (plan.segments <= 1 || dims->batch == 0 || dims->seqlen == 0) return M3_OK;
    const void* ws = workspace;
    if (!ws) {
        void* p = nullptr;
        if ((s = m3::noalloc_scratch(&p)) != M3_OK) return s;
        ws = p;
    } else if (workspace_bytes < plan.workspace_bytes) {
        return fail(M3_EWORKSPACE, "workspace %zu bytes < %zu of this plan", workspace_bytes, plan.workspace_bytes);
    }
    const m3::PrefillWorkspace w = m3::prefill_workspace_layout(dims->batch, dims->seqlen, dims->heads,
                                                                dims->headdim, dims->dstate, R, plan.segments,
                                                                plan.path);
    uint32_t flag = 0;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(&flag, static_cast<const char*>(ws) + w.ctrl_off + 4, 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(M3_EHIP, "reading the look-back flag failed: %s", hipGetErrorString(e));
    if (flag) return fail(M3_ELOOKBACK, "a look-back wait of the last call on this workspace gave up");
    return M3_OK;
}

namespace {

// m3_prefill and m3_prefill_fused: the checks and the launch. raw: dt and
// lambda are raw projections, mapped (softplus with dt_bias, sigmoid) where the
// kernels load them.
m3_status prefill_impl(const void* x, const float* dt, const float* dt_bias, const float* A, const float* omega,
                       const float* lambda, const void* B, const void* C, const float* D, int32_t R, int32_t chunk,
                       const float* h0, void* y, float* h_out, const m3_dims* dims, m3_dtype io_dtype,
                       const void* carry_B, const void* carry_x, void* workspace, size_t workspace_bytes,
                       void* stream, bool raw) {
    g_err[0] = 0;
    m3_plan plan;
    m3_status s = make_plan(dims, R, chunk, io_dtype, &plan);
    if (s != M3_OK) return s;
    const int64_t b = dims->batch, L = dims->seqlen;
    const int64_t H = dims->heads, G = dims->groups, P = dims->headdim, N = dims->dstate;
    const size_t es = io_size(io_dtype);
    const bool tokens = b > 0 && L > 0;
    const bool heads = b > 0;

    struct Req { const char* name; const void* p; bool needed; };
    // omega and lambda may be NULL: omega = 0 (real-valued state) and lambda = 1 (Euler / Mamba-2)
    const Req req[] = {{"x", x, tokens}, {"dt", dt, tokens}, {"B", B, tokens}, {"C", C, tokens},
                       {"y", y, tokens}, {"A", A, heads}, {"D", D, heads}};
    for (const Req& r : req)
        if (r.needed && !r.p) return fail(M3_EINVAL, "%s is NULL", r.name);
    if ((carry_B == nullptr) != (carry_x == nullptr))
        return fail(M3_EINVAL, "carry_B and carry_x must be given together");

    const void* ptrs[] = {x, dt, A, omega, lambda, B, C, D, h0, y, h_out, carry_B, carry_x, dt_bias};
    const char* names[] = {"x", "dt", "A", "omega", "lambda", "B", "C", "D", "h0", "y", "h_out",
                           "carry_B", "carry_x", "dt_bias"};
    for (size_t i = 0; i < sizeof ptrs / sizeof ptrs[0]; ++i)
        if (ptrs[i] && !aligned16(ptrs[i])) return fail(M3_EALIGN, "%s is not 16-byte aligned", names[i]);

    const size_t tok = size_t(b) * size_t(L);
    const Range ry = rng("y", y, tok * H * R * P * es);
    const Range inputs[] = {rng("x", x, tok * H * R * P * es), rng("dt", dt, tok * H * 4),
                            rng("lambda", lambda, tok * H * 4), rng("B", B, tok * G * R * N * es),
                            rng("C", C, tok * G * R * N * es), rng("A", A, H * 4),
                            rng("omega", omega, H * (N / 2) * 4), rng("D", D, H * 4),
                            rng("h0", h0, size_t(b) * H * N * P * 4),
                            rng("h_out", h_out, size_t(b) * H * N * P * 4),
                            rng("carry_B", carry_B, size_t(b) * G * R * N * es),
                            rng("carry_x", carry_x, size_t(b) * H * R * P * es),
                            rng("dt_bias", dt_bias, H * 4)};
    for (const Range& r : inputs)
        if (overlaps(ry, r)) return fail(M3_EINVAL, "y overlaps %s", r.name);
    const Range rh = rng("h_out", h_out, size_t(b) * H * N * P * 4);
    for (const Range& r : inputs) {
        if (!std::strcmp(r.name, "h_out")) continue;
        if (!std::strcmp(r.name, "h0") && h0 == h_out) continue;  // exact alias is allowed
        if (overlaps(rh, r)) return fail(M3_EINVAL, "h_out overlaps %s", r.name);
    }
    if (plan.workspace_bytes > 0 && b > 0) {
        if (!workspace) return fail(M3_EWORKSPACE, "workspace of %zu bytes required", plan.workspace_bytes);
        if (workspace_bytes < plan.workspace_bytes)
            return fail(M3_EWORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes,
                        plan.workspace_bytes);
        if (reinterpret_cast<uintptr_t>(workspace) & 255u)
            return fail(M3_EALIGN, "workspace is not 256-byte aligned");
    }
    if (b == 0) return M3_OK;

    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipError_t e;
    if (L == 0) {  // nothing to scan: h_L = h0
        if (h_out && h_out != h0)
            e = m3::launch_copy_or_zero(reinterpret_cast<uint32_t*>(h_out),
                                        reinterpret_cast<const uint32_t*>(h0), int64_t(b) * H * N * P, st);
        else
            e = hipSuccess;
    } else {
        const int32_t kchunk = plan.path == M3_PATH_MFMA ? m3::mfma_kernel_chunk(R, chunk) : chunk;
        m3::PrefillArgs a{x, dt, A, omega, lambda, B, C, D, h0, y, h_out, carry_B, carry_x,
                          b, L, (int32_t)H, (int32_t)G, (int32_t)P, (int32_t)N, R, kchunk, io_dtype,
                          plan, workspace, st};
        a.dt_bias = raw ? dt_bias : nullptr;
        a.raw_steps = raw ? 1 : 0;
        e = plan.path == M3_PATH_MFMA   ? m3::launch_prefill_mfma(a)
            : plan.path == M3_PATH_SCAN ? m3::launch_prefill_scan(a)
                                        : m3::launch_prefill_generic(a);
    }
    if (e != hipSuccess) return fail(M3_EHIP, "launch failed: %s", hipGetErrorString(e));
    return M3_OK;
}

}  // namespace

m3_status m3_prefill(const void* x, const float* dt, const float* A, const float* omega,
                     const float* lambda, const void* B, const void* C, const float* D,
                     int32_t R, int32_t chunk, const float* h0, void* y, float* h_out,
                     const m3_dims* dims, m3_dtype io_dtype,
                     const void* carry_B, const void* carry_x,
                     void* workspace, size_t workspace_bytes, void* stream) {
    return prefill_impl(x, dt, nullptr, A, omega, lambda, B, C, D, R, chunk, h0, y, h_out, dims, io_dtype, carry_B,
                        carry_x, workspace, workspace_bytes, stream, false);
}

m3_status m3_prefill_fused(const void* x, const float* dt_raw, const float* dt_bias, const float* A,
                           const float* omega, const float* lambda_raw, const void* B, const void* C, const float* D,
                           int32_t R, int32_t chunk, const float* h0, void* y, float* h_out, const m3_dims* dims,
                           m3_dtype io_dtype, const void* carry_B, const void* carry_x, void* workspace,
                           size_t workspace_bytes, void* stream) {
    return prefill_impl(x, dt_raw, dt_bias, A, omega, lambda_raw, B, C, D, R, chunk, h0, y, h_out, dims, io_dtype,
                        carry_B, carry_x, workspace, workspace_bytes, stream, true);
}

// m3_prefill_noalloc: m3_prefill on the fixed device array of m3_noalloc.hip
size_t m3_noalloc_scratch_bytes(void) { return size_t(M3_NOALLOC_SCRATCH_BYTES); }

m3_status m3_prefill_noalloc(const void* x, const float* dt, const float* A, const float* omega, const float* lambda,
                             const void* B, const void* C, const float* D, int32_t R, int32_t chunk, const float* h0,
                             void* y, float* h_out, const m3_dims* dims, m3_dtype io_dtype, const void* carry_B,
                             const void* carry_x, void* stream) {
    const size_t cap = size_t(M3_NOALLOC_SCRATCH_BYTES);
    m3_plan plan;
    m3_status s = m3_prefill_plan(dims, R, chunk, io_dtype, &plan);
    if (s != M3_OK) return s;
    if (plan.workspace_bytes > cap)
        return fail(M3_EWORKSPACE, "these sizes need %zu bytes of scratch, above the fixed %zu bytes of m3_prefill_noalloc",
                    plan.workspace_bytes, cap);
    void* ws = nullptr;
    if (plan.workspace_bytes > 0 && dims->batch > 0 && dims->seqlen > 0) {
        if ((s = m3::noalloc_scratch(&ws)) != M3_OK) return s;
    }
    return m3_prefill(x, dt, A, omega, lambda, B, C, D, R, chunk, h0, y, h_out, dims, io_dtype, carry_B, carry_x,
                      ws, ws ? cap : 0, stream);
}

size_t m3_decode_carry_bytes(const m3_dims* dims, int32_t R, m3_dtype io_dtype, int32_t which) {
    if (check_dims(dims, R) != M3_OK || check_dtype(io_dtype) != M3_OK) return 0;
    const size_t es = io_size(io_dtype);
    if (which == 0)  // two slots of the group's B rows, then one parity word per head
        return m3::decode_carry_B_slots_bytes(dims->batch, dims->groups, R, dims->dstate, es) +
               size_t(dims->batch) * dims->heads * 4;
    if (which == 1) return size_t(dims->batch) * dims->heads * R * dims->headdim * es;
    return 0;
}

m3_status m3_decode_state_init(m3_decode_state* st, const m3_dims* dims, int32_t R, m3_dtype io_dtype,
                               float* h_buf, void* carry_B_buf, void* carry_x_buf,
                               const float* h0, const void* B_last, const void* x_last, int64_t t0,
                               void* stream) {
    g_err[0] = 0;
    if (!st) return fail(M3_EINVAL, "state is NULL");
    m3_status s = check_dims(dims, R);
    if (s != M3_OK) return s;
    if ((s = check_dtype(io_dtype)) != M3_OK) return s;
    if (t0 < 0) return fail(M3_EINVAL, "t0 %lld < 0", (long long)t0);
    const int64_t b = dims->batch;
    if (b > 0 && (!h_buf || !carry_B_buf || !carry_x_buf))
        return fail(M3_EINVAL, "state buffers must not be NULL");
    if ((B_last == nullptr) != (x_last == nullptr))
        return fail(M3_EINVAL, "B_last and x_last must be given together");
    const void* ptrs[] = {h_buf, carry_B_buf, carry_x_buf, h0, B_last, x_last};
    const char* names[] = {"h", "carry_B", "carry_x", "h0", "B_last", "x_last"};
    for (int i = 0; i < 6; ++i)
        if (ptrs[i] && !aligned16(ptrs[i])) return fail(M3_EALIGN, "%s is not 16-byte aligned", names[i]);
    const size_t es = io_size(io_dtype);
    const size_t hbytes = size_t(b) * dims->heads * dims->dstate * dims->headdim * 4;
    const size_t rowB = size_t(R) * dims->dstate * es, rowx = size_t(R) * dims->headdim * es;  // one head's carry rows
    if (h0 && h0 != h_buf && overlaps(rng("h0", h0, hbytes), rng("h", h_buf, hbytes)))
        return fail(M3_EINVAL, "h0 partially overlaps the state buffer");
    if ((rowB % 4) || (rowx % 4)) return fail(M3_EUNSUPPORTED, "carry row size not a multiple of 4 bytes");

    st->h = h_buf;
    st->carry_B = carry_B_buf;
    st->carry_x = carry_x_buf;
    st->t = t0;
    st->dims = *dims;
    st->dims.seqlen = 1;
    st->R = R;
    st->io_dtype = io_dtype;
    if (b == 0) return M3_OK;

    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    if (h0 != h_buf)
        e = m3::launch_copy_or_zero(reinterpret_cast<uint32_t*>(h_buf), reinterpret_cast<const uint32_t*>(h0),
                                    int64_t(hbytes / 4), hs);
    // B_last into slot 0 (one row per group), every head's parity word to 0 (slot 0
    // holds B_prev), x_last per head
    const size_t slots = m3::decode_carry_B_slots_bytes(b, dims->groups, R, dims->dstate, es);
    if (e == hipSuccess)
        e = m3::launch_carry_init(carry_B_buf, B_last, b, dims->groups, dims->groups, int64_t(rowB), hs);
    if (e == hipSuccess)
        e = m3::launch_carry_init(static_cast<char*>(carry_B_buf) + slots, nullptr, 1, 1, 1,
                                  int64_t(b) * dims->heads * 4, hs);
    if (e == hipSuccess)
        e = m3::launch_carry_init(carry_x_buf, x_last, b, dims->heads, dims->heads, int64_t(rowx), hs);
    if (e != hipSuccess) return fail(M3_EHIP, "state init failed: %s", hipGetErrorString(e));
    return M3_OK;
}

namespace {

// m3_decode_step and m3_decode_step_fused: the checks and the launch; pro is
// NULL for the plain step (dt_t / lambda_t are then the step and the weight,
// B_t / C_t the normalised rows)
m3_status decode_step_impl(m3_decode_state* st, const void* x_t, const float* dt_t, const float* A,
                           const float* omega, const float* lambda_t, const void* B_t, const void* C_t,
                           const float* D, int32_t R, void* y_t, void* stream, const m3::DecodePrologue* pro) {
    g_err[0] = 0;
    if (!st) return fail(M3_EINVAL, "state is NULL");
    m3_status s = check_dims(&st->dims, st->R);
    if (s != M3_OK) return s;
    if ((s = check_dtype(st->io_dtype)) != M3_OK) return s;
    if (R != st->R) return fail(M3_ESHAPE, "R %d differs from the state's %d", R, st->R);
    const m3_dims& d = st->dims;
    const int64_t b = d.batch;
    if (pro) {
        if (!(pro->eps >= 0.f)) return fail(M3_EINVAL, "eps must be >= 0");
        if (int64_t(R) * d.dstate > m3::kDecodeFusedGenericRN)
            return fail(M3_EUNSUPPORTED, "R * N = %lld above %lld for the fused step", (long long)R * d.dstate,
                        (long long)m3::kDecodeFusedGenericRN);
    }
    if (b == 0) { st->t += 1; return M3_OK; }
    struct Req { const char* name; const void* p; bool optional; };
    // omega and lambda_t may be NULL: omega = 0 (real-valued state) and lambda = 1 (Euler / Mamba-2)
    const Req req[] = {{"x_t", x_t, false}, {pro ? "dt_raw_t" : "dt_t", dt_t, false}, {"A", A, false},
                       {"omega", omega, true}, {pro ? "lambda_raw_t" : "lambda_t", lambda_t, true},
                       {pro ? "B_raw_t" : "B_t", B_t, false}, {pro ? "C_raw_t" : "C_t", C_t, false}, {"D", D, false},
                       {"y_t", y_t, false}, {"state h", st->h, false}, {"state carry_B", st->carry_B, false},
                       {"state carry_x", st->carry_x, false}};
    for (const Req& r : req) {
        if (!r.p) {
            if (r.optional) continue;
            return fail(M3_EINVAL, "%s is NULL", r.name);
        }
        if (!aligned16(r.p)) return fail(M3_EALIGN, "%s is not 16-byte aligned", r.name);
    }
    const size_t es = io_size(st->io_dtype);
    const int64_t H = d.heads, G = d.groups, P = d.headdim, N = d.dstate;
    const Range ry = rng("y_t", y_t, size_t(b) * H * R * P * es);
    const Range others[] = {rng("x_t", x_t, size_t(b) * H * R * P * es), rng("dt_t", dt_t, size_t(b) * H * 4),
                            rng("lambda_t", lambda_t, size_t(b) * H * 4),
                            rng("B_t", B_t, size_t(b) * G * R * N * es), rng("C_t", C_t, size_t(b) * G * R * N * es),
                            rng("state h", st->h, size_t(b) * H * N * P * 4),
                            rng("state carry_B", st->carry_B, m3_decode_carry_bytes(&d, R, st->io_dtype, 0)),
                            rng("state carry_x", st->carry_x, size_t(b) * H * R * P * es)};
    for (const Range& r : others)
        if (overlaps(ry, r)) return fail(M3_EINVAL, "y_t overlaps %s", r.name);

    m3::DecodeArgs a{st->h, st->carry_B, st->carry_x, x_t, dt_t, A, omega,
                     lambda_t, B_t, C_t, D, y_t, b, (int32_t)H, (int32_t)G, (int32_t)P, (int32_t)N, R,
                     st->io_dtype, reinterpret_cast<hipStream_t>(stream), int(st->t & 1), pro};
    hipError_t e = m3::launch_decode(a);
    if (e != hipSuccess) return fail(M3_EHIP, "decode launch failed: %s", hipGetErrorString(e));
    st->t += 1;
    return M3_OK;
}

}  // namespace

m3_status m3_decode_step(m3_decode_state* st, const void* x_t, const float* dt_t, const float* A,
                         const float* omega, const float* lambda_t, const void* B_t, const void* C_t,
                         const float* D, int32_t R, void* y_t, void* stream) {
    return decode_step_impl(st, x_t, dt_t, A, omega, lambda_t, B_t, C_t, D, R, y_t, stream, nullptr);
}

m3_status m3_decode_step_fused(m3_decode_state* st, const void* x_t, const float* dt_raw_t, const float* dt_bias,
                               const float* A, const float* omega, const float* lambda_raw_t, const void* B_raw_t,
                               const void* C_raw_t, const float* B_weight, const float* B_bias,
                               const float* C_weight, const float* C_bias, float eps, const float* D, int32_t R,
                               void* y_t, void* stream) {
    const void* opt[] = {dt_bias, B_weight, B_bias, C_weight, C_bias};
    const char* names[] = {"dt_bias", "B_weight", "B_bias", "C_weight", "C_bias"};
    for (int i = 0; i < 5; ++i)
        if (opt[i] && !aligned16(opt[i])) {
            g_err[0] = 0;
            return fail(M3_EALIGN, "%s is not 16-byte aligned", names[i]);
        }
    const m3::DecodePrologue pro{B_weight, B_bias, C_weight, C_bias, dt_bias, eps};
    return decode_step_impl(st, x_t, dt_raw_t, A, omega, lambda_raw_t, B_raw_t, C_raw_t, D, R, y_t, stream, &pro);
}

size_t m3_prefill_backward_workspace_size(const m3_dims* dims, int32_t R) {
    if (check_dims(dims, R) != M3_OK) return 0;
    if (!m3::backward_supported(dims->headdim, dims->dstate, R)) return 0;
    return m3::backward_workspace_bytes(dims->batch, dims->heads, dims->seqlen);
}

m3_status m3_prefill_backward(const void* x, const float* dt, const float* A, const float* omega,
                              const float* lambda, const void* B, const void* C, const float* D,
                              int32_t R, const float* h0, const void* carry_B, const void* carry_x,
                              const void* dy, const float* dh_out,
                              float* dx, float* dB, float* dC, float* ddt, float* dlambda, float* dA,
                              float* domega, float* dD, float* dh0, float* dcarry_B, float* dcarry_x,
                              const m3_dims* dims, m3_dtype io_dtype,
                              void* workspace, size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    m3_status s = check_dims(dims, R);
    if (s != M3_OK) return s;
    if ((s = check_dtype(io_dtype)) != M3_OK) return s;
    const int64_t b = dims->batch, L = dims->seqlen;
    const int64_t H = dims->heads, G = dims->groups, P = dims->headdim, N = dims->dstate;
    if (!m3::backward_supported((int32_t)P, (int32_t)N, R))
        return fail(M3_EUNSUPPORTED, "backward supports N <= 128, P <= 64, R <= 4 (got N %lld, P %lld, R %d)",
                    (long long)N, (long long)P, R);
    if (io_dtype == M3_BF16 && (P % 2))
        return fail(M3_EUNSUPPORTED, "bf16 backward needs an even head dim P (got %lld)", (long long)P);
    const bool tokens = b > 0 && L > 0;
    struct Req { const char* name; const void* p; bool needed; };
    const Req req[] = {{"x", x, tokens}, {"dt", dt, tokens}, {"B", B, tokens}, {"C", C, tokens},
                       {"dy", dy, tokens}, {"dx", dx, tokens}, {"dB", dB, tokens}, {"dC", dC, tokens},
                       {"ddt", ddt, tokens}, {"A", A, b > 0}, {"D", D, b > 0}, {"dA", dA, b > 0}, {"dD", dD, b > 0}};
    for (const Req& r : req)
        if (r.needed && !r.p) return fail(M3_EINVAL, "%s is NULL", r.name);
    if ((carry_B == nullptr) != (carry_x == nullptr))
        return fail(M3_EINVAL, "carry_B and carry_x must be given together");
    if ((dcarry_B == nullptr) != (dcarry_x == nullptr))
        return fail(M3_EINVAL, "dcarry_B and dcarry_x must be given together");
    if (dcarry_B && !carry_B) return fail(M3_EINVAL, "dcarry_B / dcarry_x given without a carry");

    const size_t es = io_size(io_dtype);
    const size_t tok = size_t(b) * size_t(L);
    const size_t nx = tok * H * R * P, nbc = tok * G * R * N, nsc = tok * H, nst = size_t(b) * H * N * P;
    const Range in[] = {rng("x", x, nx * es), rng("dt", dt, nsc * 4), rng("A", A, H * 4),
                        rng("omega", omega, H * (N / 2) * 4), rng("lambda", lambda, nsc * 4),
                        rng("B", B, nbc * es), rng("C", C, nbc * es), rng("D", D, H * 4), rng("h0", h0, nst * 4),
                        rng("carry_B", carry_B, size_t(b) * G * R * N * es),
                        rng("carry_x", carry_x, size_t(b) * H * R * P * es), rng("dy", dy, nx * es),
                        rng("dh_out", dh_out, nst * 4), rng("workspace", workspace, workspace_bytes)};
    const Range out[] = {rng("dx", dx, nx * 4), rng("dB", dB, nbc * 4), rng("dC", dC, nbc * 4),
                         rng("ddt", ddt, nsc * 4), rng("dlambda", dlambda, nsc * 4), rng("dA", dA, H * 4),
                         rng("domega", domega, H * (N / 2) * 4), rng("dD", dD, H * 4), rng("dh0", dh0, nst * 4),
                         rng("dcarry_B", dcarry_B, size_t(b) * G * R * N * 4),
                         rng("dcarry_x", dcarry_x, size_t(b) * H * R * P * 4)};
    for (const Range& r : in)
        if (r.lo && !aligned16(reinterpret_cast<const void*>(r.lo)))
            return fail(M3_EALIGN, "%s is not 16-byte aligned", r.name);
    for (const Range& r : out)
        if (r.lo && !aligned16(reinterpret_cast<const void*>(r.lo)))
            return fail(M3_EALIGN, "%s is not 16-byte aligned", r.name);
    const int nout = int(sizeof out / sizeof out[0]);
    for (int o = 0; o < nout; ++o) {
        for (const Range& r : in)
            if (overlaps(out[o], r)) return fail(M3_EINVAL, "%s overlaps %s", out[o].name, r.name);
        for (int q = o + 1; q < nout; ++q)
            if (overlaps(out[o], out[q])) return fail(M3_EINVAL, "%s overlaps %s", out[o].name, out[q].name);
    }
    const size_t need = m3::backward_workspace_bytes(b, (int32_t)H, L);
    if (tokens && (!workspace || workspace_bytes < need))
        return fail(M3_EWORKSPACE, "backward needs %zu workspace bytes, got %zu", need, workspace_bytes);
    if (b == 0) return M3_OK;
    if (b * H > 0x7fffffff) return fail(M3_EUNSUPPORTED, "b * H above 2^31 - 1");

    m3::BackwardArgs a{x, dt, A, omega, lambda, B, C, D, h0, carry_B, carry_x, dy, dh_out,
                       dx, dB, dC, ddt, dlambda, dA, domega, dD, dh0, dcarry_B, dcarry_x,
                       b, L, (int32_t)H, (int32_t)G, (int32_t)P, (int32_t)N, R, io_dtype,
                       static_cast<float*>(workspace), reinterpret_cast<hipStream_t>(stream)};
    hipError_t e = m3::launch_backward(a);
    if (e != hipSuccess) return fail(M3_EHIP, "backward launch failed: %s", hipGetErrorString(e));
    return M3_OK;
}

m3_status m3_prologue(const m3_dims* dims, int32_t R, m3_dtype io_dtype, int64_t ntok,
                      const void* B_raw, const void* C_raw, const float* B_weight, const float* B_bias,
                      const float* C_weight, const float* C_bias, float eps,
                      const float* dt_raw, const float* dt_bias, const float* lambda_raw,
                      void* B, void* C, float* dt, float* lambda, void* stream) {
    g_err[0] = 0;
    m3_status s = check_dims(dims, R);
    if (s != M3_OK) return s;
    if ((s = check_dtype(io_dtype)) != M3_OK) return s;
    if (ntok < 0) return fail(M3_EINVAL, "ntok %lld < 0", (long long)ntok);
    if (!(eps >= 0.f) || eps > 3.0e38f) return fail(M3_EINVAL, "eps must be finite and >= 0");
    struct Pair { const char* in_name; const void* in; const char* out_name; const void* out; };
    const Pair pairs[] = {{"B_raw", B_raw, "B", B}, {"C_raw", C_raw, "C", C}, {"dt_raw", dt_raw, "dt", dt},
                          {"lambda_raw", lambda_raw, "lambda", lambda}};
    for (const Pair& p : pairs)
        if ((p.in == nullptr) != (p.out == nullptr))
            return fail(M3_EINVAL, "%s and %s must be given together", p.in_name, p.out_name);
    if (!B && (B_weight || B_bias)) return fail(M3_EINVAL, "B_weight / B_bias given without B");
    if (!C && (C_weight || C_bias)) return fail(M3_EINVAL, "C_weight / C_bias given without C");
    if (!dt && dt_bias) return fail(M3_EINVAL, "dt_bias given without dt");

    const int64_t H = dims->heads, G = dims->groups, N = dims->dstate;
    const size_t es = io_size(io_dtype);
    const size_t nrow = size_t(ntok) * size_t(G) * size_t(R) * size_t(N) * es;
    const size_t npar = size_t(G) * size_t(R) * size_t(N) * 4, nsc = size_t(ntok) * size_t(H) * 4;
    const Range in[] = {rng("B_raw", B_raw, nrow), rng("C_raw", C_raw, nrow), rng("B_weight", B_weight, npar),
                        rng("B_bias", B_bias, npar), rng("C_weight", C_weight, npar), rng("C_bias", C_bias, npar),
                        rng("dt_raw", dt_raw, nsc), rng("dt_bias", dt_bias, size_t(H) * 4),
                        rng("lambda_raw", lambda_raw, nsc)};
    const Range out[] = {rng("B", B, nrow), rng("C", C, nrow), rng("dt", dt, nsc), rng("lambda", lambda, nsc)};
    const int own[] = {0, 1, 6, 8};  // the input each output may replace in place
    for (const Range& r : in)
        if (r.lo && !aligned16(reinterpret_cast<const void*>(r.lo)))
            return fail(M3_EALIGN, "%s is not 16-byte aligned", r.name);
    for (const Range& r : out)
        if (r.lo && !aligned16(reinterpret_cast<const void*>(r.lo)))
            return fail(M3_EALIGN, "%s is not 16-byte aligned", r.name);
    for (int o = 0; o < 4; ++o) {
        for (int i = 0; i < int(sizeof in / sizeof in[0]); ++i) {
            if (!overlaps(out[o], in[i])) continue;
            if (i == own[o] && out[o].lo == in[i].lo) continue;  // in place
            return fail(M3_EINVAL, "%s overlaps %s", out[o].name, in[i].name);
        }
        for (int q = o + 1; q < 4; ++q)
            if (overlaps(out[o], out[q])) return fail(M3_EINVAL, "%s overlaps %s", out[o].name, out[q].name);
    }
    if (ntok == 0 || !(B || C || dt || lambda)) return M3_OK;  // nothing to do: no launch
    const int64_t rows = ntok * G * R;
    if ((B || C) && (rows + 15) / 16 > 0x3fffffff) return fail(M3_EUNSUPPORTED, "too many rows");
    if ((dt || lambda) && (ntok * H + 255) / 256 > 0x3fffffff) return fail(M3_EUNSUPPORTED, "too many tokens");

    m3::PrologueArgs a{B_raw, C_raw, B_weight, B_bias, C_weight, C_bias, eps, dt_raw, dt_bias, lambda_raw,
                       B, C, dt, lambda, ntok, (int32_t)H, (int32_t)(G * R), (int32_t)N, io_dtype,
                       reinterpret_cast<hipStream_t>(stream)};
    hipError_t e = m3::launch_prologue(a);
    if (e != hipSuccess) return fail(M3_EHIP, "prologue launch failed: %s", hipGetErrorString(e));
    return M3_OK;
}

}  // extern "C"
