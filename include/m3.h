/*
 * m3.h -- C ABI of libm3.so: the Mamba-3 SSM core recurrence on AMD MI355X (gfx950).
 *
 * The operation. Per (batch b, head h) the state h_t is an N x P fp32 matrix
 * whose rows (2k, 2k+1) hold one complex number per column (complex-valued SSM
 * with decay A and rotation frequency omega, real part taken at the output:
 * "复值SSM × 广义梯形离散 × MIMO，线性模型的全面重构", §2.1). Each token t
 * brings x_t (P x R), B_t and C_t (N x R), a step dt_t > 0 and a trapezoid
 * weight lambda_t in [0, 1]. With alpha = exp(dt*A_h), gamma = lambda*dt and
 * delta = (1 - lambda)*dt (exponential-trapezoidal rule, same digest §2.2 and
 * "Mamba-3架构技术解析：新一代语言建模的范式转移" §2.1):
 *
 *   h_t = alpha_t Rot(dt_t omega_h) (h_{t-1} + delta_t B_{t-1} x_{t-1}^T) + gamma_t B_t x_t^T
 *   y_t = h_t^T C_t + D_h x_t                    (y_t is P x R; MIMO rank R, digest §2.3)
 *
 * where Rot(theta) turns pair k by +theta_k = dt_t * omega_{h,k} (the 2x2 block
 * [[cos, -sin], [sin, cos]] on rows (2k, 2k+1)). Written in the rotating frame
 * (B and C turned by the cumulative angle, data-dependent RoPE: arXiv 2603.15569
 * summary page, contribution 2) this is h_t = alpha_t h_{t-1} +
 * beta_t B_{t-1}x_{t-1}^T + gamma_t B_t x_t^T with beta_t = delta_t alpha_t.
 * (B_{t-1}, x_{t-1}) of the first token is the "carry": zero unless given.
 *
 * Layout. All tensors are dense, row-major, device memory, 16-byte aligned:
 *   x, y        [b][L][H][R][P]   io dtype (bf16 or fp32)
 *   B, C        [b][L][G][R][N]   io dtype; head h uses group h / (H/G)
 *   dt, lambda  [b][L][H]         fp32
 *   A, D        [H]               fp32 (A < 0 decays)
 *   omega       [H][N/2]          fp32
 *   h0, h_out   [b][H][N][P]      fp32 (the state is always fp32)
 *   carry_B     [b][G][R][N]      io dtype; carry_x [b][H][R][P] io dtype
 * Decode-step tensors drop the L axis.
 *
 * Ownership. The caller owns every buffer (inputs, outputs, workspace, decode
 * state); the library allocates no memory and keeps no global state apart from
 * a thread-local error message. Calls are asynchronous on `stream` (a
 * hipStream_t; NULL is the null stream): a device fault surfaces at the
 * caller's next synchronisation. Nothing throws across this ABI.
 *
 * Errors. Every argument is checked before any HIP call; a bad argument returns
 * a status != M3_OK and launches nothing. m3_last_error() then names the
 * argument. Launch failures return M3_EHIP.
 */
#ifndef M3_H
#define M3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum m3_dtype { M3_F32 = 0, M3_BF16 = 1 } m3_dtype;

typedef enum m3_status {
    M3_OK = 0,
    M3_EINVAL = 1,       /* null required pointer, bad size, odd N, R < 1, chunk < 1, G not dividing H, y aliasing an input */
    M3_ESHAPE = 2,       /* inconsistent sizes (e.g. R differs from the decode state's) */
    M3_EDTYPE = 3,       /* unknown io dtype */
    M3_EALIGN = 4,       /* a tensor pointer is not 16-byte aligned */
    M3_EUNSUPPORTED = 5, /* valid but not implemented (chunk above 4096) */
    M3_EHIP = 6,         /* a HIP runtime call or kernel launch failed */
    M3_EWORKSPACE = 7,   /* workspace missing or smaller than m3_prefill_workspace_size() */
    M3_ELOOKBACK = 8     /* (m3_prefill_check) a look-back wait of the last call gave up: its outputs are not valid */
} m3_status;

/* Problem sizes. seqlen is ignored by the decode calls. */
typedef struct m3_dims {
    int64_t batch;    /* b >= 0 */
    int64_t seqlen;   /* L >= 0 */
    int32_t heads;    /* H >= 1 */
    int32_t groups;   /* G >= 1, divides H */
    int32_t headdim;  /* P >= 1 */
    int32_t dstate;   /* N >= 2, even (N/2 rotation pairs) */
} m3_dims;

/* How m3_prefill will split the work (all integers, exact). */
typedef struct m3_plan {
    int64_t n_chunks;        /* ceil(L / chunk'), chunk' the chunk the kernels walk: the chunk
                                asked for, except on the MFMA path at R 5 to 8, where chunks
                                hold at most 32 tokens (the result does not depend on it) */
    int64_t last_chunk_len;  /* L - (n_chunks - 1) * chunk', 0 when L == 0 */
    int32_t segments;        /* sequence segments per (b, h) walked in parallel; the
                                environment variable M3_PREFILL_SEGMENTS (a positive
                                integer, read at planning time) overrides the count
                                the plan would choose, where segments apply */
    int64_t chunks_per_segment;
    int32_t path;            /* M3_PATH_* below */
    size_t workspace_bytes;  /* what m3_prefill needs (0 allowed when this is 0) */
} m3_plan;

/* GENERIC: chunked, fp32 arithmetic, any sizes (the fp32 I/O path).
 * MFMA:    chunked on matrix cores, bf16 I/O, R 1 to 4, chunk <= 64, N a
 *          multiple of 8 up to 512 and P a multiple of 8 up to 1024: passes of
 *          at most 128 state rows and 64 columns (zero-padded inside the kernel
 *          where a pass holds fewer); with N above 128 the row passes' outputs
 *          are summed in fp32 in the workspace (the plan then asks for
 *          b*L*H*R*P*4 bytes); also R 5 to 8 at exactly N 128, P 64 (any
 *          chunk, walked in chunks of at most 32 tokens, no sequence segments).
 * SCAN:    token-by-token walk with the state in registers and the rank
 *          contractions on matrix cores, bf16 I/O, N and P multiples of 16 with
 *          N <= 256, P <= 64, R 5 to 8 (chunk unused; at N 128, P 64 these
 *          ranks take the MFMA path). */
enum { M3_PATH_GENERIC = 0, M3_PATH_MFMA = 1, M3_PATH_SCAN = 2 };

/*
 * m3_prefill -- chunked evaluation of the recurrence over L tokens.
 *
 * Passage: the parallel form of the trapezoid recurrence, whose mask is the
 * cumulative decay times a width-2 convolution ("复值SSM × 广义梯形离散 × MIMO",
 * Fig. 2), evaluated chunk by chunk with the fp32 state passed between chunks.
 *
 * x, dt, A, B, C, D: inputs as laid out above (required).
 * omega:  rotation rates, or NULL for omega = 0: the real-valued state of the
 *         pages' ablations (no RoPE on B and C; a faster path at R = 1).
 * lambda: trapezoid weights, or NULL for lambda = 1: the Euler rule, which the
 *         pages identify with Mamba-2 (no previous-input term).
 * R:      MIMO rank (>= 1).  chunk: tokens per chunk (1 .. 4096); any value gives
 *         the same result up to rounding; 64 is the tuned one.
 * h0:     initial state, or NULL for zero.
 * y:      output [b][L][H][R][P], must not overlap any input.
 * h_out:  final state h_L, or NULL. May alias h0.
 * dims:   sizes; io_dtype: dtype of x, B, C, y, carry_B, carry_x.
 * carry_B, carry_x: the token before the first (both or neither), else NULL.
 * workspace, workspace_bytes: device scratch of at least
 *         m3_prefill_workspace_size() bytes (may be NULL when that is 0). The
 *         library clears what it needs on `stream`; calls sharing one
 *         workspace must be ordered on one stream.
 */
m3_status m3_prefill(const void* x, const float* dt, const float* A, const float* omega,
                     const float* lambda, const void* B, const void* C, const float* D,
                     int32_t R, int32_t chunk, const float* h0, void* y, float* h_out,
                     const m3_dims* dims, m3_dtype io_dtype,
                     const void* carry_B, const void* carry_x,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * m3_prefill_fused -- m3_prefill on the raw projections of the step and the
 * trapezoid weight: the scalar part of the input prologue is applied where the
 * kernels load them, with no pass of its own.
 *
 * Passage: the block computes the step as a softplus of its projection plus a
 * learnt bias and the trapezoid weight as a sigmoid of its projection, next to
 * the QK-norm of B and C ("复值SSM × 广义梯形离散 × MIMO，线性模型的全面重构",
 * §2.4 and Fig. 4; m3_prologue's reading).
 *
 * dt_raw:     [b][L][H] fp32; the step is dt = softplus(dt_raw + dt_bias[h]).
 * dt_bias:    [H] fp32, or NULL for 0.
 * lambda_raw: [b][L][H] fp32, lambda = sigmoid(lambda_raw); or NULL for
 *             lambda = 1 (no sigmoid).
 * B, C:       the recurrence's B and C as m3_prefill takes them (the QK-norm
 *             stays with m3_prologue: at G < H it is per group, and a fused
 *             form would repeat it in every head of the group).
 * Everything else, the plan, the workspace and the errors: as m3_prefill
 * (dt_bias, when given, is checked like the other inputs: 16-byte aligned, not
 * overlapping y). Equal to m3_prologue on dt and lambda followed by m3_prefill
 * up to the rounding of softplus and sigmoid (hardware exp2 / log2 / rcp here,
 * a few ulp).
 */
m3_status m3_prefill_fused(const void* x, const float* dt_raw, const float* dt_bias, const float* A,
                           const float* omega, const float* lambda_raw, const void* B, const void* C,
                           const float* D, int32_t R, int32_t chunk, const float* h0, void* y, float* h_out,
                           const m3_dims* dims, m3_dtype io_dtype, const void* carry_B, const void* carry_x,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes m3_prefill needs for these sizes (0 on invalid sizes). Host only. */
size_t m3_prefill_workspace_size(const m3_dims* dims, int32_t R, int32_t chunk, m3_dtype io_dtype);

/*
 * m3_prefill_check -- did the last m3_prefill call on this workspace complete its
 * sequence-segment hand-offs?
 *
 * When the plan splits each sequence into segments (m3_plan.segments > 1), a
 * segment waits for its predecessors' end states (a decoupled look-back). A
 * predecessor always holds an earlier ticket and is running or done, so the wait
 * ends; it is bounded all the same (about a second of polling), and a wait that
 * gives up sets an error flag in the workspace and lets the call finish with
 * invalid outputs. This call synchronises `stream`, reads that flag and returns
 * M3_ELOOKBACK if it is set, M3_OK otherwise (at once, with no HIP call, when the
 * plan has one segment). workspace, workspace_bytes: as passed to m3_prefill;
 * NULL checks the fixed scratch of the last m3_prefill_noalloc call on the
 * current device. The environment variable M3_LOOKBACK_SPIN_LIMIT (polls, read
 * by each m3_prefill call) overrides the bound; 0 makes every wait give up at
 * once, for testing this report.
 */
m3_status m3_prefill_check(const m3_dims* dims, int32_t R, int32_t chunk, m3_dtype io_dtype,
                           const void* workspace, size_t workspace_bytes, void* stream);

/*
 * m3_prefill_noalloc -- m3_prefill for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that forbid
 * it): the same computation, arguments and results, with the workspace taken
 * from a fixed scratch array that the library holds in device memory instead of
 * a caller buffer. Nothing is allocated or freed by this call.
 *
 * The scratch is M3_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU, held from the first
 * call on that GPU until the process ends. Sizes whose m3_prefill_workspace_size()
 * exceeds it are rejected with M3_EWORKSPACE before anything is launched (at
 * the workloads' sizes the segmented long prefill of b 1, H 64, L 32768, R 4
 * needs 16 MiB; N above 128 needs b*L*H*R*P*4 bytes). Every call on one GPU
 * shares that GPU's array, which keeps the last call's contents; what must start
 * at zero is cleared by a kernel on `stream`. Calls that overlap in time on one
 * GPU (other streams, other threads) race on the scratch and must not be issued.
 */
#define M3_NOALLOC_SCRATCH_BYTES (32u << 20)
m3_status m3_prefill_noalloc(const void* x, const float* dt, const float* A, const float* omega,
                             const float* lambda, const void* B, const void* C, const float* D,
                             int32_t R, int32_t chunk, const float* h0, void* y, float* h_out,
                             const m3_dims* dims, m3_dtype io_dtype,
                             const void* carry_B, const void* carry_x, void* stream);

/* Bytes of m3_prefill_noalloc's fixed scratch (M3_NOALLOC_SCRATCH_BYTES). Host only. */
size_t m3_noalloc_scratch_bytes(void);

/* Fill *plan with the integers m3_prefill will use. Host only, no HIP call. */
m3_status m3_prefill_plan(const m3_dims* dims, int32_t R, int32_t chunk, m3_dtype io_dtype,
                          m3_plan* plan);

/*
 * Decode state: the fp32 state plus the previous token's (B, x), which the
 * trapezoid rule needs for the next step. Buffers are caller-owned device memory:
 *   h        [b][H][N][P] fp32
 *   carry_B  m3_decode_carry_bytes(.., 0) bytes, opaque: two slots [2][b][G][R][N]
 *            of the group's previous B rows (io dtype), then one 32-bit slot
 *            parity word per (b, h) at the next 16-byte boundary
 *   carry_x  [b][H][R][P] io dtype
 * Everything a step needs lives in these device buffers: a step reads B_prev
 * from the slot its parity word names and writes B_t into the other one, so
 * the kernels read no host-side counter for their results, and a step captured
 * in a HIP graph, and a graph of any number of steps, replays correctly. t
 * counts the tokens consumed by the calls made on this struct (a prefill of L
 * tokens hands over t = L); it is bookkeeping for the caller (graph replays do
 * not advance it). Its parity also picks the order in which a step walks the
 * (b, h) workgroups (backwards on odd t, so the states written last are read
 * first while the memory-side cache still holds them): a speed hint that does
 * not change any result.
 */
typedef struct m3_decode_state {
    float* h;
    void* carry_B;
    void* carry_x;
    int64_t t;
    m3_dims dims;
    int32_t R;
    m3_dtype io_dtype;
} m3_decode_state;

/* Bytes of the carry buffers (which = 0: carry_B, 1: carry_x). Host only. */
size_t m3_decode_carry_bytes(const m3_dims* dims, int32_t R, m3_dtype io_dtype, int32_t which);

/*
 * m3_decode_state_init -- bind caller buffers and set the starting point.
 *
 * Copies h0 (or zeros) into h_buf and (B_last, x_last) (or zeros) into the
 * carry (B_last into slot 0, every parity word to 0), on `stream`. B_last [b][G][R][N] and x_last
 * [b][H][R][P] are the last token already consumed (e.g. the prefill's last
 * token); both or neither. t0 >= 0 is the number of tokens already consumed.
 * h0 may equal h_buf (then it is left in place).
 */
m3_status m3_decode_state_init(m3_decode_state* st, const m3_dims* dims, int32_t R, m3_dtype io_dtype,
                               float* h_buf, void* carry_B_buf, void* carry_x_buf,
                               const float* h0, const void* B_last, const void* x_last, int64_t t0,
                               void* stream);

/*
 * m3_decode_step -- one token of the recurrence for every (b, h), in place.
 *
 * Passage: the recurrent (decode) form; the state is read and written once per
 * token, and MIMO raises the work per state byte without more state traffic
 * ("复值SSM × 广义梯形离散 × MIMO", §2.3 and §3.3; "Mamba-3架构技术解析", §2.3).
 *
 * x_t [b][H][R][P], B_t/C_t [b][G][R][N] (io dtype), dt_t/lambda_t [b][H] fp32,
 * A, D [H], omega [H][N/2]; y_t [b][H][R][P] io dtype (must not overlap the
 * inputs or the state). omega and lambda_t may be NULL (omega = 0, lambda = 1,
 * as for m3_prefill). R must equal st->R. On success st->t is incremented.
 * Steps on one state must be ordered on one stream.
 */
m3_status m3_decode_step(m3_decode_state* st, const void* x_t, const float* dt_t, const float* A,
                         const float* omega, const float* lambda_t, const void* B_t, const void* C_t,
                         const float* D, int32_t R, void* y_t, void* stream);

/*
 * m3_decode_step_fused -- m3_decode_step on the raw projections, with the
 * input prologue (m3_prologue's reading, below) computed inside the step
 * kernel instead of a separate launch.
 *
 * Passage: the QK-norm and bias sit between the B/C projection and the
 * recurrence ("复值SSM × 广义梯形离散 × MIMO，线性模型的全面重构", §2.4 and Fig. 4);
 * at decode every (b, h) workgroup normalises its group's rows itself.
 *
 * x_t [b][H][R][P], B_raw_t / C_raw_t [b][G][R][N] (io dtype); dt_raw_t and
 * lambda_raw_t [b][H] fp32 (lambda_raw_t NULL: lambda = 1); dt_bias [H],
 * B_weight / B_bias / C_weight / C_bias [G][R][N] fp32, each NULL for zero bias
 * or unit weight; eps >= 0. The step uses dt = softplus(dt_raw + dt_bias),
 * lambda = sigmoid(lambda_raw) and the normalised rows rounded to the io dtype,
 * exactly as m3_prologue would store them, so the call equals m3_prologue
 * followed by m3_decode_step (up to the summation order of the norm); the B
 * carry holds the normalised rows. Other arguments, the state and the errors
 * as for m3_decode_step; R * N above 8192 is M3_EUNSUPPORTED.
 */
m3_status m3_decode_step_fused(m3_decode_state* st, const void* x_t, const float* dt_raw_t, const float* dt_bias,
                               const float* A, const float* omega, const float* lambda_raw_t, const void* B_raw_t,
                               const void* C_raw_t, const float* B_weight, const float* B_bias,
                               const float* C_weight, const float* C_bias, float eps, const float* D, int32_t R,
                               void* y_t, void* stream);

/*
 * m3_prologue -- the input prologue in front of the recurrence, one pass over
 * the raw projections of ntok tokens (b * L for a prefill, b for a decode step).
 *
 * Passage: a QK-norm and a learnable additive bias follow the B/C projection
 * ("复值SSM × 广义梯形离散 × MIMO，线性模型的全面重构", §2.4 and Fig. 4; §3.4 on the
 * bias); the step and the trapezoid weight come through softplus and sigmoid
 * (the workloads' input recipe). The pages print no formulas; the reading
 * taken, per (token t, group g, rank r) row of N entries:
 *
 *   B[t][g][r][n] = B_raw[t][g][r][n] / sqrt(mean_n' B_raw[t][g][r][n']^2 + eps)
 *                   * B_weight[g][r][n] + B_bias[g][r][n]          (C likewise)
 *   dt[t][h]      = softplus(dt_raw[t][h] + dt_bias[h])   = log(1 + e^x)
 *   lambda[t][h]  = sigmoid(lambda_raw[t][h])             = 1 / (1 + e^-x)
 *
 * dims: heads, groups, dstate are used (batch, seqlen, headdim are not); R >= 1.
 * B_raw, C_raw -> B, C: [ntok][G][R][N] io dtype, fp32 arithmetic, the output
 *   rounded to the io dtype (nearest even). B_weight, C_weight, B_bias, C_bias:
 *   [G][R][N] fp32, each NULL for all-ones weight / zero bias. eps >= 0.
 * dt_raw -> dt: [ntok][H] fp32; dt_bias [H] fp32 or NULL.
 * lambda_raw -> lambda: [ntok][H] fp32.
 * Each of the four parts runs only when both its input and its output are
 * given (B_raw/B, C_raw/C, dt_raw/dt, lambda_raw/lambda); one of a pair alone
 * is an error. An output may be its own input (in place) but must not overlap
 * any other argument. Asynchronous on `stream`; the kernels hold no state.
 */
m3_status m3_prologue(const m3_dims* dims, int32_t R, m3_dtype io_dtype, int64_t ntok,
                      const void* B_raw, const void* C_raw, const float* B_weight, const float* B_bias,
                      const float* C_weight, const float* C_bias, float eps,
                      const float* dt_raw, const float* dt_bias, const float* lambda_raw,
                      void* B, void* C, float* dt, float* lambda, void* stream);

/*
 * m3_prefill_backward -- gradients of one m3_prefill call (training).
 *
 * Passage: the same recurrence, differentiated in reverse ("复值SSM × 广义梯形离散
 * × MIMO", §2.1-§2.3; the pages' kernels serve training as well as inference).
 * Given dy = dLoss/dy [b][L][H][R][P] (io dtype) and dh_out = dLoss/dh_out
 * [b][H][N][P] fp32 (NULL: zero), it writes dLoss/d of every input, fp32:
 *   dx [b][L][H][R][P], dB and dC [b][L][G][R][N] (summed over the heads of a
 *   group), ddt and dlambda [b][L][H], dA and dD [H] and domega [H][N/2]
 *   (summed over batch and tokens), dh0 [b][H][N][P], dcarry_B [b][G][R][N]
 *   and dcarry_x [b][H][R][P].
 * The forward inputs are those of m3_prefill (same layouts, same NULL rules for
 * omega, lambda, h0 and the carry). dlambda, domega and dh0 may be NULL (not
 * wanted); dcarry_B / dcarry_x are given together, and only with the carry.
 * Supported: N <= 128, P <= 64 (even with bf16 I/O), R <= 4 (else M3_EUNSUPPORTED). The arithmetic is
 * fp32; the states are recomputed from checkpoints kept in `workspace` (at least
 * m3_prefill_backward_workspace_size() bytes). The summed gradients are added
 * with device atomics, so their last bits can vary from call to call. No
 * output may overlap an input or another output. Asynchronous on `stream`.
 */
m3_status m3_prefill_backward(const void* x, const float* dt, const float* A, const float* omega,
                              const float* lambda, const void* B, const void* C, const float* D,
                              int32_t R, const float* h0, const void* carry_B, const void* carry_x,
                              const void* dy, const float* dh_out,
                              float* dx, float* dB, float* dC, float* ddt, float* dlambda, float* dA,
                              float* domega, float* dD, float* dh0, float* dcarry_B, float* dcarry_x,
                              const m3_dims* dims, m3_dtype io_dtype,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes m3_prefill_backward needs (0 on invalid or unsupported sizes). Host only. */
size_t m3_prefill_backward_workspace_size(const m3_dims* dims, int32_t R);

/*
 * The mixer block around the recurrence (training-free forward: prefill and
 * decode step). The PaperWeekly digest ("复值SSM × 广义梯形离散 × MIMO，线性模型的全面
 * 重构", §2.4 and Fig. 4) lists what a Mamba-3 block holds without a block
 * formula; the reading taken is the Mamba-2 block layout with those changes.
 * Per token u (d_model entries, bf16):
 *   x = u W_x^T, z = u W_z^T       [H][R][P]     (bf16)
 *   B_raw = u W_B^T, C_raw = u W_C^T   [G][R][N] (bf16)
 *   dt_raw = u W_dt^T, lambda_raw = u W_lambda^T  [H] (fp32)
 *   B, C, dt, lambda = m3_prologue(...) with the weights' B/C norm weights and biases, dt_bias, eps
 *   y = the recurrence (m3_prefill, or m3_decode_step) with A, omega, D
 *   out = (y * silu(z)) W_out^T    [d_model]     (bf16; silu(v) = v sigmoid(v))
 * Weights are bf16, row-major [out][in] as a linear layer stores them (x = u W_x^T):
 * W_x, W_z [H*R*P][d_model], W_B, W_C [G*R*N][d_model], W_dt, W_lambda
 * [H][d_model], W_out [d_model][H*R*P]. The
 * projections run as hipBLASLt GEMMs (fp32 accumulation); omega, the norm
 * weights, biases and dt_bias may be NULL as for m3_prologue / m3_prefill.
 * The intermediates live in the caller's workspace. A mixer object holds the
 * hipBLASLt handle, the GEMM algorithms chosen per shape (timed on the first
 * call of each shape, which synchronises the stream once: capture a graph only
 * after one eager call of the same sizes) and three side streams: the input
 * projections of a call with at most 1024 tokens fan out to them (fork and join
 * events on `stream`, so a captured call captures them too). Create it once,
 * use it from one thread and one call at a time, destroy it at the end.
 */
typedef struct m3_mixer m3_mixer;
typedef struct m3_mixer_weights {
    int32_t d_model;
    const void* W_x;
    const void* W_z;
    const void* W_B;
    const void* W_C;
    const void* W_dt;
    const void* W_lambda;
    const void* W_out;
    const float* B_weight;  /* [G][R][N] or NULL */
    const float* B_bias;
    const float* C_weight;
    const float* C_bias;
    const float* dt_bias;   /* [H] or NULL */
    const float* A;         /* [H] */
    const float* omega;     /* [H][N/2] or NULL */
    const float* D;         /* [H] */
    float eps;
} m3_mixer_weights;

/* Create / destroy a mixer object (host call; creates a hipBLASLt handle and three
 * default-priority streams on the current device). */
m3_status m3_mixer_create(m3_mixer** out);
void m3_mixer_destroy(m3_mixer* m);

/* Workspace bytes of m3_mixer_prefill for these sizes (dims->seqlen tokens per
 * sequence; 1 for m3_mixer_decode_step), 0 on invalid sizes. Host only. */
size_t m3_mixer_workspace_size(const m3_dims* dims, int32_t R, int32_t chunk, int32_t d_model);

/*
 * m3_mixer_prefill -- the block over u [b][L][d_model] bf16 -> out [b][L][d_model] bf16.
 * h0 (nullable) and h_out (nullable) as for m3_prefill; chunk as for m3_prefill.
 * st (nullable): a decode state whose buffers are bound (m3_decode_state_init)
 * with the same sizes; it receives h_L, the last token's (B, x) as the carry and
 * t = L, so m3_mixer_decode_step continues the sequences. Asynchronous on `stream`.
 */
m3_status m3_mixer_prefill(m3_mixer* m, const m3_mixer_weights* w, const m3_dims* dims, int32_t R, int32_t chunk,
                           const void* u, void* out, const float* h0, float* h_out, m3_decode_state* st,
                           void* workspace, size_t workspace_bytes, void* stream);

/* m3_mixer_decode_step -- the block for one token per sequence, u_t [b][d_model] ->
 * out_t [b][d_model], advancing st (bf16) by one token. Workspace: at least
 * m3_mixer_workspace_size() with seqlen 1. */
m3_status m3_mixer_decode_step(m3_mixer* m, const m3_mixer_weights* w, m3_decode_state* st, const void* u_t,
                               void* out_t, void* workspace, size_t workspace_bytes, void* stream);

/* Static text for a status code. */
const char* m3_status_string(m3_status s);

/* Detail of the last error on this thread ("" when none). */
const char* m3_last_error(void);

/* ABI version of this header (bumped on incompatible change). */
#define M3_ABI_VERSION 1
int32_t m3_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* M3_H */
