/*
 * m3_oracle.c -- CPU reference for the Mamba-3 SSM core recurrence.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, obviously correct
 * definition that the HIP library is checked against. It is linked only by the
 * tests, by the smoke check and by the bench's CPU-baseline leg; the product
 * path never calls it, and it shares no code, header or table with the HIP
 * library.
 *
 * What it computes (one independent walk per (batch, head), token by token, in
 * double precision; single-precision inputs are widened exactly):
 *
 *   The continuous SSM has a complex diagonal transition A + i*omega per state
 *   pair: A decays the state, omega rotates it, and the output takes the real
 *   part ("复值SSM × 广义梯形离散 × MIMO，线性模型的全面重构", §2.1; arXiv
 *   2603.15569 summary page, key contribution 2). A complex pair (re, im) is
 *   stored as the two real rows (2k, 2k+1) of the state, so multiplying by
 *   e^{i*theta} is the 2x2 rotation [[cos, -sin], [sin, cos]] on those rows
 *   (same digest, §2.2: block-diagonal matrix of 2x2 rotation blocks).
 *
 *   Discretisation is the exponential-trapezoidal (generalised trapezoidal)
 *   rule: the input integral is weighted at both ends of the step, lambda on
 *   the current input and (1 - lambda) on the previous one, and the previous
 *   input is carried through the step's transition ("复值SSM × ...", §2.2;
 *   "Mamba-3架构技术解析：新一代语言建模的范式转移", §2.1, whose lambda = 1/2
 *   formula multiplies the earlier B by e^{A*dt}). With
 *     alpha_t = exp(dt_t*A), gamma_t = lambda_t*dt_t, delta_t = (1-lambda_t)*dt_t,
 *   one step is
 *     g   = h_{t-1} + delta_t * B_{t-1} x_{t-1}^T        (previous input)
 *     h_t = alpha_t * Rot(dt_t*omega) g + gamma_t * B_t x_t^T
 *     y_t = h_t^T C_t + D * x_t
 *   i.e. h_t = alpha_t h_{t-1} + beta_t B_{t-1}x_{t-1}^T + gamma_t B_t x_t^T
 *   with beta_t = delta_t*alpha_t, the rotation included in alpha's complex form.
 *
 *   MIMO rank R: B_t, C_t are N x R and x_t, y_t are P x R; the input term is
 *   the N x R by R x P product B_t x_t^T ("复值SSM × ...", §2.3 and Fig. 3;
 *   "Mamba-3架构技术解析", §2.3). The R columns share dt, lambda, A, omega, D.
 *
 *   The token before the first one contributes through its (B, x) pair, the
 *   "carry"; with no carry it is zero (nothing precedes the sequence).
 *
 * Layout (row-major, contiguous):
 *   x, y [b][L][H][R][P]; B, C [b][L][G][R][N]; dt, lam [b][L][H];
 *   A, D [H]; omega [H][N/2]; h0, h_out [b][H][N][P];
 *   carry_B [b][G][R][N]; carry_x [b][H][R][P].  Head h reads group h/(H/G).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int m3o_version(void) { return 1; }

/* Returns 0 on success, -1 on bad sizes, -2 on allocation failure. */
int m3o_scan(int64_t batch, int64_t L, int64_t H, int64_t G, int64_t P, int64_t N, int64_t R,
             const float* x, const float* dt, const float* A, const float* omega,
             const float* lam, const float* B, const float* C, const float* D,
             const float* h0, const float* carry_B, const float* carry_x,
             double* y, double* h_out, int nthreads)
{
    if (batch < 0 || L < 0 || H <= 0 || G <= 0 || P <= 0 || N <= 0 || R <= 0) return -1;
    if (N % 2 != 0 || H % G != 0) return -1;
    const int64_t heads_per_group = H / G;
    const int64_t nbh = batch * H;
    int failed = 0;
    if (nthreads <= 0) nthreads = 1;

#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1) reduction(|| : failed)
    for (int64_t bh = 0; bh < nbh; ++bh) {
        const int64_t b = bh / H, h = bh % H, g = h / heads_per_group;
        double* st = (double*)malloc(sizeof(double) * (size_t)(N * P));
        double* Bp = (double*)malloc(sizeof(double) * (size_t)(R * N));
        double* xp = (double*)malloc(sizeof(double) * (size_t)(R * P));
        if (!st || !Bp || !xp) { free(st); free(Bp); free(xp); failed = 1; continue; }

        /* initial state and the previous token's input */
        for (int64_t i = 0; i < N * P; ++i)
            st[i] = h0 ? (double)h0[(b * H + h) * N * P + i] : 0.0;
        for (int64_t i = 0; i < R * N; ++i)
            Bp[i] = carry_B ? (double)carry_B[(b * G + g) * R * N + i] : 0.0;
        for (int64_t i = 0; i < R * P; ++i)
            xp[i] = carry_x ? (double)carry_x[(b * H + h) * R * P + i] : 0.0;

        const double a_h = (double)A[h];
        const double d_h = (double)D[h];
        for (int64_t t = 0; t < L; ++t) {
            const int64_t th = (b * L + t) * H + h;
            const double step = (double)dt[th];
            const double lm = (double)lam[th];
            const double alpha = exp(step * a_h);
            const double gamma = lm * step;
            const double delta = (1.0 - lm) * step;
            const float* xt = x + th * R * P;
            const float* Bt = B + ((b * L + t) * G + g) * R * N;
            const float* Ct = C + ((b * L + t) * G + g) * R * N;

            /* g = h + delta * B_{t-1} x_{t-1}^T */
            for (int64_t n = 0; n < N; ++n)
                for (int64_t p = 0; p < P; ++p) {
                    double u = 0.0;
                    for (int64_t r = 0; r < R; ++r) u += Bp[r * N + n] * xp[r * P + p];
                    st[n * P + p] += delta * u;
                }
            /* multiply pair k by alpha * e^{i * dt * omega_k} */
            for (int64_t k = 0; k < N / 2; ++k) {
                const double th_k = step * (double)omega[h * (N / 2) + k];
                const double c = cos(th_k), s = sin(th_k);
                double* re = st + (2 * k) * P;
                double* im = st + (2 * k + 1) * P;
                for (int64_t p = 0; p < P; ++p) {
                    const double a = re[p], bb = im[p];
                    re[p] = alpha * (c * a - s * bb);
                    im[p] = alpha * (s * a + c * bb);
                }
            }
            /* h += gamma * B_t x_t^T */
            for (int64_t n = 0; n < N; ++n)
                for (int64_t p = 0; p < P; ++p) {
                    double u = 0.0;
                    for (int64_t r = 0; r < R; ++r) u += (double)Bt[r * N + n] * (double)xt[r * P + p];
                    st[n * P + p] += gamma * u;
                }
            /* y[r][p] = sum_n h[n][p] C[r][n] + D x[r][p] */
            double* yt = y + th * R * P;
            for (int64_t r = 0; r < R; ++r)
                for (int64_t p = 0; p < P; ++p) {
                    double acc = 0.0;
                    for (int64_t n = 0; n < N; ++n) acc += st[n * P + p] * (double)Ct[r * N + n];
                    yt[r * P + p] = acc + d_h * (double)xt[r * P + p];
                }
            /* this token becomes the previous one */
            for (int64_t i = 0; i < R * N; ++i) Bp[i] = (double)Bt[i];
            for (int64_t i = 0; i < R * P; ++i) xp[i] = (double)xt[i];
        }
        if (h_out)
            memcpy(h_out + (b * H + h) * N * P, st, sizeof(double) * (size_t)(N * P));
        free(st); free(Bp); free(xp);
    }
    return failed ? -2 : 0;
}
