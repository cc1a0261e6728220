/*
 * CPU oracle for the Mamba-2 SSD forward: a plain step-by-step recurrence in
 * double precision.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file; it exists so that tests, the smoke check and the CPU baseline of
 * the benchmark have an independent answer to compare against.  It shares no
 * code, header, table or helper with the GPU library.
 *
 * What it computes (per batch row r and head h, independently):
 *
 *   H_t = a_t * H_{t-1} + x_t B_t^T          (P x N state, a_t scalar)
 *   y_t = H_t C_t + D_h x_t
 *   a_t = exp(dt_t * A_h),  A_h = -exp(A_log_h)
 *
 * Sources (page title, then section):
 *  - recurrence H_t = a_t H_{t-1} + B_t x_t^T, y_t = C_t^T H_t, one scalar decay
 *    per head acting on every row of the state: "088 Mamba-2: writing the
 *    recurrent state as a structured matrix" (wq-win.github.io), section 2.1
 *    "unrolling the history contribution".  The page stores the state as N x P;
 *    here it is stored transposed, P x N, which changes no value.
 *  - a_t = exp(Delta_t * A): "Mamba" paper story (ai.tomabc.com), section on
 *    the selective SSM, where the discretised decay is exp(Delta A).
 *  - skip term y = C h + D x: "Mamba and state space models" (wang-x-xia.github.io),
 *    section 2 "formal definition".
 *  - B and C shared by groups of heads: "Mamba-2 - Transformer and SSM share one
 *    algebra" (awesome.papernotes.org), key design 3 (multi-input SSM).  Head h
 *    reads group h / (H / G).
 *  - independent sequences in one packed row do not exchange state; carrying a
 *    state into the next call continues the recurrence: "088 Mamba-2", sections
 *    2.3 and 5.  At the first token of sequence k the state is replaced by
 *    init_k and then updated by that token as usual (decayed by a_t, written by
 *    x_t B_t^T), so a carried state continues a split run exactly.
 *  - optional input scaling.  The pages name the zero-order hold (ZOH) as the
 *    discretisation ("Mamba and state space models", section 2 "formal
 *    definition") without giving B-bar; the default follows the recurrence
 *    above, with no Delta on x.  Two opt-in readings:
 *      Euler: x_t -> Delta_t x_t  (B-bar = Delta B);
 *      ZOH:   x_t -> (exp(Delta_t A) - 1) / A * x_t, the exact solution over
 *             one step of h' = A h + B x with x and B held constant (for the
 *             scalar A here: h(Delta) = e^{Delta A} h(0) + (e^{Delta A} - 1)/A B x).
 *    D always multiplies the unscaled x.
 *  - optional step-size map Delta = softplus(dt + dt_bias_h): the "Mamba"
 *    paper story (ai.tomabc.com), the simplified Mamba block pseudocode, where
 *    the step size is the softplus of a projection plus a learned per-channel
 *    parameter.  Without the flag Delta = dt + dt_bias_h (dt_bias NULL = 0).
 *
 * Layouts (all contiguous, row-major):
 *   x (b,T,H,P)  dt (b,T,H)  A_log (H)  B, C (b,T,G,N)  D (H) or NULL
 *   init (nseqs,H,P,N) or NULL   seq_idx (b,T) int32 or NULL
 *   y (b,T,H,P)   final (nseqs,H,P,N) or NULL
 * Without seq_idx every row is its own sequence (nseqs == b).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int ssd_oracle_f64(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                   int64_t dstate, int64_t ngroups, int64_t nseqs,
                   const double* x, const double* dt, const double* A_log,
                   const double* B, const double* C, const double* D,
                   const double* init, const int32_t* seq_idx,
                   const double* dt_bias, int dt_softplus, int input_scaling,
                   double* y, double* final_state, int nthreads)
{
    const int64_t T = seqlen, H = nheads, P = headdim, N = dstate, G = ngroups;
    if (batch < 0 || T < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0)
        return 1;
    if (seq_idx == NULL && nseqs != batch)
        return 1;
    if (input_scaling < 0 || input_scaling > 2)
        return 1;
    const int64_t heads_per_group = H / G;
    const int64_t units = batch * H;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(|: bad)
#endif
    for (int64_t u = 0; u < units; ++u) {
        const int64_t r = u / H, h = u % H, g = h / heads_per_group;
        const double A = -exp(A_log[h]);
        const double Dh = D ? D[h] : 0.0;
        double* S = (double*)calloc((size_t)(P * N), sizeof(double));
        double* xs = (double*)malloc((size_t)P * sizeof(double));
        if (!S || !xs) { free(S); free(xs); bad |= 1; continue; }
        int64_t cur = -1;
        for (int64_t t = 0; t < T; ++t) {
            const int64_t k = seq_idx ? (int64_t)seq_idx[r * T + t] : r;
            if (k < 0 || k >= nseqs) { bad |= 1; break; }
            if (t == 0 || k != cur) {
                /* sequence boundary: hand out the finished state, load the new one */
                if (t > 0 && final_state)
                    memcpy(final_state + (cur * H + h) * P * N, S, (size_t)(P * N) * sizeof(double));
                if (init)
                    memcpy(S, init + (k * H + h) * P * N, (size_t)(P * N) * sizeof(double));
                else
                    memset(S, 0, (size_t)(P * N) * sizeof(double));
                cur = k;
            }
            double dtv = dt[(r * T + t) * H + h] + (dt_bias ? dt_bias[h] : 0.0);
            if (dt_softplus)   /* log(1 + e^v), written so that neither branch overflows */
                dtv = dtv > 0.0 ? dtv + log1p(exp(-dtv)) : log1p(exp(dtv));
            const double a = exp(dtv * A);
            /* factor on x_t in the state write (1, Delta, or the ZOH (e^{Delta A} - 1) / A) */
            const double xf = input_scaling == 1 ? dtv : (input_scaling == 2 ? expm1(dtv * A) / A : 1.0);
            const double* xt = x + ((r * T + t) * H + h) * P;
            const double* Bt = B + ((r * T + t) * G + g) * N;
            const double* Ct = C + ((r * T + t) * G + g) * N;
            double* yt = y + ((r * T + t) * H + h) * P;
            for (int64_t p = 0; p < P; ++p)
                xs[p] = xf * xt[p];
            /* decay, then write: H_t = a_t H_{t-1} + x_t B_t^T */
            for (int64_t p = 0; p < P; ++p)
                for (int64_t n = 0; n < N; ++n)
                    S[p * N + n] = a * S[p * N + n] + xs[p] * Bt[n];
            /* read after the write: y_t = H_t C_t + D x_t */
            for (int64_t p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n)
                    acc += S[p * N + n] * Ct[n];
                yt[p] = acc + Dh * xt[p];
            }
        }
        if (T > 0 && final_state && cur >= 0)
            memcpy(final_state + (cur * H + h) * P * N, S, (size_t)(P * N) * sizeof(double));
        if (T == 0 && final_state && seq_idx == NULL) {
            /* no token, no step of the recurrence: the row's state is its initial state */
            if (init)
                memcpy(final_state + (r * H + h) * P * N, init + (r * H + h) * P * N, (size_t)(P * N) * sizeof(double));
            else
                memset(final_state + (r * H + h) * P * N, 0, (size_t)(P * N) * sizeof(double));
        }
        free(S);
        free(xs);
    }
    return bad ? 2 : 0;
}

int ssd_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
