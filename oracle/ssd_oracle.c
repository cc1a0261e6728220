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

/*
 * Gradients of the same forward map (reverse-mode differentiation of the
 * recurrence above, step by step).  TEST INFRASTRUCTURE ONLY, like the forward.
 *
 * The pages give no backward algorithm; this is the chain rule applied to the
 * recurrence of "088 Mamba-2" section 2.1 (with the step-size map and input
 * scaling described above), for a loss L with dL/dy = dy and dL/dfinal = dfinal:
 *
 *   G_t = dL/dS_t = dy_t C_t^T + a_{t+1} G_{t+1}      (within a sequence; at the
 *         sequence's last token the carried term is dfinal_k instead)
 *   dC_t += S_t^T dy_t            dB_t += f_t G_t^T x_t      (summed over heads)
 *   dx_t  = f_t G_t B_t + D dy_t
 *   da_t  = <G_t, S_{t-1}>        (S_{t-1} = init_k at the sequence's first token)
 *   df_t  = x_t . (G_t B_t)
 *   dDelta_t = da_t a_t A + df_t df/dDelta      dA += da_t a_t Delta_t + df_t df/dA
 *   dA_log = dA * A,  ddt = dDelta * (softplus ? sigmoid(dt + bias) : 1)
 *   ddt_bias_h = sum of ddt over rows and tokens,  dD_h = sum dy . x
 *   dinit_k = a_t G_t at the sequence's first token t (dfinal_k for an empty row)
 *
 * with f = 1, Delta or (e^{Delta A} - 1)/A, so df/dDelta = 0, 1 or e^{Delta A}
 * and df/dA = 0, 0 or (Delta A e^{Delta A} - e^{Delta A} + 1) / A^2.
 * Every state S_t of a (row, head) is kept (T * P * N doubles): meant for test
 * sizes.  abs_sums (H x 3, or NULL) receives, per head, the sums over rows and
 * tokens of the absolute per-token terms of dA_log, ddt_bias and dD (the scale
 * against which the rounding error of those sums is judged).  dB and dC are summed over the heads of a group in increasing head
 * order, the per-head scalars over rows in increasing row order.
 */
int ssd_oracle_bwd_f64(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                       int64_t dstate, int64_t ngroups, int64_t nseqs,
                       const double* x, const double* dt, const double* A_log,
                       const double* B, const double* C, const double* D,
                       const double* init, const int32_t* seq_idx,
                       const double* dt_bias, int dt_softplus, int input_scaling,
                       const double* dy, const double* dfinal,
                       double* dx, double* ddt, double* dA_log, double* dB, double* dC,
                       double* dD, double* dinit, double* ddt_bias, double* abs_sums, int nthreads)
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
    /* per-unit contributions, reduced in a fixed order afterwards */
    double* dBu = (double*)calloc((size_t)(units * T * N) + 1, sizeof(double));
    double* dCu = (double*)calloc((size_t)(units * T * N) + 1, sizeof(double));
    double* sA = (double*)calloc((size_t)units, sizeof(double));
    double* sD = (double*)calloc((size_t)units, sizeof(double));
    double* sBias = (double*)calloc((size_t)units, sizeof(double));
    double* sAbs = (double*)calloc((size_t)units * 3, sizeof(double));
    if (!dBu || !dCu || !sA || !sD || !sBias || !sAbs) {
        free(dBu); free(dCu); free(sA); free(sD); free(sBias); free(sAbs);
        return 2;
    }
    memset(dinit, 0, (size_t)(nseqs * H * P * N) * sizeof(double));
    int bad = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(|: bad)
#endif
    for (int64_t u = 0; u < units; ++u) {
        const int64_t r = u / H, h = u % H, g = h / heads_per_group;
        const double A = -exp(A_log[h]);
        const double Dh = D ? D[h] : 0.0;
        const size_t PN = (size_t)(P * N);
        double* S = (double*)malloc((T > 0 ? (size_t)T : 1) * PN * sizeof(double));
        double* Gs = (double*)calloc(PN, sizeof(double));
        double* gb = (double*)malloc((size_t)P * sizeof(double));
        double* v = (double*)malloc((size_t)(T + 1) * 4 * sizeof(double));
        int64_t* seq = (int64_t*)malloc((size_t)(T + 1) * sizeof(int64_t));
        if (!S || !Gs || !gb || !v || !seq) {
            free(S); free(Gs); free(gb); free(v); free(seq);
            bad |= 1;
            continue;
        }
        double* Dl = v;             /* Delta_t */
        double* av = v + T;         /* a_t */
        double* fv = v + 2 * T;     /* input factor f_t */
        double* pre = v + 3 * T;    /* dt + bias (softplus argument) */
        /* forward, keeping every state */
        for (int64_t t = 0; t < T; ++t) {
            const int64_t k = seq_idx ? (int64_t)seq_idx[r * T + t] : r;
            if (k < 0 || k >= nseqs) { bad |= 1; break; }
            seq[t] = k;
            const int start = (t == 0 || k != seq[t - 1]);
            const double* prev = start ? (init ? init + (k * H + h) * P * N : NULL) : S + (size_t)(t - 1) * PN;
            double vv = dt[(r * T + t) * H + h] + (dt_bias ? dt_bias[h] : 0.0);
            pre[t] = vv;
            if (dt_softplus)
                vv = vv > 0.0 ? vv + log1p(exp(-vv)) : log1p(exp(vv));
            Dl[t] = vv;
            av[t] = exp(vv * A);
            fv[t] = input_scaling == 1 ? vv : (input_scaling == 2 ? expm1(vv * A) / A : 1.0);
            const double* xt = x + ((r * T + t) * H + h) * P;
            const double* Bt = B + ((r * T + t) * G + g) * N;
            double* St = S + (size_t)t * PN;
            for (int64_t p = 0; p < P; ++p)
                for (int64_t n = 0; n < N; ++n)
                    St[p * N + n] = av[t] * (prev ? prev[p * N + n] : 0.0) + fv[t] * xt[p] * Bt[n];
        }
        if (bad) { free(S); free(Gs); free(gb); free(v); free(seq); continue; }
        /* backward, from the last token */
        double dA = 0.0, dDs = 0.0, dbs = 0.0, aA = 0.0, aD = 0.0, ab = 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            const int64_t k = seq[t];
            const int last = (t == T - 1 || seq[t + 1] != k);
            const int start = (t == 0 || seq[t - 1] != k);
            if (last) {
                /* the state after the sequence's last token is its final state */
                for (size_t i = 0; i < PN; ++i)
                    Gs[i] = dfinal ? dfinal[(k * H + h) * (int64_t)PN + (int64_t)i] : 0.0;
            } else {
                for (size_t i = 0; i < PN; ++i)
                    Gs[i] *= av[t + 1];
            }
            const double* xt = x + ((r * T + t) * H + h) * P;
            const double* dyt = dy + ((r * T + t) * H + h) * P;
            const double* Bt = B + ((r * T + t) * G + g) * N;
            const double* Ct = C + ((r * T + t) * G + g) * N;
            for (int64_t p = 0; p < P; ++p)
                for (int64_t n = 0; n < N; ++n)
                    Gs[p * N + n] += dyt[p] * Ct[n];
            const double* St = S + (size_t)t * PN;
            const double* prev = start ? (init ? init + (k * H + h) * P * N : NULL) : S + (size_t)(t - 1) * PN;
            double* dCt = dCu + ((size_t)u * T + t) * N;
            double* dBt = dBu + ((size_t)u * T + t) * N;
            for (int64_t n = 0; n < N; ++n) {
                double sc = 0.0, sb = 0.0;
                for (int64_t p = 0; p < P; ++p) {
                    sc += St[p * N + n] * dyt[p];
                    sb += Gs[p * N + n] * xt[p];
                }
                dCt[n] = sc;
                dBt[n] = fv[t] * sb;
            }
            double df = 0.0, da = 0.0, dDt = 0.0;
            for (int64_t p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n)
                    acc += Gs[p * N + n] * Bt[n];
                gb[p] = acc;
                df += xt[p] * acc;
                dDt += dyt[p] * xt[p];
                dx[((r * T + t) * H + h) * P + p] = fv[t] * acc + Dh * dyt[p];
            }
            if (prev)
                for (size_t i = 0; i < PN; ++i)
                    da += Gs[i] * prev[i];
            const double a = av[t], Dv = Dl[t];
            double dfdD = 0.0, dfdA = 0.0;
            if (input_scaling == 1) {
                dfdD = 1.0;
            } else if (input_scaling == 2) {
                dfdD = a;
                dfdA = (Dv * A * a - a + 1.0) / (A * A);
            }
            const double dDelta = da * a * A + df * dfdD;
            dA += da * a * Dv + df * dfdA;
            aA += fabs((da * a * Dv + df * dfdA) * A);
            double g_dt = dDelta;
            if (dt_softplus)
                g_dt *= 1.0 / (1.0 + exp(-pre[t]));
            ddt[(r * T + t) * H + h] = g_dt;
            dbs += g_dt;
            dDs += dDt;
            ab += fabs(g_dt);
            aD += fabs(dDt);
            if (start) {
                double* di = dinit + (k * H + h) * P * N;
                for (size_t i = 0; i < PN; ++i)
                    di[i] = a * Gs[i];
            }
        }
        if (T == 0 && seq_idx == NULL) {
            /* no token: final = init, so dinit = dfinal */
            double* di = dinit + (r * H + h) * P * N;
            for (size_t i = 0; i < PN; ++i)
                di[i] = dfinal ? dfinal[(r * H + h) * (int64_t)PN + (int64_t)i] : 0.0;
        }
        sA[u] = dA * A;
        sD[u] = dDs;
        sBias[u] = dbs;
        sAbs[3 * u + 0] = aA;
        sAbs[3 * u + 1] = ab;
        sAbs[3 * u + 2] = aD;
        free(S); free(Gs); free(gb); free(v); free(seq);
    }
    if (!bad) {
        memset(dB, 0, (size_t)(batch * T * G * N) * sizeof(double));
        memset(dC, 0, (size_t)(batch * T * G * N) * sizeof(double));
        for (int64_t r = 0; r < batch; ++r)
            for (int64_t h = 0; h < H; ++h) {
                const int64_t u = r * H + h, g = h / heads_per_group;
                for (int64_t t = 0; t < T; ++t)
                    for (int64_t n = 0; n < N; ++n) {
                        dB[((r * T + t) * G + g) * N + n] += dBu[((size_t)u * T + t) * N + n];
                        dC[((r * T + t) * G + g) * N + n] += dCu[((size_t)u * T + t) * N + n];
                    }
            }
        for (int64_t h = 0; h < H; ++h) {
            double a = 0.0, d = 0.0, bb = 0.0;
            for (int64_t r = 0; r < batch; ++r) {
                a += sA[r * H + h];
                d += sD[r * H + h];
                bb += sBias[r * H + h];
            }
            dA_log[h] = a;
            if (dD) dD[h] = d;
            if (ddt_bias) ddt_bias[h] = bb;
            if (abs_sums) {
                double s0 = 0.0, s1 = 0.0, s2 = 0.0;
                for (int64_t r = 0; r < batch; ++r) {
                    s0 += sAbs[3 * (r * H + h) + 0];
                    s1 += sAbs[3 * (r * H + h) + 1];
                    s2 += sAbs[3 * (r * H + h) + 2];
                }
                abs_sums[3 * h + 0] = s0;
                abs_sums[3 * h + 1] = s1;
                abs_sums[3 * h + 2] = s2;
            }
        }
    }
    free(dBu); free(dCu); free(sA); free(sD); free(sBias); free(sAbs);
    return bad ? 2 : 0;
}
