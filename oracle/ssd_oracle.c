/*
 * ssd_oracle.c -- fp64 CPU oracle of the SSD layer forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code,
 * header, table or helper with the HIP path in mamba_ssd_layer_amd/csrc and
 * the product path never calls it.
 *
 * Pages cited (titles as published):
 *   [T] "Transformers是SSMs：通过结构化状态空间对偶性的广义模型和高效算法(一)"
 *       (nxbn.cn/automobile/1783.html), a translation of "Transformers are
 *       SSMs" sections 1-5.
 *   [M] "LLM(十一)——Mamba" (mztchaoqun.com.cn/posts/D49_Mamba).
 *   [S] "Mamba-2 状态空间对偶性理论" (metaphor-xennon.pages.dev).
 *
 * What is computed (the plain definition, no chunking, no logs, no cumsums):
 *   the selective SSM with a scalar-times-identity transition, [T] §2.4
 *   ("recurrent (linear) form") and §5.1, [M] §3.1.1-3.1.2, [S] §1.2:
 *       h_t = a_t * h_{t-1} + x_t (outer) B_t        h: (P, N) per head
 *       y_t = h_t . C_t                              y: (P)
 *   with a_t = exp(dt_t * A_h).  The state entering the first token of every
 *   sequence is zero (or the caller's initial state), so that token's own a_t
 *   never contributes: [T] §3.1 unrolls h_0 = B_0 x_0, and the 1-SS matrix of
 *   [T] §3.2.2 is built from a_1 .. a_{T-1} only.
 *   Each head h reads the B/C group g = h * G / H (contiguous head blocks per
 *   group: [M] §3.6.2 leaves the head-to-group map unstated; this is the
 *   reading used throughout).
 *   Variable-length batches ([M] §3.7.3): every sequence [cu[s], cu[s+1]) of
 *   the packed token axis is an independent run from a zero state.
 *
 * Parallelism: OpenMP over the independent (sequence, head) pairs.  The inner
 * arithmetic per pair is the sequential recurrence above, in fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/*
 * Layouts (all row-major, packed token axis of length Ttot):
 *   x  (Ttot, H, P)     dt (Ttot, H)     A (H)
 *   B  (Ttot, G, N)     C  (Ttot, G, N)
 *   cu_seqlens (S + 1), cu[0] = 0, non-decreasing, cu[S] = Ttot
 *   init_state (S, H, P, N) or NULL (zero)
 *   y  (Ttot, H, P)     final_state (S, H, P, N) or NULL
 * Returns 0, or -1 on inconsistent arguments (nothing written then).
 */
int ssd_oracle_recurrence(const double *x, const double *dt, const double *A,
                          const double *B, const double *C,
                          const int64_t *cu_seqlens, int64_t nseq,
                          int64_t H, int64_t P, int64_t N, int64_t G,
                          const double *init_state, double *y,
                          double *final_state, int nthreads)
{
    if (nseq < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0)
        return -1;
    if (nseq > 0 && cu_seqlens[0] != 0)
        return -1;
    for (int64_t s = 0; s < nseq; ++s)
        if (cu_seqlens[s + 1] < cu_seqlens[s])
            return -1;
    const int64_t heads_per_group = H / G;
    const int64_t npairs = nseq * H;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int failed = 0;
#pragma omp parallel
    {
        double *h = (double *)malloc(sizeof(double) * (size_t)(P * N));
        if (h == NULL) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t pair = 0; pair < npairs; ++pair) {
            if (h == NULL)
                continue;
            const int64_t s = pair / H;
            const int64_t hd = pair % H;
            const int64_t g = hd / heads_per_group; /* = hd * G / H */
            if (init_state != NULL)
                memcpy(h, init_state + (s * H + hd) * P * N, sizeof(double) * (size_t)(P * N));
            else
                memset(h, 0, sizeof(double) * (size_t)(P * N));
            for (int64_t t = cu_seqlens[s]; t < cu_seqlens[s + 1]; ++t) {
                const double a = exp(dt[t * H + hd] * A[hd]);
                const double *xt = x + (t * H + hd) * P;
                const double *Bt = B + (t * G + g) * N;
                const double *Ct = C + (t * G + g) * N;
                double *yt = y + (t * H + hd) * P;
                for (int64_t p = 0; p < P; ++p) {
                    double *hp = h + p * N;
                    double acc = 0.0;
                    for (int64_t n = 0; n < N; ++n) {
                        hp[n] = a * hp[n] + xt[p] * Bt[n];
                        acc += hp[n] * Ct[n];
                    }
                    yt[p] = acc;
                }
            }
            if (final_state != NULL)
                memcpy(final_state + (s * H + hd) * P * N, h, sizeof(double) * (size_t)(P * N));
        }
        free(h);
    }
    return failed ? -1 : 0;
}

/* Number of OpenMP threads a parallel region would use (for reporting). */
int ssd_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Backward pass of the recurrence above (the chain rule taken through it in
 * reverse token order, i.e. the adjoint recurrence), for a loss whose
 * gradients dy = dL/dy and dfinal = dL/dh_last are given:
 *     G_t  = dy_t (outer) C_t + a_{t+1} G_{t+1}     (G = dL/dh_t, (P, N);
 *                                                   G past the last token = dfinal)
 *     dx_t = G_t . B_t            (sum over n)
 *     dB_t += G_t^T x_t           (sum over p; per head here, the caller sums a group)
 *     dC_t += h_t^T dy_t          (sum over p; per head)
 *     da_t = <G_t, h_{t-1}>,  d(dt_t) = A_h a_t da_t,  dA_h += dt_t a_t da_t
 *     dL/d(initial state) = a_first G_first
 * The states h_t are recomputed from checkpoints kept every kCk tokens (no
 * division by a_t, which may be 0).
 * Layouts as for the forward; dy (Ttot, H, P); dfinal and dinit (S, H, P, N)
 * or NULL; outputs dx (Ttot, H, P), ddt (Ttot, H), dA (S, H) per sequence,
 * dB and dC (Ttot, H, N) per head.  Returns 0, or -1 on bad arguments or
 * memory exhaustion.
 */
#define kCk 64
int ssd_oracle_backward(const double *x, const double *dt, const double *A,
                        const double *B, const double *C,
                        const int64_t *cu_seqlens, int64_t nseq,
                        int64_t H, int64_t P, int64_t N, int64_t G,
                        const double *init_state, const double *dy,
                        const double *dfinal, double *dx, double *ddt,
                        double *dA, double *dB, double *dC, double *dinit,
                        int nthreads)
{
    if (nseq < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0)
        return -1;
    if (nseq > 0 && cu_seqlens[0] != 0)
        return -1;
    int64_t maxlen = 0;
    for (int64_t s = 0; s < nseq; ++s) {
        if (cu_seqlens[s + 1] < cu_seqlens[s])
            return -1;
        if (cu_seqlens[s + 1] - cu_seqlens[s] > maxlen)
            maxlen = cu_seqlens[s + 1] - cu_seqlens[s];
    }
    const int64_t heads_per_group = H / G;
    const int64_t npairs = nseq * H;
    const int64_t PN = P * N;
    const int64_t nck_max = (maxlen + kCk - 1) / kCk + 1;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int failed = 0;
#pragma omp parallel
    {
        double *ck = (double *)malloc(sizeof(double) * (size_t)(nck_max * PN));
        double *seg = (double *)malloc(sizeof(double) * (size_t)(kCk * PN));
        double *g = (double *)malloc(sizeof(double) * (size_t)PN);
        double *h = (double *)malloc(sizeof(double) * (size_t)PN);
        if (!ck || !seg || !g || !h) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t pair = 0; pair < npairs; ++pair) {
            if (!ck || !seg || !g || !h)
                continue;
            const int64_t s = pair / H;
            const int64_t hd = pair % H;
            const int64_t gr = hd / heads_per_group;
            const int64_t t0 = cu_seqlens[s], L = cu_seqlens[s + 1] - t0;
            const int64_t nck = (L + kCk - 1) / kCk;
            /* forward: the state entering tokens t0, t0 + kCk, ... */
            if (init_state != NULL)
                memcpy(h, init_state + (s * H + hd) * PN, sizeof(double) * (size_t)PN);
            else
                memset(h, 0, sizeof(double) * (size_t)PN);
            for (int64_t i = 0; i < L; ++i) {
                const int64_t t = t0 + i;
                if (i % kCk == 0)
                    memcpy(ck + (i / kCk) * PN, h, sizeof(double) * (size_t)PN);
                const double a = exp(dt[t * H + hd] * A[hd]);
                for (int64_t p = 0; p < P; ++p)
                    for (int64_t n = 0; n < N; ++n)
                        h[p * N + n] = a * h[p * N + n] + x[(t * H + hd) * P + p] * B[(t * G + gr) * N + n];
            }
            /* backward, one checkpoint segment at a time */
            if (dfinal != NULL)
                memcpy(g, dfinal + (s * H + hd) * PN, sizeof(double) * (size_t)PN);
            else
                memset(g, 0, sizeof(double) * (size_t)PN);
            double dA_acc = 0.0;
            for (int64_t c = nck - 1; c >= 0; --c) {
                const int64_t i0 = c * kCk;
                const int64_t i1 = (i0 + kCk < L) ? i0 + kCk : L;
                /* states after each token of the segment */
                const double *prev = ck + c * PN;
                for (int64_t i = i0; i < i1; ++i) {
                    const int64_t t = t0 + i;
                    const double a = exp(dt[t * H + hd] * A[hd]);
                    double *cur = seg + (i - i0) * PN;
                    for (int64_t p = 0; p < P; ++p)
                        for (int64_t n = 0; n < N; ++n)
                            cur[p * N + n] = a * prev[p * N + n] + x[(t * H + hd) * P + p] * B[(t * G + gr) * N + n];
                    prev = cur;
                }
                for (int64_t i = i1 - 1; i >= i0; --i) {
                    const int64_t t = t0 + i;
                    const double a = exp(dt[t * H + hd] * A[hd]);
                    const double *ht = seg + (i - i0) * PN;
                    const double *hprev = (i > i0) ? seg + (i - 1 - i0) * PN : ck + c * PN;
                    const double *xt = x + (t * H + hd) * P;
                    const double *dyt = dy + (t * H + hd) * P;
                    const double *Bt = B + (t * G + gr) * N;
                    const double *Ct = C + (t * G + gr) * N;
                    double *dBt = dB + (t * H + hd) * N;
                    double *dCt = dC + (t * H + hd) * N;
                    for (int64_t n = 0; n < N; ++n) {
                        dBt[n] = 0.0;
                        dCt[n] = 0.0;
                    }
                    double da = 0.0;
                    for (int64_t p = 0; p < P; ++p) {
                        double dxp = 0.0;
                        for (int64_t n = 0; n < N; ++n) {
                            const double gv = g[p * N + n] + dyt[p] * Ct[n];
                            g[p * N + n] = gv;
                            dxp += gv * Bt[n];
                            dBt[n] += gv * xt[p];
                            dCt[n] += ht[p * N + n] * dyt[p];
                            da += gv * hprev[p * N + n];
                        }
                        dx[(t * H + hd) * P + p] = dxp;
                    }
                    const double dl = a * da;
                    ddt[t * H + hd] = A[hd] * dl;
                    dA_acc += dt[t * H + hd] * dl;
                    for (int64_t e = 0; e < PN; ++e)
                        g[e] *= a;
                }
            }
            dA[s * H + hd] = dA_acc;
            if (dinit != NULL)
                memcpy(dinit + (s * H + hd) * PN, g, sizeof(double) * (size_t)PN);
        }
        free(ck);
        free(seg);
        free(g);
        free(h);
    }
    return failed ? -1 : 0;
}

/*
 * Selective scan with a diagonal transition (Mamba-1's S6 layer), the
 * comparator of the SSD layer: [M] §3.1.1 (diagonal structure, A stored as its
 * N diagonal entries), §3.1.2 (SSD restricts that diagonal to one scalar) and
 * §2.1.2-2.1.3 (an independent SSM per channel d of D, step size Delta per
 * token and channel, B and C per token shared by the channels).  With
 * a_t[d][n] = exp(Delta_t[d] * A[d][n]) and the first-order input term:
 *       h_t[d][n] = a_t[d][n] * h_{t-1}[d][n] + Delta_t[d] * B_t[n] * x_t[d]
 *       y_t[d]    = sum_n C_t[n] * h_t[d][n]
 * from a zero state at the start of every sequence.  SSD with the dt-scaled
 * input is the special case A[d][n] = A_h for every n and Delta_t[d] = dt_t[h]
 * for the channels d of head h.
 * Layouts: x, Delta (b, T, D); A (D, N); B, C (b, T, N); y (b, T, D);
 * final_state (b, D, N) or NULL.  Returns 0, or -1 on bad sizes.
 * OpenMP over the independent (sequence, channel) pairs.
 */
int ssd_oracle_selective_scan(const double *x, const double *delta, const double *A,
                              const double *B, const double *C, int64_t nbatch,
                              int64_t T, int64_t D, int64_t N, double *y,
                              double *final_state, int nthreads)
{
    if (nbatch < 0 || T < 0 || D <= 0 || N <= 0)
        return -1;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    const int64_t pairs = nbatch * D;
#pragma omp parallel
    {
        double *h = (double *)malloc((size_t)N * sizeof(double));
#pragma omp for schedule(static)
        for (int64_t q = 0; q < pairs; ++q) {
            const int64_t b = q / D, d = q % D;
            for (int64_t n = 0; n < N; ++n)
                h[n] = 0.0;
            for (int64_t t = 0; t < T; ++t) {
                const int64_t tok = b * T + t;
                const double dl = delta[tok * D + d];
                const double u = dl * x[tok * D + d];
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    h[n] = exp(dl * A[d * N + n]) * h[n] + u * B[tok * N + n];
                    acc += C[tok * N + n] * h[n];
                }
                y[tok * D + d] = acc;
            }
            if (final_state)
                for (int64_t n = 0; n < N; ++n)
                    final_state[(b * D + d) * N + n] = h[n];
        }
        free(h);
    }
    return 0;
}
