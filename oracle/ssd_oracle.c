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
