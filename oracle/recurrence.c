/*
 * ORACLE -- test infrastructure only.  Nothing in the product path may link,
 * load or call this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg do.
 *
 * Plain fp64 token-by-token evaluation of the gated delta rule, the recurrence
 * that the chunkwise Map-Reduce-Map method ("Empowering Hybrid Attention Models
 * on NPUs", section 2.1) reaches up to rounding.  The state of one head is
 * S_t = S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T and the
 * output is o_t = scale * S_t q_t, with alpha_t = exp(g_t): g is a per-token
 * log-decay, a scalar per head (GDN) or a vector over the key channels (KDA).
 * The state is stored transposed, H = S^T, as a [d_k][d_v] row-major block per
 * (sequence, head).  Expanding the product gives the step used below:
 *     H <- Diag(alpha) H                    (decay on the key axis)
 *     u  = beta * (v - H^T k)               (delta-rule error)
 *     H <- H + k u^T                        (rank-one write)
 *     o  = scale * H^T q                    (read-out of the updated state)
 *
 * Varlen packing follows the FLA graph-capture RFC ("[RFC] Add Graph Capture
 * Support for FLA Prefill and Training Paths on Ascend NPUs", section
 * "Fixed-capacity execution"): tokens of all sequences are packed along T and
 * cu_seqlens[N+1] gives sequence boundaries; each sequence starts from its own
 * initial state (or zero).  Zero-length sequences are skipped: their final
 * state is not written.
 *
 * Token inputs are float32 arrays (bf16 and fp32 inputs are exact in float32);
 * the initial state is fp64 so a carried fp64 state can be fed back; all
 * arithmetic is fp64.  Parallel over independent (sequence, head) pairs only.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* 0 if cu_seqlens is a valid packing of at most T tokens into N sequences. */
int oracle_check_cu(const int32_t *cu, int N, int T)
{
    if (N < 1 || cu[0] != 0) return 1;
    for (int n = 0; n < N; ++n)
        if (cu[n + 1] < cu[n]) return 2;
    if (cu[N] > T) return 3;
    return 0;
}

static void one_unit(int kda, const float *q, const float *k, const float *v,
                     const float *g, const float *beta, int bos, int eos,
                     int h, int H, int dk, int dv, double scale,
                     const double *h0, double *o, double *ht, double *S,
                     double *a, double *u)
{
    /* S holds H = S^T of the recurrence, [dk][dv] */
    if (h0) {
        memcpy(S, h0, sizeof(double) * (size_t)dk * dv);
    } else {
        memset(S, 0, sizeof(double) * (size_t)dk * dv);
    }
    for (int t = bos; t < eos; ++t) {
        const float *qt = q + ((size_t)t * H + h) * dk;
        const float *kt = k + ((size_t)t * H + h) * dk;
        const float *vt = v + ((size_t)t * H + h) * dv;
        const double bt = (double)beta[(size_t)t * H + h];
        /* alpha_t = exp(g_t) on the key axis */
        if (kda) {
            const float *gt = g + ((size_t)t * H + h) * dk;
            for (int i = 0; i < dk; ++i) a[i] = exp((double)gt[i]);
        } else {
            const double at = exp((double)g[(size_t)t * H + h]);
            for (int i = 0; i < dk; ++i) a[i] = at;
        }
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[i * dv + j] *= a[i];
        /* u = beta (v - H^T k) */
        for (int j = 0; j < dv; ++j) u[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
            const double ki = (double)kt[i];
            for (int j = 0; j < dv; ++j) u[j] += S[i * dv + j] * ki;
        }
        for (int j = 0; j < dv; ++j) u[j] = bt * ((double)vt[j] - u[j]);
        /* H += k u^T */
        for (int i = 0; i < dk; ++i) {
            const double ki = (double)kt[i];
            for (int j = 0; j < dv; ++j) S[i * dv + j] += ki * u[j];
        }
        /* o = scale H^T q */
        double *ot = o + ((size_t)t * H + h) * dv;
        for (int j = 0; j < dv; ++j) ot[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
            const double qi = (double)qt[i];
            for (int j = 0; j < dv; ++j) ot[j] += S[i * dv + j] * qi;
        }
        for (int j = 0; j < dv; ++j) ot[j] *= scale;
    }
    if (ht) memcpy(ht, S, sizeof(double) * (size_t)dk * dv);
}

/*
 * q, k: [T][H][dk]; v: [T][H][dv]; g: [T][H] (GDN) or [T][H][dk] (KDA);
 * beta: [T][H]; cu: [N+1]; h0: [N][H][dk][dv] fp64 or NULL (zero state).
 * o: [T][H][dv] fp64, written for rows cu[0]..cu[N]-1 only.
 * ht: [N][H][dk][dv] fp64 or NULL, written only for non-empty sequences.
 * nthreads <= 0 means the OpenMP default.  Returns 0, or the
 * oracle_check_cu code (nothing written), or -1 on allocation failure.
 */
int oracle_gated_delta_fwd(int kda, const float *q, const float *k,
                           const float *v, const float *g, const float *beta,
                           const int32_t *cu, int N, int T, int H, int dk,
                           int dv, double scale, const double *h0, double *o,
                           double *ht, int nthreads)
{
    int bad = oracle_check_cu(cu, N, T);
    if (bad) return bad;
    const int units = N * H;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#else
    nthreads = 1;
#endif
    if (nthreads < 1) nthreads = 1;
    /* per-thread scratch, allocated before the parallel region */
    const size_t per = (size_t)dk * dv + (size_t)dk + (size_t)dv;
    double *scratch = (double *)malloc(sizeof(double) * per * (size_t)nthreads);
    if (!scratch) return -1;
#ifdef _OPENMP
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
#endif
    for (int w = 0; w < units; ++w) {
#ifdef _OPENMP
        double *S = scratch + per * (size_t)omp_get_thread_num();
#else
        double *S = scratch;
#endif
        double *a = S + (size_t)dk * dv;
        double *u = a + dk;
        const int n = w / H, h = w % H;
        const int bos = cu[n], eos = cu[n + 1];
        if (eos == bos) continue;
        const double *h0u = h0 ? h0 + ((size_t)n * H + h) * dk * dv : NULL;
        double *htu = ht ? ht + ((size_t)n * H + h) * dk * dv : NULL;
        one_unit(kda, q, k, v, g, beta, bos, eos, h, H, dk, dv, scale, h0u, o,
                 htu, S, a, u);
    }
    free(scratch);
    return 0;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
