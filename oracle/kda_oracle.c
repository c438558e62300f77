/*
 * kda_oracle.c -- fp64 CPU oracle for Kimi Delta Attention (KDA).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * bench's CPU-baseline leg load this library.  It shares no code with the
 * HIP path and must never be used as a fallback for it.
 *
 * What it computes: the token-by-token recurrence, in double precision,
 * one (sequence, head) pair at a time.
 *
 *   gate    g_t = g_min * sigmoid(exp(A_h) * z_t),  g_min = -5,
 *           alpha_t = exp(g_t)                     (per key channel)
 *     -- "Kimi K3：架构、训练与推理系统研究" §3.2; devpress K3 walk-through
 *        §3.2, Eq 5; "Hybrid KDA–MLA：Kimi K3 注意力机制解析", decay design.
 *
 *   update  Sbar  = Diag(alpha_t) S_{t-1}
 *           e_t   = v_t - Sbar^T k_t              (prediction error)
 *           S_t   = Sbar + beta_t k_t e_t^T
 *   readout o_t   = S_t^T q_t
 *     -- the prediction-error form of "Hybrid KDA–MLA", core update, and
 *        "Kimi K3：架构…" §3.1 (second display); algebraically the same as
 *        S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *        (devpress walk-through §3.1, Eq 1; "Kimi K3：架构…" §3.1).
 *
 * S is d_k x d_v in the mathematics.  In memory every state tensor
 * (h0, hT, the decode state) is [N][H][d_v][d_k]: element (n, h, j, i)
 * holds S_{i,j}.  Sequence n covers tokens [cu[n], cu[n+1]) of the packed
 * inputs and starts from h0[n] (zeros when h0 is NULL); its final state
 * goes to hT[n].  Sequences and heads are independent.
 *
 * Inputs q, k, v are read either as IEEE binary32 (io_dtype 1) or as
 * bfloat16 bit patterns (io_dtype 0); both widen to double exactly.
 * z, A, beta are binary32.  The initial state (h0, or the decode state)
 * is double, so that a state carried from one call to the next stays exact;
 * binary32 states widen to it without loss.  Outputs o and hT are double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KDA_ORACLE_GMIN (-5.0)

static double widen(const void *p, int io_dtype, size_t idx) {
    if (io_dtype == 1) return (double)((const float *)p)[idx];
    uint32_t u = (uint32_t)((const uint16_t *)p)[idx] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* g = g_min * sigmoid(exp(A_h) * z), sigmoid(x) = 1 / (1 + exp(-x)). */
double kda_oracle_gate(double A_h, double z) {
    double x = exp(A_h) * z;
    double s = 1.0 / (1.0 + exp(-x));
    return KDA_ORACLE_GMIN * s;
}

/* One (sequence, head) pair over tokens [t0, t1). */
static void run_pair(int io_dtype, const void *q, const void *k, const void *v,
                     const float *z, const float *A, const float *beta,
                     const double *h0, int n, int h, int t0, int t1,
                     int H, int dk, int dv, double *o, double *hT,
                     double *S, double *a, double *kk, double *qq, double *vv,
                     double *e) {
    /* S[i * dv + j] = S_{i,j} */
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            S[(size_t)i * dv + j] =
                h0 ? h0[(((size_t)n * H + h) * dv + j) * dk + i] : 0.0;

    for (int t = t0; t < t1; ++t) {
        size_t row_k = ((size_t)t * H + h) * dk;
        size_t row_v = ((size_t)t * H + h) * dv;
        double b = (double)beta[(size_t)t * H + h];
        for (int i = 0; i < dk; ++i) {
            a[i] = exp(kda_oracle_gate((double)A[h], (double)z[row_k + i]));
            kk[i] = widen(k, io_dtype, row_k + i);
            qq[i] = widen(q, io_dtype, row_k + i);
        }
        for (int j = 0; j < dv; ++j) vv[j] = widen(v, io_dtype, row_v + j);

        /* Sbar = Diag(alpha) S */
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= a[i];

        /* e = v - Sbar^T k */
        for (int j = 0; j < dv; ++j) {
            double p = 0.0;
            for (int i = 0; i < dk; ++i) p += S[(size_t)i * dv + j] * kk[i];
            e[j] = vv[j] - p;
        }

        /* S = Sbar + beta k e^T */
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += b * kk[i] * e[j];

        /* o = S^T q */
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i) acc += S[(size_t)i * dv + j] * qq[i];
            o[row_v + j] = acc;
        }
    }

    if (hT)
        for (int j = 0; j < dv; ++j)
            for (int i = 0; i < dk; ++i)
                hT[(((size_t)n * H + h) * dv + j) * dk + i] = S[(size_t)i * dv + j];
}

/*
 * Prefill over packed sequences.
 *   q, k : [T_tot][H][dk]   v : [T_tot][H][dv]   (io_dtype)
 *   z    : [T_tot][H][dk]   A : [H]   beta : [T_tot][H]      (binary32)
 *   h0   : [N][H][dv][dk] double, or NULL for zeros
 *   cu   : [N+1] non-decreasing, cu[0] = 0
 *   o    : [T_tot][H][dv] double (out)      hT : [N][H][dv][dk] double or NULL
 *   nthreads <= 0 leaves the OpenMP default.
 * Returns 0, or -1 on a bad argument or allocation failure.
 */
int kda_oracle_prefill(int io_dtype, const void *q, const void *k, const void *v,
                       const float *z, const float *A, const float *beta,
                       const double *h0, const int32_t *cu, int N, int H, int dk,
                       int dv, double *o, double *hT, int nthreads) {
    if (N < 0 || H <= 0 || dk <= 0 || dv <= 0 || !cu || !A) return -1;
    for (int n = 0; n < N; ++n)
        if (cu[n + 1] < cu[n]) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int npairs = N * H;
    int failed = 0;
#pragma omp parallel
    {
        double *S = malloc(sizeof(double) * (size_t)dk * dv);
        double *a = malloc(sizeof(double) * dk), *kk = malloc(sizeof(double) * dk);
        double *qq = malloc(sizeof(double) * dk), *vv = malloc(sizeof(double) * dv);
        double *e = malloc(sizeof(double) * dv);
        if (!S || !a || !kk || !qq || !vv || !e) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int p = 0; p < npairs; ++p) {
                int n = p / H, h = p % H;
                run_pair(io_dtype, q, k, v, z, A, beta, h0, n, h, cu[n], cu[n + 1],
                         H, dk, dv, o, hT, S, a, kk, qq, vv, e);
            }
        }
        free(S); free(a); free(kk); free(qq); free(vv); free(e);
    }
    return failed ? -1 : 0;
}

/*
 * One decode step: every sequence advances by exactly one token, starting
 * from S_in (double [N][H][dv][dk]); the new state goes to S_out (double,
 * same layout) and the readout to o ([N][H][dv] double).  This is the
 * prefill above with cu = 0, 1, ..., N ("Kimi K3：架构…" §11.2: the
 * recurrent state is read and updated in place once per new token).
 */
int kda_oracle_decode(int io_dtype, const void *q, const void *k, const void *v,
                      const float *z, const float *A, const float *beta,
                      const double *S_in, int N, int H, int dk, int dv, double *o,
                      double *S_out, int nthreads) {
    if (N <= 0) return 0;
    int32_t *cu = malloc(sizeof(int32_t) * (size_t)(N + 1));
    if (!cu) return -1;
    for (int n = 0; n <= N; ++n) cu[n] = n;
    int rc = kda_oracle_prefill(io_dtype, q, k, v, z, A, beta, S_in, cu, N, H, dk,
                                dv, o, S_out, nthreads);
    free(cu);
    return rc;
}

int kda_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
