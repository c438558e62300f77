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

/*
 * Backward (reverse mode) of the prefill, one (sequence, head) pair.
 *
 * The pages give no backward formula; this is the exact derivative of the
 * token recurrence above, taken step by step in reverse.  With Lambda the
 * gradient of the loss with respect to S_t (d_k x d_v), per token t from the
 * last to the first:
 *   Lambda += q_t do_t^T                       (o_t = S_t^T q_t)
 *   dq_t    = S_t do_t
 *   Sbar = Diag(alpha_t) S_{t-1},  p = Sbar^T k_t,  e = v_t - p
 *   dbeta_t = k_t^T Lambda e                   (S_t = Sbar + beta k e^T)
 *   de      = beta Lambda^T k_t,  dv_t = de,  dp = -de
 *   dk_t    = beta Lambda e + Sbar dp
 *   dSbar   = Lambda + k_t dp^T
 *   dalpha  = rowsum(dSbar .* S_{t-1}),  Lambda <- Diag(alpha_t) dSbar
 *   dg      = alpha .* dalpha, and through g = g_min sigmoid(x), x = e^A z:
 *   dz      = dg g_min s (1 - s) e^A,   dA_h += sum dg g_min s (1 - s) x
 * and finally dh0 = Lambda.  The states S_{t-1}, S_t are recomputed from
 * checkpoints taken every KDA_ORACLE_CK tokens of the forward pass.
 */
#define KDA_ORACLE_CK 64

static void back_pair(int io_dtype, const void *q, const void *k, const void *v, const float *z,
                      const float *A, const float *beta, const double *h0, const double *dO,
                      const double *dhT, int n, int h, int t0, int t1, int H, int dk, int dv,
                      double *gq, double *gk, double *gv, double *gz, double *gbeta, double *gA_pair,
                      double *gh0, double *ck, double *st, double *L, double *a, double *kk,
                      double *qq, double *vv, double *e, double *w1, double *w2) {
    const size_t SS = (size_t)dk * dv;
    const int len = t1 - t0;
    const int nck = len / KDA_ORACLE_CK + 1;
    const double eA = exp((double)A[h]);
    /* forward: the state before every KDA_ORACLE_CK-th token */
    double *S = st;   /* scratch: current state */
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            S[(size_t)i * dv + j] = h0 ? h0[(((size_t)n * H + h) * dv + j) * dk + i] : 0.0;
    for (int t = 0; t < len; ++t) {
        if (t % KDA_ORACLE_CK == 0) memcpy(ck + (size_t)(t / KDA_ORACLE_CK) * SS, S, sizeof(double) * SS);
        const int tg = t0 + t;
        const size_t row_k = ((size_t)tg * H + h) * dk, row_v = ((size_t)tg * H + h) * dv;
        const double b = (double)beta[(size_t)tg * H + h];
        for (int i = 0; i < dk; ++i) {
            a[i] = exp(kda_oracle_gate((double)A[h], (double)z[row_k + i]));
            kk[i] = widen(k, io_dtype, row_k + i);
        }
        for (int j = 0; j < dv; ++j) vv[j] = widen(v, io_dtype, row_v + j);
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= a[i];
        for (int j = 0; j < dv; ++j) {
            double p = 0.0;
            for (int i = 0; i < dk; ++i) p += S[(size_t)i * dv + j] * kk[i];
            e[j] = vv[j] - p;
        }
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += b * kk[i] * e[j];
    }
    (void)nck;

    /* Lambda = dhT */
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            L[(size_t)i * dv + j] = dhT ? dhT[(((size_t)n * H + h) * dv + j) * dk + i] : 0.0;
    double gA = 0.0;
    /* chunks in reverse; inside a chunk, states recomputed into st[0..C] */
    for (int c0 = (len - 1) / KDA_ORACLE_CK * KDA_ORACLE_CK; len > 0 && c0 >= 0; c0 -= KDA_ORACLE_CK) {
        const int c1 = c0 + KDA_ORACLE_CK < len ? c0 + KDA_ORACLE_CK : len;
        memcpy(st, ck + (size_t)(c0 / KDA_ORACLE_CK) * SS, sizeof(double) * SS);
        for (int t = c0; t < c1; ++t) {   /* st[t - c0 + 1] = S after token t */
            const int tg = t0 + t;
            const size_t row_k = ((size_t)tg * H + h) * dk, row_v = ((size_t)tg * H + h) * dv;
            const double b = (double)beta[(size_t)tg * H + h];
            const double *Sp = st + (size_t)(t - c0) * SS;
            double *Sn = st + (size_t)(t - c0 + 1) * SS;
            for (int i = 0; i < dk; ++i) {
                a[i] = exp(kda_oracle_gate((double)A[h], (double)z[row_k + i]));
                kk[i] = widen(k, io_dtype, row_k + i);
            }
            for (int j = 0; j < dv; ++j) vv[j] = widen(v, io_dtype, row_v + j);
            for (int j = 0; j < dv; ++j) {
                double p = 0.0;
                for (int i = 0; i < dk; ++i) p += a[i] * Sp[(size_t)i * dv + j] * kk[i];
                e[j] = vv[j] - p;
            }
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j)
                    Sn[(size_t)i * dv + j] = a[i] * Sp[(size_t)i * dv + j] + b * kk[i] * e[j];
        }
        for (int t = c1 - 1; t >= c0; --t) {
            const int tg = t0 + t;
            const size_t row_k = ((size_t)tg * H + h) * dk, row_v = ((size_t)tg * H + h) * dv;
            const double b = (double)beta[(size_t)tg * H + h];
            const double *Sp = st + (size_t)(t - c0) * SS;      /* S_{t-1} */
            const double *Sn = st + (size_t)(t - c0 + 1) * SS;  /* S_t */
            for (int i = 0; i < dk; ++i) {
                a[i] = exp(kda_oracle_gate((double)A[h], (double)z[row_k + i]));
                kk[i] = widen(k, io_dtype, row_k + i);
                qq[i] = widen(q, io_dtype, row_k + i);
            }
            for (int j = 0; j < dv; ++j) vv[j] = widen(v, io_dtype, row_v + j);
            const double *dOt = dO + row_v;
            /* Lambda += q do^T;  dq = S_t do */
            for (int i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int j = 0; j < dv; ++j) {
                    L[(size_t)i * dv + j] += qq[i] * dOt[j];
                    acc += Sn[(size_t)i * dv + j] * dOt[j];
                }
                gq[row_k + i] = acc;
            }
            /* e = v - Sbar^T k,  w1 = Lambda^T k */
            for (int j = 0; j < dv; ++j) {
                double p = 0.0, lk = 0.0;
                for (int i = 0; i < dk; ++i) {
                    p += a[i] * Sp[(size_t)i * dv + j] * kk[i];
                    lk += L[(size_t)i * dv + j] * kk[i];
                }
                e[j] = vv[j] - p;
                w1[j] = lk;
            }
            double db = 0.0;
            for (int j = 0; j < dv; ++j) db += w1[j] * e[j];
            gbeta[(size_t)tg * H + h] = db;
            /* dv = beta Lambda^T k;  dp = -dv (kept in w1) */
            for (int j = 0; j < dv; ++j) {
                gv[row_v + j] = b * w1[j];
                w1[j] = -b * w1[j];
            }
            /* dk = beta Lambda e + Sbar dp */
            for (int i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int j = 0; j < dv; ++j)
                    acc += b * L[(size_t)i * dv + j] * e[j] + a[i] * Sp[(size_t)i * dv + j] * w1[j];
                gk[row_k + i] = acc;
            }
            /* dSbar = Lambda + k dp^T;  dalpha = rowsum(dSbar .* S_{t-1});  Lambda = Diag(alpha) dSbar */
            for (int i = 0; i < dk; ++i) {
                double da = 0.0;
                for (int j = 0; j < dv; ++j) {
                    const double ds = L[(size_t)i * dv + j] + kk[i] * w1[j];
                    da += ds * Sp[(size_t)i * dv + j];
                    L[(size_t)i * dv + j] = a[i] * ds;
                }
                w2[i] = a[i] * da;   /* dg */
            }
            /* through the gate */
            for (int i = 0; i < dk; ++i) {
                const double x = eA * (double)z[row_k + i];
                const double s = 1.0 / (1.0 + exp(-x));
                const double dx = w2[i] * KDA_ORACLE_GMIN * s * (1.0 - s);
                gz[row_k + i] = dx * eA;
                gA += dx * x;
            }
        }
    }
    *gA_pair = gA;
    if (gh0)
        for (int j = 0; j < dv; ++j)
            for (int i = 0; i < dk; ++i)
                gh0[(((size_t)n * H + h) * dv + j) * dk + i] = L[(size_t)i * dv + j];
}

/*
 * Gradients of L = sum(dO . o) + sum(dhT . hT) for the prefill above.
 *   dO : [T_tot][H][dv] double;  dhT : [N][H][dv][dk] double or NULL
 *   gq, gk : [T_tot][H][dk];  gv : [T_tot][H][dv];  gz : [T_tot][H][dk];
 *   gbeta : [T_tot][H];  gA : [H];  gh0 : [N][H][dv][dk] or NULL   (double, out)
 * gA sums the (sequence, head) contributions in sequence order.
 */
int kda_oracle_backward(int io_dtype, const void *q, const void *k, const void *v, const float *z,
                        const float *A, const float *beta, const double *h0, const int32_t *cu, int N,
                        int H, int dk, int dv, const double *dO, const double *dhT, double *gq, double *gk,
                        double *gv, double *gz, double *gbeta, double *gA, double *gh0, int nthreads) {
    if (N < 0 || H <= 0 || dk <= 0 || dv <= 0 || !cu || !A || !dO) return -1;
    for (int n = 0; n < N; ++n)
        if (cu[n + 1] < cu[n]) return -1;
    int maxlen = 0;
    for (int n = 0; n < N; ++n)
        if (cu[n + 1] - cu[n] > maxlen) maxlen = cu[n + 1] - cu[n];
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    const size_t SS = (size_t)dk * dv;
    const int nck = maxlen / KDA_ORACLE_CK + 1;
    double *gA_pairs = calloc((size_t)N * H + 1, sizeof(double));
    if (!gA_pairs) return -1;
    int failed = 0;
    const int npairs = N * H;
#pragma omp parallel
    {
        double *ck = malloc(sizeof(double) * SS * (size_t)nck);
        double *st = malloc(sizeof(double) * SS * (KDA_ORACLE_CK + 1));
        double *L = malloc(sizeof(double) * SS);
        double *a = malloc(sizeof(double) * dk), *kk = malloc(sizeof(double) * dk);
        double *qq = malloc(sizeof(double) * dk), *w2 = malloc(sizeof(double) * dk);
        double *vv = malloc(sizeof(double) * dv), *e = malloc(sizeof(double) * dv);
        double *w1 = malloc(sizeof(double) * dv);
        if (!ck || !st || !L || !a || !kk || !qq || !w2 || !vv || !e || !w1) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int p = 0; p < npairs; ++p) {
                const int n = p / H, h = p % H;
                back_pair(io_dtype, q, k, v, z, A, beta, h0, dO, dhT, n, h, cu[n], cu[n + 1], H, dk, dv,
                          gq, gk, gv, gz, gbeta, gA_pairs + p, gh0, ck, st, L, a, kk, qq, vv, e, w1, w2);
            }
        }
        free(ck); free(st); free(L); free(a); free(kk); free(qq); free(w2); free(vv); free(e); free(w1);
    }
    if (!failed)
        for (int h = 0; h < H; ++h) {
            double s = 0.0;
            for (int n = 0; n < N; ++n) s += gA_pairs[(size_t)n * H + h];
            gA[h] = s;
        }
    free(gA_pairs);
    return failed ? -1 : 0;
}

int kda_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
