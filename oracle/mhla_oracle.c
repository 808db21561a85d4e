/*
 * mhla_oracle.c -- plain, slow, binary64 CPU oracle for the MHLA forward pass.
 *
 * TEST INFRASTRUCTURE ONLY: called by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product path.  It shares no
 * code with the GPU library.
 *
 * The four steps follow "MHLA: Restoring Expressivity of Linear Attention via
 * Token-Level Multi-Head" in the order of its §4.1:
 *   1. feature map        phi = ELU + 1                ("Linear Attention 笔记" §2)
 *   2. local summaries    S_b = sum_{j in b} phi(k_j) v_j^T,  z_b = sum_{j in b} phi(k_j)
 *   3. multi-head mixing  S~_i = sum_b m_{i,b} S_b,           z~_i = sum_b m_{i,b} z_b
 *   4. output             y_t = phi(q_t)^T S~_i / (phi(q_t)^T z~_i + 1e-6)
 * The causal variant takes App. C: the mix runs over earlier blocks b < i, and
 * within block i the running summary is updated token by token,
 * S_i <- S_i + phi(k_t) v_t^T, and re-mixed with m_{i,i} before token t reads it
 * (the prefix therefore includes t itself, as in the recurrence of
 * "Linear Attention 笔记" §4).  The 1e-6 guard sits after the complete mixed
 * dot product, as in that page's §4 and §5.
 */
#include "mhla_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

double mhla_oracle_phi(double x) {
    /* ELU with alpha = 1 is x for x > 0 and exp(x) - 1 otherwise; plus one. */
    return x > 0.0 ? x + 1.0 : exp(x);
}

static int sizes_ok(long BH, long N, long d, long M) {
    return BH >= 1 && N >= 1 && d >= 1 && M >= 1 && N % M == 0;
}

int mhla_oracle_summaries(const float* k, const float* v, long BH, long N, long d, long M,
                          double* S, double* z) {
    if (!sizes_ok(BH, N, d, M) || !k || !v || !S || !z) return -1;
    const long C = N / M;
    double* fk = (double*)malloc(sizeof(double) * d);
    if (!fk) return -1;
    for (long p = 0; p < BH; ++p) {
        for (long b = 0; b < M; ++b) {
            double* Sb = S + (p * M + b) * d * d;
            double* zb = z + (p * M + b) * d;
            memset(Sb, 0, sizeof(double) * d * d);
            memset(zb, 0, sizeof(double) * d);
            for (long j = b * C; j < (b + 1) * C; ++j) {
                const float* kj = k + (p * N + j) * d;
                const float* vj = v + (p * N + j) * d;
                for (long r = 0; r < d; ++r) fk[r] = mhla_oracle_phi((double)kj[r]);
                for (long r = 0; r < d; ++r) {
                    for (long c = 0; c < d; ++c) Sb[r * d + c] += fk[r] * (double)vj[c];
                    zb[r] += fk[r];
                }
            }
        }
    }
    free(fk);
    return 0;
}

int mhla_oracle_mix(const double* S, const double* z, const float* W, long BH, long d, long M,
                    int causal, double* St, double* zt) {
    if (BH < 1 || d < 1 || M < 1 || !S || !z || !W || !St || !zt) return -1;
    for (long p = 0; p < BH; ++p) {
        for (long i = 0; i < M; ++i) {
            double* Si = St + (p * M + i) * d * d;
            double* zi = zt + (p * M + i) * d;
            memset(Si, 0, sizeof(double) * d * d);
            memset(zi, 0, sizeof(double) * d);
            const long bend = causal ? i : M; /* causal: earlier blocks only */
            for (long b = 0; b < bend; ++b) {
                const double w = (double)W[i * M + b];
                const double* Sb = S + (p * M + b) * d * d;
                const double* zb = z + (p * M + b) * d;
                for (long e = 0; e < d * d; ++e) Si[e] += w * Sb[e];
                for (long r = 0; r < d; ++r) zi[r] += w * zb[r];
            }
        }
    }
    return 0;
}

/* One (batch, head) pair; q, k, v, out point at its [N][d] slices. */
static int forward_pair(const float* q, const float* k, const float* v, const float* W,
                        double* out, long N, long d, long M, int causal, int normalise) {
    const long C = N / M;
    double* S = (double*)malloc(sizeof(double) * M * d * d);
    double* z = (double*)malloc(sizeof(double) * M * d);
    double* St = (double*)malloc(sizeof(double) * M * d * d);
    double* zt = (double*)malloc(sizeof(double) * M * d);
    double* P = (double*)malloc(sizeof(double) * d * d);
    double* pz = (double*)malloc(sizeof(double) * d);
    double* fq = (double*)malloc(sizeof(double) * d);
    double* fk = (double*)malloc(sizeof(double) * d);
    int rc = -1;
    if (!S || !z || !St || !zt || !P || !pz || !fq || !fk) goto done;

    if (mhla_oracle_summaries(k, v, 1, N, d, M, S, z) != 0) goto done;
    if (mhla_oracle_mix(S, z, W, 1, d, M, causal, St, zt) != 0) goto done;

    for (long i = 0; i < M; ++i) {
        const double* Si = St + i * d * d;
        const double* zi = zt + i * d;
        const double wii = (double)W[i * M + i];
        memset(P, 0, sizeof(double) * d * d);
        memset(pz, 0, sizeof(double) * d);
        for (long t = i * C; t < (i + 1) * C; ++t) {
            for (long r = 0; r < d; ++r) fq[r] = mhla_oracle_phi((double)q[t * d + r]);
            if (causal) {
                /* App. C inference: fold token t into its block's running summary. */
                for (long r = 0; r < d; ++r) fk[r] = mhla_oracle_phi((double)k[t * d + r]);
                for (long r = 0; r < d; ++r) {
                    for (long c = 0; c < d; ++c) P[r * d + c] += fk[r] * (double)v[t * d + c];
                    pz[r] += fk[r];
                }
            }
            double den = 0.0;
            for (long r = 0; r < d; ++r)
                den += fq[r] * (causal ? zi[r] + wii * pz[r] : zi[r]);
            den += MHLA_ORACLE_EPS;
            for (long c = 0; c < d; ++c) {
                double num = 0.0;
                for (long r = 0; r < d; ++r)
                    num += fq[r] * (causal ? Si[r * d + c] + wii * P[r * d + c] : Si[r * d + c]);
                /* Without the normaliser (the [MHLA] §4.1 remark on long sequences) the
                   output is the mixed numerator itself. */
                out[t * d + c] = normalise ? num / den : num;
            }
        }
    }
    rc = 0;
done:
    free(S); free(z); free(St); free(zt); free(P); free(pz); free(fq); free(fk);
    return rc;
}

/* One (batch, head) pair with an explicit block assignment: token t belongs to block
 * blk[t] ([MHLA] §4.1: blocks of N_b tokens along spatial or spatio-temporal axes, of
 * any sizes).  Non-causal. */
static int forward_pair_blocks(const float* q, const float* k, const float* v, const float* W,
                               double* out, long N, long d, long M, const int* blk, int normalise) {
    double* S = (double*)calloc((size_t)(M * d * d), sizeof(double));
    double* z = (double*)calloc((size_t)(M * d), sizeof(double));
    double* St = (double*)malloc(sizeof(double) * M * d * d);
    double* zt = (double*)malloc(sizeof(double) * M * d);
    double* fq = (double*)malloc(sizeof(double) * d);
    double* fk = (double*)malloc(sizeof(double) * d);
    int rc = -1;
    if (!S || !z || !St || !zt || !fq || !fk) goto done;
    for (long j = 0; j < N; ++j) { /* step 2: every token into its own block's summary */
        const long b = blk[j];
        if (b < 0 || b >= M) goto done;
        for (long r = 0; r < d; ++r) fk[r] = mhla_oracle_phi((double)k[j * d + r]);
        for (long r = 0; r < d; ++r) {
            for (long c = 0; c < d; ++c) S[(b * d + r) * d + c] += fk[r] * (double)v[j * d + c];
            z[b * d + r] += fk[r];
        }
    }
    if (mhla_oracle_mix(S, z, W, 1, d, M, 0, St, zt) != 0) goto done;
    for (long t = 0; t < N; ++t) { /* step 4 with the mixed summary of t's block */
        const long i = blk[t];
        const float* qt = q + t * d;
        for (long r = 0; r < d; ++r) fq[r] = mhla_oracle_phi((double)qt[r]);
        double dot = 0.0;
        for (long r = 0; r < d; ++r) dot += fq[r] * zt[i * d + r];
        const double guarded = dot + MHLA_ORACLE_EPS;
        for (long c = 0; c < d; ++c) {
            double acc = 0.0;
            for (long r = 0; r < d; ++r) acc += fq[r] * St[(i * d + r) * d + c];
            out[t * d + c] = normalise ? acc / guarded : acc;
        }
    }
    rc = 0;
done:
    free(S); free(z); free(St); free(zt); free(fq); free(fk);
    return rc;
}

int mhla_oracle_forward_blocks(const float* q, const float* k, const float* v, const float* W,
                               double* out, long B, long H, long N, long d, long M, const int* blk,
                               int options, int nthreads) {
    if (B < 1 || H < 1 || N < 1 || d < 1 || M < 1 || !q || !k || !v || !W || !out || !blk) return -1;
    if (options & ~(MHLA_ORACLE_NO_NORMALISER | MHLA_ORACLE_W_PER_HEAD)) return -1; /* non-causal */
    const int normalise = !(options & MHLA_ORACLE_NO_NORMALISER);
    const int per_head = (options & MHLA_ORACLE_W_PER_HEAD) != 0;
    const long BH = B * H;
    int failures = 0;
    (void)nthreads;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1) \
    reduction(+ : failures)
#endif
    for (long p = 0; p < BH; ++p) {
        const long off = p * N * d;
        const float* Wq = per_head ? W + (p % H) * M * M : W;
        failures += forward_pair_blocks(q + off, k + off, v + off, Wq, out + off, N, d, M, blk, normalise) != 0;
    }
    return failures ? -1 : 0;
}

int mhla_oracle_forward_ex(const float* q, const float* k, const float* v, const float* W,
                           double* out, long B, long H, long N, long d, long M, int options,
                           int nthreads) {
    if (B < 1 || H < 1 || !sizes_ok(B * H, N, d, M) || !q || !k || !v || !W || !out) return -1;
    if (options & ~(MHLA_ORACLE_CAUSAL | MHLA_ORACLE_NO_NORMALISER | MHLA_ORACLE_W_PER_HEAD)) return -1;
    const int causal = (options & MHLA_ORACLE_CAUSAL) != 0;
    const int normalise = (options & MHLA_ORACLE_NO_NORMALISER) == 0;
    const int per_head = (options & MHLA_ORACLE_W_PER_HEAD) != 0;
    const long BH = B * H;
    int failures = 0;
    (void)nthreads;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1) \
    reduction(+ : failures)
#endif
    for (long p = 0; p < BH; ++p) {
        const long off = p * N * d;
        /* pair p is (batch p / H, head p % H); with one matrix per head it uses W[p % H] */
        const float* Wp = per_head ? W + (p % H) * M * M : W;
        failures += forward_pair(q + off, k + off, v + off, Wp, out + off, N, d, M, causal, normalise) != 0;
    }
    return failures ? -1 : 0;
}

int mhla_oracle_forward(const float* q, const float* k, const float* v, const float* W,
                        double* out, long B, long H, long N, long d, long M, int causal,
                        int nthreads) {
    return mhla_oracle_forward_ex(q, k, v, W, out, B, H, N, d, M, causal ? MHLA_ORACLE_CAUSAL : 0,
                                  nthreads);
}
