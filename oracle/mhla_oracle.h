/*
 * mhla_oracle.h -- plain CPU oracle for the MHLA forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This code exists so that tests, the smoke check
 * and the benchmark's CPU-baseline leg can check the GPU library against an
 * independent, obviously correct implementation.  The product path never
 * calls it, and it shares no code, header, table or helper with the HIP
 * library.
 *
 * Sources (page titles as published):
 *   [MHLA]  "MHLA: Restoring Expressivity of Linear Attention via Token-Level
 *           Multi-Head" -- §4.1 (local KV summaries, multi-head mixing, the
 *           output ratio), §4.2 (coefficient matrix M_c, token-level
 *           expansion Eq. 5, chunkwise form), App. C (causal mixing and the
 *           streaming inference update).
 *   [LA]    "Linear Attention（线性注意力）笔记" -- §2 (feature map ELU+1),
 *           §4 (causal recurrence with the 1e-6 guard in the denominator),
 *           §5 (parallel form).
 *
 * Arithmetic is IEEE binary64 throughout; inputs are binary32 arrays whose
 * values the generator made exactly representable (bf16 or fp32 draws).
 *
 * Layouts (all row-major, contiguous):
 *   q, k, v, out : [B][H][N][d]
 *   W            : [M][M], W[i*M + b] = weight of block b's summary for query block i
 *   S            : [BH][M][d][d], S[..][b][r][c] = sum_{j in b} phi(k_j)[r] * v_j[c]
 *   z            : [BH][M][d]
 * Block b holds tokens [b*C, (b+1)*C) with C = N / M; N must be a multiple of M.
 *
 * Return value: 0 on success, -1 on invalid sizes or a failed allocation.
 */
#ifndef MHLA_ORACLE_H
#define MHLA_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Added to the denominator after the full mixed dot product ([LA] §4, §5). */
#define MHLA_ORACLE_EPS 1e-6

/* phi(x) = ELU(x) + 1 with alpha = 1 ([LA] §2). */
double mhla_oracle_phi(double x);

/* Step 2 of [MHLA] §4.1: per-block KV summary S_b and normaliser z_b. */
int mhla_oracle_summaries(const float* k, const float* v, long BH, long N, long d, long M,
                          double* S, double* z);

/* Step 3 of [MHLA] §4.1 / App. C: mixed summaries.  Non-causal sums over every
 * block b; causal sums over b < i only (the current block's own contribution is
 * the within-block prefix, added per token in the causal output). */
int mhla_oracle_mix(const double* S, const double* z, const float* W, long BH, long d, long M,
                    int causal, double* St, double* zt);

/* The whole forward pass.  nthreads > 1 runs independent (batch, head) pairs on
 * that many OpenMP threads (same arithmetic, different pairs per thread). */
int mhla_oracle_forward(const float* q, const float* k, const float* v, const float* W,
                        double* out, long B, long H, long N, long d, long M, int causal,
                        int nthreads);

/* Options of mhla_oracle_forward_ex (bit flags). */
#define MHLA_ORACLE_CAUSAL 1        /* the causal variant ([MHLA] App. C) */
#define MHLA_ORACLE_NO_NORMALISER 2 /* y_t = phi(q_t)^T S~_i (plus the causal prefix term), no
                                       division: [MHLA] §4.1, remark on the output for long sequences */
#define MHLA_ORACLE_W_PER_HEAD 4    /* W is [H][M][M]: head h applies §4.1 with its own matrix
                                       W + h*M*M (the pages describe one matrix for all heads) */

/* The non-causal forward pass with an explicit block assignment: token t of every
 * (batch, head) pair belongs to block blk[t] (0 <= blk[t] < M; blocks of any sizes and
 * shapes, [MHLA] §4.1).  options: MHLA_ORACLE_NO_NORMALISER, MHLA_ORACLE_W_PER_HEAD. */
int mhla_oracle_forward_blocks(const float* q, const float* k, const float* v, const float* W,
                               double* out, long B, long H, long N, long d, long M, const int* blk,
                               int options, int nthreads);

/* The forward pass with options; mhla_oracle_forward(.., causal, ..) is
 * mhla_oracle_forward_ex(.., causal ? MHLA_ORACLE_CAUSAL : 0, ..). */
int mhla_oracle_forward_ex(const float* q, const float* k, const float* v, const float* W,
                           double* out, long B, long H, long N, long d, long M, int options,
                           int nthreads);

#ifdef __cplusplus
}
#endif
#endif
