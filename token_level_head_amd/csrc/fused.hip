// fused.hip -- the whole MHLA forward pass for short blocks in one kernel, with
// the block summaries kept on chip ("MHLA: Restoring Expressivity of Linear
// Attention via Token-Level Multi-Head", §4.1: phi, local KV summaries
// S_b = sum_{j in b} phi(k_j) v_j^T and z_b, multi-head mixing with M_c, output
// ratio; guard as in "Linear Attention 笔记" §4/§5).  Non-causal only.
//
// When blocks are shorter than d (DiT-S/2 at 256x256: 16 tokens, d = 64) the d x d
// summaries are several times larger than the tokens they summarise, and
// round-tripping them through HBM dominates the three-stage pass.  Here one
// workgroup of eight waves owns one (batch, head) pair; wave w owns blocks w and
// w + 8.  Each wave loads its K, V and Q once and computes phi(k) and phi(q) once
// (bf16, in registers).  The d x d summary space is then walked in P*P sub-tiles
// of 16 features x 16 value columns (d = 16P; sub-tile (ia, c) holds features
// P*m + ia and columns P*n + c, the lane layout of the summary MFMA), each in
// three barrier-separated steps through LDS:
//   1. every wave computes the sub-tile of S_b for its blocks (one 16x16x16 bf16
//      MFMA: tokens along k) and, for c == 0, z_b (an MFMA against ones);
//   2. the 16 entry tiles (+ the z tile) of the sub-tile are mixed,
//      S~_i = sum_b W[i, b] S_b, on float32 MFMA (16x16x4, blocks along k:
//      exact products); each result is split into bf16 hi + lo for step 3;
//   3. every wave adds phi(Q_i) S~_i (sub-tile) into its output accumulators
//      (2 bf16 MFMAs: hi and lo) and, for c == 0, phi(Q_i) z~_i into the
//      denominator (an MFMA whose A rows all equal z~_i).
// The output MFMA puts value columns on rows and tokens on columns, so after the
// last sub-tile each lane holds 4P consecutive columns of one token; it scales
// them by 1 / (den + 1e-6) and writes them with 16-byte stores.  K, V, Q and W
// are read with buffer loads (scalar descriptor, 32-bit offsets; an offset past
// the end reads zero).
#include "common.hpp"
#include "kernels.hpp"

namespace mhla {

namespace {

constexpr int kMaxBlocks = 16;  // M: one 16-row MFMA tile of W and S~
constexpr int kWaves = 8;
constexpr int kBlocksPerWave = kMaxBlocks / kWaves;
// LDS layout, in 4-byte words.  Strides are chosen so that every LDS access of
// the three steps touches 64 distinct banks per wave (or, for 8-byte accesses,
// 64 distinct banks per half wave).
constexpr int kRSA = 20;              // S sub-tile: one feature row of 16 columns (+4)
constexpr int kBSA = 16 * kRSA + 1;   // S sub-tile: one block (= 1 mod 4)
constexpr int kBSB = 130;             // S~ hi (and lo): one query block, [4 feature quads][16 columns] x 2 words
constexpr int kBZA = 16;              // z sub-tile: one block
constexpr int kBZB = 12;              // z~ hi (and lo): one query block, 4 feature quads x 2 words
constexpr int kLdsWords = kMaxBlocks * kBSA + 2 * kMaxBlocks * kBSB + kMaxBlocks * kBZA + 2 * kMaxBlocks * kBZB;

__device__ __forceinline__ float half_to_f32(uint32_t word, int half) {
    return __uint_as_float(half ? (word & 0xffff0000u) : (word << 16));
}

}  // namespace

template <int D, bool FULL>
__global__ __launch_bounds__(512) void fused_small_kernel(const uint16_t* __restrict__ Q,
                                                          const uint16_t* __restrict__ K,
                                                          const uint16_t* __restrict__ V,
                                                          const float* __restrict__ W, float* __restrict__ Y,
                                                          int N, int M) {
    constexpr int P = D / 16;
    constexpr int BPW = kBlocksPerWave;
    __shared__ __align__(16) float lds[kLdsWords];
    float* A = lds;                                           // [16 blocks][16 features][kRSA]
    uint2* Bhi = reinterpret_cast<uint2*>(lds + kMaxBlocks * kBSA);  // [16 query blocks][kBSB / 2]
    uint2* Blo = Bhi + kMaxBlocks * kBSB / 2;
    float* Az = reinterpret_cast<float*>(Blo + kMaxBlocks * kBSB / 2);  // [16 blocks][kBZA]
    uint2* Zhi = reinterpret_cast<uint2*>(Az + kMaxBlocks * kBZA);      // [16 query blocks][kBZB / 2]
    uint2* Zlo = Zhi + kMaxBlocks * kBZB / 2;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, n = lane & 15;
    const int64_t pair = blockIdx.x;
    const int C = FULL ? 16 : N / M;  // tokens per block, <= 16

    // Blocks M .. 15 take part in the mixing MFMAs with weight zero: clear their rows.
    for (int x = threadIdx.x; x < (kMaxBlocks - M) * kBSA; x += 512) A[M * kBSA + x] = 0.f;
    for (int x = threadIdx.x; x < (kMaxBlocks - M) * kBZA; x += 512) Az[M * kBZA + x] = 0.f;

    // ---- loads: K and V (lane: P features / columns of tokens 4g .. 4g+3), Q (lane:
    // features 4Pg .. 4Pg + 4P - 1 of token n), W (lane: W[n][4kb + g]) ----
    const uint32_t pair_bytes = (uint32_t)N * D * 2;
    const rsrc_t rK = make_rsrc(K + pair * N * D, pair_bytes);
    const rsrc_t rV = make_rsrc(V + pair * N * D, pair_bytes);
    const rsrc_t rQ = make_rsrc(Q + pair * N * D, pair_bytes);
    const rsrc_t rW = make_rsrc(W, (uint32_t)M * M * 4);
    u32x2 kw[BPW][4], vw[BPW][4];
    u32x4 qw[BPW][P == 4 ? 2 : 1];
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
        const int b = wave + kWaves * j;  // b >= M reads past the end: zeros
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t off = ((uint32_t)(b * C + 4 * g + e) * D + P * n) * 2;
            if constexpr (P == 4) {
                kw[j][e] = buf_load64(rK, off);
                vw[j][e] = buf_load64(rV, off);
            } else if constexpr (P == 2) {
                kw[j][e] = u32x2{buf_load32(rK, off), 0u};
                vw[j][e] = u32x2{buf_load32(rV, off), 0u};
            } else {
                kw[j][e] = u32x2{buf_load16(rK, off), 0u};
                vw[j][e] = u32x2{buf_load16(rV, off), 0u};
            }
        }
        const uint32_t qoff = ((uint32_t)(b * C + n) * D + 4 * P * g) * 2;
        if constexpr (P == 4) {
            qw[j][0] = buf_load128(rQ, qoff);
            qw[j][1] = buf_load128(rQ, qoff + 16);
        } else if constexpr (P == 2) {
            qw[j][0] = buf_load128(rQ, qoff);
        } else {
            const u32x2 x = buf_load64(rQ, qoff);
            qw[j][0] = u32x4{x.x, x.y, 0u, 0u};
        }
    }
    float wf[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        const int b = 4 * kb + g;
        wf[kb] = __uint_as_float(buf_load32(rW, off_if(n < M && b < M, (uint32_t)(n * M + b) * 4)));
    }
    issue_fence();

    // ---- phi(k) as the summary MFMA's A operand: ak[j][ia][e] = phi(K[4g + e][P n + ia]);
    // phi(q) as the output MFMA's B operand: bq[j][ia][e] = phi(Q[n][P (4g + e) + ia]) ----
    bf16x4 ak[BPW][P], bq[BPW][P];
#pragma unroll
    for (int j = 0; j < BPW; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool ok = FULL || 4 * g + e < C;
#pragma unroll
            for (int ia = 0; ia < P; ++ia) {
                const uint32_t kword = (P == 4 && ia >= 2) ? kw[j][e].y : kw[j][e].x;
                const float x = half_to_f32(kword, P == 1 ? 0 : ia & 1);
                ak[j][ia][e] = (__bf16)(ok ? phi_fast(x) : 0.f);
                const int fl = P * e + ia;
                const uint32_t qword = qw[j][fl / 8][(fl % 8) / 2];
                bq[j][ia][e] = (__bf16)phi_fast(half_to_f32(qword, fl & 1));
            }
        }

    const bf16x4 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
    f32x4 oacc[BPW][P], dacc[BPW];
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
        dacc[j] = zero4();
#pragma unroll
        for (int c = 0; c < P; ++c) oacc[j][c] = zero4();
    }

#pragma unroll
    for (int s = 0; s < P * P; ++s) {
        const int c = s / P, ia = s % P;
        // 1. sub-tile (ia, c) of S_b: lane (g, n) gets S_b[P (4g + r) + ia][P n + c]
#pragma unroll
        for (int j = 0; j < BPW; ++j) {
            const int b = wave + kWaves * j;
            if (b < M) {  // uniform
                bf16x4 bv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t vword = (P == 4 && c >= 2) ? vw[j][e].y : vw[j][e].x;
                    bv[e] = bits_to_bf16((uint16_t)((P > 1 && (c & 1)) ? vword >> 16 : vword));
                }
                const f32x4 sa = mfma16(ak[j][ia], bv, zero4());
                float* dst = A + b * kBSA + 4 * g * kRSA + n;
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[r * kRSA] = sa[r];
                if (c == 0) {
                    const f32x4 za = mfma16(ak[j][ia], ones, zero4());
                    if (n == 0) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) Az[b * kBZA + 4 * g + r] = za[r];
                    }
                }
            }
        }
        __syncthreads();

        // 2. mixing: tile t < 16 is value column P t + c of the sub-tile, tile 16 is z.
        //    Lane (g, n) gets S~_{i = n}[feature P (4g + r) + ia][column P t + c].
        const int ntile = c == 0 ? 17 : 16;
        for (int t = wave; t < ntile; t += kWaves) {  // uniform
            const float* src = t < 16 ? A + n * kRSA + t : Az + n;
            const int bstride = t < 16 ? kBSA : kBZA;
            f32x4 acc = zero4();
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(src[(4 * kb + g) * bstride], wf[kb], acc, 0, 0, 0);
            bf16x4 h, l;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bf16pair p = split_bf16(acc[r]);
                h[r] = p.hi;
                l[r] = p.lo;
            }
            if (t < 16) {
                Bhi[n * (kBSB / 2) + g * 16 + t] = __builtin_bit_cast(uint2, h);
                Blo[n * (kBSB / 2) + g * 16 + t] = __builtin_bit_cast(uint2, l);
            } else {
                Zhi[n * (kBZB / 2) + g] = __builtin_bit_cast(uint2, h);
                Zlo[n * (kBZB / 2) + g] = __builtin_bit_cast(uint2, l);
            }
        }
        __syncthreads();

        // 3. output: D[column P (4g + r) + c][token n] += sum_m S~_i[P m + ia][.] phi(q_n)[P m + ia]
#pragma unroll
        for (int j = 0; j < BPW; ++j) {
            const int b = wave + kWaves * j;
            if (b < M) {  // uniform
                const bf16x4 sh = __builtin_bit_cast(bf16x4, Bhi[b * (kBSB / 2) + g * 16 + n]);
                const bf16x4 sl = __builtin_bit_cast(bf16x4, Blo[b * (kBSB / 2) + g * 16 + n]);
                oacc[j][c] = mfma16(sh, bq[j][ia], oacc[j][c]);
                oacc[j][c] = mfma16(sl, bq[j][ia], oacc[j][c]);
                if (c == 0) {
                    const bf16x4 zh = __builtin_bit_cast(bf16x4, Zhi[b * (kBZB / 2) + g]);
                    const bf16x4 zl = __builtin_bit_cast(bf16x4, Zlo[b * (kBZB / 2) + g]);
                    dacc[j] = mfma16(zh, bq[j][ia], dacc[j]);
                    dacc[j] = mfma16(zl, bq[j][ia], dacc[j]);
                }
            }
        }
        // The next sub-tile's step 1 overwrites only the S and z sub-tiles, whose
        // last reader (step 2) finished before the barrier above.
    }

    // ---- y = numerator / (den + 1e-6): lane (g, n) holds columns 4Pg .. 4Pg + 4P - 1 of token n ----
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
        const int b = wave + kWaves * j;
        if (b < M && (FULL || n < C)) {
            const float rden = fast_rcp(dacc[j][0] + kEps);
            float* dst = Y + (pair * N + b * C + n) * D + 4 * P * g;
#pragma unroll
            for (int h = 0; h < P; ++h) {
                f32x4 o;
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const int col = 4 * h + x;  // = P r + c
                    o[x] = oacc[j][col % P][col / P] * rden;
                }
                *reinterpret_cast<f32x4*>(dst + 4 * h) = o;
            }
        }
    }
}

bool fused_applicable(int D, int64_t BH, int64_t N, int64_t M) {
    (void)D;
    (void)BH;
    // Blocks of at most 16 tokens (one 16-deep k-step and one query tile per
    // block) and at most 16 blocks (one 16-row tile of W).
    return M <= kMaxBlocks && N / M <= 16;
}

hipError_t launch_fused(const void* q, const void* k, const void* v, const float* W, float* out, int64_t BH,
                        int64_t N, int D, int64_t M, hipStream_t stream) {
    const bool full = N / M == 16;
    const uint16_t* qq = (const uint16_t*)q;
    const uint16_t* kk = (const uint16_t*)k;
    const uint16_t* vv = (const uint16_t*)v;
    const dim3 grid((unsigned)BH), block(64 * kWaves);
#define MHLA_FUSED_CASE(DD)                                                                              \
    case DD:                                                                                             \
        if (full)                                                                                        \
            fused_small_kernel<DD, true><<<grid, block, 0, stream>>>(qq, kk, vv, W, out, (int)N, (int)M);  \
        else                                                                                             \
            fused_small_kernel<DD, false><<<grid, block, 0, stream>>>(qq, kk, vv, W, out, (int)N, (int)M); \
        break;
    switch (D) {
        MHLA_FUSED_CASE(16)
        MHLA_FUSED_CASE(32)
        MHLA_FUSED_CASE(64)
        default: return hipErrorInvalidValue;
    }
#undef MHLA_FUSED_CASE
    return hipGetLastError();
}

}  // namespace mhla
