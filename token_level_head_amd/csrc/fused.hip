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
// w + 8.  Each wave loads its K, V and W, stages V once through LDS (so that each
// lane holds one value column of its tokens), and only then issues its Q loads, so
// that the K and V requests of all workgroups reach memory first; phi(k) and phi(q)
// are computed once (bf16, in registers).  The d x d summary space is walked in P*P
// sub-tiles (d = 16P; sub-tile (ia, c) holds features P*m + ia and value columns
// 16c .. 16c + 15), in column-chunk-major order, two sub-tiles of one column chunk
// at a time, each batch in three barrier-separated steps through LDS:
//   1. every wave computes both sub-tiles of S_b for its blocks (one 16x16x16 bf16
//      MFMA each, tokens along k) and, for c == 0, z_b (an MFMA against ones), and
//      stores them as float32;
//   2. each sub-tile's 16 column tiles (+ the z tile) are mixed,
//      S~_i = sum_b W[i, b] S_b, with blocks along k: S and W split into bf16
//      hi + lo, three MFMAs (hi.hi + lo.hi + hi.lo); the result is split into
//      hi + lo again for step 3;
//   3. every wave adds phi(Q_i) S~_i (both sub-tiles) into the accumulators of the
//      current column chunk (MFMAs on hi and lo) and, for c == 0, phi(Q_i) z~_i into
//      the denominator (an MFMA whose A rows all equal z~_i).
// The output MFMA puts value columns on rows and tokens on columns, so once a
// column chunk is complete each lane holds 4 consecutive columns of one token: it
// scales them by 1 / (den + 1e-6) and writes them with one 16-byte store while the
// next chunks are computed.  K, V, Q and W are read with buffer loads (scalar
// descriptor, 32-bit offsets; an offset past the end reads zero).  Blocks M .. 15
// run through the same steps on zero K/V (finite summaries) and carry zero mixing
// weight.  LDS holds two batch slots (80 KiB), so two workgroups share a CU.
// With between one and two pairs per CU (DiT-S/2: 384 pairs on 256 CUs) the CUs
// holding two whole pairs would set the time, so 2 * CUs - B*H pairs are split into
// column halves run by two workgroups (each recomputes phi and z for its half), and
// every CU gets one whole pair and one half (measured: 24.3 -> 22.2 us).
//
// Sequences of at most 256 tokens whose blocks are 2 to 4 whole 16-token tiles
// (C = 32, 48, 64) run through the same kernel with the tiles as its blocks
// (M = N / 16 here, T = C / 16 tiles per block) and tile weights W[i / T][b / T]:
// a block's summary is the sum of its tiles' summaries, so the mix of tile i is
// exactly S~ of its block.
#include "common.hpp"
#include "kernels.hpp"

namespace mhla {

namespace {

constexpr int kMaxBlocks = 16;  // M: one 16-row MFMA tile of W and S~
constexpr int kWaves = 8;
constexpr int kBlocksPerWave = kMaxBlocks / kWaves;

// LDS layout, in 4-byte words.  Strides are chosen so that the accesses of the
// three steps hit distinct banks.
constexpr int kRSA = 20;             // S sub-tile: one value column, 16 features (+4)
constexpr int kBSA = 16 * kRSA + 4;  // S sub-tile: one block (4 blocks apart = 16 banks apart)
constexpr int kBSB = 130;            // S~ hi (and lo): one query block, [4 feature quads][16 columns] x 2 words
constexpr int kBZA = 20;             // z sub-tile: one block
constexpr int kBZB = 12;             // z~ hi (and lo): one query block, 4 feature quads x 2 words
// One batch slot: an S sub-tile, the S~ sub-tile (hi, lo), a z sub-tile, z~ (hi, lo).
constexpr int kSlotS = kMaxBlocks * kBSA;
constexpr int kSlotSt = 2 * kMaxBlocks * kBSB;
constexpr int kSlotZ = kMaxBlocks * kBZA;
constexpr int kSlotZt = 2 * kMaxBlocks * kBZB;
constexpr int kSlotWords = kSlotS + kSlotSt + kSlotZ + kSlotZt;

__device__ __forceinline__ float half_to_f32(uint32_t word, int half) {
    return __uint_as_float(half ? (word & 0xffff0000u) : (word << 16));
}

__device__ __forceinline__ bf16x4 as_bf16x4(uint32_t lo_pair, uint32_t hi_pair) {
    return __builtin_bit_cast(bf16x4, u32x2{lo_pair, hi_pair});
}


}  // namespace

// One (batch, head) pair, value columns of column chunks [C0, C1) (HC = 0: all P
// chunks; 1 and 2: the first and second half, for pairs split over two workgroups).
// `lds` holds SB batch slots.
template <int D, bool FULL, int HC>
__device__ __forceinline__ void fused_pair(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                           const uint16_t* __restrict__ V, const float* __restrict__ W,
                                           const OutSpec& o, int N, int M, int heads, int T, float* lds,
                                           int64_t pair) {
    constexpr int P = D / 16;
    constexpr int BPW = kBlocksPerWave;
    constexpr int SB = P > 1 ? 2 : 1;  // sub-tiles per batch (same column chunk)
    constexpr int NB = P * P / SB;     // batches
    static_assert(HC == 0 || P >= 2, "column halves need at least two column chunks");
    constexpr int BT0 = HC == 2 ? NB / 2 : 0, BT1 = HC == 1 ? NB / 2 : NB;  // this workgroup's batches
    constexpr int C0 = BT0 * SB / P;                                         // its first column chunk
    float* const A = lds;                                                   // [SB][16 blocks][16 columns][kRSA]
    uint2* const Bhi = reinterpret_cast<uint2*>(lds + SB * kSlotS);        // [SB][hi, lo][16 query blocks][kBSB / 2]
    float* const Az = lds + SB * (kSlotS + kSlotSt);                       // [SB][16 blocks][kBZA]
    uint2* const Zhi = reinterpret_cast<uint2*>(Az + SB * kSlotZ);         // [SB][hi, lo][16 query blocks][kBZB / 2]

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, n = lane & 15;
    const int C = FULL ? 16 : N / M;  // tokens per block, <= 16

    // ---- loads: K and V (lane: P features / columns of tokens 4g .. 4g+3), W (lane:
    // W[n][4g + e]); Q (lane: features 4Pg .. 4Pg + 4P - 1 of token n) after V has gone
    // through LDS, so that the K and V requests of all workgroups come first ----
    const uint32_t pair_bytes = (uint32_t)N * D * 2;
    const rsrc_t rK = make_rsrc(K + pair * N * D, pair_bytes);
    const rsrc_t rV = make_rsrc(V + pair * N * D, pair_bytes);
    const rsrc_t rQ = make_rsrc(Q + pair * N * D, pair_bytes);
    const int MW = M / T;  // blocks of W (M counts 16-token tiles when T > 1)
    const rsrc_t rW = make_rsrc(pair_w(W, pair, heads, MW), (uint32_t)MW * MW * 4);
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
    }
    float wv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int b = 4 * g + e;
        wv[e] = __uint_as_float(buf_load32(rW, off_if(n < M && b < M, (uint32_t)((n / T) * MW + b / T) * 4)));
    }
    auto load_q = [&]() {
#pragma unroll
        for (int j = 0; j < BPW; ++j) {
            const int b = wave + kWaves * j;
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
    };
    issue_fence();

    // Mixing B operand: W[i = n][b = 4g + e] split into hi + lo.
    uint32_t w01h, w01l, w23h, w23l;
    split2_bf16(wv[0], wv[1], w01h, w01l);
    split2_bf16(wv[2], wv[3], w23h, w23l);
    const bf16x4 wh = as_bf16x4(w01h, w23h), wl = as_bf16x4(w01l, w23l);

    // phi(k) as the summary MFMA's A operand: ak[j][ia][e] = phi(K[4g + e][P n + ia]).
    bf16x4 ak[BPW][P], bq[BPW][P];
#pragma unroll
    for (int j = 0; j < BPW; ++j)
#pragma unroll
        for (int ia = 0; ia < P; ++ia) {
            float fk[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t kword = (P == 4 && ia >= 2) ? kw[j][e].y : kw[j][e].x;
                const float pk = phi_fast(half_to_f32(kword, P == 1 ? 0 : ia & 1));
                fk[e] = (FULL || 4 * g + e < C) ? pk : 0.f;
            }
            ak[j][ia] = as_bf16x4(pack_bf16(fk[0], fk[1]), pack_bf16(fk[2], fk[3]));
        }
    // V as the summary MFMA's B operand for column chunk c (value columns 16c .. 16c+15):
    // vb[j][c][e] = V[4g + e][16c + n].  The coalesced loads gave lane n columns
    // Pn .. Pn + P - 1, so the tile goes once through LDS (each wave its own region,
    // inside the S~ buffers, which are first written after the first batch's barrier)
    // in token-major order and is read back by column.
    bf16x4 vb[BPW][P];
    {
        uint16_t* vt = reinterpret_cast<uint16_t*>(Bhi) + (size_t)wave * BPW * 16 * D;  // [j][token][column]
#pragma unroll
        for (int j = 0; j < BPW; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint16_t* dst = vt + (j * 16 + 4 * g + e) * D + P * n;
                if constexpr (P == 4)
                    *reinterpret_cast<uint2*>(dst) = uint2{vw[j][e].x, vw[j][e].y};
                else if constexpr (P == 2)
                    *reinterpret_cast<uint32_t*>(dst) = vw[j][e].x;
                else
                    *dst = (uint16_t)vw[j][e].x;
            }
        __syncthreads();
        load_q();
#pragma unroll
        for (int j = 0; j < BPW; ++j)
#pragma unroll
            for (int c = 0; c < P; ++c) {
                uint32_t h[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) h[e] = vt[(j * 16 + 4 * g + e) * D + 16 * c + n];
                vb[j][c] = as_bf16x4(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
            }
    }

    // phi(q) as the output MFMA's B operand, bq[j][ia][e] = phi(Q[n][P (4g + e) + ia]);
    // formed just before the first output step.
    auto make_bq = [&]() {
#pragma unroll
        for (int j = 0; j < BPW; ++j)
#pragma unroll
            for (int ia = 0; ia < P; ++ia) {
                float fq[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int fl = P * e + ia;
                    fq[e] = phi_fast(half_to_f32(qw[j][fl / 8][(fl % 8) / 2], fl & 1));
                }
                bq[j][ia] = as_bf16x4(pack_bf16(fq[0], fq[1]), pack_bf16(fq[2], fq[3]));
            }
    };

    const bf16x4 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
    f32x4 oacc[BPW], dacc[BPW];  // output accumulators of the current column chunk; denominator
    float rden[BPW];

    // Mixing of one 16-column tile: four blocks' values, split hi + lo, against the
    // split W; the result split again for the output step.
    auto mix_tile = [&](const float* src, int bstride, uint2* hi_dst, uint2* lo_dst) {
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = src[e * bstride];
        uint32_t h01, l01, h23, l23;
        split2_bf16(x[0], x[1], h01, l01);
        split2_bf16(x[2], x[3], h23, l23);
        const bf16x4 sh = as_bf16x4(h01, h23), sl = as_bf16x4(l01, l23);
        f32x4 acc = mfma16(sh, wh, zero4());
        acc = mfma16(sl, wh, acc);
        acc = mfma16(sh, wl, acc);
        uint32_t o01h, o01l, o23h, o23l;
        split2_bf16(acc[0], acc[1], o01h, o01l);
        split2_bf16(acc[2], acc[3], o23h, o23l);
        *hi_dst = uint2{o01h, o23h};
        *lo_dst = uint2{o01l, o23l};
    };

#pragma unroll
    for (int bt = BT0; bt < BT1; ++bt) {
        // 1. sub-tile (ia, c) of S_b: lane (g, n) gets S_b[P (4g + r) + ia][16 c + n], r = 0..3
#pragma unroll
        for (int u = 0; u < SB; ++u) {
            const int s = bt * SB + u, c = s / P, ia = s % P;
            float* const a_wr = A + u * kSlotS + n * kRSA + 4 * g;
            float* const z_wr = Az + u * kSlotZ + 4 * g;
#pragma unroll
            for (int j = 0; j < BPW; ++j) {
                const int b = wave + kWaves * j;
                *reinterpret_cast<f32x4*>(a_wr + b * kBSA) = mfma16(ak[j][ia], vb[j][c], zero4());
                if (c == C0) {
                    const f32x4 za = mfma16(ak[j][ia], ones, zero4());
                    if (n == 0) *reinterpret_cast<f32x4*>(z_wr + b * kBZA) = za;
                }
            }
        }
        __syncthreads();

        // 2. mixing.  Column tile t < 16 (value column 16 c + t), and for c == 0 the z
        //    tile: lane (g, n) gets S~_{i = n}[feature P (4g + r) + ia][.], r = 0..3.
#pragma unroll
        for (int u = 0; u < SB; ++u) {
            const int s = bt * SB + u, c = s / P, ia = s % P;
            const float* const a_rd = A + u * kSlotS + 4 * g * kBSA + n;
            uint2* const bhi = Bhi + u * (kSlotSt / 2) + n * (kBSB / 2) + g * 16;
            uint2* const blo = bhi + kMaxBlocks * kBSB / 2;
#pragma unroll
            for (int j = 0; j < 16 / kWaves; ++j) {
                const int t = wave + kWaves * j;
                mix_tile(a_rd + t * kRSA, kBSA, bhi + t, blo + t);
            }
            if (c == C0 && wave == (ia + 4 * u) % kWaves) {
                uint2* const zhi = Zhi + u * (kSlotZt / 2) + n * (kBZB / 2) + g;
                mix_tile(Az + u * kSlotZ + 4 * g * kBZA + n, kBZA, zhi, zhi + kMaxBlocks * kBZB / 2);
            }
        }
        __syncthreads();

        // 3. output: D[column 16 c + 4g + r][token n] += sum_m S~_i[P m + ia][.] phi(q_n)[P m + ia]
        if (bt == BT0) make_bq();
#pragma unroll
        for (int u = 0; u < SB; ++u) {
            const int s = bt * SB + u, c = s / P, ia = s % P;
            const uint2* const bhi = Bhi + u * (kSlotSt / 2);
            const uint2* const blo = bhi + kMaxBlocks * kBSB / 2;
            const uint2* const zhi = Zhi + u * (kSlotZt / 2);
            const uint2* const zlo = zhi + kMaxBlocks * kBZB / 2;
#pragma unroll
            for (int j = 0; j < BPW; ++j) {
                const int b = wave + kWaves * j;
                const uint2 sh = bhi[b * (kBSB / 2) + g * 16 + n];
                const uint2 sl = blo[b * (kBSB / 2) + g * 16 + n];
                oacc[j] = mfma16(as_bf16x4(sh.x, sh.y), bq[j][ia], ia == 0 ? zero4() : oacc[j]);
                oacc[j] = mfma16(as_bf16x4(sl.x, sl.y), bq[j][ia], oacc[j]);
                if (c == C0) {
                    const uint2 zh = zhi[b * (kBZB / 2) + g];
                    const uint2 zl = zlo[b * (kBZB / 2) + g];
                    dacc[j] = mfma16(as_bf16x4(zh.x, zh.y), bq[j][ia], ia == 0 ? zero4() : dacc[j]);
                    dacc[j] = mfma16(as_bf16x4(zl.x, zl.y), bq[j][ia], dacc[j]);
                }
            }
            // The next batch's step 1 overwrites only the S and z sub-tiles, whose last
            // reader (step 2) finished before the barrier above.

            // Column chunk c is complete after its last feature group (the denominator
            // after chunk 0): write it now, so the stores overlap the remaining chunks.
            if (ia == P - 1) {
                if (c == C0) {
#pragma unroll
                    for (int j = 0; j < BPW; ++j) rden[j] = out_scale(o, dacc[j][0] + kEps);
                }
#pragma unroll
                for (int j = 0; j < BPW; ++j) {
                    const int b = wave + kWaves * j;
                    if (b < M && (FULL || n < C)) {
                        const int64_t e = (pair * N + b * C + n) * D + 16 * c + 4 * g;
                        const f32x4 a = oacc[j];
                        store_out(o, e, f32x4{a[0] * rden[j], a[1] * rden[j], a[2] * rden[j], a[3] * rden[j]});
                    }
                }
            }
        }
    }
}

// Workgroups [0, nfull) each run the whole pair of their index; the rest run the
// remaining pairs in column halves, two workgroups per pair (dispatched after all
// the whole pairs, so that a CU holding two workgroups gets a whole pair and a half;
// the two halves of a pair are numbered 8 apart, which keeps them on one XCD).
template <int D, bool FULL>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(4))) void fused_small_kernel(
                                                          const uint16_t* __restrict__ Q,
                                                          const uint16_t* __restrict__ K,
                                                          const uint16_t* __restrict__ V,
                                                          const float* __restrict__ W, OutSpec o,
                                                          int N, int M, int heads, int T, int nfull) {
    constexpr int P = D / 16;
    constexpr int SB = P > 1 ? 2 : 1;
    __shared__ __align__(16) float lds[SB * kSlotWords];
    const int w = blockIdx.x;
    if (w < nfull) {
        fused_pair<D, FULL, 0>(Q, K, V, W, o, N, M, heads, T, lds, w);
    } else if constexpr (P >= 2) {
        // Halves of one pair are 8 workgroups apart, so that round-robin dispatch puts
        // both on the same XCD and the second reads the pair's inputs from that L2.
        const int u = w - nfull;
        const int nh = ((int)gridDim.x - nfull) / 2;  // pairs run in halves
        const int g16 = (nh / 8) * 16;
        int j, h;
        if (u < g16) {
            j = 8 * (u / 16) + (u % 8);
            h = (u / 8) & 1;
        } else {
            j = (nh / 8) * 8 + (u - g16) / 2;
            h = (u - g16) & 1;
        }
        const int64_t pair = nfull + j;
        if (h)
            fused_pair<D, FULL, 2>(Q, K, V, W, o, N, M, heads, T, lds, pair);
        else
            fused_pair<D, FULL, 1>(Q, K, V, W, o, N, M, heads, T, lds, pair);
    }
}

bool fused_applicable(int D, int64_t BH, int64_t N, int64_t M) {
    (void)D;
    (void)BH;
    // Blocks of at most 16 tokens (one 16-deep k-step and one query tile per
    // block) and at most 16 blocks (one 16-row tile of W); or at most 256 tokens in
    // blocks of 2 to 4 whole 16-token tiles, run as tiles: a block's summary is the
    // sum of its tiles' summaries, so mixing the tiles with W[block(i), block(b)]
    // gives every tile of block i exactly S~_i.  Longer blocks stay on the staged
    // path, whose summaries are then small next to the tokens (one block of 256
    // tokens: 12% faster staged than fused, measured).
    const int64_t C = N / M;
    return (M <= kMaxBlocks && C <= 16) || (N <= 16 * kMaxBlocks && C % 16 == 0 && C <= 64);
}

hipError_t launch_fused(const void* q, const void* k, const void* v, const float* W, const OutSpec& out,
                        int64_t BH, int64_t N, int D, int64_t M, int heads, hipStream_t stream) {
    const int64_t C = N / M;
    const int T = C > 16 ? (int)(C / 16) : 1;  // 16-token tiles per block
    const bool full = C >= 16;
    M = M * T;
    const uint16_t* qq = (const uint16_t*)q;
    const uint16_t* kk = (const uint16_t*)k;
    const uint16_t* vv = (const uint16_t*)v;
    // Between one and two pairs per CU, the CUs holding two whole pairs would set the
    // time: split 2 * CUs - BH pairs into column halves, so that every CU gets a whole
    // pair and a half (d >= 32; d = 16 has a single column chunk).
    const int cus = device_cu_count();
    const int64_t nhalf = (D >= 32 && BH > cus && BH < 2 * (int64_t)cus) ? 2 * cus - BH : 0;
    const int nfull = (int)(BH - nhalf);
    const dim3 grid((unsigned)(nfull + 2 * nhalf)), block(64 * kWaves);
#define MHLA_FUSED_CASE(DD)                                                                              \
    case DD:                                                                                             \
        if (full)                                                                                        \
            fused_small_kernel<DD, true><<<grid, block, 0, stream>>>(qq, kk, vv, W, out, (int)N, (int)M, heads, T, nfull);  \
        else                                                                                             \
            fused_small_kernel<DD, false><<<grid, block, 0, stream>>>(qq, kk, vv, W, out, (int)N, (int)M, heads, T, nfull); \
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
