// causal.hip -- stage 3 of the causal MHLA forward pass for blocks of at most 256
// tokens ("MHLA: Restoring Expressivity of Linear Attention via Token-Level
// Multi-Head", §4.1 causal form and App. C; guard as in "Linear Attention 笔记"
// §4/§5):
//
//   y_t = [phi(q_t) S~_i + W[i,i] sum_{j in i, j <= t} (phi(q_t).phi(k_j)) v_j]
//         / [phi(q_t) z~_i + W[i,i] sum_{j in i, j <= t} phi(q_t).phi(k_j) + 1e-6]
//
// with S~_i, z~_i the mix of the earlier blocks (b < i).  The within-block prefix is
// evaluated as one masked C x C product per block (the chunkwise form), which for
// C <= 256 costs less than walking a d x d running state and needs no sequential
// dependence between the block's 16-token tiles.
//
// One workgroup of four waves owns one block.  Before a single barrier the waves
// split S~_i into bf16 hi + lo MFMA operands in LDS and each wave applies phi to
// the keys of its own tiles (tile t belongs to wave t mod 8 < 4 ? t mod 4 : 7 - t
// mod 8, which balances the triangular work) and leaves them in LDS, together with
// the tiles' V rows already packed as score x V operands.  Then each
// wave, for each of its query tiles t:
//   * numerator phi(Q_t) S~_i (16x16x32 MFMAs, hi and lo) and denominator
//     phi(Q_t) z~_i (an MFMA whose B columns all equal z~_i);
//   * for key tiles u <= t, two at a time: scores phi(K_u) phi(Q_t)^T (MFMA),
//     masked to key <= query on the diagonal tile, scaled by W[i,i] and split
//     into hi + lo; these are the A operand of the score x V MFMA (keys along
//     k) and of an MFMA against ones that adds their row sums to the
//     denominator, so numerator and denominator use the same rounded weights.
// The MFMA results put query rows 4g + r and value columns P n + jb in lane
// (g, n), so each lane writes P consecutive floats per row.
//
// The feature order along the MFMA k axis is the same for Q, K, S~ and z~: k-step
// ks, slot e = 8g + e' holds feature P (4g + e' mod 4) + 2 ks + e' / 4, which are
// the 4P consecutive features 4Pg .. 4Pg + 4P - 1 of lane group g, and also two
// packed chunks (ia = 2ks, 2ks + 1) of the summary layout.
#include "common.hpp"
#include "kernels.hpp"

namespace mhla {

namespace {

constexpr int kQuadMaxTiles = 16;  // blocks of up to 256 tokens
constexpr int kQuadMaxOwn = kQuadMaxTiles / 4;

// The tile a wave handles in its slot s (s < kQuadMaxOwn): slots alternate between
// the rising and the falling half of each group of eight tiles.
__device__ __forceinline__ int own_tile(int wave, int s) { return 8 * (s >> 1) + ((s & 1) ? 7 - wave : wave); }

// 4P consecutive bf16 of one token row, as 2P words.
template <int P, bool NT>
__device__ __forceinline__ void load_row(rsrc_t r, uint32_t off, uint32_t (&w)[2 * P]) {
    if constexpr (P == 4) {
        const u32x4 a = buf_load128<NT>(r, off), b = buf_load128<NT>(r, off + 16);
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    } else if constexpr (P == 2) {
        const u32x4 a = buf_load128<NT>(r, off);
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    } else {
        const u32x2 a = buf_load64<NT>(r, off);
        w[0] = a.x; w[1] = a.y;
    }
}

// Operand slot (ks, e) -> feature index within the lane group's 4P features, or -1.
template <int P>
__device__ __forceinline__ constexpr int slot_feature(int ks, int e) {
    return (2 * ks + e / 4 < P) ? P * (e % 4) + 2 * ks + e / 4 : -1;
}

// phi of a row as MFMA operands (zero where the slot is padding or !ok).
template <int P, int KS>
__device__ __forceinline__ void phi_operand(const uint32_t (&w)[2 * P], bool ok, bf16x8 (&op)[KS]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        uint32_t pk[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
            float f[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int fl = slot_feature<P>(ks, 2 * e2 + h);
                if (fl < 0) {
                    f[h] = 0.f;
                } else {
                    const uint32_t word = w[fl / 2];
                    const float x = __uint_as_float((fl & 1) ? (word & 0xffff0000u) : (word << 16));
                    f[h] = ok ? phi_fast(x) : 0.f;
                }
            }
            pk[e2] = pack_bf16(f[0], f[1]);
        }
        op[ks] = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
    }
}

// Eight floats -> bf16x8 hi and lo.
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split2_bf16(x[2 * i], x[2 * i + 1], h[i], l[i]);
    hi = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
    lo = __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], l[2], l[3]});
}

}  // namespace

size_t causal_quad_lds_bytes(int D, int64_t C) {
    const int P = D / 16, KS = D >= 32 ? D / 32 : 1;
    const int64_t T = (C + 15) / 16;
    return (size_t)(2 * KS * P + T * KS) * 64 * 16 + (size_t)T * P * 64 * 8;
}

bool causal_quad_applicable(int64_t C) { return C <= 16 * kQuadMaxTiles; }

template <int D, bool NT>
__global__ __launch_bounds__(256) void output_causal_quad_kernel(const uint16_t* __restrict__ Q,
                                                                 const uint16_t* __restrict__ K,
                                                                 const uint16_t* __restrict__ V,
                                                                 const float* __restrict__ St,
                                                                 const float* __restrict__ W, OutSpec o,
                                                                 int64_t BH, int N, int M, int heads) {
    constexpr int P = D / 16;
    constexpr int KS = D >= 32 ? D / 32 : 1;
    constexpr int L = D * D + D;
    extern __shared__ uint4 lds4[];
    uint4* sh = lds4;                // [KS][P][64]: S~ operand, hi
    uint4* sl = sh + KS * P * 64;    //              lo
    uint4* kb = sl + KS * P * 64;    // [T][KS][64]: phi(K) operand per key tile

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, n = lane & 15;
    const int64_t unit = blockIdx.x;  // pair * M + block
    const int64_t pair = unit / M;
    const int blk = (int)(unit % M);
    const int C = N / M;
    const int T = (C + 15) / 16;
    u32x2* vbuf = reinterpret_cast<u32x2*>(kb + T * KS * 64);  // [T][P][64]: V operand halves per key tile
    const int bstart = blk * C;
    const float wii = pair_w(W, pair, heads, M)[(int64_t)blk * M + blk];
    const float* sv = St + ((int64_t)blk * BH + summary_row(pair, heads, BH)) * L;

    const uint32_t pair_bytes = (uint32_t)N * D * 2;
    const rsrc_t rQ = make_rsrc(Q + pair * N * D, pair_bytes);
    const rsrc_t rK = make_rsrc(K + pair * N * D, pair_bytes);
    const rsrc_t rV = make_rsrc(V + pair * N * D, pair_bytes);
    const int64_t ybase = pair * N * D;
    // Lane (g, n) of a row load reads features 4Pg .. 4Pg + 4P - 1 of token row n.
    auto row_off = [&](int tile, int r) { return ((uint32_t)(bstart + 16 * tile + r) * D + 4 * P * g) * 2; };

    // ---- before the barrier: S~ operands into LDS, phi(K) and V of own tiles into LDS ----
    // Every load of this part is issued first -- the S~ chunks the wave splits, z~, the K
    // and V rows of its first two tiles (reading zero where a tile or row is absent) and
    // the first Q row -- so that their latencies overlap instead of forming a chain.
    constexpr int PRE = 2;                  // own tiles whose rows are loaded up front
    constexpr int NPI = (KS * P + 3) / 4;   // S~ chunks per wave
    f32x4 sc[NPI][2];
#pragma unroll
    for (int q = 0; q < NPI; ++q) {
        const int pi = wave + 4 * q, ks = pi / P, jb = pi % P;
        const bool has = pi < KS * P, has1 = has && 2 * ks + 1 < P;
        sc[q][0] = *reinterpret_cast<const f32x4*>(sv + (has ? ((2 * ks) * P + jb) * 256 : 0) + lane * 4);
        sc[q][1] = *reinterpret_cast<const f32x4*>(sv + (has1 ? ((2 * ks + 1) * P + jb) * 256 : 0) + lane * 4);
        if (!has1) sc[q][1] = zero4();
    }
    f32x4 z4[P];
#pragma unroll
    for (int h = 0; h < P; ++h) z4[h] = *reinterpret_cast<const f32x4*>(sv + D * D + 4 * P * g + 4 * h);
    typedef uint32_t VRun[P == 4 ? 2 : 1];
    auto load_own = [&](int t, uint32_t (&kraw)[2 * P], VRun (&vr)[4]) {
        load_row<P, NT>(rK, off_if(t < T && 16 * t + n < C, row_off(t, n)), kraw);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * t + 4 * g + e;
            const uint32_t off = off_if(t < T && row < C, ((uint32_t)(bstart + row) * D + P * n) * 2);
            if constexpr (P == 4) {
                const u32x2 x = buf_load64<NT>(rV, off);
                vr[e][0] = x.x;
                vr[e][1] = x.y;
            } else if constexpr (P == 2) {
                vr[e][0] = buf_load32<NT>(rV, off);
            } else {
                vr[e][0] = buf_load16<NT>(rV, off);
            }
        }
    };
    uint32_t kpre[PRE][2 * P];
    VRun vpre[PRE][4];
#pragma unroll
    for (int s = 0; s < PRE; ++s) load_own(own_tile(wave, s), kpre[s], vpre[s]);
    uint32_t qraw[2 * P];  // Q row of the first own tile
    load_row<P, NT>(rQ, off_if(16 * own_tile(wave, 0) + n < C, row_off(own_tile(wave, 0), n)), qraw);
    issue_fence();

#pragma unroll
    for (int q = 0; q < NPI; ++q) {
        const int pi = wave + 4 * q;
        if (pi < KS * P) {  // uniform
            const float x[8] = {sc[q][0][0], sc[q][0][1], sc[q][0][2], sc[q][0][3],
                                sc[q][1][0], sc[q][1][1], sc[q][1][2], sc[q][1][3]};
            bf16x8 hi, lo;
            split8(x, hi, lo);
            sh[pi * 64 + lane] = __builtin_bit_cast(uint4, hi);
            sl[pi * 64 + lane] = __builtin_bit_cast(uint4, lo);
        }
    }
#pragma unroll
    for (int s = 0; s < kQuadMaxOwn; ++s) {
        const int t = own_tile(wave, s);
        if (t < T) {  // uniform
            uint32_t kraw[2 * P];
            VRun vr[4];
            if (s < PRE) {
#pragma unroll
                for (int w = 0; w < 2 * P; ++w) kraw[w] = kpre[s < PRE ? s : 0][w];
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int h = 0; h < (P == 4 ? 2 : 1); ++h) vr[e][h] = vpre[s < PRE ? s : 0][e][h];
            } else {
                load_own(t, kraw, vr);
            }
            const bool ok = 16 * t + n < C;
            bf16x8 ak[KS];
            phi_operand<P, KS>(kraw, ok, ak);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) kb[(t * KS + ks) * 64 + lane] = __builtin_bit_cast(uint4, ak[ks]);
            // V of keys 4g + e (e < 4) of tile t, value columns P n + jb, packed per column
            // block as the four bf16 of one half of the score x V B operand.
#pragma unroll
            for (int jb = 0; jb < P; ++jb) {
                uint32_t hv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t word = vr[e][jb / 2];
                    hv[e] = (P > 1 && (jb & 1)) ? word >> 16 : word & 0xffffu;
                }
                vbuf[(t * P + jb) * 64 + lane] = u32x2{hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16)};
            }
        }
    }
    // z~ operand (every B column equal to z~), hi and lo.
    bf16x8 zh[KS], zl[KS];
    {
        float zf[4 * P];
#pragma unroll
        for (int h = 0; h < P; ++h)
#pragma unroll
            for (int u = 0; u < 4; ++u) zf[4 * h + u] = z4[h][u];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int fl = slot_feature<P>(ks, e);
                x[e] = fl < 0 ? 0.f : zf[fl];
            }
            split8(x, zh[ks], zl[ks]);
        }
    }
    const bf16x8 ones8 = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                          (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
    __syncthreads();

    // ---- own query tiles ----
#pragma unroll
    for (int s = 0; s < kQuadMaxOwn; ++s) {
        const int t = own_tile(wave, s);
        if (t >= T) continue;  // uniform
        bf16x8 aq[KS];
        phi_operand<P, KS>(qraw, true, aq);
        if (s + 1 < kQuadMaxOwn) {  // next own tile's Q row, in flight while this tile computes
            const int tn = own_tile(wave, s + 1);
            load_row<P, NT>(rQ, off_if(tn < T && 16 * tn + n < C, row_off(tn, n)), qraw);
        }

        f32x4 acc[P], dacc = zero4();
#pragma unroll
        for (int jb = 0; jb < P; ++jb) acc[jb] = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int jb = 0; jb < P; ++jb) {
                acc[jb] = mfma32(aq[ks], __builtin_bit_cast(bf16x8, sh[(ks * P + jb) * 64 + lane]), acc[jb]);
                acc[jb] = mfma32(aq[ks], __builtin_bit_cast(bf16x8, sl[(ks * P + jb) * 64 + lane]), acc[jb]);
            }
            dacc = mfma32(aq[ks], zh[ks], dacc);
            dacc = mfma32(aq[ks], zl[ks], dacc);
        }

        // Key tiles u, u + 1 <= t: k slot e < 4 is key 4g + e of tile u, e >= 4 key 4g + e - 4 of u + 1.
        for (int u = 0; u <= t; u += 2) {
            const bool two = u + 1 <= t;  // uniform
            float a[8];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int uu = u + h;
                f32x4 sc = zero4();
                if (h == 0 || two) {
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
                        sc = mfma32(__builtin_bit_cast(bf16x8, kb[(uu * KS + ks) * 64 + lane]), aq[ks], sc);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // lane (g, n): query n, key 4g + i of tile uu; the diagonal tile keeps key <= query
                    const bool keep = (h == 0 || two) && (uu < t || 4 * g + i <= n);
                    a[4 * h + i] = keep ? wii * sc[i] : 0.f;
                }
            }
            bf16x8 ahi, alo;
            split8(a, ahi, alo);
#pragma unroll
            for (int jb = 0; jb < P; ++jb) {  // V operand: keys of tile u, then of tile u + 1 (zero if absent)
                const u32x2 v0 = vbuf[(u * P + jb) * 64 + lane];
                const u32x2 v1 = two ? vbuf[((u + 1) * P + jb) * 64 + lane] : u32x2{0u, 0u};
                const bf16x8 bv = __builtin_bit_cast(bf16x8, u32x4{v0.x, v0.y, v1.x, v1.y});
                acc[jb] = mfma32(ahi, bv, acc[jb]);
                acc[jb] = mfma32(alo, bv, acc[jb]);
            }
            dacc = mfma32(ahi, ones8, dacc);
            dacc = mfma32(alo, ones8, dacc);
        }

        // lane (g, n): rows 16t + 4g + r, columns P n .. P n + P - 1
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * t + 4 * g + r;
            if (row < C) {
                const float rd = out_scale(o, dacc[r] + kEps);
                const int64_t e = ybase + (int64_t)(bstart + row) * D + P * n;
                if constexpr (P == 4) {
                    store_out(o, e, f32x4{acc[0][r] * rd, acc[1][r] * rd, acc[2][r] * rd, acc[3][r] * rd});
                } else if constexpr (P == 2) {
                    store_out(o, e, f32x2{acc[0][r] * rd, acc[1][r] * rd});
                } else {
                    store_out(o, e, acc[0][r] * rd);
                }
            }
        }
    }
}

hipError_t launch_causal_quad(const void* q, const void* k, const void* v, const float* St, const float* W,
                              const OutSpec& out, int64_t BH, int64_t N, int D, int64_t M, int heads,
                              hipStream_t stream) {
    const uint16_t* qq = (const uint16_t*)q;
    const uint16_t* kk = (const uint16_t*)k;
    const uint16_t* vv = (const uint16_t*)v;
    const size_t lds = causal_quad_lds_bytes(D, N / M);
    const dim3 grid((unsigned)(BH * M)), block(256);
    const bool nt = stream_token_inputs(BH, N, D, 2);
#define MHLA_QUAD_CASE(DD)                                                                                     \
    case DD:                                                                                                   \
        if (nt)                                                                                                \
            output_causal_quad_kernel<DD, true><<<grid, block, lds, stream>>>(qq, kk, vv, St, W, out, BH, (int)N, (int)M, heads);  \
        else                                                                                                   \
            output_causal_quad_kernel<DD, false><<<grid, block, lds, stream>>>(qq, kk, vv, St, W, out, BH, (int)N, (int)M, heads); \
        break;
    switch (D) {
        MHLA_QUAD_CASE(16)
        MHLA_QUAD_CASE(32)
        MHLA_QUAD_CASE(64)
        default: return hipErrorInvalidValue;
    }
#undef MHLA_QUAD_CASE
    return hipGetLastError();
}

}  // namespace mhla
