// output.hip -- stage 3 of the MHLA forward pass: the output ratio
//   y_t = phi(q_t)^T S~_i / (phi(q_t)^T z~_i + 1e-6),  i = block of t
// ("MHLA: Restoring Expressivity of Linear Attention via Token-Level Multi-Head",
// §4.1; guard as in "Linear Attention 笔记" §4/§5), and its causal variant
// (same page, App. C): S~_i mixes only blocks b < i, and token t adds
// W[i,i] * (phi(q_t)^T P_t, phi(q_t)^T p_t) with P_t the summary of block i's
// tokens up to and including t.
//
// Non-causal, one wave per run of up to four 16-token tiles of one block:
//   * phi(Q) rows are the MFMA A operand (lane n = token, lane group g = a run of
//     4P features, read as one or two 16-byte loads);
//   * S~_i enters as the B operand, split once per wave into bf16 hi + lo parts
//     (two MFMAs), read straight from the packed layout with 16-byte loads: the
//     features a lane's group needs are exactly the ones the summary kernel left
//     in that lane;
//   * the denominator phi(q).z~ is a per-lane dot product plus a reduction over
//     the four lane groups with wavefront shuffles;
//   * one reciprocal per row, written once with 16-byte stores.
// Causal: see output_causal_kernel below.
#include "common.hpp"
#include "kernels.hpp"

namespace mhla {

// B operands from packed chunks: slot e of k-step ks is group-local feature
// fl = 8*ks + e, held in chunk (fl % P, jb) at row fl / P (zero past 4P).
template <int P, int KS>
__device__ __forceinline__ void build_b(const f32x4 (&ch)[P * P], bf16x8 (&bh)[KS][P], bf16x8 (&bl)[KS][P]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int jb = 0; jb < P; ++jb)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int fl = 8 * ks + e;
                const float x = fl < 4 * P ? ch[(fl % P) * P + jb][fl / P] : 0.f;
                const bf16pair h = split_bf16(x);
                bh[ks][jb][e] = h.hi;
                bl[ks][jb][e] = h.lo;
            }
}

// Lane (g, n) holds acc[jj][i] = numerator of row t0 + 4g + i at column
// P*n + jb0 + jj (jj < PJ); `den` is the guarded denominator of row t0 + n (any
// lane group).  PJ consecutive values are stored per row, from element offset
// ybase (the pair's first element of Y).
template <int P, int PJ>
__device__ __forceinline__ void store_rows(const OutSpec& o, int64_t ybase, int t0, int bend, int g, int n,
                                           int jb0, const f32x4 (&acc)[PJ], float den,
                                           const BlockLayout& lay = BlockLayout{nullptr, nullptr}, int N = 0) {
    constexpr int D = 16 * P;
    const float rden = out_scale(o, den);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float r = __shfl(rden, 4 * g + i, 64);
        const int entry = t0 + 4 * g + i;  // list entry; the row of Y it fills:
        const int row = entry < bend ? token_row(lay, entry, N) : -1;
        if (row >= 0) {
            const int64_t e = ybase + row * D + P * n + jb0;
            if constexpr (PJ == 4) {
                store_out(o, e, f32x4{acc[0][i] * r, acc[1][i] * r, acc[2][i] * r, acc[3][i] * r});
            } else if constexpr (PJ == 2) {
                store_out(o, e, f32x2{acc[0][i] * r, acc[1][i] * r});
            } else {
                store_out(o, e, acc[0][i] * r);
            }
        }
    }
}

// Offsets inside one (batch, head) pair fit in 32 bits (the API limits N*d).
template <int D, bool NT>
__global__ __launch_bounds__(256) void output_bf16_kernel(const uint16_t* __restrict__ Q,
                                                          const float* __restrict__ St, OutSpec o,
                                                          int64_t BH, int N, int64_t M, int tpw, int wpu, int heads,
                                                          BlockLayout lay) {
    constexpr int P = D / 16;
    constexpr int FL = 4 * P;                 // features per lane group
    constexpr int KS = D >= 32 ? D / 32 : 1;  // 16x16x32 k-steps (d = 16 pads to 32)
    constexpr int L = D * D + D;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, n = lane & 15;
    const int64_t w = (int64_t)blockIdx.x * 4 + wave;
    const int64_t unit = w / wpu;  // unit = pair * M + block
    const int s = (int)(w % wpu);
    if (unit >= BH * M) return;  // whole wave; no barriers in this kernel
    const int64_t pair = unit / M;
    const int blk = (int)(unit % M);
    int bstart, bend;  // the block's range in the token list
    block_range(lay, blk, N, M, bstart, bend);
    const int ntiles = (bend - bstart + 15) / 16;
    const int tile_beg = s * tpw;
    const int tile_end = min(ntiles, tile_beg + tpw);

    const float* sv = St + ((int64_t)blk * BH + summary_row(pair, heads, BH)) * L;
    f32x4 sch[P * P];
#pragma unroll
    for (int c4 = 0; c4 < P * P; ++c4) sch[c4] = *reinterpret_cast<const f32x4*>(sv + c4 * 256 + lane * 4);
    float zt[FL];
#pragma unroll
    for (int h = 0; h < FL / 4; ++h) {
        const f32x4 zz = *reinterpret_cast<const f32x4*>(sv + D * D + FL * g + 4 * h);
#pragma unroll
        for (int u = 0; u < 4; ++u) zt[4 * h + u] = zz[u];
    }
    bf16x8 bh[KS][P], bl[KS][P];
    build_b<P, KS>(sch, bh, bl);

    const int64_t ybase = pair * N * D;
    // Q rows through a per-pair buffer descriptor: a row outside the block reads zero
    // with no mask, so the next tile's loads stay in flight while this tile computes.
    const rsrc_t rQ = make_rsrc(Q + pair * N * D, (uint32_t)N * D * 2);
    auto qload = [&](int tile, uint32_t (&w)[2 * P], bool& ok) {
        const int tq = bstart + 16 * tile + n;  // list entry
        const int qrow = (tile < tile_end && tq < bend) ? token_row(lay, tq, N) : -1;
        ok = qrow >= 0;
        const uint32_t off = off_if(ok, ((uint32_t)(ok ? qrow : 0) * D + FL * g) * 2);
        if constexpr (P == 4) {
            const u32x4 a = buf_load128<NT>(rQ, off), b = buf_load128<NT>(rQ, off + 16);
            w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
            w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
        } else if constexpr (P == 2) {
            const u32x4 a = buf_load128<NT>(rQ, off);
            w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        } else {
            const u32x2 a = buf_load64<NT>(rQ, off);
            w[0] = a.x; w[1] = a.y;
        }
    };
    uint32_t qcur[2 * P], qnext[2 * P];
    bool okcur = false, oknext = false;
    if (tile_beg < tile_end) qload(tile_beg, qcur, okcur);
    for (int tile = tile_beg; tile < tile_end; ++tile) {
        const int t0 = bstart + 16 * tile;
        qload(tile + 1, qnext, oknext);  // the next tile's rows (none past the last: zero)
        issue_fence();
        // phi(Q) as the A operand: token t0 + n, group-local features of group g.
        bf16x8 aq[KS];
        float den = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int fl = 8 * ks + e;
                float x = 0.f;
                if (fl < FL) {
                    const uint32_t word = qcur[fl / 2];
                    x = __uint_as_float((fl & 1) ? (word & 0xffff0000u) : (word << 16));
                }
                const __bf16 ph = (__bf16)((fl < FL && okcur) ? phi_fast(x) : 0.f);
                aq[ks][e] = ph;
                if (fl < FL) den = fmaf(bf16v_to_f32(ph), zt[fl], den);
            }
        den = sum_over_groups(den) + kEps;

        f32x4 acc[P];
#pragma unroll
        for (int jb = 0; jb < P; ++jb) {
            acc[jb] = zero4();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                acc[jb] = mfma32(aq[ks], bh[ks][jb], acc[jb]);
                acc[jb] = mfma32(aq[ks], bl[ks][jb], acc[jb]);
            }
        }
        store_rows<P, P>(o, ybase, t0, bend, g, n, 0, acc, den, lay, N);
#pragma unroll
        for (int h = 0; h < 2 * P; ++h) qcur[h] = qnext[h];
        okcur = oknext;
    }
}

// Causal: P waves share one block, wave jb computing value columns P*n + jb.
// The workgroup walks the block's 16-token tiles in order.  For each tile the
// P waves load Q and K once between them (one 16-byte chunk per lane), apply
// phi once, and leave the bf16 tiles in LDS (double-buffered, one barrier per
// tile); every wave then reads the layouts it needs: phi(Q) and phi(K) rows as
// MFMA operands for the numerator and the 16 x 16 scores, and phi(K) with tokens
// along k for the state update.
//
// The B operand S~_i + W[i,i] P (P = the block's summary over the tiles already
// done) is one running float32 accumulator set `comb` in the packed layout: it
// starts as S~_i and each tile adds bf16(W[i,i] phi(k))^T v with MFMA, so it is
// formed lane-locally with no separate copy of S~_i.  The normaliser works the
// same way (start z~_i, add with an MFMA against ones).  Inside the tile the
// masked product (phi(Q) phi(K)^T) V covers the inclusive prefix exactly; its
// weights are carried as bf16 hi + lo and its row sums come from the same
// rounded values (chunkwise form of App. C).
template <int D, bool NT>
__global__ __launch_bounds__(256) void output_causal_kernel(const uint16_t* __restrict__ Q,
                                                            const uint16_t* __restrict__ K,
                                                            const uint16_t* __restrict__ V,
                                                            const float* __restrict__ St,
                                                            const float* __restrict__ W, OutSpec o,
                                                            int64_t BH, int N, int64_t M, int heads) {
    constexpr int P = D / 16;
    constexpr int FL = 4 * P;
    constexpr int KS = D >= 32 ? D / 32 : 1;
    constexpr int L = D * D + D;
    constexpr int BPW = 4 / P;    // blocks per workgroup
    constexpr int TILE = 16 * D;  // bf16 elements of one 16-token tile
    __shared__ __align__(16) uint16_t lds[2][BPW][2][TILE];  // [buffer][block slot][phi(Q), phi(K)]

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, n = lane & 15;
    const int bw = wave / P, jb = wave % P;
    const int64_t unit = (int64_t)blockIdx.x * BPW + bw;  // pair * M + block
    const bool active = unit < BH * M;                      // inactive slots still meet the barriers
    const int64_t pair = active ? unit / M : 0;
    const int blk = active ? (int)(unit % M) : 0;
    const int C = (int)(N / M);
    const int ntiles = (C + 15) / 16;
    const int bstart = blk * C, bend = bstart + C;
    const float wii = active ? pair_w(W, pair, heads, M)[(int64_t)blk * M + blk] : 0.f;

    const float* sv = St + ((int64_t)blk * BH + summary_row(pair, heads, BH)) * L;
    f32x4 comb[P];  // comb[ia] = chunk (ia, jb) of S~_i + W[i,i] P
#pragma unroll
    for (int ia = 0; ia < P; ++ia)
        comb[ia] = load_or_zero(reinterpret_cast<const f32x4*>(sv + (ia * P + jb) * 256 + lane * 4), active,
                                reinterpret_cast<const f32x4*>(St));
    f32x4 zacc[P];  // zacc[ia][i] = running normaliser at group-local feature P*i + ia
#pragma unroll
    for (int h = 0; h < FL / 4; ++h) {
        const f32x4 zz = load_or_zero(reinterpret_cast<const f32x4*>(sv + D * D + FL * g + 4 * h), active,
                                      reinterpret_cast<const f32x4*>(St));
#pragma unroll
        for (int u = 0; u < 4; ++u) zacc[(4 * h + u) % P][(4 * h + u) / P] = zz[u];
    }

    const uint16_t* Qp = Q + pair * N * D;
    const uint16_t* Kp = K + pair * N * D;
    const uint16_t* Vp = V + pair * N * D;
    const int64_t ybase = pair * N * D;
    const bf16x4 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};

    // This lane's share of the tile: one 16-byte chunk of Q or K.
    constexpr int CPR = D / 8;                    // 8-element chunks per row
    const int chunk = jb * 64 + lane;             // 0 .. 4D - 1
    const int which = chunk / (16 * CPR);         // 0: Q, 1: K
    const int crow = (chunk % (16 * CPR)) / CPR;  // token within the tile
    const int ccol = 8 * (chunk % CPR);           // first feature
    const uint16_t* src = which ? Kp : Qp;

    for (int tile = 0; tile < ntiles; ++tile) {
        const int t0 = bstart + 16 * tile;
        uint16_t* buf = &lds[tile & 1][bw][0][0];
        {  // phi of this lane's chunk into LDS
            const bool ok = active && t0 + crow < bend;
            const uint4 x = load_token_or_zero<NT>(reinterpret_cast<const uint4*>(src + (t0 + crow) * D + ccol), ok,
                                         reinterpret_cast<const uint4*>(Q));
            const uint32_t wv[4] = {x.x, x.y, x.z, x.w};
            uint32_t o[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const __bf16 lo = (__bf16)(ok ? phi_fast(__uint_as_float(wv[u] << 16)) : 0.f);
                const __bf16 hi = (__bf16)(ok ? phi_fast(__uint_as_float(wv[u] & 0xffff0000u)) : 0.f);
                o[u] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
            }
            *reinterpret_cast<uint4*>(buf + which * TILE + crow * D + ccol) = make_uint4(o[0], o[1], o[2], o[3]);
        }
        // This wave's value column for tokens t0 + 4g + e (tokens along k).
        bf16x4 bv4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int tok = t0 + 4 * g + e;
            bv4[e] = bits_to_bf16(load_token_or_zero<NT>(Vp + tok * D + P * n + jb, active && tok < bend, V));
        }
        __syncthreads();

        const uint16_t* tq = buf;
        const uint16_t* tk = buf + TILE;
        bf16x8 aq[KS], ak[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if constexpr (FL >= 8) {
                aq[ks] = *reinterpret_cast<const bf16x8*>(tq + n * D + FL * g + 8 * ks);
                ak[ks] = *reinterpret_cast<const bf16x8*>(tk + n * D + FL * g + 8 * ks);
            } else {  // d = 16: four features per group, zero-padded to the 32-deep MFMA
                const bf16x4 a4 = *reinterpret_cast<const bf16x4*>(tq + n * D + FL * g);
                const bf16x4 k4 = *reinterpret_cast<const bf16x4*>(tk + n * D + FL * g);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    aq[ks][e] = e < 4 ? a4[e & 3] : (__bf16)0.f;
                    ak[ks][e] = e < 4 ? k4[e & 3] : (__bf16)0.f;
                }
            }
        }
        bf16x4 ak4[P];  // bf16(W[i,i] phi(k)) for tokens t0 + 4g + e, features P*n + ia
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
            for (int ia = 0; ia < P; ++ia)
                ak4[ia][e] = (__bf16)(wii * bf16_to_f32(tk[(4 * g + e) * D + P * n + ia]));
        }

        // Numerator and denominator against S~_i + W[i,i] P (tiles before this one).
        f32x4 acc[1];
        acc[0] = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            bf16x8 bh, bl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int fl = 8 * ks + e;
                const float x = fl < FL ? comb[fl % P][fl / P] : 0.f;
                const bf16pair hp = split_bf16(x);
                bh[e] = hp.hi;
                bl[e] = hp.lo;
            }
            acc[0] = mfma32(aq[ks], bh, acc[0]);
            acc[0] = mfma32(aq[ks], bl, acc[0]);
        }
        float den = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int fl = 8 * ks + e;
                if (fl < FL) den = fmaf(bf16v_to_f32(aq[ks][e]), zacc[fl % P][fl / P], den);
            }
        den = sum_over_groups(den);

        // Inside the tile: lane (g, n) gets A[query n][key 4g + i], kept for key <= query.
        f32x4 at = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) at = mfma32(ak[ks], aq[ks], at);
        bf16x4 ahi, alo;
        float rs = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float a = (4 * g + i <= n) ? wii * at[i] : 0.f;
            const bf16pair hp = split_bf16(a);
            ahi[i] = hp.hi;
            alo[i] = hp.lo;
            rs += bf16v_to_f32(hp.hi) + bf16v_to_f32(hp.lo);
        }
        den += sum_over_groups(rs) + kEps;
        acc[0] = mfma16(ahi, bv4, acc[0]);
        acc[0] = mfma16(alo, bv4, acc[0]);

        // Fold this tile into the running operand and normaliser.
#pragma unroll
        for (int ia = 0; ia < P; ++ia) {
            comb[ia] = mfma16(ak4[ia], bv4, comb[ia]);
            zacc[ia] = mfma16(ak4[ia], ones, zacc[ia]);
        }
        if (active) store_rows<P, 1>(o, ybase, t0, bend, g, n, jb, acc, den);
    }
}

// float32 path: one thread per output element, float32 arithmetic throughout.
__global__ __launch_bounds__(256) void output_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                         const float* __restrict__ V, const float* __restrict__ St,
                                                         const float* __restrict__ W, OutSpec o,
                                                         int64_t BH, int64_t N, int64_t M, int D, int causal,
                                                         int heads, BlockLayout lay) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= BH * N * D) return;
    const int c = (int)(idx % D);
    const int64_t pair = idx / ((int64_t)N * D);
    int64_t t = (idx / D) % N, blk;  // without a token list: token t of block t / C
    if (lay.offsets) {
        // list entry p = t: its block by binary search over the offsets, its row in the sequence
        const int p = (int)t;
        int lo = 0, hi = (int)M;  // the last b with offsets[b] <= p
        while (hi - lo > 1) {
            const int mid = (lo + hi) / 2;
            if (lay.offsets[mid] <= p) lo = mid; else hi = mid;
        }
        blk = lo;
        t = token_row(lay, p, (int)N);
        if (t < 0) return;
    } else {
        blk = t / (N / M);
    }
    const int64_t C = N / M;
    const int P = D / 16;
    const float* sv = St + (blk * BH + summary_row(pair, heads, BH)) * (int64_t)(D * D + D);
    const float* q = Q + (pair * N + t) * D;
    float num = 0.f, den = 0.f;
    for (int r = 0; r < D; ++r) {
        const float fq = phi_precise(q[r]);
        num = fmaf(fq, sv[packed_index(P, r, c)], num);
        den = fmaf(fq, sv[D * D + r], den);
    }
    if (causal) {
        const float wii = pair_w(W, pair, heads, M)[blk * M + blk];
        float ni = 0.f, di = 0.f;
        for (int64_t j = blk * C; j <= t; ++j) {
            const float* kj = K + (pair * N + j) * D;
            float a = 0.f;
            for (int r = 0; r < D; ++r) a = fmaf(phi_precise(q[r]), phi_precise(kj[r]), a);
            ni = fmaf(a, V[(pair * N + j) * D + c], ni);
            di += a;
        }
        num = fmaf(wii, ni, num);
        den = fmaf(wii, di, den);
    }
    store_out(o, (pair * N + t) * D + c, o.norm ? num / (den + kEps) : num);
}

hipError_t launch_output(int dtype, const void* q, const void* k, const void* v, const float* St,
                         const float* W, const OutSpec& out, int64_t BH, int64_t N, int D, int64_t M, bool causal,
                         int heads, const BlockLayout& lay, int64_t cmax, hipStream_t stream) {
    if (dtype == kDtypeF32) {
        const int64_t total = BH * N * D;
        output_f32_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream>>>(
            (const float*)q, (const float*)k, (const float*)v, St, W, out, BH, N, M, D, causal ? 1 : 0, heads, lay);
        return hipGetLastError();
    }
    const uint16_t* qq = (const uint16_t*)q;
    const uint16_t* kk = (const uint16_t*)k;
    const uint16_t* vv = (const uint16_t*)v;
    const bool nt = stream_token_inputs(BH, N, D, 2);
    if (causal && causal_quad_applicable(N / M))
        return launch_causal_quad(q, k, v, St, W, out, BH, N, D, M, heads, stream);
    if (causal) {  // d/16 waves per block, 4 / (d/16) blocks per workgroup
        const int bpw = 4 / (D / 16);
        const dim3 grid((unsigned)((BH * M + bpw - 1) / bpw));
#define MHLA_LAUNCH_OUT(DD)                                                                                   \
    if (nt)                                                                                                   \
        output_causal_kernel<DD, true><<<grid, dim3(256), 0, stream>>>(qq, kk, vv, St, W, out, BH, (int)N, M, heads);  \
    else                                                                                                      \
        output_causal_kernel<DD, false><<<grid, dim3(256), 0, stream>>>(qq, kk, vv, St, W, out, BH, (int)N, M, heads)
        switch (D) {
            case 16: MHLA_LAUNCH_OUT(16); break;
            case 32: MHLA_LAUNCH_OUT(32); break;
            case 64: MHLA_LAUNCH_OUT(64); break;
            default: return hipErrorInvalidValue;
        }
#undef MHLA_LAUNCH_OUT
        return hipGetLastError();
    }
    // Up to four tiles per wave, amortising the summary operand over 64 tokens.
    const int64_t C = cmax;
    const int ntiles = (int)((C + 15) / 16);
    const int tpw = min(ntiles, 4);
    const int wpu = (ntiles + tpw - 1) / tpw;
    const dim3 grid((unsigned)((BH * M * wpu + 3) / 4));
#define MHLA_LAUNCH_OUT(DD)                                                                        \
    if (nt)                                                                                        \
        output_bf16_kernel<DD, true><<<grid, dim3(256), 0, stream>>>(qq, St, out, BH, (int)N, M, tpw, wpu, heads, lay); \
    else                                                                                           \
        output_bf16_kernel<DD, false><<<grid, dim3(256), 0, stream>>>(qq, St, out, BH, (int)N, M, tpw, wpu, heads, lay)
    switch (D) {
        case 16: MHLA_LAUNCH_OUT(16); break;
        case 32: MHLA_LAUNCH_OUT(32); break;
        case 64: MHLA_LAUNCH_OUT(64); break;
        default: return hipErrorInvalidValue;
    }
#undef MHLA_LAUNCH_OUT
    return hipGetLastError();
}

}  // namespace mhla
