// output.hip -- stage 3 of the MHLA forward pass: the output ratio
//   y_t = phi(q_t)^T S~_i / (phi(q_t)^T z~_i + 1e-6),  i = block of t
// ("MHLA: Restoring Expressivity of Linear Attention via Token-Level Multi-Head",
// §4.1; guard as in "Linear Attention 笔记" §4/§5), and its causal variant
// (same page, App. C): S~_i mixes only blocks b < i, and token t adds
// W[i,i] * (phi(q_t)^T P_t, phi(q_t)^T p_t) with P_t the summary of block i's
// tokens up to and including t.
//
// bf16 path, one wave per 16-token tile sequence of one block:
//   * phi(Q) rows are the MFMA A operand (lane n = token, lane group g = a run of
//     4P features, read as one or two 16-byte loads);
//   * S~_i enters as the B operand, split into bf16 hi + lo parts (two MFMAs),
//     and it is read straight from the packed layout with 16-byte loads: the
//     features a lane's group needs are exactly the ones the summary kernel left
//     in that lane;
//   * the denominator phi(q).z~ is a per-lane dot product plus a reduction over
//     the four lane groups with wavefront shuffles;
//   * one float32 divide per output, written once with 16-byte stores.
// Causal: the wave walks its block's tiles in order and keeps the running block
// summary P (and p) in MFMA accumulators in the packed layout, so the operand
// S~_i + W[i,i] P is formed lane-locally each tile.  Inside a tile the strictly
// causal part is the masked 16 x 16 product (phi(Q) phi(K)^T) V (chunkwise form
// of App. C), with A kept as bf16 hi + lo and its row sums taken from the same
// rounded values that multiply V.
#include "common.hpp"
#include "kernels.hpp"

namespace mhla {

// 4P consecutive bf16 values starting at p (P = d/16): 8, 16 or 32 bytes.
template <int P>
__device__ __forceinline__ void load_group(const uint16_t* p, bool ok, const uint16_t* safe, uint16_t (&out)[4 * P]) {
    if constexpr (P == 1) {
        const uint2 x = load_or_zero(reinterpret_cast<const uint2*>(p), ok, reinterpret_cast<const uint2*>(safe));
        out[0] = (uint16_t)x.x; out[1] = (uint16_t)(x.x >> 16);
        out[2] = (uint16_t)x.y; out[3] = (uint16_t)(x.y >> 16);
    } else {
#pragma unroll
        for (int h = 0; h < P / 2; ++h) {
            const uint4 x = load_or_zero(reinterpret_cast<const uint4*>(p + 8 * h), ok, reinterpret_cast<const uint4*>(safe));
            const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                out[8 * h + 2 * u] = (uint16_t)w[u];
                out[8 * h + 2 * u + 1] = (uint16_t)(w[u] >> 16);
            }
        }
    }
}

// P consecutive bf16 values (2P bytes).
template <int P>
__device__ __forceinline__ void load_feat3(const uint16_t* p, bool ok, const uint16_t* safe, uint16_t (&out)[P]) {
    if constexpr (P == 4) {
        const uint2 x = load_or_zero(reinterpret_cast<const uint2*>(p), ok, reinterpret_cast<const uint2*>(safe));
        out[0] = (uint16_t)x.x; out[1] = (uint16_t)(x.x >> 16);
        out[2] = (uint16_t)x.y; out[3] = (uint16_t)(x.y >> 16);
    } else if constexpr (P == 2) {
        const uint32_t x = load_or_zero(reinterpret_cast<const uint32_t*>(p), ok, reinterpret_cast<const uint32_t*>(safe));
        out[0] = (uint16_t)x; out[1] = (uint16_t)(x >> 16);
    } else {
        out[0] = load_or_zero(p, ok, safe);
    }
}

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

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void output_bf16_kernel(const uint16_t* __restrict__ Q,
                                                          const uint16_t* __restrict__ K,
                                                          const uint16_t* __restrict__ V,
                                                          const float* __restrict__ St,
                                                          const float* __restrict__ W, float* __restrict__ Y,
                                                          int64_t BH, int64_t N, int64_t M, int tpw, int wpu) {
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
    const int64_t pair = unit / M, blk = unit % M;
    const int64_t C = N / M;
    const int ntiles = (int)((C + 15) / 16);
    const int tile_beg = s * tpw;
    const int tile_end = min(ntiles, tile_beg + tpw);
    const int64_t bstart = blk * C, bend = bstart + C;

    const float* sv = St + (blk * BH + pair) * (int64_t)L;
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
    if constexpr (!CAUSAL) build_b<P, KS>(sch, bh, bl);

    float wii = 0.f;
    f32x4 pst[P * P];  // running summary of this block's earlier tiles (packed layout)
    f32x4 pz[P];       // its normaliser: pz[ia][i] = p[P*(4g + i) + ia]
    if constexpr (CAUSAL) {
        wii = W[blk * M + blk];
#pragma unroll
        for (int c4 = 0; c4 < P * P; ++c4) pst[c4] = zero4();
#pragma unroll
        for (int a = 0; a < P; ++a) pz[a] = zero4();
    }

    const uint16_t* Qp = Q + pair * N * D;
    const uint16_t* Kp = K + pair * N * D;
    const uint16_t* Vp = V + pair * N * D;
    float* Yp = Y + pair * N * D;

    for (int tile = tile_beg; tile < tile_end; ++tile) {
        const int64_t t0 = bstart + 16 * (int64_t)tile;

        // phi(Q) as the A operand: token t0 + n, group-local features of group g.
        const int64_t tq = t0 + n;
        const bool qok = tq < bend;
        uint16_t qr[FL];
        load_group<P>(Qp + tq * D + FL * g, qok, Q, qr);
        issue_fence();
        bf16x8 aq[KS];
        float qf[FL];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int fl = 8 * ks + e;
                const __bf16 ph = (__bf16)((fl < FL && qok) ? phi_fast(bf16_to_f32(qr[fl < FL ? fl : 0])) : 0.f);
                aq[ks][e] = ph;
                if (fl < FL) qf[fl] = bf16v_to_f32(ph);
            }

        float zc[FL];
        if constexpr (CAUSAL) {
            f32x4 comb[P * P];
#pragma unroll
            for (int c4 = 0; c4 < P * P; ++c4)
#pragma unroll
                for (int i = 0; i < 4; ++i) comb[c4][i] = fmaf(wii, pst[c4][i], sch[c4][i]);
            build_b<P, KS>(comb, bh, bl);
#pragma unroll
            for (int fl = 0; fl < FL; ++fl) zc[fl] = fmaf(wii, pz[fl % P][fl / P], zt[fl]);
        } else {
#pragma unroll
            for (int fl = 0; fl < FL; ++fl) zc[fl] = zt[fl];
        }

        float den = 0.f;
#pragma unroll
        for (int fl = 0; fl < FL; ++fl) den = fmaf(qf[fl], zc[fl], den);
        den = sum_over_groups(den);

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

        if constexpr (CAUSAL) {
            // phi(K) rows (keys t0 + n) as an A operand for A^T = phi(K) phi(Q)^T.
            const int64_t tk = t0 + n;
            const bool kok = tk < bend;
            uint16_t kr[FL];
            load_group<P>(Kp + tk * D + FL * g, kok, K, kr);
            bf16x8 ak[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int fl = 8 * ks + e;
                    ak[ks][e] = (__bf16)((fl < FL && kok) ? phi_fast(bf16_to_f32(kr[fl < FL ? fl : 0])) : 0.f);
                }
            // The tile's K and V with tokens along k: lane holds tokens t0 + 4g + e
            // (e < 4) at features / columns P*n .. P*n + P - 1.
            bf16x4 ak16[P], bv16[P];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t tok = t0 + 4 * g + e;
                const bool ok = tok < bend;
                uint16_t k16[P], v16[P];
                load_feat3<P>(Kp + tok * D + P * n, ok, K, k16);
                load_feat3<P>(Vp + tok * D + P * n, ok, V, v16);
#pragma unroll
                for (int f = 0; f < P; ++f) {
                    ak16[f][e] = (__bf16)(ok ? phi_fast(bf16_to_f32(k16[f])) : 0.f);
                    bv16[f][e] = bits_to_bf16(v16[f]);
                }
            }
            // Lane (g, n) receives A[query n][key 4g + i], i = 0..3.
            f32x4 at = zero4();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) at = mfma32(ak[ks], aq[ks], at);
            bf16x4 ahi, alo;
            float rs = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float a = (4 * g + i <= n) ? wii * at[i] : 0.f;
                const bf16pair h = split_bf16(a);
                ahi[i] = h.hi;
                alo[i] = h.lo;
                rs += bf16v_to_f32(h.hi) + bf16v_to_f32(h.lo);
            }
            den += sum_over_groups(rs);
#pragma unroll
            for (int jb = 0; jb < P; ++jb) {
                acc[jb] = mfma16(ahi, bv16[jb], acc[jb]);
                acc[jb] = mfma16(alo, bv16[jb], acc[jb]);
            }
            // Fold this tile into the running block summary.
            const bf16x4 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
#pragma unroll
            for (int ia = 0; ia < P; ++ia) {
#pragma unroll
                for (int jb = 0; jb < P; ++jb) pst[ia * P + jb] = mfma16(ak16[ia], bv16[jb], pst[ia * P + jb]);
                pz[ia] = mfma16(ak16[ia], ones, pz[ia]);
            }
        }

        den += kEps;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float dd = __shfl(den, 4 * g + i, 64);
            const int64_t row = t0 + 4 * g + i;
            if (row < bend) {
                float* dst = Yp + row * D + P * n;
                if constexpr (P == 4) {
                    *reinterpret_cast<f32x4*>(dst) = f32x4{acc[0][i] / dd, acc[1][i] / dd, acc[2][i] / dd, acc[3][i] / dd};
                } else if constexpr (P == 2) {
                    *reinterpret_cast<float2*>(dst) = make_float2(acc[0][i] / dd, acc[1][i] / dd);
                } else {
                    dst[0] = acc[0][i] / dd;
                }
            }
        }
    }
}

// float32 path: one thread per output element, float32 arithmetic throughout.
__global__ __launch_bounds__(256) void output_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                         const float* __restrict__ V, const float* __restrict__ St,
                                                         const float* __restrict__ W, float* __restrict__ Y,
                                                         int64_t BH, int64_t N, int64_t M, int D, int causal) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= BH * N * D) return;
    const int c = (int)(idx % D);
    const int64_t t = (idx / D) % N, pair = idx / ((int64_t)N * D);
    const int64_t C = N / M, blk = t / C;
    const int P = D / 16;
    const float* sv = St + (blk * BH + pair) * (int64_t)(D * D + D);
    const float* q = Q + (pair * N + t) * D;
    float num = 0.f, den = 0.f;
    for (int r = 0; r < D; ++r) {
        const float fq = phi_precise(q[r]);
        num = fmaf(fq, sv[packed_index(P, r, c)], num);
        den = fmaf(fq, sv[D * D + r], den);
    }
    if (causal) {
        const float wii = W[blk * M + blk];
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
    Y[idx] = num / (den + kEps);
}

hipError_t launch_output(int dtype, const void* q, const void* k, const void* v, const float* St,
                         const float* W, float* out, int64_t BH, int64_t N, int D, int64_t M, bool causal,
                         hipStream_t stream) {
    if (dtype == kDtypeF32) {
        const int64_t total = BH * N * D;
        output_f32_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream>>>(
            (const float*)q, (const float*)k, (const float*)v, St, W, out, BH, N, M, D, causal ? 1 : 0);
        return hipGetLastError();
    }
    const int64_t C = N / M;
    const int ntiles = (int)((C + 15) / 16);
    // Causal: one wave walks all of a block's tiles in order.  Otherwise up to
    // four tiles per wave, amortising the summary operand over 64 tokens.
    const int tpw = causal ? ntiles : min(ntiles, 4);
    const int wpu = (ntiles + tpw - 1) / tpw;
    const int64_t waves = BH * M * wpu;
    const dim3 grid((unsigned)((waves + 3) / 4));
    const uint16_t* qq = (const uint16_t*)q;
    const uint16_t* kk = (const uint16_t*)k;
    const uint16_t* vv = (const uint16_t*)v;
#define MHLA_LAUNCH_OUT(DD, CC) \
    output_bf16_kernel<DD, CC><<<grid, dim3(256), 0, stream>>>(qq, kk, vv, St, W, out, BH, N, M, tpw, wpu)
    if (causal) {
        switch (D) {
            case 16: MHLA_LAUNCH_OUT(16, true); break;
            case 32: MHLA_LAUNCH_OUT(32, true); break;
            case 64: MHLA_LAUNCH_OUT(64, true); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (D) {
            case 16: MHLA_LAUNCH_OUT(16, false); break;
            case 32: MHLA_LAUNCH_OUT(32, false); break;
            case 64: MHLA_LAUNCH_OUT(64, false); break;
            default: return hipErrorInvalidValue;
        }
    }
#undef MHLA_LAUNCH_OUT
    return hipGetLastError();
}

}  // namespace mhla
