// fused.hip -- the whole MHLA forward pass for short blocks in one kernel, with
// the block summaries kept on chip ("MHLA: Restoring Expressivity of Linear
// Attention via Token-Level Multi-Head", §4.1: phi, local KV summaries
// S_b = sum_{j in b} phi(k_j) v_j^T and z_b, multi-head mixing with M_c, output
// ratio; guard as in "Linear Attention 笔记" §4/§5).  Non-causal only.
//
// When blocks are shorter than d (DiT-S/2 at 256x256: 16 tokens, d = 64) the d x d
// summaries are several times larger than the tokens they summarise, and
// round-tripping them through HBM dominates the three-stage pass.  Here one
// workgroup owns one (batch, head) pair and a slice of 16 consecutive value
// columns (16*slice .. 16*slice + 15) and runs the same four steps with the
// summaries in LDS:
//   1. phi(K) and the summaries of every block restricted to the slice's
//      columns, plus z_b, on 16x16x16 bf16 MFMA (tokens along k; lane holds P
//      features of 4 tokens, MFMA ia treats row m as feature P*m + ia);
//   2. the mixing GEMM S~ = W S over the flattened [feature][column] + z
//      columns, bf16 hi/lo on both operands (three MFMAs), in place in LDS;
//   3. phi(Q) S~_i / (phi(Q) z~_i + 1e-6) for every query block, S~_i split
//      into hi/lo as the B operand.
// The d/16 workgroups of a pair are numbered to run on one XCD, so the second
// and later reads of the pair's K and Q come from its L2.
#include "common.hpp"
#include "kernels.hpp"

namespace mhla {

template <int D>
struct FusedShape {
    static constexpr int P = D / 16;
    static constexpr int NCOL = 16 * D + D;  // flattened S: [feature][16 columns], then z[feature]
    static constexpr int STR = NCOL + 4;     // LDS row stride in floats (staggers banks across rows)
    static constexpr int MAXM = 1024 / D;    // rows that fit in ~70 KiB of LDS
};

int fused_max_blocks(int D) { return 1024 / D; }

size_t fused_lds_bytes(int D, int64_t M) { return (size_t)M * (17 * D + 4) * sizeof(float); }

template <int D>
__global__ __launch_bounds__(256) void fused_small_kernel(const uint16_t* __restrict__ Q,
                                                          const uint16_t* __restrict__ K,
                                                          const uint16_t* __restrict__ V,
                                                          const float* __restrict__ W, float* __restrict__ Y,
                                                          int64_t BH, int N, int M) {
    using Sh = FusedShape<D>;
    constexpr int P = Sh::P, NCOL = Sh::NCOL, STR = Sh::STR, MAXM = Sh::MAXM;
    constexpr int FL = 4 * P;
    constexpr int KS = D >= 32 ? D / 32 : 1;
    constexpr int RT = (MAXM + 15) / 16;  // 16-row tiles of W / S~ (also 16-deep k-chunks over blocks)
    extern __shared__ __align__(16) float lds[];  // [M][STR]

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, n = lane & 15;
    // Workgroup b runs on XCD b % 8; the P slices of one pair share that XCD.
    const int64_t bid = blockIdx.x;
    const int slice = (int)((bid >> 3) % P);
    const int64_t pair = ((bid >> 3) / P) * 8 + (bid & 7);
    if (pair >= BH) return;  // uniform over the workgroup: no barrier is skipped by part of it
    const int C = N / M;
    const int col0 = 16 * slice;
    const uint16_t* Kp = K + pair * N * D;
    const uint16_t* Vp = V + pair * N * D;
    const uint16_t* Qp = Q + pair * N * D;
    float* Yp = Y + pair * N * D;
    const bf16x4 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};

    // Blocks hold at most 16 tokens (one 16-deep MFMA k-step, one query tile), and
    // wave w owns blocks w, w + 4, ...; both token phases work on groups of four of
    // its blocks, with all loads of a group issued before any of them is used.
    const int nb = (M - wave + 3) / 4;  // blocks of this wave

    // Q of the first group of query blocks, loaded now and used after the mixing.
    uint16_t qpre[4][FL];
    auto load_q = [&](int j0, uint16_t (&qr)[4][FL]) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = wave + 4 * (j0 + u);
            const bool ok = j0 + u < nb && n < C;
            const int tq = i * C + n;
            if constexpr (P == 1) {
                const uint2 x = load_or_zero(reinterpret_cast<const uint2*>(Qp + tq * D + FL * g), ok,
                                             reinterpret_cast<const uint2*>(Q));
                qr[u][0] = (uint16_t)x.x; qr[u][1] = (uint16_t)(x.x >> 16);
                qr[u][2] = (uint16_t)x.y; qr[u][3] = (uint16_t)(x.y >> 16);
            } else {
#pragma unroll
                for (int h = 0; h < P / 2; ++h) {
                    const uint4 x = load_or_zero(reinterpret_cast<const uint4*>(Qp + tq * D + FL * g + 8 * h), ok,
                                                 reinterpret_cast<const uint4*>(Q));
                    const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                    for (int v2 = 0; v2 < 4; ++v2) {
                        qr[u][8 * h + 2 * v2] = (uint16_t)w4[v2];
                        qr[u][8 * h + 2 * v2 + 1] = (uint16_t)(w4[v2] >> 16);
                    }
                }
            }
        }
    };
    load_q(0, qpre);

    // ---- 1. summaries of every block over this slice's columns ----
    for (int j0 = 0; j0 < nb; j0 += 4) {
        uint16_t kr[4][4][P], vr[4][4];  // [block of the group][token e][feature]
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int b = wave + 4 * (j0 + u);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int tl = 4 * g + e;
                const bool ok = j0 + u < nb && tl < C;
                const int t = b * C + tl;
                if constexpr (P == 4) {
                    const uint2 x = load_or_zero(reinterpret_cast<const uint2*>(Kp + t * D + P * n), ok,
                                                 reinterpret_cast<const uint2*>(K));
                    kr[u][e][0] = (uint16_t)x.x; kr[u][e][1] = (uint16_t)(x.x >> 16);
                    kr[u][e][2] = (uint16_t)x.y; kr[u][e][3] = (uint16_t)(x.y >> 16);
                } else if constexpr (P == 2) {
                    const uint32_t x = load_or_zero(reinterpret_cast<const uint32_t*>(Kp + t * D + P * n), ok,
                                                    reinterpret_cast<const uint32_t*>(K));
                    kr[u][e][0] = (uint16_t)x; kr[u][e][1] = (uint16_t)(x >> 16);
                } else {
                    kr[u][e][0] = load_or_zero(Kp + t * D + n, ok, K);
                }
                vr[u][e] = load_or_zero(Vp + t * D + col0 + n, ok, V);
            }
        }
        issue_fence();
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (j0 + u < nb) {  // uniform
                const int b = wave + 4 * (j0 + u);
                bf16x4 a[P], bv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool ok = 4 * g + e < C;
#pragma unroll
                    for (int ia = 0; ia < P; ++ia)
                        a[ia][e] = (__bf16)(ok ? phi_fast(bf16_to_f32(kr[u][e][ia])) : 0.f);
                    bv[e] = bits_to_bf16(vr[u][e]);
                }
                // lane (g, n) gets S_b[P*(4g + i) + ia][col0 + n] and z_b at the same features.
                float* row = lds + b * STR;
#pragma unroll
                for (int ia = 0; ia < P; ++ia) {
                    const f32x4 sa = mfma16(a[ia], bv, zero4());
                    const f32x4 za = mfma16(a[ia], ones, zero4());
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int f = P * (4 * g + i) + ia;
                        row[f * 16 + n] = sa[i];
                        if (n == 0) row[16 * D + f] = za[i];
                    }
                }
            }
        }
    }
    __syncthreads();

    // ---- 2. mixing, in place: S~[i][c] = sum_b W[i, b] S[b][c] ----
    bf16x4 wh[RT][RT], wl[RT][RT];  // W fragments: row tile rt, k-chunk kc
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int kc = 0; kc < RT; ++kc)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * rt + n, bb = 16 * kc + 4 * g + e;
                const bf16pair p = split_bf16(load_or_zero(W + i * M + bb, i < M && bb < M, W));
                wh[rt][kc][e] = p.hi;
                wl[rt][kc][e] = p.lo;
            }
    const int rtn = (M + 15) / 16;
    for (int ct = wave; ct < NCOL / 16; ct += 4) {
        const int c = 16 * ct + n;
        f32x4 acc[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt] = zero4();
#pragma unroll
        for (int kc = 0; kc < RT; ++kc) {
            if (kc < rtn) {  // uniform
                bf16x4 bh, bl;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int bb = 16 * kc + 4 * g + e;
                    const bf16pair p = split_bf16(bb < M ? lds[bb * STR + c] : 0.f);
                    bh[e] = p.hi;
                    bl[e] = p.lo;
                }
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    if (rt < rtn) {
                        acc[rt] = mfma16(wh[rt][kc], bh, acc[rt]);
                        acc[rt] = mfma16(wh[rt][kc], bl, acc[rt]);
                        acc[rt] = mfma16(wl[rt][kc], bh, acc[rt]);
                    }
                }
            }
        }
        // Every row of column c has been read by this wave; only it writes column c.
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * rt + 4 * g + r;
                if (rt < rtn && i < M) lds[i * STR + c] = acc[rt][r];
            }
    }
    __syncthreads();

    // ---- 3. output of every query block for this slice ----
    for (int j0 = 0; j0 < nb; j0 += 4) {
        uint16_t qr[4][FL];
        if (j0 == 0) {
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int f = 0; f < FL; ++f) qr[u][f] = qpre[u][f];
        } else {
            load_q(j0, qr);
            issue_fence();
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (j0 + u < nb) {  // uniform
                const int i = wave + 4 * (j0 + u);
                const float* row = lds + i * STR;
                bf16x8 aq[KS], bh[KS], bl[KS];
                float den = 0.f;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int fl = 8 * ks + e;
                        const bf16pair p = split_bf16(fl < FL ? row[(FL * g + fl) * 16 + n] : 0.f);
                        bh[ks][e] = p.hi;
                        bl[ks][e] = p.lo;
                        const __bf16 ph =
                            (__bf16)((fl < FL && n < C) ? phi_fast(bf16_to_f32(qr[u][fl < FL ? fl : 0])) : 0.f);
                        aq[ks][e] = ph;
                        if (fl < FL) den = fmaf(bf16v_to_f32(ph), row[16 * D + FL * g + fl], den);
                    }
                den = sum_over_groups(den) + kEps;
                f32x4 acc = zero4();
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    acc = mfma32(aq[ks], bh[ks], acc);
                    acc = mfma32(aq[ks], bl[ks], acc);
                }
                const float rden = fast_rcp(den);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float rr = __shfl(rden, 4 * g + r, 64);
                    if (4 * g + r < C) Yp[(i * C + 4 * g + r) * D + col0 + n] = acc[r] * rr;
                }
            }
        }
    }
}

bool fused_applicable(int D, int64_t BH, int64_t N, int64_t M) {
    const int64_t C = N / M;
    // Blocks of at most 16 tokens (summaries outweigh the tokens; one MFMA k-step
    // and one query tile per block), all rows in LDS, and enough workgroups
    // (BH * d/16) to fill the chip.
    return M <= fused_max_blocks(D) && C <= 16 && BH * (D / 16) >= 256;
}

hipError_t launch_fused(const void* q, const void* k, const void* v, const float* W, float* out, int64_t BH,
                        int64_t N, int D, int64_t M, hipStream_t stream) {
    const int P = D / 16;
    const size_t lds = fused_lds_bytes(D, M);
    hipError_t e = hipSuccess;
    switch (D) {  // allow more than the default 64 KiB of dynamic LDS
        case 16: e = hipFuncSetAttribute((const void*)fused_small_kernel<16>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); break;
        case 32: e = hipFuncSetAttribute((const void*)fused_small_kernel<32>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); break;
        case 64: e = hipFuncSetAttribute((const void*)fused_small_kernel<64>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)(((BH + 7) / 8) * 8 * P));
    const uint16_t* qq = (const uint16_t*)q;
    const uint16_t* kk = (const uint16_t*)k;
    const uint16_t* vv = (const uint16_t*)v;
    switch (D) {
        case 16: fused_small_kernel<16><<<grid, dim3(256), lds, stream>>>(qq, kk, vv, W, out, BH, (int)N, (int)M); break;
        case 32: fused_small_kernel<32><<<grid, dim3(256), lds, stream>>>(qq, kk, vv, W, out, BH, (int)N, (int)M); break;
        case 64: fused_small_kernel<64><<<grid, dim3(256), lds, stream>>>(qq, kk, vv, W, out, BH, (int)N, (int)M); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace mhla
