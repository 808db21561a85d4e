// bwd_fused.hip -- gradients of the MHLA forward pass for short sequences (N <= 256,
// at most 16 blocks of whole 16-token tiles, non-causal, bf16 inputs) in one kernel,
// in the token-level form of "MHLA: Restoring Expressivity of Linear Attention via
// Token-Level Multi-Head" (§4.2, Eq. 5).  With b(t) the block of token t,
//
//   s_tj = phi(q_t) . phi(k_j),   A_tj = W[b(t), b(j)] s_tj,   g_tj = dy_t . v_j
//   den_t = sum_j A_tj + 1e-6,    dn_t = sum_j A_tj g_tj          (dn_t = dy_t . num_t)
//   dnum_t = dy_t / den_t,        dden_t = -dn_t / den_t^2
//   dA_tj = g_tj / den_t + dden_t  (without the normaliser: den_t = 1, dA_tj = g_tj)
//   dv_j        = sum_t A_tj dnum_t
//   d phi(q_t)  = sum_j W[b(t), b(j)] dA_tj phi(k_j)
//               = (sum_j W g_tj phi(k_j)) / den_t + dden_t z~_b(t),   z~_i = sum_b W[i, b] z_b
//   d phi(k_j)  = sum_t W[b(t), b(j)] dA_tj phi(q_t)
//   dW[i, b]   += sum_{t in i, j in b} dA_tj s_tj                      (summed over pairs)
//
// which is the chain rule through the four steps of §4.1 regrouped by token, as the
// forward's token-level kernel regroups the forward ("Linear Attention 笔记" §2 for
// phi = ELU + 1, §4/§5 for the guard).  For blocks shorter than d the summary form
// moves four d x d summaries per block (S, S~, dS~, dS) through HBM; this form needs
// none, only the N x N scores of each pair, which never leave the registers.
//
// One workgroup of eight waves per (batch, head) pair, two passes:
//   pass A (queries): wave w owns query tiles w and w + 8.  phi(K) (bf16 hi + lo) and V
//     sit in LDS; per pair of key tiles the wave forms s^T and g^T (keys x queries) on
//     MFMA, accumulates den_t and dn_t per lane, and adds the product of phi(K)^T with
//     (W g)^T into its d phi(q)^T accumulators.  It then writes dq and leaves den_t,
//     dden_t in LDS.
//   pass B (keys): phi(Q) and dy (bf16 hi + lo) replace phi(K) and V in LDS; wave w owns
//     key tiles w and w + 8, forms s and g (queries x keys) per pair of query tiles, and
//     accumulates dv^T += dy^T (A / den) and d phi(k)^T += phi(Q)^T (W dA), then writes
//     dk and dv; sum dA s goes into wave-private dW bins in LDS.
// Every product runs on 16x16x32 bf16 MFMA with float32 operands split into bf16 hi + lo
// (three products; two when one side is an exact bf16 input) and float32 accumulation
// in a fixed order, so the result is bit-reproducible.  dW leaves the kernel as one
// partial per pair, summed over pairs in a fixed order by bwd_fused_dw_kernel.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"
#include "lds_tiles.hpp"

namespace mhla {

namespace {

constexpr int kBW = 8;         // waves per workgroup
constexpr int kBMaxRows = 256; // N
constexpr int kBMaxBlocks = 16;

template <int D>
struct BwdCfg {
    static constexpr int P = D / 16;   // 16-wide feature (or value) tiles
    static constexpr int KS = D / 32;  // 32-deep k-steps over features
    static constexpr int CPR = D / 8;  // 16-byte pieces per row
    static constexpr int kPlane = kBMaxRows * D * 2;  // one bf16 [256][D] array
    // LDS: four planes (pass A: phi(K) hi, phi(K) lo, V; pass B: phi(Q) hi, phi(Q) lo,
    // dy hi, dy lo), then 1 / den and dden per token, z~ per block, W, dW bins per wave.
    static constexpr int kDen = 4 * kPlane;
    static constexpr int kDden = kDen + kBMaxRows * 4;
    static constexpr int kZt = kDden + kBMaxRows * 4;
    static constexpr int kW = kZt + kBMaxBlocks * D * 4;
    static constexpr int kBins = kW + kBMaxBlocks * kBMaxBlocks * 4;
    static constexpr int kBytes = kBins + kBW * kBMaxBlocks * kBMaxBlocks * 4;
};

struct BwdShape {
    int N, M, C, QT, norm;  // QT: 16-token tiles (queries and keys alike)
    int nwhole;             // workgroups that take a whole pair (the rest take halves)
};

// phi(x) = ELU(x) + 1 and phi'(x) (1 above zero, exp(x) = phi(x) at or below), float32.
__device__ __forceinline__ float phi_d(float x, float& dphi) {
    const float p = phi_fast(x);
    dphi = x > 0.f ? 1.f : p;
    return p;
}

// Rows r0 .. r0 + 15 (one tile) of a [N][D] bf16 matrix into LDS planes: phi split into
// hi and lo (PHI), or the values as they are (hi only).  16 bytes per lane and piece.
template <int D, bool PHI>
__device__ __forceinline__ void stage_rows(const uint16_t* __restrict__ X, int64_t base, int nrows,
                                           unsigned char* hi, unsigned char* lo) {
    constexpr int CPR = BwdCfg<D>::CPR;
    for (int u = threadIdx.x; u < nrows * CPR; u += 64 * kBW) {
        const int row = u / CPR, pc = u % CPR;
        const u32x4 w = *reinterpret_cast<const u32x4*>(X + base + (int64_t)row * D + 8 * pc);
        const int off = 16 * swz(row, pc, CPR);
        if constexpr (PHI) {
            uint32_t h[4], l[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) split2_bf16(phi_fast(lo_bf16(w[e])), phi_fast(hi_bf16(w[e])), h[e], l[e]);
            *reinterpret_cast<u32x4*>(hi + off) = u32x4{h[0], h[1], h[2], h[3]};
            *reinterpret_cast<u32x4*>(lo + off) = u32x4{l[0], l[1], l[2], l[3]};
        } else {
            *reinterpret_cast<u32x4*>(hi + off) = w;
        }
    }
}

// Rows of the float32 dy into LDS planes as bf16 hi and lo.
template <int D>
__device__ __forceinline__ void stage_dy(const float* __restrict__ dY, int64_t base, int nrows, unsigned char* hi,
                                         unsigned char* lo) {
    constexpr int CPR = BwdCfg<D>::CPR;
    for (int u = threadIdx.x; u < nrows * CPR; u += 64 * kBW) {
        const int row = u / CPR, pc = u % CPR;
        const f32x4* src = reinterpret_cast<const f32x4*>(dY + base + (int64_t)row * D + 8 * pc);
        const f32x4 a = src[0], b = src[1];
        uint32_t h[4], l[4];
        split2_bf16(a[0], a[1], h[0], l[0]);
        split2_bf16(a[2], a[3], h[1], l[1]);
        split2_bf16(b[0], b[1], h[2], l[2]);
        split2_bf16(b[2], b[3], h[3], l[3]);
        const int off = 16 * swz(row, pc, CPR);
        *reinterpret_cast<u32x4*>(hi + off) = u32x4{h[0], h[1], h[2], h[3]};
        *reinterpret_cast<u32x4*>(lo + off) = u32x4{l[0], l[1], l[2], l[3]};
    }
}

// A 16 x 32 operand read straight from an LDS plane: lane (g, n) takes row r0 + n,
// k-slots 8g .. 8g + 7 = columns 32 ks + 8g .. +7.
template <int D>
__device__ __forceinline__ bf16x8 lds_rows(const unsigned char* plane, int r0, int ks, int g, int n) {
    return *reinterpret_cast<const bf16x8*>(plane + 16 * swz(r0 + n, 4 * ks + g, BwdCfg<D>::CPR));
}

// The same operand from global memory: bf16 row (phi applied, split into hi and lo).
template <int D>
__device__ __forceinline__ void row_phi_operand(const uint16_t* __restrict__ X, int64_t row, int ks, int g, bf16x8& h,
                                                bf16x8& l) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(X + row * D + 32 * ks + 8 * g);
    uint32_t hh[4], ll[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) split2_bf16(phi_fast(lo_bf16(w[e])), phi_fast(hi_bf16(w[e])), hh[e], ll[e]);
    h = __builtin_bit_cast(bf16x8, u32x4{hh[0], hh[1], hh[2], hh[3]});
    l = __builtin_bit_cast(bf16x8, u32x4{ll[0], ll[1], ll[2], ll[3]});
}

// Eight float32 values (k-slots of a 16x16x32 operand) split into bf16 hi and lo.
__device__ __forceinline__ void split8(const f32x4& a, const f32x4& b, bf16x8& h, bf16x8& l) {
    uint32_t hh[4], ll[4];
    split2_bf16(a[0], a[1], hh[0], ll[0]);
    split2_bf16(a[2], a[3], hh[1], ll[1]);
    split2_bf16(b[0], b[1], hh[2], ll[2]);
    split2_bf16(b[2], b[3], hh[3], ll[3]);
    h = __builtin_bit_cast(bf16x8, u32x4{hh[0], hh[1], hh[2], hh[3]});
    l = __builtin_bit_cast(bf16x8, u32x4{ll[0], ll[1], ll[2], ll[3]});
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes of the wave, in a fixed order, returned in every lane: each row of
// 16 lanes by DPP moves within the row (quad swaps, half-row then row mirror), then the
// four row sums read from lanes 0, 16, 32, 48.  No LDS round trips.
__device__ __forceinline__ float wave_total(float x) {
    x += dpp_f32<0xB1>(x);   // quad_perm [1, 0, 3, 2]
    x += dpp_f32<0x4E>(x);   // quad_perm [2, 3, 0, 1]
    x += dpp_f32<0x141>(x);  // row_half_mirror
    x += dpp_f32<0x140>(x);  // row_mirror
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ f32x4 mfma3(const bf16x8& ah, const bf16x8& al, const bf16x8& bh, const bf16x8& bl,
                                       f32x4 c) {
    c = mfma32(ah, bh, c);
    c = mfma32(ah, bl, c);
    return mfma32(al, bh, c);
}

// LDS areas of the kernel (see BwdCfg).
struct BwdLds {
    unsigned char *pl0, *pl1, *pl2, *pl3;
    float *rden, *dden, *zt, *wl, *bins;
};

// The row-layout operands of two 16-row tiles (hi and lo planes of one matrix).
template <int D>
struct TileOps {
    bf16x8 h[2][BwdCfg<D>::KS], l[2][BwdCfg<D>::KS];
};

// Pass A for NT query tiles qts[0 .. NT) of the wave: phi(K) hi/lo in pl0/pl1, V in pl2.
// Writes 1 / den_t, dden_t of the tiles' queries, and dq of the first NX tiles (the
// others only need their normaliser terms, for pass B).  The tiles' phi(q) and dy
// operands are left in qo and yo for pass B's planes.
template <int D, int NT, int NX>
__device__ __forceinline__ void bwd_pass_a(const BwdLds& L, const uint16_t* __restrict__ Q,
                                           const float* __restrict__ dY, float* __restrict__ dQ, const BwdShape& sh,
                                           int64_t pair, const int (&qts)[NT], int g, int n, TileOps<D>& qo,
                                           TileOps<D>& yo) {
    using Cfg = BwdCfg<D>;
    constexpr int P = Cfg::P, KS = Cfg::KS, CPR = Cfg::CPR;
    const int M = sh.M, QT = sh.QT, CT = sh.C / 16;
    const bool norm = sh.norm != 0;
    auto& bqh = qo.h;  // phi(q) and dy as B operands: query n
    auto& bql = qo.l;
    auto& byh = yo.h;
    auto& byl = yo.l;
    int64_t qrow[NT];
    int bt[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) {
        const int qt = qts[u];
        bt[u] = qt / CT;
        qrow[u] = pair * sh.N + 16 * qt + n;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            row_phi_operand<D>(Q, qrow[u], ks, g, bqh[u][ks], bql[u][ks]);
            const f32x4* src = reinterpret_cast<const f32x4*>(dY + qrow[u] * D + 32 * ks + 8 * g);
            split8(src[0], src[1], byh[u][ks], byl[u][ks]);
        }
    }
    f32x4 xacc[NX][P];  // (sum_j W g_tj phi(k_j))^T: features 16f + 4g + i, query n
    float dsum[NT], nsum[NT];  // this lane's keys' part of den_t and dn_t (query n)
#pragma unroll
    for (int u = 0; u < NT; ++u) dsum[u] = nsum[u] = 0.f;
#pragma unroll
    for (int u = 0; u < NX; ++u)
#pragma unroll
        for (int f = 0; f < P; ++f) xacc[u][f] = zero4();
    for (int jp = 0; jp < QT / 2; ++jp) {
        f32x4 wg[NX][2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int kt = 2 * jp + hh;
            bf16x8 akh[KS], akl[KS], av[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                akh[ks] = lds_rows<D>(L.pl0, 16 * kt, ks, g, n);
                akl[ks] = lds_rows<D>(L.pl1, 16 * kt, ks, g, n);
                av[ks] = lds_rows<D>(L.pl2, 16 * kt, ks, g, n);
            }
#pragma unroll
            for (int u = 0; u < NT; ++u) {
                f32x4 s = zero4(), gg = zero4();  // keys 16 kt + 4g + e, query n
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    s = mfma3(akh[ks], akl[ks], bqh[u][ks], bql[u][ks], s);
                    gg = mfma32(av[ks], byh[u][ks], gg);
                    gg = mfma32(av[ks], byl[u][ks], gg);
                }
                const float w = L.wl[bt[u] * M + kt / CT];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float a = w * s[e];
                    dsum[u] += a;
                    nsum[u] = fmaf(a, gg[e], nsum[u]);
                    if (u < NX) wg[u < NX ? u : 0][hh][e] = w * gg[e];
                }
            }
        }
        bf16x8 gh[NX], gl[NX];  // (W g)^T as B: k-slot 8g + 4hh + e = key 32 jp + 16 hh + 4g + e
#pragma unroll
        for (int u = 0; u < NX; ++u) split8(wg[u][0], wg[u][1], gh[u], gl[u]);
#pragma unroll
        for (int f = 0; f < P; ++f) {
            const bf16x8 kth = lds_operand_t(L.pl0, 32 * jp, 16 * f, CPR, g, n);
            const bf16x8 ktl = lds_operand_t(L.pl1, 32 * jp, 16 * f, CPR, g, n);
#pragma unroll
            for (int u = 0; u < NX; ++u) xacc[u][f] = mfma3(kth, ktl, gh[u], gl[u], xacc[u][f]);
        }
    }
#pragma unroll
    for (int u = 0; u < NT; ++u) {
        const int qt = qts[u];
        // den_t, dn_t for query n: the four lane groups hold disjoint keys
        const float dtot = sum_over_groups(dsum[u]), ntot = sum_over_groups(nsum[u]);
        const float rden = norm ? 1.f / (dtot + kEps) : 1.f;
        const float dden = norm ? -ntot * rden * rden : 0.f;
        if (g == 0) {
            L.rden[16 * qt + n] = rden;
            L.dden[16 * qt + n] = dden;
        }
        if (u >= NX) continue;
        // d phi(q)^T = X^T / den + dden z~_b(t), times phi'(q); 16-byte stores
#pragma unroll
        for (int f = 0; f < P; ++f) {
            const int f0 = 16 * f + 4 * g;
            const u32x2 qw = *reinterpret_cast<const u32x2*>(Q + qrow[u] * D + f0);
            const float qv[4] = {lo_bf16(qw[0]), hi_bf16(qw[0]), lo_bf16(qw[1]), hi_bf16(qw[1])};
            f32x4 out;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float dp;
                (void)phi_d(qv[i], dp);
                out[i] = fmaf(xacc[u < NX ? u : 0][f][i], rden, dden * L.zt[bt[u] * D + f0 + i]) * dp;
            }
            *reinterpret_cast<f32x4*>(dQ + qrow[u] * D + f0) = out;
        }
    }
}

// Pass B for NT key tiles kt0, kt0 + 8 (NT = 2) of the wave: phi(Q) hi/lo in pl0/pl1, dy
// hi/lo in pl2/pl3; the tiles' phi(k) operands in ko (hi, lo) and their v in vo.h.
// Writes dk, dv and adds sum dA s to the wave's dW bins.
template <int D, int NT>
__device__ __forceinline__ void bwd_pass_b(const BwdLds& L, const uint16_t* __restrict__ K, float* __restrict__ dK,
                                           float* __restrict__ dV, float* mybins, const BwdShape& sh, int64_t pair,
                                           int kt0, int lane, int g, int n, const TileOps<D>& ko,
                                           const TileOps<D>& vo) {
    using Cfg = BwdCfg<D>;
    constexpr int P = Cfg::P, KS = Cfg::KS, CPR = Cfg::CPR;
    const int M = sh.M, QT = sh.QT, CT = sh.C / 16;
    const auto& bkh = ko.h;  // phi(k) and v as B operands: key n
    const auto& bkl = ko.l;
    const auto& bv = vo.h;
    int64_t krow[NT];
    int bj[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) {
        const int kt = kt0 + kBW * u;
        bj[u] = kt / CT;
        krow[u] = pair * sh.N + 16 * kt + n;
    }
    f32x4 vacc[NT][P], kacc[NT][P];  // dv^T, d phi(k)^T: values / features 16c + 4g + i, key n
    float dwl[NT];  // this lane's part of sum dA s for block pair (bcur, bj)
#pragma unroll
    for (int u = 0; u < NT; ++u) {
        dwl[u] = 0.f;
#pragma unroll
        for (int c = 0; c < P; ++c) vacc[u][c] = kacc[u][c] = zero4();
    }
    int bcur = 0;
    // The query blocks come in order, so each (query block, key block) bin of the wave is
    // written once: plain stores, no read-modify-write (both tiles' parts summed first when
    // they fall in one key block).
    auto flush = [&]() {
        if (NT == 2 && bj[0] == bj[NT - 1]) {
            const float tot = wave_total(dwl[0] + dwl[NT - 1]);
            if (lane == 0) mybins[bcur * kBMaxBlocks + bj[0]] = tot;
        } else {
#pragma unroll
            for (int u = 0; u < NT; ++u) {
                const float tot = wave_total(dwl[u]);
                if (lane == 0) mybins[bcur * kBMaxBlocks + bj[u]] = tot;
            }
        }
#pragma unroll
        for (int u = 0; u < NT; ++u) dwl[u] = 0.f;
    };
    for (int tp = 0; tp < QT / 2; ++tp) {
        f32x4 ad[NT][2], ds[NT][2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int qt = 2 * tp + hh, bt = qt / CT;
            if (bt != bcur) {  // uniform: the previous block pair's dW parts to the bins
                flush();
                bcur = bt;
            }
            bf16x8 aqh[KS], aql[KS], ayh[KS], ayl[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                aqh[ks] = lds_rows<D>(L.pl0, 16 * qt, ks, g, n);
                aql[ks] = lds_rows<D>(L.pl1, 16 * qt, ks, g, n);
                ayh[ks] = lds_rows<D>(L.pl2, 16 * qt, ks, g, n);
                ayl[ks] = lds_rows<D>(L.pl3, 16 * qt, ks, g, n);
            }
            const f32x4 rd4 = *reinterpret_cast<const f32x4*>(L.rden + 16 * qt + 4 * g);
            const f32x4 dd4 = *reinterpret_cast<const f32x4*>(L.dden + 16 * qt + 4 * g);
#pragma unroll
            for (int u = 0; u < NT; ++u) {
                f32x4 s = zero4(), gg = zero4();  // queries 16 qt + 4g + e, key n
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    s = mfma3(aqh[ks], aql[ks], bkh[u][ks], bkl[u][ks], s);
                    gg = mfma32(ayh[ks], bv[u][ks], gg);
                    gg = mfma32(ayl[ks], bv[u][ks], gg);
                }
                const float w = L.wl[bt * M + bj[u]];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float da = fmaf(gg[e], rd4[e], dd4[e]);  // dA_tj
                    ad[u][hh][e] = w * s[e] * rd4[e];              // A_tj / den_t
                    ds[u][hh][e] = w * da;
                    dwl[u] = fmaf(da, s[e], dwl[u]);
                }
            }
        }
        bf16x8 adh[NT], adl[NT], dsh[NT], dsl[NT];  // B: k-slot 8g + 4hh + e = query 32 tp + 16 hh + 4g + e
#pragma unroll
        for (int u = 0; u < NT; ++u) {
            split8(ad[u][0], ad[u][1], adh[u], adl[u]);
            split8(ds[u][0], ds[u][1], dsh[u], dsl[u]);
        }
#pragma unroll
        for (int c = 0; c < P; ++c) {
            const bf16x8 yth = lds_operand_t(L.pl2, 32 * tp, 16 * c, CPR, g, n);
            const bf16x8 ytl = lds_operand_t(L.pl3, 32 * tp, 16 * c, CPR, g, n);
#pragma unroll
            for (int u = 0; u < NT; ++u) vacc[u][c] = mfma3(yth, ytl, adh[u], adl[u], vacc[u][c]);
            const bf16x8 qth = lds_operand_t(L.pl0, 32 * tp, 16 * c, CPR, g, n);
            const bf16x8 qtl = lds_operand_t(L.pl1, 32 * tp, 16 * c, CPR, g, n);
#pragma unroll
            for (int u = 0; u < NT; ++u) kacc[u][c] = mfma3(qth, qtl, dsh[u], dsl[u], kacc[u][c]);
        }
    }
    flush();
    // dk = d phi(k) phi'(k), dv; 16-byte stores
#pragma unroll
    for (int u = 0; u < NT; ++u)
#pragma unroll
        for (int c = 0; c < P; ++c) {
            const int f0 = 16 * c + 4 * g;
            const u32x2 kw = *reinterpret_cast<const u32x2*>(K + krow[u] * D + f0);
            const float kv[4] = {lo_bf16(kw[0]), hi_bf16(kw[0]), lo_bf16(kw[1]), hi_bf16(kw[1])};
            f32x4 dkv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float dp;
                (void)phi_d(kv[i], dp);
                dkv[i] = kacc[u][c][i] * dp;
            }
            *reinterpret_cast<f32x4*>(dK + krow[u] * D + f0) = dkv;
            *reinterpret_cast<f32x4*>(dV + krow[u] * D + f0) = vacc[u][c];
        }
}

template <int D>
__global__ __launch_bounds__(64 * kBW) void bwd_fused_kernel(const uint16_t* __restrict__ Q,
                                                             const uint16_t* __restrict__ K,
                                                             const uint16_t* __restrict__ V,
                                                             const float* __restrict__ W,
                                                             const float* __restrict__ dY, float* __restrict__ dQ,
                                                             float* __restrict__ dK, float* __restrict__ dV,
                                                             float* __restrict__ dWpart, BwdShape sh) {
    using Cfg = BwdCfg<D>;
    constexpr int P = Cfg::P, CPR = Cfg::CPR;
    __shared__ __align__(16) unsigned char lds[Cfg::kBytes];
    unsigned char* const pl0 = lds;
    unsigned char* const pl1 = lds + Cfg::kPlane;
    unsigned char* const pl2 = lds + 2 * Cfg::kPlane;
    unsigned char* const pl3 = lds + 3 * Cfg::kPlane;
    float* const rden_s = reinterpret_cast<float*>(lds + Cfg::kDen);
    float* const dden_s = reinterpret_cast<float*>(lds + Cfg::kDden);
    float* const zt = reinterpret_cast<float*>(lds + Cfg::kZt);
    float* const wl = reinterpret_cast<float*>(lds + Cfg::kW);
    float* const bins = reinterpret_cast<float*>(lds + Cfg::kBins);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, n = lane & 15;
    // Workgroups below nwhole take a whole pair; the rest take half of one (the split
    // pairs' two halves 8 workgroups apart, on one XCD): query tiles 8h .. 8h + 7 in
    // pass A (plus the normaliser terms of the other half's tiles) and the same key tiles
    // in pass B.  Pair counts between one and two rounds of workgroups thus end in a
    // second round of shorter halves instead of a half-empty round of whole pairs.
    int64_t pair;
    int half = -1;
    if ((int)blockIdx.x < sh.nwhole) {
        pair = blockIdx.x;
    } else {
        const int idx = (int)blockIdx.x - sh.nwhole;
        pair = sh.nwhole + (idx / 16) * 8 + idx % 8;
        half = (idx / 8) % 2;
    }
    const int64_t base = pair * sh.N * D;
    const int N = sh.N, M = sh.M, QT = sh.QT;

    // ---- set-up: phi(K) hi/lo and V to LDS, W, cleared dW bins ----
    stage_rows<D, true>(K, base, N, pl0, pl1);
    stage_rows<D, false>(V, base, N, pl2, nullptr);
    for (int t = threadIdx.x; t < M * M; t += 64 * kBW) wl[t] = W[t];
    for (int t = threadIdx.x; t < kBW * kBMaxBlocks * kBMaxBlocks; t += 64 * kBW) bins[t] = 0.f;
    __syncthreads();
    // z~_i = sum_b W[i, b] z_b = sum_r W[i, b(r)] phi(k_r): one [M x N] x [N x D] product on
    // MFMA, wave w < P taking features 16w .. 16w + 15 (W and phi(K) as hi/lo bf16).
    if (wave < P) {
        f32x4 acc = zero4();  // rows (i) 4g + e, feature 16 wave + n
        for (int kp = 0; kp < N / 32; ++kp) {
            f32x4 w2[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                // k-slots 8g + 4hh + e are rows 32 kp + 16 hh + 4g + e (one block: C % 16 = 0)
                const float w = n < M ? wl[n * M + (32 * kp + 16 * hh + 4 * g) / sh.C] : 0.f;
                w2[hh] = f32x4{w, w, w, w};
            }
            bf16x8 wh, wlo;
            split8(w2[0], w2[1], wh, wlo);
            const bf16x8 kh = lds_operand_t(pl0, 32 * kp, 16 * wave, CPR, g, n);
            const bf16x8 kl = lds_operand_t(pl1, 32 * kp, 16 * wave, CPR, g, n);
            acc = mfma3(wh, wlo, kh, kl, acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (4 * g + e < M) zt[(4 * g + e) * D + 16 * wave + n] = acc[e];
    }
    __syncthreads();

    // ---- pass A: the wave's query tiles (w, and w + 8 when there is one) ----
    const BwdLds L{pl0, pl1, pl2, pl3, rden_s, dden_s, zt, wl, bins};
    // Query tiles of the wave in pass A (every tile of the pair has exactly one owner), and
    // its key tiles in pass B.
    int nq = 0, nk = 0, qt_[2] = {0, 0}, kt0 = wave;
    if (half >= 0) {  // (QT = 16)
        nq = 2, qt_[0] = 8 * half + wave, qt_[1] = 8 * (1 - half) + wave;
        nk = 1, kt0 = 8 * half + wave;
    } else if (wave < QT) {
        nq = nk = wave + kBW < QT ? 2 : 1;
        qt_[0] = wave, qt_[1] = wave + kBW;
    }
    TileOps<D> qo, yo;
    if (half >= 0) {
        const int qts[2] = {qt_[0], qt_[1]};
        bwd_pass_a<D, 2, 1>(L, Q, dY, dQ, sh, pair, qts, g, n, qo, yo);
    } else if (nq == 2) {
        const int qts[2] = {qt_[0], qt_[1]};
        bwd_pass_a<D, 2, 2>(L, Q, dY, dQ, sh, pair, qts, g, n, qo, yo);
    } else if (nq == 1) {
        const int qts[1] = {qt_[0]};
        bwd_pass_a<D, 1, 1>(L, Q, dY, dQ, sh, pair, qts, g, n, qo, yo);
    }
    // Pass B's key operands -- phi(K) hi/lo and V rows of the wave's key tiles -- are taken
    // from the planes before pass B's operands replace them.
    TileOps<D> ko, vo;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        if (u < nk) {  // uniform
#pragma unroll
            for (int ks = 0; ks < Cfg::KS; ++ks) {
                ko.h[u][ks] = lds_rows<D>(pl0, 16 * (kt0 + kBW * u), ks, g, n);
                ko.l[u][ks] = lds_rows<D>(pl1, 16 * (kt0 + kBW * u), ks, g, n);
                vo.h[u][ks] = lds_rows<D>(pl2, 16 * (kt0 + kBW * u), ks, g, n);
            }
        }
    }
    __syncthreads();  // every wave is done with phi(K) and V in LDS; 1 / den, dden written

    // ---- pass B: phi(Q) hi/lo and dy hi/lo to LDS from pass A's operands (each query tile
    // has one owner, and the row-layout operand is what lds_rows reads back) ----
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        if (u < nq) {  // uniform
#pragma unroll
            for (int ks = 0; ks < Cfg::KS; ++ks) {
                const int off = 16 * swz(16 * qt_[u] + n, 4 * ks + g, CPR);
                *reinterpret_cast<bf16x8*>(pl0 + off) = qo.h[u][ks];
                *reinterpret_cast<bf16x8*>(pl1 + off) = qo.l[u][ks];
                *reinterpret_cast<bf16x8*>(pl2 + off) = yo.h[u][ks];
                *reinterpret_cast<bf16x8*>(pl3 + off) = yo.l[u][ks];
            }
        }
    }
    __syncthreads();
    float* const mybins = bins + wave * kBMaxBlocks * kBMaxBlocks;
    if (nk == 2)
        bwd_pass_b<D, 2>(L, K, dK, dV, mybins, sh, pair, kt0, lane, g, n, ko, vo);
    else if (nk == 1)
        bwd_pass_b<D, 1>(L, K, dK, dV, mybins, sh, pair, kt0, lane, g, n, ko, vo);
    __syncthreads();
    // the pair's dW: the waves' bins in wave order
    for (int t = threadIdx.x; t < M * M; t += 64 * kBW) {
        const int i = t / M, b = t % M;
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < kBW; ++w) s += bins[w * kBMaxBlocks * kBMaxBlocks + i * kBMaxBlocks + b];
        dWpart[(int64_t)blockIdx.x * M * M + t] = s;  // one partial per workgroup
    }
}

// dW = sum over pairs of the per-pair partials: one workgroup per entry, each thread a
// strided run of pairs, then a fixed tree over the threads (the same order every call).
__global__ __launch_bounds__(256) void bwd_fused_dw_kernel(const float* __restrict__ part, float* __restrict__ dW,
                                                          int64_t BH, int MM) {
    __shared__ float red[256];
    const int t = blockIdx.x;
    float s = 0.f;
    for (int64_t p = threadIdx.x; p < BH; p += 256) s += part[p * MM + t];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0) dW[t] = red[0];
}

}  // namespace

bool bwd_fused_applicable(int dtype, int D, int64_t N, int64_t M, bool causal) {
    // Short sequences in blocks of whole 16-token tiles: the scores of a pair fit one
    // workgroup; longer sequences or other blocks take the summary-form kernels.
    if (dtype != kDtypeBF16 || causal || (D != 32 && D != 64)) return false;
    if (N > kBMaxRows || M > kBMaxBlocks || N % M) return false;
    const int64_t C = N / M;
    return C % 16 == 0 && (N / 16) % 2 == 0;
}

size_t bwd_fused_workspace_floats(int64_t BH, int64_t M) { return (size_t)(2 * BH * M * M); }

hipError_t launch_bwd_fused(const void* q, const void* k, const void* v, const float* W, const float* dy, float* dq,
                            float* dk, float* dv, float* dW, int64_t BH, int64_t N, int D, int64_t M, bool normalize,
                            float* ws, hipStream_t stream) {
    BwdShape sh;
    sh.N = (int)N;
    sh.M = (int)M;
    sh.C = (int)(N / M);
    sh.QT = (int)(N / 16);
    sh.norm = normalize ? 1 : 0;
    // Between one and two rounds of workgroups (one per CU): split the pairs that would
    // run alone in the second round into halves (a multiple of 8 of them).
    const int64_t cus = device_cu_count();
    int64_t nsplit = 0;
    if (sh.QT == 16 && BH > cus && BH < 2 * cus) nsplit = (2 * cus - BH) / 8 * 8;
    sh.nwhole = (int)(BH - nsplit);
    const uint16_t* qq = static_cast<const uint16_t*>(q);
    const uint16_t* kk = static_cast<const uint16_t*>(k);
    const uint16_t* vv = static_cast<const uint16_t*>(v);
    const int64_t nwg = BH + nsplit;
    const dim3 grid((unsigned)nwg), block(64 * kBW);
    switch (D) {
        case 32: bwd_fused_kernel<32><<<grid, block, 0, stream>>>(qq, kk, vv, W, dy, dq, dk, dv, ws, sh); break;
        case 64: bwd_fused_kernel<64><<<grid, block, 0, stream>>>(qq, kk, vv, W, dy, dq, dk, dv, ws, sh); break;
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int MM = (int)(M * M);
    bwd_fused_dw_kernel<<<dim3((unsigned)MM), dim3(256), 0, stream>>>(ws, dW, nwg, MM);
    return hipGetLastError();
}

}  // namespace mhla
