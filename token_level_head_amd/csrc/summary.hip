// summary.hip -- stage 1 of the MHLA forward pass: phi(K) fused with the
// per-block KV summaries ("MHLA: Restoring Expressivity of Linear Attention via
// Token-Level Multi-Head", §4.1: S_b = sum_{j in b} phi(k_j) v_j^T, z_b = sum phi(k_j)).
//
// bf16 path.  S_b = phi(K_b)^T V_b is a d x d product whose reduction runs over
// tokens, while K and V are stored token-major.  Instead of transposing tiles
// through LDS, each lane loads P = d/16 consecutive features of 8 tokens (one
// 8-byte load per token for d = 64; 16 lanes cover a whole 128-byte row; lane
// group g takes tokens t + 4e + g, so each load instruction reads four
// consecutive rows) and
// repacks them in registers: MFMA (ia, ib) of the P x P set treats its row m as
// feature P*m + ia and its column n as value column P*n + ib.  The accumulators
// then hold S in the packed layout of common.hpp, which is written with
// full-wave 1 KiB stores.  phi(k) is rounded to bf16 once; the same rounded
// values feed both S_b (MFMA) and z_b (bf16 dot products against (1, 1)), so
// numerator and denominator stay consistent.  Accumulation is float32.
//
// K and V are read through one buffer descriptor per (batch, head) pair with
// 32-bit offsets; a token past the segment gets an out-of-range offset and reads
// zero.  Only the last 32-token step of a segment needs the phi mask.
//
// A block of C tokens may be split over `wpb` waves of one workgroup
// (wpb in {1, 2, 4}, chosen so that enough waves exist); their partial sums are
// added in LDS in a fixed order, so results do not depend on scheduling.  When
// even that leaves too few workgroups (long blocks, few (batch, head) pairs:
// global linear attention over a long sequence), each block is also cut into
// `nseg` token segments handled by different workgroups, which write partial
// summaries in the summary layout; summary_reduce_kernel then adds the partials
// in segment order.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace mhla {

template <int P>
struct TokenWords;  // raw bits of P consecutive bf16 features of one token
template <>
struct TokenWords<4> { typedef u32x2 type; };
template <>
struct TokenWords<2> { typedef uint32_t type; };
template <>
struct TokenWords<1> { typedef uint16_t type; };

template <int P, bool NT>
__device__ __forceinline__ typename TokenWords<P>::type load_token(rsrc_t r, uint32_t off) {
    if constexpr (P == 4) return buf_load64<NT>(r, off);
    else if constexpr (P == 2) return buf_load32<NT>(r, off);
    else return buf_load16<NT>(r, off);
}

// Feature f (< P) of a token's raw bits, as a float.
template <int P>
__device__ __forceinline__ float token_feature(const typename TokenWords<P>::type& w, int f) {
    if constexpr (P == 4) return __uint_as_float((f & 1) ? ((f < 2 ? w.x : w.y) & 0xffff0000u) : ((f < 2 ? w.x : w.y) << 16));
    else if constexpr (P == 2) return __uint_as_float((f & 1) ? (w & 0xffff0000u) : (w << 16));
    else return __uint_as_float((uint32_t)w << 16);
}

// Raw bf16 bits of feature f (< P) of a token.
template <int P>
__device__ __forceinline__ uint32_t token_bits(const typename TokenWords<P>::type& w, int f) {
    if constexpr (P == 4) return (f & 1) ? ((f < 2 ? w.x : w.y) >> 16) : ((f < 2 ? w.x : w.y) & 0xffffu);
    else if constexpr (P == 2) return (f & 1) ? (w >> 16) : (w & 0xffffu);
    else return w;
}

// TR: the transposed summary S_b^T[c][r] = sum_j v_j[c] phi(k_j)[r] in the same packed
// layout (value features along the MFMA rows, key features along its columns), with
// phi(k) split into bf16 hi + lo (two products; v is an exact bf16 operand) and z
// summed in float32: the operand the backward pass contracts over the value index.
template <int D, bool PIPE, bool NT, bool TR = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(TR && D == 64 ? 3 : 4))) void summaries_bf16_kernel(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ V, float* __restrict__ S, int64_t BH, int N, int M,
    int wpb, int nseg, int segC, int heads, BlockLayout lay) {
    constexpr int P = D / 16;
    constexpr int L = D * D + D;
    typedef typename TokenWords<P>::type TW;
    extern __shared__ float red[];  // (4 - 4/wpb) partials of 64 lanes x (4 P^2 + P) floats

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, n = lane & 15;
    const int per_wg = 4 / wpb;
    // nseg > 1 only with wpb == 4 (one unit per workgroup): workgroup -> (unit, token segment).
    const int64_t unit = nseg > 1 ? (int64_t)blockIdx.x / nseg
                                  : (int64_t)blockIdx.x * per_wg + wave / wpb;  // unit = pair * M + block
    const int wseg = nseg > 1 ? (int)(blockIdx.x % nseg) : 0;
    const int seg = wave % wpb;
    const bool active = unit < BH * M;

    f32x4 acc[P][P];
#pragma unroll
    for (int a = 0; a < P; ++a)
#pragma unroll
        for (int b = 0; b < P; ++b) acc[a][b] = zero4();
    float zacc[P];
#pragma unroll
    for (int a = 0; a < P; ++a) zacc[a] = 0.f;
    uint32_t ones = 0x3f803f80u;  // (1, 1) as packed bf16, kept in a register (see split2_bf16)
    asm("" : "+v"(ones));

    int64_t pair = 0, blk = 0;
    if (active) {
        pair = unit / M;
        blk = unit % M;
        int bstart, bend;  // the block's range in the token list
        block_range(lay, blk, N, M, bstart, bend);
        const int base = bstart + wseg * segC;  // this workgroup's token range
        const int len = max(0, nseg > 1 ? min(segC, bend - bstart - wseg * segC) : bend - bstart);
        const int seg_len = ((len + wpb - 1) / wpb + 31) / 32 * 32;
        const int t_beg = base + seg * seg_len;
        const int t_end = min(base + len, t_beg + seg_len);
        const uint32_t pair_bytes = (uint32_t)N * D * 2;
        const rsrc_t rK = make_rsrc(K + pair * N * D, pair_bytes);
        const rsrc_t rV = make_rsrc(V + pair * N * D, pair_bytes);
        // One 32-token step: lane (g, n) holds tokens t + 4e + g, e = 0..7 (the MFMA's
        // k index 8g + e; any token order works, as A and B use the same one).
        auto load = [&](TW (&kr)[8], TW (&vr)[8], int t) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int tok = t + 4 * e + g;  // list entry; its row in the sequence:
                const int row = token_row(lay, tok < t_end ? tok : 0, N);
                const uint32_t off = off_if(tok < t_end && row >= 0, ((uint32_t)row * D + P * n) * 2);
                kr[e] = load_token<P, NT>(rK, off);
                vr[e] = load_token<P, NT>(rV, off);
            }
        };
        auto compute = [&](const TW (&kr)[8], const TW (&vr)[8], int t, auto masked_c) {
            constexpr bool masked = decltype(masked_c)::value;
            if constexpr (TR) {
#pragma unroll
                for (int ib = 0; ib < P; ++ib) {  // B operand: phi(k) feature Pn + ib, hi and lo
                    uint32_t fh[4], fl[4];
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) {
                        float f0 = phi_fast(token_feature<P>(kr[2 * e2], ib));
                        float f1 = phi_fast(token_feature<P>(kr[2 * e2 + 1], ib));
                        if constexpr (masked) {
                            f0 = t + 8 * e2 + g < t_end ? f0 : 0.f;
                            f1 = t + 8 * e2 + 4 + g < t_end ? f1 : 0.f;
                        }
                        zacc[ib] += f0 + f1;
                        split2_bf16(f0, f1, fh[e2], fl[e2]);
                    }
                    const bf16x8 bh = __builtin_bit_cast(bf16x8, u32x4{fh[0], fh[1], fh[2], fh[3]});
                    const bf16x8 bl = __builtin_bit_cast(bf16x8, u32x4{fl[0], fl[1], fl[2], fl[3]});
#pragma unroll
                    for (int ia = 0; ia < P; ++ia) {  // A operand: v feature Pn + ia
                        uint32_t vb[4];
#pragma unroll
                        for (int e2 = 0; e2 < 4; ++e2)
                            vb[e2] = token_bits<P>(vr[2 * e2], ia) | (token_bits<P>(vr[2 * e2 + 1], ia) << 16);
                        const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{vb[0], vb[1], vb[2], vb[3]});
                        acc[ia][ib] = mfma32(a, bh, acc[ia][ib]);
                        acc[ia][ib] = mfma32(a, bl, acc[ia][ib]);
                    }
                }
                return;
            }
#pragma unroll
            for (int ia = 0; ia < P; ++ia) {
                uint32_t pk[4];
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    float f0 = phi_fast(token_feature<P>(kr[2 * e2], ia));
                    float f1 = phi_fast(token_feature<P>(kr[2 * e2 + 1], ia));
                    if constexpr (masked) {  // tokens past the segment read zero, but phi(0) = 1
                        f0 = t + 8 * e2 + g < t_end ? f0 : 0.f;
                        f1 = t + 8 * e2 + 4 + g < t_end ? f1 : 0.f;
                    }
                    pk[e2] = pack_bf16(f0, f1);
                    zacc[ia] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[e2]),
                                                               __builtin_bit_cast(bf16x2, ones), zacc[ia], false);
                }
                const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
#pragma unroll
                for (int ib = 0; ib < P; ++ib) {
                    uint32_t vb[4];
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2)
                        vb[e2] = token_bits<P>(vr[2 * e2], ib) | (token_bits<P>(vr[2 * e2 + 1], ib) << 16);
                    const bf16x8 b = __builtin_bit_cast(bf16x8, u32x4{vb[0], vb[1], vb[2], vb[3]});
                    acc[ia][ib] = mfma32(a, b, acc[ia][ib]);
                }
            }
        };
        auto run = [&](const TW (&kr)[8], const TW (&vr)[8], int t) {
            if (t + 32 <= t_end)
                compute(kr, vr, t, std::false_type{});
            else
                compute(kr, vr, t, std::true_type{});
        };
        int t = t_beg;
        if constexpr (PIPE) {
            // Two register sets: the loads of step s + 1 are issued before step s computes,
            // unconditionally (a step past the segment reads zero), so that every path
            // keeps the same loads in flight and each wait covers the current step only.
            const int nsteps = (t_end - t_beg + 31) / 32;
            TW k0[8], v0[8], k1[8], v1[8];
            load(k0, v0, t);
            for (int s = 0; s < nsteps; s += 2, t += 64) {
                load(k1, v1, t + 32);
                issue_fence();
                run(k0, v0, t);
                if (s + 1 >= nsteps) break;
                load(k0, v0, t + 64);
                issue_fence();
                run(k1, v1, t + 32);
            }
        } else {
            for (; t + 32 <= t_end; t += 32) {
                TW kr[8], vr[8];
                load(kr, vr, t);
                issue_fence();
                compute(kr, vr, t, std::false_type{});
            }
            if (t < t_end) {
                TW kr[8], vr[8];
                load(kr, vr, t);
                issue_fence();
                compute(kr, vr, t, std::true_type{});
            }
        }
    }
    // z: sum the four token groups; lanes (., n) then hold z[P*n + f].
#pragma unroll
    for (int f = 0; f < P; ++f) zacc[f] = sum_over_groups(zacc[f]);

    if (wpb > 1) {
        constexpr int PER_LANE = 4 * P * P + P;
        const int unit_in_wg = wave / wpb;
        if (seg > 0) {
            float* part = red + (size_t)((unit_in_wg * (wpb - 1) + seg - 1) * 64) * PER_LANE;
            f32x4* dst = reinterpret_cast<f32x4*>(part);
#pragma unroll
            for (int a = 0; a < P; ++a)
#pragma unroll
                for (int b = 0; b < P; ++b) dst[(a * P + b) * 64 + lane] = acc[a][b];
            float* zd = part + 4 * P * P * 64;
#pragma unroll
            for (int f = 0; f < P; ++f) zd[f * 64 + lane] = zacc[f];
        }
        __syncthreads();
        if (seg == 0) {
            for (int s = 1; s < wpb; ++s) {
                const float* part = red + (size_t)((unit_in_wg * (wpb - 1) + s - 1) * 64) * PER_LANE;
                const f32x4* src = reinterpret_cast<const f32x4*>(part);
#pragma unroll
                for (int a = 0; a < P; ++a)
#pragma unroll
                    for (int b = 0; b < P; ++b) acc[a][b] += src[(a * P + b) * 64 + lane];
                const float* zs = part + 4 * P * P * 64;
#pragma unroll
                for (int f = 0; f < P; ++f) zacc[f] += zs[f * 64 + lane];
            }
        }
    }
    if (!active || seg != 0) return;

    // With token segments, S points at the partial array [nseg][M][BH][L].
    float* out = S + ((int64_t)wseg * M * BH + blk * BH + summary_row(pair, heads, BH)) * (int64_t)L;
#pragma unroll
    for (int a = 0; a < P; ++a)
#pragma unroll
        for (int b = 0; b < P; ++b)
            *reinterpret_cast<f32x4*>(out + (a * P + b) * 256 + lane * 4) = acc[a][b];
    if (g == 0) {
#pragma unroll
        for (int f = 0; f < P; ++f) out[D * D + P * n + f] = zacc[f];
    }
}

// float32 path: plain float32 arithmetic, one thread per summary entry.
__global__ __launch_bounds__(256) void summaries_f32_kernel(const float* __restrict__ K,
                                                            const float* __restrict__ V,
                                                            float* __restrict__ S, int64_t BH, int64_t N,
                                                            int64_t M, int D, int heads, BlockLayout lay) {
    const int64_t unit = blockIdx.x;  // pair * M + block
    const int64_t pair = unit / M, blk = unit % M;
    int bstart, bend;
    block_range(lay, blk, (int)N, M, bstart, bend);
    const int P = D / 16, L = D * D + D;
    const float* Kp = K + pair * N * D;
    const float* Vp = V + pair * N * D;
    float* out = S + (blk * BH + summary_row(pair, heads, BH)) * (int64_t)L;
    for (int e = threadIdx.x; e < L; e += blockDim.x) {
        float acc = 0.f;
        if (e < D * D) {
            const int chunk = e / 256, rem = e % 256, ln = rem / 4, i = rem % 4;
            const int ia = chunk / P, ib = chunk % P;
            const int r = P * (4 * (ln / 16) + i) + ia, c = P * (ln % 16) + ib;
            for (int j = bstart; j < bend; ++j) {
                const int64_t row = token_row(lay, j, (int)N);
                if (row >= 0) acc = fmaf(phi_precise(Kp[row * D + r]), Vp[row * D + c], acc);
            }
        } else {
            const int r = e - D * D;
            for (int j = bstart; j < bend; ++j) {
                const int64_t row = token_row(lay, j, (int)N);
                if (row >= 0) acc += phi_precise(Kp[row * D + r]);
            }
        }
        out[e] = acc;
    }
}

// S[i] = sum over s of part[s][i] (i < n4 float4 groups), in segment order.
__global__ __launch_bounds__(256) void summary_reduce_kernel(const f32x4* __restrict__ part, f32x4* __restrict__ S,
                                                             int64_t n4, int nseg) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    f32x4 acc = part[i];
    for (int s = 1; s < nseg; ++s) acc += part[(int64_t)s * n4 + i];
    S[i] = acc;
}

namespace {

struct SummarySplit {
    int wpb, nseg, segC;
};

// Waves per block (1, 2, 4) and, for long blocks on few (batch, head) pairs, token
// segments over several workgroups, so that about 1024 workgroups exist.  A block is
// split further only while the waves stay within 4096 (the resident slots at 4 waves
// per SIMD), so that all of them run in one round: 1536 blocks of 256 tokens in 6144
// waves left the second round half empty.  Every wave keeps at least two 32-token
// steps; segments are multiples of 128 tokens.
SummarySplit summary_split(int64_t BH, int64_t C, int64_t M) {
    const int64_t units = BH * M;
    SummarySplit sp{1, 1, (int)C};
    while (sp.wpb < 4 && units * sp.wpb * 2 <= 4096 && C >= 64 * (2 * sp.wpb)) sp.wpb *= 2;
    if (sp.wpb == 4 && units < 1024 && C >= 512) {
        const int64_t want = (1024 + units - 1) / units;
        const int64_t segC = ((C + want - 1) / want + 127) / 128 * 128;
        const int64_t seg = (C + segC - 1) / segC;
        if (seg > 1) {
            sp.nseg = (int)seg;
            sp.segC = (int)std::max<int64_t>(segC, 256);
            sp.nseg = (int)((C + sp.segC - 1) / sp.segC);
        }
    }
    return sp;
}

}  // namespace

bool summaries_t_fits(int64_t BH, int64_t N, int D, int64_t M) {
    return (D == 16 || D == 32 || D == 64) && M > 0 && N % M == 0 && summary_split(BH, N / M, M).nseg == 1;
}

hipError_t launch_summaries_t(const uint16_t* k, const uint16_t* v, float* St, int64_t BH, int64_t N, int D,
                              int64_t M, hipStream_t stream) {
    if (!summaries_t_fits(BH, N, D, M)) return hipErrorInvalidValue;
    const int64_t units = BH * M;
    const SummarySplit sp = summary_split(BH, N / M, M);
    const int per_wg = 4 / sp.wpb;
    const int64_t grid = (units + per_wg - 1) / per_wg;
    const int P = D / 16;
    const size_t lds = sp.wpb > 1 ? (size_t)(4 - per_wg) * 64 * (4 * P * P + P) * sizeof(float) : 0;
    const BlockLayout lay{nullptr, nullptr};
    const bool nt = stream_token_inputs(BH, N, D, 2);
#define MHLA_SUMMARIES_T_CASE(DD, PIPE)                                                                      \
    case DD:                                                                                               \
        if (nt)                                                                                            \
            summaries_bf16_kernel<DD, PIPE, true, true><<<dim3((unsigned)grid), dim3(256), lds, stream>>>( \
                k, v, St, BH, (int)N, (int)M, sp.wpb, 1, (int)(N / M), 0, lay);                            \
        else                                                                                               \
            summaries_bf16_kernel<DD, PIPE, false, true><<<dim3((unsigned)grid), dim3(256), lds, stream>>>(\
                k, v, St, BH, (int)N, (int)M, sp.wpb, 1, (int)(N / M), 0, lay);                            \
        break;
    switch (D) {
        MHLA_SUMMARIES_T_CASE(16, true)
        MHLA_SUMMARIES_T_CASE(32, true)
        MHLA_SUMMARIES_T_CASE(64, false)
        default: return hipErrorInvalidValue;
    }
#undef MHLA_SUMMARIES_T_CASE
    return hipGetLastError();
}

size_t summary_partial_bytes(int dtype, int64_t BH, int64_t C, int D, int64_t M) {
    if (dtype == kDtypeF32) return 0;
    const SummarySplit sp = summary_split(BH, C, M);
    return sp.nseg > 1 ? (size_t)sp.nseg * (size_t)(M * BH) * (size_t)(D * D + D) * sizeof(float) : 0;
}

hipError_t launch_summaries(int dtype, const void* k, const void* v, float* S, int64_t BH, int64_t N,
                            int D, int64_t M, int heads, const BlockLayout& lay, int64_t cmax, float* partial,
                            hipStream_t stream) {
    const int64_t units = BH * M;
    if (dtype == kDtypeF32) {
        summaries_f32_kernel<<<dim3((unsigned)units), dim3(256), 0, stream>>>(
            (const float*)k, (const float*)v, S, BH, N, M, D, heads, lay);
        return hipGetLastError();
    }
    const SummarySplit sp = summary_split(BH, cmax, M);
    if (sp.nseg > 1 && !partial) return hipErrorInvalidValue;
    const int per_wg = 4 / sp.wpb;
    const int64_t grid = sp.nseg > 1 ? units * sp.nseg : (units + per_wg - 1) / per_wg;
    const int P = D / 16;
    const size_t lds = sp.wpb > 1 ? (size_t)(4 - per_wg) * 64 * (4 * P * P + P) * sizeof(float) : 0;
    const uint16_t* kk = (const uint16_t*)k;
    const uint16_t* vv = (const uint16_t*)v;
    float* dst = sp.nseg > 1 ? partial : S;
    const bool nt = stream_token_inputs(BH, N, D, 2);
#define MHLA_SUMMARIES_CASE(DD, PIPE)                                                                           \
    case DD:                                                                                                  \
        if (nt)                                                                                               \
            summaries_bf16_kernel<DD, PIPE, true><<<dim3((unsigned)grid), dim3(256), lds, stream>>>(          \
                kk, vv, dst, BH, (int)N, (int)M, sp.wpb, sp.nseg, sp.segC, heads, lay);                                   \
        else                                                                                                  \
            summaries_bf16_kernel<DD, PIPE, false><<<dim3((unsigned)grid), dim3(256), lds, stream>>>(         \
                kk, vv, dst, BH, (int)N, (int)M, sp.wpb, sp.nseg, sp.segC, heads, lay);                                   \
        break;
    switch (D) {
        MHLA_SUMMARIES_CASE(16, true)
        MHLA_SUMMARIES_CASE(32, true)
        MHLA_SUMMARIES_CASE(64, false)
        default: return hipErrorInvalidValue;
    }
#undef MHLA_SUMMARIES_CASE
    if (sp.nseg > 1) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t n4 = units * (D * D + D) / 4;
        summary_reduce_kernel<<<dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream>>>(
            reinterpret_cast<const f32x4*>(partial), reinterpret_cast<f32x4*>(S), n4, sp.nseg);
    }
    return hipGetLastError();
}

}  // namespace mhla
