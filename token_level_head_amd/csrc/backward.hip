// backward.hip -- gradients of the MHLA forward pass ("MHLA: Restoring Expressivity
// of Linear Attention via Token-Level Multi-Head", §4.1 steps, App. C causal form;
// the coefficient matrix M_c is learned end to end, §4.2).  For L = sum(dY * Y),
// token t in block i, A_t = S~_i (+ W_ii P_t causal), a_t = z~_i (+ W_ii p_t causal),
// P_t, p_t = the summary of block i's tokens up to and including t:
//
//   U_t = A_t dy_t,  den_t = phi(q_t).a_t + 1e-6,  dy_t.num_t = phi(q_t).U_t
//   dden_t = -(phi(q_t).U_t) / den_t^2,  dnum_t = dy_t / den_t
//   d phi(q_t) = U_t / den_t + dden_t a_t
//   dS~_i = sum_{t in i} phi(q_t) dnum_t^T,  dz~_i = sum_{t in i} dden_t phi(q_t)
//   dS_b = sum_i W[i,b] dS~_i (causal: i > b),  dW[i,b] = sum_pairs <dS~_i | dz~_i, S_b | z_b>
//   d phi(k_j) = dS_b v_j + dz_b,  dv_j = dS_b^T phi(k_j)                 (j in block b)
//   causal, keys j of block b, R_j = sum_{t in b, t >= j} phi(q_t) dnum_t^T, r_j likewise
//   with dden_t:  d phi(k_j) += W_bb (R_j v_j + r_j),  dv_j += W_bb R_j^T phi(k_j),
//   dW[b,b] += sum_t phi(q_t).(P_t dnum_t) + dden_t phi(q_t).p_t
//   dq = d phi(q) * phi'(q), dk = d phi(k) * phi'(k), phi'(x) = 1 (x > 0) or exp(x).
//
// The numerator phi(q_t)^T A_t itself is never formed: its only use, dy_t.num_t, equals
// phi(q_t).U_t.  Every d x d operand is therefore contracted over its value index c,
// which is why the summaries here are stored transposed: X^T[c][r] (rows = value
// column c, columns = feature r) in the packed layout of common.hpp, so that a
// lane's packed chunks are exactly the B operand of U = dy X^T-style products.
//
// Precision: every product runs on bf16 MFMA with both operands split into hi + lo
// bf16 parts (three products; two when an operand is an exact bf16 input), with
// float32 accumulation in a fixed order -- about 16 significant bits per operand and
// bit-reproducible results.  phi and the reciprocals use the hardware exp2 and rcp.
//
// Tiles are 16 tokens.  Two register layouts of a tile are used (lane l, g = l / 16,
// n = l % 16, d = 16P, FL = 4P):
//   row layout (RL):  lane holds token n, features FL*g .. FL*g + FL - 1; it is the A
//                     (or B) operand of the 16x16x32 MFMA with tokens along m (or n);
//   dot layout (DL):  lane holds tokens 4g + i (i < 4), features P*n .. P*n + P - 1;
//                     it is the result layout of those MFMAs (with the packed B
//                     operand) and the A/B operand of the 16x16x16 MFMA with tokens
//                     along k (the summary-type products).
// Each tile is read through its own buffer descriptor whose range ends at the block's
// last token: rows past it read as zero and stores to them are dropped.
//
// Kernels: bwd_sum_kernel recomputes S_b^T, z_b; the mixing GEMM (mix.hip) forms S~;
// bwd_query_kernel / bwd_query_causal_kernel produce dq and dS~^T, dz~ (causal: also
// per-token den, dden and the diagonal part of dW); the mixing GEMM with W^T forms dS;
// bwd_key_kernel / bwd_key_causal_kernel produce dk, dv; bwd_dw_kernel and
// bwd_dw_reduce1_kernel / bwd_dw_reduce_kernel form dW as a split-K MFMA GEMM with a
// two-level fixed-order reduction.
// Non-causal kernels spread a block's tiles over up to four waves of one workgroup
// (partial sums added in LDS in a fixed order).  Causal kernels walk a block's tiles
// in order (queries: two waves splitting the feature columns) or in reverse (keys: one
// wave per orientation of the running sum), carrying the running summary.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "lds_tiles.hpp"

namespace mhla {

namespace {

template <int D>
struct Dim {
    static constexpr int P = D / 16;
    static constexpr int FL = 4 * P;                 // features per lane group (row layout)
    static constexpr int KS = D >= 32 ? D / 32 : 1;  // 16x16x32 k-steps over features (d = 16 pads to 32)
    static constexpr int L = D * D + D;              // floats per summary vector
};

// CNT consecutive elements (bf16 or float) at byte offset `off`, as floats.
template <typename T, int CNT>
__device__ __forceinline__ void load_run(rsrc_t r, uint32_t off, float (&x)[CNT]) {
    constexpr int BYTES = CNT * (int)sizeof(T);
    constexpr int WORDS = BYTES >= 4 ? BYTES / 4 : 1;
    uint32_t w[WORDS];
    if constexpr (BYTES >= 16) {
#pragma unroll
        for (int h = 0; h < BYTES / 16; ++h) {
            const u32x4 v = buf_load128(r, off + 16 * h);
            w[4 * h] = v.x;
            w[4 * h + 1] = v.y;
            w[4 * h + 2] = v.z;
            w[4 * h + 3] = v.w;
        }
    } else if constexpr (BYTES == 8) {
        const u32x2 v = buf_load64(r, off);
        w[0] = v.x;
        w[1] = v.y;
    } else if constexpr (BYTES == 4) {
        w[0] = buf_load32(r, off);
    } else {
        w[0] = buf_load16(r, off);
    }
#pragma unroll
    for (int c = 0; c < CNT; ++c) {
        if constexpr (std::is_same<T, float>::value)
            x[c] = __uint_as_float(w[c]);
        else
            x[c] = __uint_as_float((c & 1) ? (w[c >> 1] & 0xffff0000u) : (w[c >> 1] << 16));
    }
}

// load_run in two halves: the loads (raw words, kept in registers) and, later, the
// conversion to floats, so that a tile's loads can be issued a whole tile ahead.
template <typename T, int CNT>
struct RawRun {
    static constexpr int BYTES = CNT * (int)sizeof(T);
    static constexpr int WORDS = BYTES >= 4 ? BYTES / 4 : 1;
    uint32_t w[WORDS];
};

template <typename T, int CNT>
__device__ __forceinline__ void raw_load(rsrc_t r, uint32_t off, RawRun<T, CNT>& x) {
    constexpr int BYTES = RawRun<T, CNT>::BYTES;
    if constexpr (BYTES >= 16) {
#pragma unroll
        for (int h = 0; h < BYTES / 16; ++h) {
            const u32x4 v = buf_load128(r, off + 16 * h);
            x.w[4 * h] = v.x;
            x.w[4 * h + 1] = v.y;
            x.w[4 * h + 2] = v.z;
            x.w[4 * h + 3] = v.w;
        }
    } else if constexpr (BYTES == 8) {
        const u32x2 v = buf_load64(r, off);
        x.w[0] = v.x;
        x.w[1] = v.y;
    } else if constexpr (BYTES == 4) {
        x.w[0] = buf_load32(r, off);
    } else {
        x.w[0] = buf_load16(r, off);
    }
}

template <typename T, int CNT>
__device__ __forceinline__ void raw_cvt(const RawRun<T, CNT>& x, float (&y)[CNT]) {
#pragma unroll
    for (int c = 0; c < CNT; ++c) {
        if constexpr (std::is_same<T, float>::value)
            y[c] = __uint_as_float(x.w[c]);
        else
            y[c] = __uint_as_float((c & 1) ? (x.w[c >> 1] & 0xffff0000u) : (x.w[c >> 1] << 16));
    }
}

template <int CNT>
__device__ __forceinline__ void store_run(rsrc_t r, uint32_t off, const float (&x)[CNT]) {
    if constexpr (CNT == 4) {
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])}, r,
            (int)off, 0, 0);
    } else if constexpr (CNT == 2) {
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(x[0]), __float_as_uint(x[1])}, r, (int)off, 0, 0);
    } else {
        static_assert(CNT == 1, "runs of 1, 2 or 4 floats");
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x[0]), r, (int)off, 0, 0);
    }
}

// Descriptor over `rows` rows of width D starting at row `row0` of X.
template <typename T>
__device__ __forceinline__ rsrc_t tile_rsrc(const T* X, int64_t row0, int rows, int width) {
    return make_rsrc(X + row0 * width, (uint32_t)(rows * width * (int)sizeof(T)));
}

template <typename T, int D>
__device__ __forceinline__ void load_rl(rsrc_t r, int g, int n, float (&x)[D / 4]) {
    load_run<T, D / 4>(r, (uint32_t)((n * D + (D / 4) * g) * (int)sizeof(T)), x);
}

template <typename T, int D>
__device__ __forceinline__ void load_dl(rsrc_t r, int g, int n, float (&x)[4][D / 16]) {
    constexpr int P = D / 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) load_run<T, P>(r, (uint32_t)(((4 * g + i) * D + P * n) * (int)sizeof(T)), x[i]);
}

template <int D>
__device__ __forceinline__ void store_dl(rsrc_t r, int g, int n, int i, const float (&x)[D / 16]) {
    constexpr int P = D / 16;
    store_run<P>(r, (uint32_t)(((4 * g + i) * D + P * n) * 4), x);
}

// phi(x) = ELU(x) + 1 = max(x, 0) + exp(min(x, 0)) and its derivative, with the
// hardware exp2 (relative error about |x| 2^-24 + 1 ulp, far inside what the split
// products keep).  min(x, 0) is taken as x - max(x, 0), exact for finite x, so that
// a NaN input stays NaN (max(NaN, 0) is 0 under IEEE maxNum); relu0 as in common.hpp.
__device__ __forceinline__ float bexp(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }
__device__ __forceinline__ float phi_b(float x) {
    const float m = relu0(x);
    return m + bexp(x - m);
}
__device__ __forceinline__ float phi_grad(float x, float& dphi) {
    const float m = relu0(x);
    const float e = bexp(x - m);
    dphi = x > 0.f ? 1.f : e;
    return m + e;
}

// Row-layout values as 16x16x32 operands (slot 8ks + e = group-local feature); the
// hi + lo split is done two values at a time (split2_bf16).
template <int FL, int KS>
__device__ __forceinline__ void split_rl(const float (&x)[FL], bf16x8 (&hi)[KS], bf16x8 (&lo)[KS]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        uint32_t h[4], l[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int f = 8 * ks + 2 * e;
            if (f < FL) {
                split2_bf16(x[f], x[f + 1], h[e], l[e]);
            } else {
                h[e] = l[e] = 0u;
            }
        }
        hi[ks] = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
        lo[ks] = __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], l[2], l[3]});
    }
}

__device__ __forceinline__ void split4(float a, float b, float c, float d, bf16x4& hi, bf16x4& lo) {
    uint32_t h0, l0, h1, l1;
    split2_bf16(a, b, h0, l0);
    split2_bf16(c, d, h1, l1);
    hi = __builtin_bit_cast(bf16x4, u32x2{h0, h1});
    lo = __builtin_bit_cast(bf16x4, u32x2{l0, l1});
}

// Dot-layout values as 16x16x16 operands, one per feature block.
template <int P>
__device__ __forceinline__ void split_dl(const float (&x)[4][P], bf16x4 (&hi)[P], bf16x4 (&lo)[P]) {
#pragma unroll
    for (int b = 0; b < P; ++b) split4(x[0][b], x[1][b], x[2][b], x[3][b], hi[b], lo[b]);
}

__device__ __forceinline__ void split4(const f32x4& x, bf16x4& hi, bf16x4& lo) { split4(x[0], x[1], x[2], x[3], hi, lo); }

// The 8 B-operand slots of k-step ks, column block jb, from packed chunks of X: slot
// (ks, e) is X[FL*g + 8ks + e][P*n + jb], held in chunk (f % P, jb) at position f / P.
template <int P>
__device__ __forceinline__ void packed_slots(const f32x4 (&ch)[P * P], int ks, int jb, bf16x8& bh, bf16x8& bl) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int f = 8 * ks + 2 * e;
        if (f < 4 * P) {
            split2_bf16(ch[(f % P) * P + jb][f / P], ch[((f + 1) % P) * P + jb][(f + 1) / P], h[e], l[e]);
        } else {
            h[e] = l[e] = 0u;
        }
    }
    bh = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
    bl = __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], l[2], l[3]});
}

// B operands from packed chunks of X (all k-steps and column blocks).
template <int P, int KS>
__device__ __forceinline__ void packed_b(const f32x4 (&ch)[P * P], bf16x8 (&bh)[KS][P], bf16x8 (&bl)[KS][P]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int jb = 0; jb < P; ++jb) packed_slots<P>(ch, ks, jb, bh[ks][jb], bl[ks][jb]);
}

// acc[jb] += A (row layout, tokens along m) x X (packed B operands), column block jb
// = columns P*n + jb.  ALO: the A operand has a lo part (else it is exact in bf16).
template <int P, int KS, bool ALO>
__device__ __forceinline__ void gemm_rl(const bf16x8 (&ah)[KS], const bf16x8 (&al)[KS], const bf16x8 (&bh)[KS][P],
                                        const bf16x8 (&bl)[KS][P], f32x4 (&acc)[P]) {
#pragma unroll
    for (int jb = 0; jb < P; ++jb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            acc[jb] = mfma32(ah[ks], bh[ks][jb], acc[jb]);
            acc[jb] = mfma32(ah[ks], bl[ks][jb], acc[jb]);
            if constexpr (ALO) acc[jb] = mfma32(al[ks], bh[ks][jb], acc[jb]);
        }
}

// gemm_rl with the B operands built from packed float32 chunks of X one (k-step,
// column block) at a time, so that no full split copy of X is live.
template <int P, int KS, bool ALO>
__device__ __forceinline__ void gemm_packed(const bf16x8 (&ah)[KS], const bf16x8 (&al)[KS], const f32x4 (&ch)[P * P],
                                            f32x4 (&acc)[P]) {
#pragma unroll
    for (int jb = 0; jb < P; ++jb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            bf16x8 bh, bl;
            packed_slots<P>(ch, ks, jb, bh, bl);
            acc[jb] = mfma32(ah[ks], bh, acc[jb]);
            acc[jb] = mfma32(ah[ks], bl, acc[jb]);
            if constexpr (ALO) acc[jb] = mfma32(al[ks], bh, acc[jb]);
        }
}

// B operands of packed chunks of X, split once into LDS in lane order: entry (ks, jb,
// hi/lo) of lane l at sb[2 (ks P + jb) + hl][l].  The nw waves of the workgroup build
// the entries (ks P + jb) = w, w + nw, ... between them; a barrier must follow.
template <int P, int KS>
__device__ __forceinline__ void packed_b_lds(const f32x4 (&ch)[P * P], u32x4 (*sb)[64], int lane, int w, int nw) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int jb = 0; jb < P; ++jb)
            if ((ks * P + jb) % nw == w) {
                bf16x8 h, l;
                packed_slots<P>(ch, ks, jb, h, l);
                sb[2 * (ks * P + jb)][lane] = __builtin_bit_cast(u32x4, h);
                sb[2 * (ks * P + jb) + 1][lane] = __builtin_bit_cast(u32x4, l);
            }
}

// gemm_rl with the B operands read from LDS (laid out by packed_b_lds).
template <int P, int KS, bool ALO>
__device__ __forceinline__ void gemm_lds(const bf16x8 (&ah)[KS], const bf16x8 (&al)[KS], const u32x4 (*sb)[64],
                                         int lane, f32x4 (&acc)[P]) {
#pragma unroll
    for (int jb = 0; jb < P; ++jb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 bh = __builtin_bit_cast(bf16x8, sb[2 * (ks * P + jb)][lane]);
            const bf16x8 bl = __builtin_bit_cast(bf16x8, sb[2 * (ks * P + jb) + 1][lane]);
            acc[jb] = mfma32(ah[ks], bh, acc[jb]);
            acc[jb] = mfma32(ah[ks], bl, acc[jb]);
            if constexpr (ALO) acc[jb] = mfma32(al[ks], bh, acc[jb]);
        }
}

// acc (packed chunks of X) += sum over the tile's tokens of a_t b_t^T, X[r][c] with
// r from the A side and c from the B side (both in dot layout).
template <int P, bool ALO>
__device__ __forceinline__ void acc_outer(const bf16x4 (&ah)[P], const bf16x4 (&al)[P], const bf16x4 (&bh)[P],
                                          const bf16x4 (&bl)[P], f32x4 (&acc)[P * P]) {
#pragma unroll
    for (int ia = 0; ia < P; ++ia)
#pragma unroll
        for (int ib = 0; ib < P; ++ib) {
            f32x4 c = acc[ia * P + ib];
            c = mfma16(ah[ia], bh[ib], c);
            c = mfma16(ah[ia], bl[ib], c);
            if constexpr (ALO) c = mfma16(al[ia], bh[ib], c);
            acc[ia * P + ib] = c;
        }
}

// Sum over the 16 lanes of a lane group.
__device__ __forceinline__ float sum16(float x) {
    x += __shfl_xor(x, 1, 64);
    x += __shfl_xor(x, 2, 64);
    x += __shfl_xor(x, 4, 64);
    x += __shfl_xor(x, 8, 64);
    return x;
}

template <int P>
__device__ __forceinline__ void load_packed(const float* X, int lane, f32x4 (&ch)[P * P]) {
#pragma unroll
    for (int c = 0; c < P * P; ++c) ch[c] = *reinterpret_cast<const f32x4*>(X + c * 256 + lane * 4);
}

// Packed chunks of Y = X^T from the packed X: chunk (ia, ib) position i of lane (g, n)
// is Y[P(4g + i) + ia][Pn + ib] = X[Pn + ib][P(4g + i) + ia].
template <int P>
__device__ __forceinline__ void load_packed_t(const float* X, int g, int n, f32x4 (&ch)[P * P]) {
#pragma unroll
    for (int ia = 0; ia < P; ++ia)
#pragma unroll
        for (int ib = 0; ib < P; ++ib)
#pragma unroll
            for (int i = 0; i < 4; ++i) ch[ia * P + ib][i] = X[packed_index(P, P * n + ib, P * (4 * g + i) + ia)];
}

template <int P>
__device__ __forceinline__ void store_packed(float* X, int lane, int g, int n, const f32x4 (&ch)[P * P],
                                             const float (&z)[P]) {
    constexpr int D = 16 * P;
#pragma unroll
    for (int c = 0; c < P * P; ++c) *reinterpret_cast<f32x4*>(X + c * 256 + lane * 4) = ch[c];
    if (g == 0)
#pragma unroll
        for (int b = 0; b < P; ++b) X[D * D + P * n + b] = z[b];
}

// Adds the partial summaries of the `wpu` waves of a workgroup into wave 0, pairwise
// through LDS in a fixed order.  z must already be summed over the lane groups.
template <int P>
__device__ void reduce_waves(f32x4 (&acc)[P * P], float (&z)[P], float* lds, int wave, int wpu, int lane, int g,
                             int n) {
    constexpr int D = 16 * P, L = D * D + D;
    for (int s = wpu >> 1; s >= 1; s >>= 1) {
        if (wave >= s && wave < 2 * s) {
            float* dst = lds + (wave - s) * L;
#pragma unroll
            for (int c = 0; c < P * P; ++c) *reinterpret_cast<f32x4*>(dst + c * 256 + lane * 4) = acc[c];
            if (g == 0)
#pragma unroll
                for (int b = 0; b < P; ++b) dst[D * D + P * n + b] = z[b];
        }
        __syncthreads();
        if (wave < s) {
            const float* src = lds + wave * L;
#pragma unroll
            for (int c = 0; c < P * P; ++c) acc[c] += *reinterpret_cast<const f32x4*>(src + c * 256 + lane * 4);
#pragma unroll
            for (int b = 0; b < P; ++b) z[b] += src[D * D + P * n + b];
        }
        __syncthreads();
    }
}

}  // namespace

// S_b^T, z_b (packed, transposed) for one (pair, block) per workgroup of wpu waves.
template <int D, typename T>
__global__ __launch_bounds__(256) void bwd_sum_kernel(const T* __restrict__ K, const T* __restrict__ V,
                                                      float* __restrict__ S, int64_t BH, int N, int M, int wpu) {
    using Dm = Dim<D>;
    constexpr int P = Dm::P, L = Dm::L;
    constexpr bool VLO = !std::is_same<T, uint16_t>::value;  // bf16 inputs are exact bf16 operands
    extern __shared__ float red[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, n = lane & 15;
    const int64_t unit = blockIdx.x, pair = unit / M;
    const int blk = (int)(unit % M), C = N / M;
    const int64_t row0 = pair * N + (int64_t)blk * C;
    const int ntiles = (C + 15) / 16;
    f32x4 acc[P * P];
    float z[P];
#pragma unroll
    for (int c = 0; c < P * P; ++c) acc[c] = zero4();
#pragma unroll
    for (int b = 0; b < P; ++b) z[b] = 0.f;
    for (int tile = wave; tile < ntiles; tile += wpu) {
        const int t0 = 16 * tile, rows = min(16, C - t0);
        const rsrc_t rk = tile_rsrc(K, row0 + t0, rows, D), rv = tile_rsrc(V, row0 + t0, rows, D);
        float kx[4][P], vx[4][P];
        load_dl<T, D>(rk, g, n, kx);
        load_dl<T, D>(rv, g, n, vx);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int b = 0; b < P; ++b) {
                kx[i][b] = 4 * g + i < rows ? phi_b(kx[i][b]) : 0.f;
                z[b] += kx[i][b];
            }
        bf16x4 kh[P], kl[P], vh[P], vl[P];
        split_dl<P>(kx, kh, kl);
        split_dl<P>(vx, vh, vl);
        acc_outer<P, VLO>(vh, vl, kh, kl, acc);
    }
#pragma unroll
    for (int b = 0; b < P; ++b) z[b] = sum_over_groups(z[b]);
    if (wpu > 1) reduce_waves<P>(acc, z, red, wave, wpu, lane, g, n);
    if (wave == 0) store_packed<P>(S + ((int64_t)blk * BH + pair) * L, lane, g, n, acc, z);
}

// dq and dS~_i^T, dz~_i for one (pair, block i) per workgroup of wpu waves (non-causal).
template <int D, typename T>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void bwd_query_kernel(const T* __restrict__ Q, const float* __restrict__ dY,
                                                        const float* __restrict__ St, float* __restrict__ dQ,
                                                        float* __restrict__ dSt, int64_t BH, int N, int M, int wpu,
                                                        int norm) {
    using Dm = Dim<D>;
    constexpr int P = Dm::P, FL = Dm::FL, KS = Dm::KS, L = Dm::L;
    extern __shared__ float red[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, n = lane & 15;
    const int64_t unit = blockIdx.x, pair = unit / M;
    const int blk = (int)(unit % M), C = N / M;
    const int64_t row0 = pair * N + (int64_t)blk * C;
    const int ntiles = (C + 15) / 16;

    const float* sv = St + ((int64_t)blk * BH + pair) * L;
    __shared__ u32x4 sb[2 * KS * P][64];  // B[k = c][col = r] = S~[r][c], shared by the waves
    float zt[P];
    {
        f32x4 ch[P * P];
        load_packed<P>(sv, lane, ch);
        packed_b_lds<P, KS>(ch, sb, lane, wave, wpu);
#pragma unroll
        for (int b = 0; b < P; ++b) zt[b] = sv[D * D + P * n + b];
    }
    __syncthreads();
    f32x4 acc[P * P];
    float zacc[P];
#pragma unroll
    for (int c = 0; c < P * P; ++c) acc[c] = zero4();
#pragma unroll
    for (int b = 0; b < P; ++b) zacc[b] = 0.f;

    // For d <= 32 the tile's operands are loaded one tile ahead as raw words (at d = 64
    // the registers for them would push the kernel below three waves per SIMD).
    constexpr bool PRE = D <= 32;
    RawRun<float, FL> pyr;
    RawRun<float, P> pyd[4];
    RawRun<T, P> pqd[4];
    auto prefetch = [&](int tile) {
        const int t0 = 16 * tile, rows = min(16, C - t0);
        const rsrc_t rq = tile_rsrc(Q, row0 + t0, rows, D), ry = tile_rsrc(dY, row0 + t0, rows, D);
        raw_load<float, FL>(ry, (uint32_t)((n * D + FL * g) * 4), pyr);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            raw_load<float, P>(ry, (uint32_t)(((4 * g + i) * D + P * n) * 4), pyd[i]);
            raw_load<T, P>(rq, (uint32_t)(((4 * g + i) * D + P * n) * (int)sizeof(T)), pqd[i]);
        }
    };
    if constexpr (PRE) {
        if (wave < ntiles) prefetch(wave);
    }
    for (int tile = wave; tile < ntiles; tile += wpu) {
        const int t0 = 16 * tile, rows = min(16, C - t0);
        const rsrc_t rdq = tile_rsrc(dQ, row0 + t0, rows, D);
        float yr[FL], yd[4][P], qd[4][P];
        if constexpr (PRE) {
            raw_cvt<float, FL>(pyr, yr);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                raw_cvt<float, P>(pyd[i], yd[i]);
                raw_cvt<T, P>(pqd[i], qd[i]);
            }
            if (tile + wpu < ntiles) prefetch(tile + wpu);
        } else {
            const rsrc_t rq = tile_rsrc(Q, row0 + t0, rows, D), ry = tile_rsrc(dY, row0 + t0, rows, D);
            load_rl<float, D>(ry, g, n, yr);
            load_dl<float, D>(ry, g, n, yd);
            load_dl<T, D>(rq, g, n, qd);
        }
        bf16x8 yh[KS], yl[KS];
        split_rl<FL, KS>(yr, yh, yl);
        f32x4 u[P];  // U[4g + i][Pn + jb] = (S~_i dy_t)[r]
#pragma unroll
        for (int jb = 0; jb < P; ++jb) u[jb] = zero4();
        gemm_lds<P, KS, true>(yh, yl, sb, lane, u);

        float fq[4][P], dp[4][P], dn[4][P], dden[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float den = 0.f, dyn = 0.f;
#pragma unroll
            for (int b = 0; b < P; ++b) {
                fq[i][b] = phi_grad(qd[i][b], dp[i][b]);
                den = fmaf(fq[i][b], zt[b], den);
                dyn = fmaf(fq[i][b], u[b][i], dyn);
            }
            den = sum16(den) + kEps;
            dyn = sum16(dyn);
            // without the normaliser y = num: dnum = dy, no den terms
            const float rden = norm ? fast_rcp(den) : 1.f;
            dden[i] = norm ? -dyn * rden * rden : 0.f;
            float out[P];
#pragma unroll
            for (int b = 0; b < P; ++b) {
                out[b] = fmaf(u[b][i], rden, dden[i] * zt[b]) * dp[i][b];
                dn[i][b] = yd[i][b] * rden;
            }
            store_dl<D>(rdq, g, n, i, out);
        }
        bf16x4 nh[P], nl[P], qh[P], ql[P];
        split_dl<P>(dn, nh, nl);
        split_dl<P>(fq, qh, ql);
        acc_outer<P, true>(nh, nl, qh, ql, acc);  // dS~^T[c][r] += dnum[c] phi(q)[r]
#pragma unroll
        for (int b = 0; b < P; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) zacc[b] = fmaf(dden[i], fq[i][b], zacc[b]);
    }
#pragma unroll
    for (int b = 0; b < P; ++b) zacc[b] = sum_over_groups(zacc[b]);
    if (wpu > 1) reduce_waves<P>(acc, zacc, red, wave, wpu, lane, g, n);
    if (wave == 0) store_packed<P>(dSt + ((int64_t)blk * BH + pair) * L, lane, g, n, acc, zacc);
}

// dk, dv for one (pair, key block b) from dS_b^T, dz_b (non-causal); waves of the
// workgroup take the block's tiles in turn.
template <int D, typename T, bool SHARED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void bwd_key_kernel(const T* __restrict__ K, const T* __restrict__ V,
                                                      const float* __restrict__ dS, float* __restrict__ dK,
                                                      float* __restrict__ dV, int64_t BH, int N, int M, int wpu) {
    using Dm = Dim<D>;
    constexpr int P = Dm::P, FL = Dm::FL, KS = Dm::KS, L = Dm::L;
    constexpr bool VLO = !std::is_same<T, uint16_t>::value;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, n = lane & 15;
    const int64_t unit = blockIdx.x, pair = unit / M;
    const int blk = (int)(unit % M), C = N / M;
    const int64_t row0 = pair * N + (int64_t)blk * C;
    const int ntiles = (C + 15) / 16;

    // The B operands of dS in both orientations: per wave in registers, or (SHARED, when
    // several waves share the block) split once into LDS for all of them.
    const float* sv = dS + ((int64_t)blk * BH + pair) * L;
    bf16x8 b1h[SHARED ? 1 : KS][P], b1l[SHARED ? 1 : KS][P];  // B[k = c][col = r] = dS[r][c]  (d phi(k))
    bf16x8 b2h[SHARED ? 1 : KS][P], b2l[SHARED ? 1 : KS][P];  // B[k = r][col = c] = dS[r][c]  (dv)
    __shared__ u32x4 sb1[SHARED ? 2 * KS * P : 1][64], sb2[SHARED ? 2 * KS * P : 1][64];
    float dz[P];
    {
        f32x4 ch[P * P];
        load_packed<P>(sv, lane, ch);
        if constexpr (SHARED) packed_b_lds<P, KS>(ch, sb1, lane, wave, wpu);
        else packed_b<P, KS>(ch, b1h, b1l);
        load_packed_t<P>(sv, g, n, ch);
        if constexpr (SHARED) packed_b_lds<P, KS>(ch, sb2, lane, wave, wpu);
        else packed_b<P, KS>(ch, b2h, b2l);
#pragma unroll
        for (int b = 0; b < P; ++b) dz[b] = sv[D * D + P * n + b];
    }
    if constexpr (SHARED) __syncthreads();
    if (wave >= ntiles) return;  // no barriers past this point
    // The tile's k and v are loaded one tile ahead as raw words (not for float32 inputs
    // at d = 64, where their registers would spill).
    constexpr bool PRE = D <= 32 || !VLO;
    RawRun<T, FL> pvr, pkr;
    RawRun<T, P> pkd[4];
    auto prefetch = [&](int tile) {
        const int t0 = 16 * tile, rows = min(16, C - t0);
        const rsrc_t rk = tile_rsrc(K, row0 + t0, rows, D), rv = tile_rsrc(V, row0 + t0, rows, D);
        raw_load<T, FL>(rv, (uint32_t)((n * D + FL * g) * (int)sizeof(T)), pvr);
        raw_load<T, FL>(rk, (uint32_t)((n * D + FL * g) * (int)sizeof(T)), pkr);
#pragma unroll
        for (int i = 0; i < 4; ++i) raw_load<T, P>(rk, (uint32_t)(((4 * g + i) * D + P * n) * (int)sizeof(T)), pkd[i]);
    };
    if constexpr (PRE) prefetch(wave);
    for (int tile = wave; tile < ntiles; tile += wpu) {
        const int t0 = 16 * tile, rows = min(16, C - t0);
        const rsrc_t rdk = tile_rsrc(dK, row0 + t0, rows, D), rdv = tile_rsrc(dV, row0 + t0, rows, D);
        float vr[FL], kr[FL], kd[4][P];
        if constexpr (PRE) {
            raw_cvt<T, FL>(pvr, vr);
            raw_cvt<T, FL>(pkr, kr);
#pragma unroll
            for (int i = 0; i < 4; ++i) raw_cvt<T, P>(pkd[i], kd[i]);
            if (tile + wpu < ntiles) prefetch(tile + wpu);
        } else {
            const rsrc_t rk = tile_rsrc(K, row0 + t0, rows, D), rv = tile_rsrc(V, row0 + t0, rows, D);
            load_rl<T, D>(rv, g, n, vr);
            load_rl<T, D>(rk, g, n, kr);
            load_dl<T, D>(rk, g, n, kd);
        }
#pragma unroll
        for (int f = 0; f < FL; ++f) kr[f] = phi_b(kr[f]);
        bf16x8 vh[KS], vl[KS], kh[KS], kl[KS];
        split_rl<FL, KS>(vr, vh, vl);
        split_rl<FL, KS>(kr, kh, kl);
        f32x4 a1[P], a2[P];
#pragma unroll
        for (int b = 0; b < P; ++b) a1[b] = a2[b] = zero4();
        if constexpr (SHARED) {
            gemm_lds<P, KS, VLO>(vh, vl, sb1, lane, a1);
            gemm_lds<P, KS, true>(kh, kl, sb2, lane, a2);
        } else {
            gemm_rl<P, KS, VLO>(vh, vl, b1h, b1l, a1);
            gemm_rl<P, KS, true>(kh, kl, b2h, b2l, a2);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float ok[P], ov[P];
#pragma unroll
            for (int b = 0; b < P; ++b) {
                float dp;
                phi_grad(kd[i][b], dp);
                ok[b] = (a1[b][i] + dz[b]) * dp;
                ov[b] = a2[b][i];
            }
            store_dl<D>(rdk, g, n, i, ok);
            store_dl<D>(rdv, g, n, i, ov);
        }
    }
}

// Causal, CP waves per (pair, query block i) (CP = 2 for d >= 32, else 1), tiles in
// order.  Wave w owns the feature blocks b = w*P/CP .. (w+1)*P/CP - 1 (features P*n + b
// of lane n): those columns of U_t = A_t dy_t and dq, those columns of the running
// P^T of the earlier tiles, of dS~_i^T and of dz~_i.  The per-row sums over all
// features (den_t, phi(q_t).U_t and the within-block parts that dW[i,i] needs) are
// formed from the waves' partial sums, exchanged through LDS (one barrier per tile,
// double-buffered, added in wave order).  The constant S~_i^T is split once into
// per-lane B operands kept in LDS.  Inside a tile the masked scores (v_j . dy_t,
// j <= t) carry the rest of P_t dy_t.  Wave 0 also stores (den_t, dden_t) per token
// for the key pass and the block's part of dW[i,i].
template <int D>
struct QcShared {
    static constexpr int P = D / 16, KS = D >= 32 ? D / 32 : 1, CP = P >= 2 ? 2 : 1, PH = P / CP;
    u32x4 sb[2 * KS * PH][CP][64];  // S~_i B operands of each wave's column blocks
    float xch[2][CP][4][16];        // [tile parity][wave][quantity][row]
};

// The body of wave w (a template parameter, so that the owned blocks index registers
// statically).
template <int D, typename T, int w>
__device__ __forceinline__ void query_causal_wave(const T* __restrict__ Q, const T* __restrict__ K,
                                                  const T* __restrict__ V, const float* __restrict__ dY,
                                                  const float* __restrict__ W, const float* __restrict__ St,
                                                  float* __restrict__ dQ, float* __restrict__ dSt,
                                                  float* __restrict__ G, float* __restrict__ dWdiag, int64_t BH,
                                                  int N, int M, int norm, QcShared<D>& sh) {
    using Dm = Dim<D>;
    constexpr int P = Dm::P, FL = Dm::FL, KS = Dm::KS, L = Dm::L;
    constexpr int CP = QcShared<D>::CP, PH = QcShared<D>::PH;
    constexpr bool VLO = !std::is_same<T, uint16_t>::value;
    auto& sb = sh.sb;
    auto& xch = sh.xch;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, n = lane & 15;
    const int64_t unit = blockIdx.x, pair = unit / M;
    const int blk = (int)(unit % M), C = N / M;
    const int64_t row0 = pair * N + (int64_t)blk * C;
    const int ntiles = (C + 15) / 16;
    const float wii = W[(int64_t)blk * M + blk];
    constexpr int b0 = w * PH;  // first owned feature block

    const float* sv = St + ((int64_t)blk * BH + pair) * L;
    float zt[PH];
    {
        f32x4 ch[P * P];
        load_packed<P>(sv, lane, ch);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int j = 0; j < PH; ++j) {
                bf16x8 h, l;
                packed_slots<P>(ch, ks, b0 + j, h, l);
                sb[2 * (ks * PH + j)][w][lane] = __builtin_bit_cast(u32x4, h);
                sb[2 * (ks * PH + j) + 1][w][lane] = __builtin_bit_cast(u32x4, l);
            }
#pragma unroll
        for (int j = 0; j < PH; ++j) zt[j] = sv[D * D + P * n + b0 + j];
    }
    f32x4 pt[P * PH], acc[P * PH];  // chunks (ia, b0 + j) at [ia * PH + j]
    float pz[PH], zacc[PH], dwl = 0.f;
#pragma unroll
    for (int c = 0; c < P * PH; ++c) pt[c] = acc[c] = zero4();
#pragma unroll
    for (int j = 0; j < PH; ++j) pz[j] = zacc[j] = 0.f;
    __syncthreads();

    // The tile's first operands (dy and v in row layout, k and q in dot layout) are
    // loaded one tile ahead, as raw words, and converted when the tile starts.
    RawRun<float, FL> pyr;
    RawRun<T, FL> pvr;
    RawRun<T, P> pkd[4], pqd[4];
    auto prefetch = [&](int tile) {
        const int t0 = 16 * tile, rows = min(16, C - t0);
        const int64_t r0 = row0 + t0;
        const rsrc_t rq = tile_rsrc(Q, r0, rows, D), rk = tile_rsrc(K, r0, rows, D), rv = tile_rsrc(V, r0, rows, D);
        const rsrc_t ry = tile_rsrc(dY, r0, rows, D);
        raw_load<float, FL>(ry, (uint32_t)((n * D + FL * g) * 4), pyr);
        raw_load<T, FL>(rv, (uint32_t)((n * D + FL * g) * (int)sizeof(T)), pvr);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            raw_load<T, P>(rk, (uint32_t)(((4 * g + i) * D + P * n) * (int)sizeof(T)), pkd[i]);
            raw_load<T, P>(rq, (uint32_t)(((4 * g + i) * D + P * n) * (int)sizeof(T)), pqd[i]);
        }
    };
    prefetch(0);
    for (int tile = 0; tile < ntiles; ++tile) {
        const int t0 = 16 * tile, rows = min(16, C - t0);
        const int64_t r0 = row0 + t0;
        const rsrc_t rv = tile_rsrc(V, r0, rows, D);
        const rsrc_t ry = tile_rsrc(dY, r0, rows, D);
        float yr[FL], vr[FL], kd[4][P], qd[4][P];
        raw_cvt<float, FL>(pyr, yr);
        raw_cvt<T, FL>(pvr, vr);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            raw_cvt<T, P>(pkd[i], kd[i]);
            raw_cvt<T, P>(pqd[i], qd[i]);
        }
        if (tile + 1 < ntiles) prefetch(tile + 1);

        bf16x8 yh[KS], yl[KS];
        split_rl<FL, KS>(yr, yh, yl);
        f32x4 ui[PH], us[PH];  // S~_i dy_t and P_t dy_t (owned columns), dot layout
#pragma unroll
        for (int j = 0; j < PH; ++j) ui[j] = us[j] = zero4();
#pragma unroll
        for (int j = 0; j < PH; ++j)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 bh = __builtin_bit_cast(bf16x8, sb[2 * (ks * PH + j)][w][lane]);
                const bf16x8 bl = __builtin_bit_cast(bf16x8, sb[2 * (ks * PH + j) + 1][w][lane]);
                ui[j] = mfma32(yh[ks], bh, ui[j]);
                ui[j] = mfma32(yh[ks], bl, ui[j]);
                ui[j] = mfma32(yl[ks], bh, ui[j]);
            }
        // P_{<tile} dy_t: B slot (ks, e) of column block b0 + j is P^T[FL g + 8ks + e][P n + b0 + j],
        // held in chunk ((8ks + e) % P, b0 + j) at position (8ks + e) / P
#pragma unroll
        for (int j = 0; j < PH; ++j)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                uint32_t h[4], l[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int f = 8 * ks + 2 * e;
                    if (f < FL) {
                        split2_bf16(pt[(f % P) * PH + j][f / P], pt[((f + 1) % P) * PH + j][(f + 1) / P], h[e], l[e]);
                    } else {
                        h[e] = l[e] = 0u;
                    }
                }
                const bf16x8 bh = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
                const bf16x8 bl = __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], l[2], l[3]});
                us[j] = mfma32(yh[ks], bh, us[j]);
                us[j] = mfma32(yh[ks], bl, us[j]);
                us[j] = mfma32(yl[ks], bh, us[j]);
            }
        // scores v_j . dy_t: lane (g, n) holds j = 4g + e, t = n, kept for j <= t
        f32x4 gy = zero4();
        {
            bf16x8 vh[KS], vl[KS];
            split_rl<FL, KS>(vr, vh, vl);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                gy = mfma32(vh[ks], yh[ks], gy);
                gy = mfma32(vh[ks], yl[ks], gy);
                if constexpr (VLO) gy = mfma32(vl[ks], yh[ks], gy);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) gy[e] = 4 * g + e <= n ? gy[e] : 0.f;
        }
        float fk[4][P];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int b = 0; b < P; ++b) fk[i][b] = 4 * g + i < rows ? phi_b(kd[i][b]) : 0.f;
        bf16x4 kh[P], kl[P];
        split_dl<P>(fk, kh, kl);
        {
            bf16x4 gh, gl;
            split4(gy, gh, gl);
#pragma unroll
            for (int j = 0; j < PH; ++j) {  // us += sum_{j' <= t in tile} (v_j' . dy_t) phi(k_j')
                us[j] = mfma16(gh, kh[b0 + j], us[j]);
                us[j] = mfma16(gh, kl[b0 + j], us[j]);
                us[j] = mfma16(gl, kh[b0 + j], us[j]);
            }
        }
        // p_t = the block's phi(k) sum up to and including t (owned features)
        float pin[4][PH];
#pragma unroll
        for (int j = 0; j < PH; ++j) {
            float run = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                run += fk[i][b0 + j];
                pin[i][j] = run;
            }
            float excl = 0.f;
#pragma unroll
            for (int h = 0; h < 3; ++h) {
                const float t = __shfl(run, 16 * h + n, 64);
                excl += h < g ? t : 0.f;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) pin[i][j] += pz[j] + excl;
            pz[j] += sum_over_groups(run);
        }

        // per-row partial sums over the owned features, exchanged between the waves
        float fq[4][PH], dp[4][PH], part[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float den = 0.f, idn = 0.f, dyn = 0.f, idy = 0.f;
#pragma unroll
            for (int j = 0; j < PH; ++j) {
                fq[i][j] = phi_grad(qd[i][b0 + j], dp[i][j]);
                const float a = fmaf(wii, pin[i][j], zt[j]);
                const float uu = fmaf(wii, us[j][i], ui[j][i]);
                den = fmaf(fq[i][j], a, den);
                idn = fmaf(fq[i][j], pin[i][j], idn);
                dyn = fmaf(fq[i][j], uu, dyn);
                idy = fmaf(fq[i][j], us[j][i], idy);
            }
            part[0][i] = sum16(den);
            part[1][i] = sum16(idn);
            part[2][i] = sum16(dyn);
            part[3][i] = sum16(idy);
        }
        float tot[4][4];
        if constexpr (CP == 2) {
            float(*x)[4][16] = xch[tile & 1];
            if (n == 0)
#pragma unroll
                for (int qn = 0; qn < 4; ++qn)
#pragma unroll
                    for (int i = 0; i < 4; ++i) x[w][qn][4 * g + i] = part[qn][i];
            __syncthreads();
#pragma unroll
            for (int qn = 0; qn < 4; ++qn)
#pragma unroll
                for (int i = 0; i < 4; ++i) tot[qn][i] = x[0][qn][4 * g + i] + x[1][qn][4 * g + i];
        } else {
#pragma unroll
            for (int qn = 0; qn < 4; ++qn)
#pragma unroll
                for (int i = 0; i < 4; ++i) tot[qn][i] = part[qn][i];
        }
        const rsrc_t rdq = tile_rsrc(dQ, r0, rows, D), rg = tile_rsrc(G, r0, rows, 2);
        float yd[4][P], dn[4][P], dden[4];
        load_dl<float, D>(ry, g, n, yd);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // without the normaliser: den = 1 (stored, so that the key kernel's dnum = dy), dden = 0
            const float den = norm ? tot[0][i] + kEps : 1.f;
            const float rden = norm ? fast_rcp(den) : 1.f;
            dden[i] = norm ? -tot[2][i] * rden * rden : 0.f;
            float out[PH];
#pragma unroll
            for (int j = 0; j < PH; ++j) {
                const float a = fmaf(wii, pin[i][j], zt[j]);
                const float uu = fmaf(wii, us[j][i], ui[j][i]);
                out[j] = fmaf(uu, rden, dden[i] * a) * dp[i][j];
            }
#pragma unroll
            for (int b = 0; b < P; ++b) dn[i][b] = yd[i][b] * rden;
            store_run<PH>(rdq, (uint32_t)(((4 * g + i) * D + P * n + b0) * 4), out);
            if (w == 0 && n == 0) {
                dwl += fmaf(tot[3][i], rden, dden[i] * tot[1][i]);
                const float gd[2] = {den, dden[i]};
                store_run<2>(rg, (uint32_t)((4 * g + i) * 8), gd);
            }
        }
        {  // dS~^T chunks (ia, b0 + j) += dnum[c] phi(q)[r]
            bf16x4 nh[P], nl[P];
            split_dl<P>(dn, nh, nl);
#pragma unroll
            for (int j = 0; j < PH; ++j) {
                bf16x4 qh, ql;
                split4(fq[0][j], fq[1][j], fq[2][j], fq[3][j], qh, ql);
#pragma unroll
                for (int ia = 0; ia < P; ++ia) {
                    f32x4 c = acc[ia * PH + j];
                    c = mfma16(nh[ia], qh, c);
                    c = mfma16(nh[ia], ql, c);
                    c = mfma16(nl[ia], qh, c);
                    acc[ia * PH + j] = c;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) zacc[j] = fmaf(dden[i], fq[i][j], zacc[j]);
            }
        }
        {  // P^T chunks (ia, b0 + j) += v[c] phi(k)[r] over this tile
            float vd[4][P];
            load_dl<T, D>(rv, g, n, vd);
            bf16x4 vh[P], vl[P];
            split_dl<P>(vd, vh, vl);
#pragma unroll
            for (int j = 0; j < PH; ++j)
#pragma unroll
                for (int ia = 0; ia < P; ++ia) {
                    f32x4 c = pt[ia * PH + j];
                    c = mfma16(vh[ia], kh[b0 + j], c);
                    c = mfma16(vh[ia], kl[b0 + j], c);
                    if constexpr (VLO) c = mfma16(vl[ia], kh[b0 + j], c);
                    pt[ia * PH + j] = c;
                }
        }
    }
    float* out = dSt + ((int64_t)blk * BH + pair) * L;
#pragma unroll
    for (int ia = 0; ia < P; ++ia)
#pragma unroll
        for (int j = 0; j < PH; ++j)
            *reinterpret_cast<f32x4*>(out + (ia * P + b0 + j) * 256 + lane * 4) = acc[ia * PH + j];
#pragma unroll
    for (int j = 0; j < PH; ++j) {
        const float z = sum_over_groups(zacc[j]);
        if (g == 0) out[D * D + P * n + b0 + j] = z;
    }
    if constexpr (w == 0) {
        dwl = sum_over_groups(sum16(dwl));
        if (lane == 0) dWdiag[pair * M + blk] = dwl;
    }
}

template <int D, typename T>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2))) void bwd_query_causal_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, const float* __restrict__ dY,
    const float* __restrict__ W, const float* __restrict__ St, float* __restrict__ dQ, float* __restrict__ dSt,
    float* __restrict__ G, float* __restrict__ dWdiag, int64_t BH, int N, int M, int norm) {
    __shared__ QcShared<D> sh;
    if (threadIdx.x < 64)
        query_causal_wave<D, T, 0>(Q, K, V, dY, W, St, dQ, dSt, G, dWdiag, BH, N, M, norm, sh);
    else if constexpr (QcShared<D>::CP == 2)
        query_causal_wave<D, T, 1>(Q, K, V, dY, W, St, dQ, dSt, G, dWdiag, BH, N, M, norm, sh);
}

// Causal query side in the token-level form, for blocks of an even number of whole
// 16-token tiles (C <= CMAX).  With A_t = S~_i + W[i,i] P_t (P_t: the block's phi(k) v^T
// up to and including t), the within-block parts of U_t = A_t dy_t and of the normaliser
// a_t = z~_i + W[i,i] p_t are sums over keys j <= t of the block,
//
//   P_t dy_t = sum_{j <= t} g_tj phi(k_j),  g_tj = v_j . dy_t,    p_t = sum_{j <= t} phi(k_j),
//   phi(q_t).P_t dy_t = sum_{j <= t} s_tj g_tj,  phi(q_t).p_t = sum_{j <= t} s_tj,  s_tj = phi(q_t).phi(k_j),
//
// formed as masked products over the block's key tiles rather than by carrying P_t tile
// by tile, so that the block's query tiles are independent.  One workgroup of four waves
// per (pair, block): phi(K) hi/lo, V and S~_i hi/lo (row-major [r][c]) in LDS; wave w
// takes the query tiles of its snake slots.  Per tile, in the transposed layout (features
// 16F + 4g + i of query n): U^T = S~ dy^T + sum_j W g phi(k_j) and p^T (the masked product
// with ones); den, dden, dq.  A second loop over the same tiles then adds, in the dot
// layout of the other kernels, the tiles' parts of dS~_i^T = sum_t phi(q_t) dnum_t^T and
// dz~_i (so that their accumulators do not share registers with the first loop's), and
// the waves' parts are added in a fixed order at the end.  Outputs as bwd_query_causal_kernel: dq, dS~^T and dz~ of
// the block, (den, dden) per token, and the block's part of dW[i,i].
// Eight float32 values (k-slots 0-3 from a, 4-7 from b) as bf16 hi and lo operands.
__device__ __forceinline__ void split_pair8(const f32x4& a, const f32x4& b, bf16x8& h, bf16x8& l) {
    uint32_t hh[4], ll[4];
    split2_bf16(a[0], a[1], hh[0], ll[0]);
    split2_bf16(a[2], a[3], hh[1], ll[1]);
    split2_bf16(b[0], b[1], hh[2], ll[2]);
    split2_bf16(b[2], b[3], hh[3], ll[3]);
    h = __builtin_bit_cast(bf16x8, u32x4{hh[0], hh[1], hh[2], hh[3]});
    l = __builtin_bit_cast(bf16x8, u32x4{ll[0], ll[1], ll[2], ll[3]});
}

template <int D, int CMAX>
struct QcTl {
    static constexpr int P = D / 16, KS = D / 32, CPR = D / 8;
    static constexpr int kPlane = CMAX * D * 2;  // one bf16 [CMAX][D] plane
    static constexpr int kSt = D * D * 2;        // one bf16 [D][D] plane
    // phi(K) hi, phi(K) lo, V, S~ hi, S~ lo, z~ (D floats), per-wave dW parts (4 floats)
    static constexpr int kBytes = 3 * kPlane + 2 * kSt + D * 4 + 16;
};

template <int D, int CMAX>
__global__ __launch_bounds__(256) void bwd_query_causal_tl_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const float* __restrict__ dY, const float* __restrict__ W, const float* __restrict__ St, float* __restrict__ dQ,
    float* __restrict__ dSt, float* __restrict__ G, float* __restrict__ dWdiag, int64_t BH, int N, int M, int norm) {
    using Cf = QcTl<D, CMAX>;
    constexpr int P = Cf::P, KS = Cf::KS, CPR = Cf::CPR, L = D * D + D;
    __shared__ __align__(16) unsigned char lds[Cf::kBytes];
    unsigned char* const pkh = lds;
    unsigned char* const pkl = lds + Cf::kPlane;
    unsigned char* const pv = lds + 2 * Cf::kPlane;
    unsigned char* const sth = lds + 3 * Cf::kPlane;
    unsigned char* const stl = sth + Cf::kSt;
    float* const zts = reinterpret_cast<float*>(stl + Cf::kSt);
    float* const dwp = zts + D;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, n = lane & 15;
    const int64_t unit = blockIdx.x, pair = unit / M;
    const int blk = (int)(unit % M), C = N / M, T = C / 16;
    const int64_t tok0 = pair * N + (int64_t)blk * C;
    const float wii = W[(int64_t)blk * M + blk];
    const float* sv = St + ((int64_t)blk * BH + pair) * L;

    // ---- staging: phi(K) hi/lo and V rows of the block, S~_i to [r][c] hi/lo, z~_i ----
    {
        constexpr int NU = CMAX * CPR / 256, NS = D * D / 1024;
        u32x4 kw[NU], vw[NU];
        f32x4 sw[NS];
#pragma unroll
        for (int j = 0; j < NU; ++j) {
            const int u = threadIdx.x + 256 * j, row = min(u / CPR, C - 1), pc = u % CPR;  // (rows past C: unused)
            kw[j] = *reinterpret_cast<const u32x4*>(K + (tok0 + row) * D + 8 * pc);
            vw[j] = *reinterpret_cast<const u32x4*>(V + (tok0 + row) * D + 8 * pc);
        }
#pragma unroll
        for (int j = 0; j < NS; ++j) sw[j] = *reinterpret_cast<const f32x4*>(sv + (threadIdx.x + 256 * j) * 4);
        if ((int)threadIdx.x < D) zts[threadIdx.x] = sv[D * D + threadIdx.x];
#pragma unroll
        for (int j = 0; j < NU; ++j) {
            const int u = threadIdx.x + 256 * j, row = u / CPR, pc = u % CPR;
            if (row >= C) break;  // (uniform in j: C is a multiple of 32 rows)
            const int off = 16 * swz(row, pc, CPR);
            uint32_t h[4], l[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                split2_bf16(phi_b(__uint_as_float(kw[j][e] << 16)), phi_b(__uint_as_float(kw[j][e] & 0xffff0000u)),
                            h[e], l[e]);
            *reinterpret_cast<u32x4*>(pkh + off) = u32x4{h[0], h[1], h[2], h[3]};
            *reinterpret_cast<u32x4*>(pkl + off) = u32x4{l[0], l[1], l[2], l[3]};
            *reinterpret_cast<u32x4*>(pv + off) = vw[j];
        }
        // S~_i is stored transposed in the packed layout: chunk (ia, ib), lane l, element i
        // holds S~[r = P (l % 16) + ib][c = P (4 (l / 16) + i) + ia].
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const int x = threadIdx.x + 256 * j;
            const int chunk = x / 64, l = x % 64, ia = chunk / P, ib = chunk % P;
            const int r = P * (l % 16) + ib;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = P * (4 * (l / 16) + i) + ia;
                const int off = 16 * swz(r, c >> 3, CPR) + 2 * (c & 7);
                uint32_t h, lo;
                split2_bf16(sw[j][i], 0.f, h, lo);
                *reinterpret_cast<uint16_t*>(sth + off) = (uint16_t)h;
                *reinterpret_cast<uint16_t*>(stl + off) = (uint16_t)lo;
            }
        }
    }
    __syncthreads();
    // A 16 x 32 operand from a plane: lane (g, n) takes row r0 + n, k-slots 8g .. 8g + 7
    // (columns 32 ks + 8g ..).
    auto rows_op = [&](const unsigned char* plane, int r0, int ks) {
        return *reinterpret_cast<const bf16x8*>(plane + 16 * swz(r0 + n, 4 * ks + g, CPR));
    };

    float dwl = 0.f, rden_q[4], dden_q[4];  // (query n of the wave's slots)
#pragma unroll
    for (int slot = 0; slot < 4; ++slot) {
        rden_q[slot] = dden_q[slot] = 0.f;
        const int qt = 8 * (slot >> 1) + ((slot & 1) ? 7 - wave : wave);  // snake order balances the triangle
        if (qt >= T) continue;                                               // uniform
        const int64_t qrow = tok0 + 16 * qt + n;                             // query n of the tile
        bf16x8 bqh[KS], bql[KS], byh[KS], byl[KS];  // phi(q) and dy as B operands (features 32 ks + 8g ..)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(Q + qrow * D + 32 * ks + 8 * g);
            uint32_t h[4], l[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                split2_bf16(phi_b(__uint_as_float(w[e] << 16)), phi_b(__uint_as_float(w[e] & 0xffff0000u)), h[e],
                            l[e]);
            bqh[ks] = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
            bql[ks] = __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], l[2], l[3]});
            const f32x4* src = reinterpret_cast<const f32x4*>(dY + qrow * D + 32 * ks + 8 * g);
            const f32x4 a = src[0], b = src[1];
            split2_bf16(a[0], a[1], h[0], l[0]);
            split2_bf16(a[2], a[3], h[1], l[1]);
            split2_bf16(b[0], b[1], h[2], l[2]);
            split2_bf16(b[2], b[3], h[3], l[3]);
            byh[ks] = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
            byl[ks] = __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], l[2], l[3]});
        }
        // U^T = S~ dy^T, to which the within-block sum_j W g phi(k_j) is added below, and p^T
        // (features 16F + 4g + i, query n)
        f32x4 us[P], ps[P];
#pragma unroll
        for (int F = 0; F < P; ++F) {
            f32x4 a = zero4();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 sh = rows_op(sth, 16 * F, ks), sl = rows_op(stl, 16 * F, ks);
                a = mfma32(sh, byh[ks], a);
                a = mfma32(sh, byl[ks], a);
                a = mfma32(sl, byh[ks], a);
            }
            us[F] = a;
            ps[F] = zero4();
        }
        // phi(q) and phi'(q) at features 16F + 4g + i of query n; its dots with z~ and S~ dy
        float fq[P][4], dpq[P][4], pz = 0.f, pu = 0.f;
#pragma unroll
        for (int F = 0; F < P; ++F) {
            const u32x2 qw = *reinterpret_cast<const u32x2*>(Q + qrow * D + 16 * F + 4 * g);
            const float qv[4] = {__uint_as_float(qw[0] << 16), __uint_as_float(qw[0] & 0xffff0000u),
                                 __uint_as_float(qw[1] << 16), __uint_as_float(qw[1] & 0xffff0000u)};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                fq[F][i] = phi_grad(qv[i], dpq[F][i]);
                pz = fmaf(fq[F][i], zts[16 * F + 4 * g + i], pz);
                pu = fmaf(fq[F][i], us[F][i], pu);
            }
        }
        const float pzt = sum_over_groups(pz), pst = sum_over_groups(pu);
        float ssum = 0.f, sgsum = 0.f;  // this lane's keys of sum_j s_tj, sum_j s_tj g_tj (query n)
        for (int jp = 0; 2 * jp <= qt; ++jp) {
            f32x4 wg2[2], mk2[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int kt = 2 * jp + hh;
                wg2[hh] = mk2[hh] = zero4();
                if (kt > qt) continue;  // uniform
                f32x4 sc = zero4(), gg = zero4();  // keys 16 kt + 4g + e, query n
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 akh = rows_op(pkh, 16 * kt, ks), akl = rows_op(pkl, 16 * kt, ks);
                    const bf16x8 av = rows_op(pv, 16 * kt, ks);
                    sc = mfma32(akh, bqh[ks], sc);
                    sc = mfma32(akh, bql[ks], sc);
                    sc = mfma32(akl, bqh[ks], sc);
                    gg = mfma32(av, byh[ks], gg);
                    gg = mfma32(av, byl[ks], gg);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool keep = 16 * kt + 4 * g + e <= 16 * qt + n;  // key <= query
                    const float s1 = keep ? sc[e] : 0.f, g1 = keep ? gg[e] : 0.f;
                    ssum += s1;
                    sgsum = fmaf(s1, g1, sgsum);
                    wg2[hh][e] = wii * g1;
                    mk2[hh][e] = keep ? 1.f : 0.f;
                }
            }
            bf16x8 gh, gl, mh, ml;  // k-slot 8g + 4hh + e = key 32 jp + 16 hh + 4g + e
            split_pair8(wg2[0], wg2[1], gh, gl);
            split_pair8(mk2[0], mk2[1], mh, ml);  // (0 and 1 are exact: ml is zero)
#pragma unroll
            for (int F = 0; F < P; ++F) {
                const bf16x8 kth = lds_operand_t(pkh, 32 * jp, 16 * F, CPR, g, n);
                const bf16x8 ktl = lds_operand_t(pkl, 32 * jp, 16 * F, CPR, g, n);
                us[F] = mfma32(kth, gh, us[F]);
                us[F] = mfma32(kth, gl, us[F]);
                us[F] = mfma32(ktl, gh, us[F]);
                ps[F] = mfma32(kth, mh, ps[F]);
                ps[F] = mfma32(ktl, mh, ps[F]);
            }
        }
        const float st = sum_over_groups(ssum), sgt = sum_over_groups(sgsum);
        // den_t = phi(q).a_t + eps = phi(q).z~ + W sum_j s_tj + eps, and phi(q).U_t =
        // phi(q).S~ dy_t + W sum_j s_tj g_tj (the within-block parts from the same sums that
        // dW[i,i] takes, so that they cancel there as they should); without the normaliser
        // den = 1 (stored so that the key pass's dnum = dy) and dden = 0
        const float den = norm ? fmaf(wii, st, pzt) + kEps : 1.f;
        const float rden = norm ? fast_rcp(den) : 1.f;
        const float dden = norm ? -fmaf(wii, sgt, pst) * rden * rden : 0.f;
        rden_q[slot] = rden;
        dden_q[slot] = dden;
        // dq = (U / den + dden (z~ + W p)) phi'(q)
#pragma unroll
        for (int F = 0; F < P; ++F) {
            f32x4 out;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float a = fmaf(wii, ps[F][i], zts[16 * F + 4 * g + i]);
                out[i] = fmaf(us[F][i], rden, dden * a) * dpq[F][i];
            }
            *reinterpret_cast<f32x4*>(dQ + qrow * D + 16 * F + 4 * g) = out;
        }
        if (g == 0) {
            *reinterpret_cast<float2*>(G + qrow * 2) = make_float2(den, dden);
            dwl += fmaf(sgt, rden, dden * st);  // this query's part of dW[i,i]
        }
    }
    // dS~^T += dnum phi(q)^T, dz~ += dden phi(q) over the wave's tiles, in the dot layout
    // (tokens 4g + i, features P n + b): chunk (ia, ib) of the packed layout directly
    f32x4 acc[P * P];
    float zacc[P];
#pragma unroll
    for (int c = 0; c < P * P; ++c) acc[c] = zero4();
#pragma unroll
    for (int b = 0; b < P; ++b) zacc[b] = 0.f;
#pragma unroll
    for (int slot = 0; slot < 4; ++slot) {
        const int qt = 8 * (slot >> 1) + ((slot & 1) ? 7 - wave : wave);
        if (qt >= T) continue;  // uniform
        {
            const rsrc_t rq = tile_rsrc(Q, tok0 + 16 * qt, 16, D), ry = tile_rsrc(dY, tok0 + 16 * qt, 16, D);
            float qd[4][P], yd[4][P];
            load_dl<uint16_t, D>(rq, g, n, qd);
            load_dl<float, D>(ry, g, n, yd);
            float dn[4][P], fd[4][P], ddi[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float ri = __shfl(rden_q[slot], 4 * g + i, 64);  // lane 4g + i holds query 4g + i
                ddi[i] = __shfl(dden_q[slot], 4 * g + i, 64);
#pragma unroll
                for (int b = 0; b < P; ++b) {
                    fd[i][b] = phi_b(qd[i][b]);
                    dn[i][b] = yd[i][b] * ri;
                }
            }
            bf16x4 nh[P], nl[P];
            split_dl<P>(dn, nh, nl);
#pragma unroll
            for (int j = 0; j < P; ++j) {
                bf16x4 qh, ql;
                split4(fd[0][j], fd[1][j], fd[2][j], fd[3][j], qh, ql);
#pragma unroll
                for (int ia = 0; ia < P; ++ia) {
                    f32x4 c = acc[ia * P + j];
                    c = mfma16(nh[ia], qh, c);
                    c = mfma16(nh[ia], ql, c);
                    c = mfma16(nl[ia], qh, c);
                    acc[ia * P + j] = c;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) zacc[j] = fmaf(ddi[i], fd[i][j], zacc[j]);
            }
        }
    }
    // ---- the block's dS~^T, dz~ and dW[i,i] part: the waves' parts added in wave order ----
#pragma unroll
    for (int b = 0; b < P; ++b) zacc[b] = sum_over_groups(zacc[b]);
    dwl = sum_over_groups(sum16(dwl));
    if (lane == 0) dwp[wave] = dwl;
    __syncthreads();  // the planes are free for the reduction below
    reduce_waves<P>(acc, zacc, reinterpret_cast<float*>(lds), wave, 4, lane, g, n);
    if (wave == 0) {
        store_packed<P>(dSt + ((int64_t)blk * BH + pair) * L, lane, g, n, acc, zacc);
        if (lane == 0) dWdiag[pair * M + blk] = ((dwp[0] + dwp[1]) + dwp[2]) + dwp[3];
    }
}

// Causal, two waves per (pair, key block b), tiles in reverse order.  The running
// dS_b + W_bb R_{>tile} is needed in two orientations: rows c for d phi(k) (contracted
// over c with v) and rows r for dv (contracted over r with phi(k)).  Wave 0 keeps the
// first and produces dk, wave 1 keeps the second and produces dv, each folding the
// tile's W_bb phi(q) dnum^T into its own copy; inside a tile the masked scores
// dnum_t . v_j + dden_t (wave 0) and phi(q_t).phi(k_j) (wave 1), t >= j, carry the rest.
template <int D, typename T>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2))) void bwd_key_causal_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, const float* __restrict__ dY,
    const float* __restrict__ W, const float* __restrict__ G, const float* __restrict__ dS, float* __restrict__ dK,
    float* __restrict__ dV, int64_t BH, int N, int M) {
    using Dm = Dim<D>;
    constexpr int P = Dm::P, FL = Dm::FL, KS = Dm::KS, L = Dm::L;
    constexpr bool VLO = !std::is_same<T, uint16_t>::value;
    const int lane = threadIdx.x & 63, role = threadIdx.x >> 6;
    const int g = lane >> 4, n = lane & 15;
    const int64_t unit = blockIdx.x, pair = unit / M;
    const int blk = (int)(unit % M), C = N / M;
    const int64_t row0 = pair * N + (int64_t)blk * C;
    const int ntiles = (C + 15) / 16;
    const float wbb = W[(int64_t)blk * M + blk];

    const float* sv = dS + ((int64_t)blk * BH + pair) * L;
    f32x4 st[P * P];  // role 0: rows c (dS^T + W R^T); role 1: rows r (dS + W R)
    float s1z[P];     // role 0: dz_b + W r
    if (role == 0) {
        load_packed<P>(sv, lane, st);
#pragma unroll
        for (int b = 0; b < P; ++b) s1z[b] = sv[D * D + P * n + b];
    } else {
        load_packed_t<P>(sv, g, n, st);
    }

    for (int tile = ntiles - 1; tile >= 0; --tile) {
        const int t0 = 16 * tile, rows = min(16, C - t0);
        const int64_t r0 = row0 + t0;
        const rsrc_t rq = tile_rsrc(Q, r0, rows, D), rk = tile_rsrc(K, r0, rows, D);
        const rsrc_t ry = tile_rsrc(dY, r0, rows, D), rg = tile_rsrc(G, r0, rows, 2);
        float qd[4][P], yd[4][P], gd[4][2];
        load_dl<T, D>(rq, g, n, qd);
        load_dl<float, D>(ry, g, n, yd);
#pragma unroll
        for (int i = 0; i < 4; ++i) load_run<float, 2>(rg, (uint32_t)((4 * g + i) * 8), gd[i]);
        float dden[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // dnum (dot layout; rows past the block: zero)
            const float ri = 4 * g + i < rows ? fast_rcp(gd[i][0]) : 0.f;
            dden[i] = gd[i][1];
#pragma unroll
            for (int b = 0; b < P; ++b) {
                yd[i][b] *= ri;
                qd[i][b] = phi_b(qd[i][b]);
            }
        }
        bf16x4 qdh[P], qdl[P];
        split_dl<P>(qd, qdh, qdl);
        f32x4 a[P];
#pragma unroll
        for (int b = 0; b < P; ++b) a[b] = zero4();
        if (role == 0) {
            // d phi(k_j) = (dS + W R_{>tile}) v_j + dz + W r + W sum_{t >= j} (dnum_t . v_j + dden_t) phi(q_t)
            const rsrc_t rv = tile_rsrc(V, r0, rows, D), rdk = tile_rsrc(dK, r0, rows, D);
            float vr[FL], yr[FL], kd[4][P], gn[2];
            load_rl<T, D>(rv, g, n, vr);
            load_rl<float, D>(ry, g, n, yr);
            load_dl<T, D>(rk, g, n, kd);
            load_run<float, 2>(rg, (uint32_t)(n * 8), gn);
            const float rn = n < rows ? fast_rcp(gn[0]) : 0.f;
#pragma unroll
            for (int f = 0; f < FL; ++f) yr[f] *= rn;
            bf16x8 vh[KS], vl[KS];
            split_rl<FL, KS>(vr, vh, vl);
            gemm_packed<P, KS, VLO>(vh, vl, st, a);
            f32x4 gg = zero4();  // lane (g, n): t = 4g + e, j = n
            {
                bf16x8 nh[KS], nl[KS];
                split_rl<FL, KS>(yr, nh, nl);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    gg = mfma32(nh[ks], vh[ks], gg);
                    gg = mfma32(nl[ks], vh[ks], gg);
                    if constexpr (VLO) gg = mfma32(nh[ks], vl[ks], gg);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) gg[e] = 4 * g + e >= n ? wbb * (gg[e] + dden[e]) : 0.f;
            {
                bf16x4 gh, gl;
                split4(gg, gh, gl);
#pragma unroll
                for (int b = 0; b < P; ++b) {
                    a[b] = mfma16(gh, qdh[b], a[b]);
                    a[b] = mfma16(gh, qdl[b], a[b]);
                    a[b] = mfma16(gl, qdh[b], a[b]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float o[P];
#pragma unroll
                for (int b = 0; b < P; ++b) {
                    float dp;
                    phi_grad(kd[i][b], dp);
                    o[b] = (a[b][i] + s1z[b]) * dp;
                }
                store_dl<D>(rdk, g, n, i, o);
            }
        } else {
            // dv_j = (dS + W R_{>tile})^T phi(k_j) + W sum_{t >= j} (phi(q_t) . phi(k_j)) dnum_t
            const rsrc_t rdv = tile_rsrc(dV, r0, rows, D);
            float kr[FL], qr[FL];
            load_rl<T, D>(rk, g, n, kr);
            load_rl<T, D>(rq, g, n, qr);
#pragma unroll
            for (int f = 0; f < FL; ++f) {
                kr[f] = phi_b(kr[f]);
                qr[f] = phi_b(qr[f]);
            }
            bf16x8 kh[KS], kl[KS];
            split_rl<FL, KS>(kr, kh, kl);
            gemm_packed<P, KS, true>(kh, kl, st, a);
            f32x4 sc = zero4();  // lane (g, n): t = 4g + e, j = n
            {
                bf16x8 qh[KS], ql[KS];
                split_rl<FL, KS>(qr, qh, ql);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    sc = mfma32(qh[ks], kh[ks], sc);
                    sc = mfma32(qh[ks], kl[ks], sc);
                    sc = mfma32(ql[ks], kh[ks], sc);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) sc[e] = 4 * g + e >= n ? wbb * sc[e] : 0.f;
            {
                bf16x4 ndh[P], ndl[P], sh, sl;
                split_dl<P>(yd, ndh, ndl);
                split4(sc, sh, sl);
#pragma unroll
                for (int b = 0; b < P; ++b) {
                    a[b] = mfma16(sh, ndh[b], a[b]);
                    a[b] = mfma16(sh, ndl[b], a[b]);
                    a[b] = mfma16(sl, ndh[b], a[b]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float o[P];
#pragma unroll
                for (int b = 0; b < P; ++b) o[b] = a[b][i];
                store_dl<D>(rdv, g, n, i, o);
            }
        }
        // fold this tile into the running sum, times W_bb
        float wdn[4][P];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int b = 0; b < P; ++b) wdn[i][b] = wbb * yd[i][b];
        bf16x4 wh[P], wl[P];
        split_dl<P>(wdn, wh, wl);
        if (role == 0) {
            acc_outer<P, true>(wh, wl, qdh, qdl, st);  // rows c: dnum[c] phi(q)[r]
#pragma unroll
            for (int b = 0; b < P; ++b) {
                float z = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) z = fmaf(dden[i], qd[i][b], z);
                s1z[b] = fmaf(wbb, sum_over_groups(z), s1z[b]);
            }
        } else {
            acc_outer<P, true>(qdh, qdl, wh, wl, st);  // rows r: phi(q)[r] dnum[c]
        }
    }
}

// Wt[b][i] = W[i][b] for the summaries that block b feeds (causal: i > b), else 0.
__global__ __launch_bounds__(256) void bwd_wt_kernel(const float* __restrict__ W, float* __restrict__ Wt, int M,
                                                     int causal) {
    const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= (int64_t)M * M) return;
    const int b = (int)(x / M), i = (int)(x % M);
    Wt[x] = (!causal || i > b) ? W[(int64_t)i * M + b] : 0.f;
}

// dW partials: part[ch][i][b] = sum over columns of chunk ch of dSt[i][col] S[b][col],
// one 64 x 64 output block per workgroup (wave w: rows 16w .. 16w + 15), on MFMA
// with hi + lo operands.  ncols and chunk are multiples of 8.  Each step's loads are
// issued two steps ahead (unconditional loads: a column or row out of range reads a
// valid address and is masked to zero when used).
struct DwRun {  // 8 consecutive floats of one row, loaded ahead; masked when used
    f32x4 x[2];
    bool ok;
};

__device__ __forceinline__ void dw_load(const float* X, int64_t ncols, int row, int M, int64_t k, int64_t k1,
                                        DwRun& r) {
    r.ok = row < M && k < k1;
    const f32x4* p = reinterpret_cast<const f32x4*>(X + (r.ok ? (int64_t)row * ncols + k : 0));
    r.x[0] = p[0];
    r.x[1] = p[1];
}

__device__ __forceinline__ void dw_split(const DwRun& r, bf16x8& hi, bf16x8& lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float a = r.ok ? r.x[e >> 1][2 * (e & 1)] : 0.f, b = r.ok ? r.x[e >> 1][2 * (e & 1) + 1] : 0.f;
        split2_bf16(a, b, h[e], l[e]);
    }
    hi = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
    lo = __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], l[2], l[3]});
}

template <int JT>
__global__ __launch_bounds__(256) void bwd_dw_kernel(const float* __restrict__ dSt, const float* __restrict__ S,
                                                     float* __restrict__ part, int64_t ncols, int M, int64_t chunk,
                                                     int nb, int rt) {
    // rt row tiles of 16 per workgroup (min(4, ceil(M / 16))); the 4 / rt wave slots
    // left over take consecutive column chunks of their own.
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, n = lane & 15;
    const int ob = (int)(blockIdx.x % (nb * nb));
    const int64_t ch = (blockIdx.x / (nb * nb)) * (4 / rt) + wave / rt;
    const int i0 = 64 * (ob / nb) + 16 * (wave % rt), b0 = 64 * (ob % nb);
    // JT column tiles of 16 per block (tiles past M read zero and are not stored)
    const int64_t k0 = ch * chunk, k1 = min(ncols, k0 + chunk);
    f32x4 acc[JT];
#pragma unroll
    for (int jb = 0; jb < JT; ++jb) acc[jb] = zero4();
    if (i0 < M && k0 < ncols) {
        const int nsteps = (int)((k1 - k0 + 31) / 32);
        // two register sets: the loads of step s + 2 are issued while step s computes
        DwRun xa[2], xb[2][JT];
        int64_t k = k0 + 8 * g;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            dw_load(dSt, ncols, i0 + n, M, k + 32 * h, k1, xa[h]);
#pragma unroll
            for (int jb = 0; jb < JT; ++jb) dw_load(S, ncols, b0 + 16 * jb + n, M, k + 32 * h, k1, xb[h][jb]);
        }
        auto step = [&](DwRun& a, DwRun (&b)[JT], int64_t knext) {
            bf16x8 ah, al, bh[JT], bl[JT];
            dw_split(a, ah, al);
#pragma unroll
            for (int jb = 0; jb < JT; ++jb) dw_split(b[jb], bh[jb], bl[jb]);
            dw_load(dSt, ncols, i0 + n, M, knext, k1, a);
#pragma unroll
            for (int jb = 0; jb < JT; ++jb) dw_load(S, ncols, b0 + 16 * jb + n, M, knext, k1, b[jb]);
            issue_fence();
#pragma unroll
            for (int jb = 0; jb < JT; ++jb) {
                acc[jb] = mfma32(ah, bh[jb], acc[jb]);
                acc[jb] = mfma32(ah, bl[jb], acc[jb]);
                acc[jb] = mfma32(al, bh[jb], acc[jb]);
            }
        };
        for (int st = 0; st < nsteps; st += 2, k += 64) {
            step(xa[0], xb[0], k + 64);
            if (st + 1 >= nsteps) break;
            step(xa[1], xb[1], k + 96);
        }
    }
    if (k0 >= ncols) return;
#pragma unroll
    for (int jb = 0; jb < JT; ++jb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = i0 + 4 * g + i, col = b0 + 16 * jb + n;
            if (row < M && col < M) part[(ch * M + row) * (int64_t)M + col] = acc[jb][i];
        }
}

// The same partials for four row tiles per workgroup (M > 32): the waves take row tiles
// 16w of one 64 x 64 output block and share its S rows.  Wave w loads S rows
// b0 + 16w .. + 15, splits them into the B operand of column tile w and hands it to
// the other waves through LDS (double-buffered, one LDS-scoped barrier per 32-column
// step, so the loads issued two steps ahead stay in flight), so each S row is read once
// per workgroup instead of once per wave.  Same products in the same order as above.
__global__ __launch_bounds__(256) void bwd_dw_shared_kernel(const float* __restrict__ dSt,
                                                            const float* __restrict__ S, float* __restrict__ part,
                                                            int64_t ncols, int M, int64_t chunk, int nb) {
    __shared__ bf16x8 bop[2][4][2][64];  // [buffer][column tile][hi, lo][lane]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, n = lane & 15;
    const int ob = (int)(blockIdx.x % (nb * nb));
    const int64_t ch = blockIdx.x / (nb * nb);
    const int i0 = 64 * (ob / nb) + 16 * wave, b0 = 64 * (ob % nb);
    const int64_t k0 = ch * chunk, k1 = min(ncols, k0 + chunk);
    if (k0 >= ncols) return;  // the whole workgroup
    f32x4 acc[4];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) acc[jb] = zero4();
    const int nsteps = (int)((k1 - k0 + 31) / 32);
    DwRun xa[2], xs[2];
    int64_t k = k0 + 8 * g;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        dw_load(dSt, ncols, i0 + n, M, k + 32 * h, k1, xa[h]);
        dw_load(S, ncols, b0 + 16 * wave + n, M, k + 32 * h, k1, xs[h]);
    }
    auto step = [&](DwRun& a, DwRun& sr, int64_t knext, int buf) {
        bf16x8 ah, al, sh, sl;
        dw_split(a, ah, al);
        dw_split(sr, sh, sl);
        dw_load(dSt, ncols, i0 + n, M, knext, k1, a);
        dw_load(S, ncols, b0 + 16 * wave + n, M, knext, k1, sr);
        issue_fence();
        bop[buf][wave][0][lane] = sh;
        bop[buf][wave][1][lane] = sl;
        lds_barrier();
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
            const bf16x8 bh = bop[buf][jb][0][lane], bl = bop[buf][jb][1][lane];
            acc[jb] = mfma32(ah, bh, acc[jb]);
            acc[jb] = mfma32(ah, bl, acc[jb]);
            acc[jb] = mfma32(al, bh, acc[jb]);
        }
    };
    for (int st = 0; st < nsteps; st += 2, k += 64) {  // nsteps is uniform: every wave meets every barrier
        step(xa[0], xs[0], k + 64, 0);
        if (st + 1 >= nsteps) break;
        step(xa[1], xs[1], k + 96, 1);
    }
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = i0 + 4 * g + i, col = b0 + 16 * jb + n;
            if (row < M && col < M) part[(ch * M + row) * (int64_t)M + col] = acc[jb][i];
        }
}

// First reduction level: part2[s][x] = sum of part[ch][x] over chunks ch of group s
// (cps chunks per group), in chunk order; consecutive threads take consecutive x.
__global__ __launch_bounds__(256) void bwd_dw_reduce1_kernel(const float* __restrict__ part,
                                                             float* __restrict__ part2, int64_t MM, int64_t nchunks,
                                                             int64_t cps, int64_t ngroups) {
    const int64_t x = (int64_t)(blockIdx.x % ngroups) * 256 + threadIdx.x;
    const int64_t s = blockIdx.x / ngroups;
    if (x >= MM) return;
    const int64_t c0 = s * cps, c1 = min(nchunks, c0 + cps);
    float acc = 0.f;
#pragma unroll 8
    for (int64_t c = c0; c < c1; ++c) acc += part[c * MM + x];
    part2[s * MM + x] = acc;
}

// dW[i][b] = sum of the first-level sums in group order; causal: b < i only, plus the
// diagonal from the per-pair partials (in pair order).
__global__ __launch_bounds__(256) void bwd_dw_reduce_kernel(const float* __restrict__ part2,
                                                            const float* __restrict__ dWdiag, float* __restrict__ dW,
                                                            int M, int64_t nsplit, int64_t BH, int causal) {
    const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= (int64_t)M * M) return;
    const int i = (int)(x / M), b = (int)(x % M);
    float s = 0.f;
    if (!causal || b < i) {
#pragma unroll 8
        for (int64_t p = 0; p < nsplit; ++p) s += part2[p * M * M + x];
    }
    if (causal && b == i) {
#pragma unroll 8
        for (int64_t p = 0; p < BH; ++p) s += dWdiag[p * M + i];
    }
    dW[x] = s;
}

namespace {

struct DwPlan {
    int nb;           // 64 x 64 output blocks per dimension
    int rt;           // row tiles of 16 per workgroup; 4 / rt chunks per workgroup
    int64_t chunk;    // columns per partial
    int64_t nchunks;
    int64_t cps;      // chunks per first-level reduction group
    int64_t nsplit;   // first-level groups
};

DwPlan dw_plan(int64_t ncols, int64_t M) {
    DwPlan p;
    p.nb = (int)((M + 63) / 64);
    p.rt = (int)std::min<int64_t>(4, (M + 15) / 16);
    if (p.rt == 3) p.rt = 4;
    const int64_t subs = 4 / p.rt;
    const int64_t nblk = (int64_t)p.nb * p.nb;
    // One round of resident workgroups: 256 CUs x (waves per SIMD of bwd_dw_kernel<rt>
    // and bwd_dw_shared_kernel: 6, 4, 4 for rt = 1, 2, 4) four-wave workgroups; a few
    // workgroups past it would form a second round alone.
    const int64_t round = 256 * (p.rt == 1 ? 6 : 4);
    const int64_t want = std::max<int64_t>(1, round / nblk) * subs;  // partials (one per wave slot)
    const int64_t most = std::max<int64_t>(1, ncols / 256);          // at least 256 columns per partial
    const int64_t nch = std::min(want, most);
    p.chunk = ((ncols + nch - 1) / nch + 31) / 32 * 32;
    p.nchunks = (ncols + p.chunk - 1) / p.chunk;
    // first level: up to 2048 workgroups, and about sqrt(nchunks) groups so that
    // neither level sums a long run per thread
    const int64_t groups = (M * M + 255) / 256;
    int64_t root = 1;
    while (root * root < p.nchunks) ++root;
    const int64_t split = std::max<int64_t>(1, std::min<int64_t>(root, 2048 / groups));
    p.cps = (p.nchunks + split - 1) / split;
    p.nsplit = (p.nchunks + p.cps - 1) / p.cps;
    return p;
}

// Waves per (pair, block) for the non-causal kernels: enough waves in flight for the
// memory system, never more than the block has tiles.
int waves_per_unit(int64_t units, int64_t ntiles) {
    int w = 1;
    while (w < 4 && 2 * w <= ntiles && units * w < 8192) w *= 2;
    return w;
}

constexpr int64_t align64(int64_t x) { return (x + 63) / 64 * 64; }

struct BwdLayout {
    int64_t S, St, dSt, dS, Wt, G, dWdiag, part, part2, total;  // float offsets
};

BwdLayout bwd_layout(int64_t BH, int64_t N, int D, int64_t M, bool causal) {
    const int64_t L = (int64_t)D * D + D;
    const int64_t arr = align64(M * BH * L);
    const DwPlan p = dw_plan(BH * L, M);
    BwdLayout o;
    o.S = 0;
    o.St = o.S + arr;
    o.dSt = o.St + arr;
    o.dS = o.dSt + arr;
    o.Wt = o.dS + arr;
    o.G = o.Wt + align64(M * M);
    o.dWdiag = o.G + (causal ? align64(2 * BH * N) : 0);
    o.part = o.dWdiag + align64(BH * M);
    o.part2 = o.part + align64(p.nchunks * M * M);
    o.total = o.part2 + align64(p.nsplit * M * M);
    return o;
}

template <int D, typename T>
hipError_t run_backward(const T* q, const T* k, const T* v, const float* W, const float* dy, float* dq, float* dk,
                        float* dv, float* dW, int64_t BH, int64_t N, int64_t M, bool causal, bool normalize, float* ws,
                        void* frag_ws, hipStream_t stream) {
    constexpr int L = D * D + D;
    const BwdLayout o = bwd_layout(BH, N, D, M, causal);
    float *S = ws + o.S, *St = ws + o.St, *dSt = ws + o.dSt, *dS = ws + o.dS, *Wt = ws + o.Wt;
    float *G = ws + o.G, *dWdiag = ws + o.dWdiag, *part = ws + o.part, *part2 = ws + o.part2;
    const int64_t units = BH * M, C = N / M, ntiles = (C + 15) / 16;
    const int wpu = waves_per_unit(units, ntiles);
    const size_t red = (size_t)(wpu / 2) * L * sizeof(float);
    const dim3 grid((unsigned)units), block(64 * wpu);
    hipError_t e;
    if (std::is_same<T, uint16_t>::value && summaries_t_fits(BH, N, D, M)) {
        e = launch_summaries_t((const uint16_t*)k, (const uint16_t*)v, S, BH, N, D, M, stream);
    } else {
        bwd_sum_kernel<D, T><<<grid, block, red, stream>>>(k, v, S, BH, (int)N, (int)M, wpu);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    if ((e = launch_mix(S, W, St, BH, D, M, causal, false, 0, frag_ws, stream)) != hipSuccess) return e;
    if (causal && std::is_same<T, uint16_t>::value && (D == 32 || D == 64) && C % 32 == 0 && C <= 256) {
        // token-level form of the within-block part (blocks of an even number of whole tiles)
        const uint16_t* q16 = reinterpret_cast<const uint16_t*>(q);
        const uint16_t* k16 = reinterpret_cast<const uint16_t*>(k);
        const uint16_t* v16 = reinterpret_cast<const uint16_t*>(v);
#define MHLA_QCTL(DD, CM)                                                                                      \
        bwd_query_causal_tl_kernel<DD, CM><<<grid, dim3(256), 0, stream>>>(q16, k16, v16, dy, W, St, dq, dSt, G, \
                                                                            dWdiag, BH, (int)N, (int)M,          \
                                                                            normalize ? 1 : 0)
        if constexpr (D == 32) {
            if (C <= 128) MHLA_QCTL(32, 128); else MHLA_QCTL(32, 256);
        } else if constexpr (D == 64) {
            if (C <= 128) MHLA_QCTL(64, 128); else MHLA_QCTL(64, 256);
        }
#undef MHLA_QCTL
    } else if (causal)
        bwd_query_causal_kernel<D, T><<<grid, dim3(D >= 32 ? 128 : 64), 0, stream>>>(
            q, k, v, dy, W, St, dq, dSt, G, dWdiag, BH, (int)N, (int)M, normalize ? 1 : 0);
    else
        bwd_query_kernel<D, T><<<grid, block, red, stream>>>(q, dy, St, dq, dSt, BH, (int)N, (int)M, wpu,
                                                             normalize ? 1 : 0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    bwd_wt_kernel<<<dim3((unsigned)((M * M + 255) / 256)), dim3(256), 0, stream>>>(W, Wt, (int)M, causal);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = launch_mix(dSt, Wt, dS, BH, D, M, false, false, 0, frag_ws, stream)) != hipSuccess) return e;
    if (causal)
        bwd_key_causal_kernel<D, T><<<grid, dim3(128), 0, stream>>>(q, k, v, dy, W, G, dS, dk, dv, BH, (int)N,
                                                                      (int)M);
    else
        if (wpu > 1)
            bwd_key_kernel<D, T, true><<<grid, block, 0, stream>>>(k, v, dS, dk, dv, BH, (int)N, (int)M, wpu);
        else
            bwd_key_kernel<D, T, false><<<grid, block, 0, stream>>>(k, v, dS, dk, dv, BH, (int)N, (int)M, wpu);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const DwPlan p = dw_plan(BH * L, M);
    const int64_t subs = 4 / p.rt;
    const dim3 dw_grid((unsigned)((p.nchunks + subs - 1) / subs * p.nb * p.nb));
    if (p.rt == 1)
        bwd_dw_kernel<1><<<dw_grid, dim3(256), 0, stream>>>(dSt, S, part, BH * L, (int)M, p.chunk, p.nb, p.rt);
    else if (p.rt == 2)
        bwd_dw_kernel<2><<<dw_grid, dim3(256), 0, stream>>>(dSt, S, part, BH * L, (int)M, p.chunk, p.nb, p.rt);
    else
        bwd_dw_shared_kernel<<<dw_grid, dim3(256), 0, stream>>>(dSt, S, part, BH * L, (int)M, p.chunk, p.nb);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t groups = (M * M + 255) / 256;
    bwd_dw_reduce1_kernel<<<dim3((unsigned)(groups * p.nsplit)), dim3(256), 0, stream>>>(part, part2, M * M,
                                                                                        p.nchunks, p.cps, groups);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    bwd_dw_reduce_kernel<<<dim3((unsigned)((M * M + 255) / 256)), dim3(256), 0, stream>>>(part2, dWdiag, dW, (int)M,
                                                                                         p.nsplit, BH,
                                                                                         causal ? 1 : 0);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(int dtype, const void* q, const void* k, const void* v, const float* W, const float* dy,
                           float* dq, float* dk, float* dv, float* dW, int64_t BH, int64_t N, int D, int64_t M,
                           bool causal, bool normalize, float* ws, void* frag_ws, hipStream_t stream) {
    if (bwd_fused_applicable(dtype, D, N, M, causal))
        return launch_bwd_fused(q, k, v, W, dy, dq, dk, dv, dW, BH, N, D, M, normalize, ws, stream);
#define MHLA_BWD(T)                                                                                             \
    switch (D) {                                                                                                \
        case 16:                                                                                                \
            return run_backward<16, T>((const T*)q, (const T*)k, (const T*)v, W, dy, dq, dk, dv, dW, BH, N, M,  \
                                       causal, normalize, ws, frag_ws, stream);                                 \
        case 32:                                                                                                \
            return run_backward<32, T>((const T*)q, (const T*)k, (const T*)v, W, dy, dq, dk, dv, dW, BH, N, M,  \
                                       causal, normalize, ws, frag_ws, stream);                                 \
        case 64:                                                                                                \
            return run_backward<64, T>((const T*)q, (const T*)k, (const T*)v, W, dy, dq, dk, dv, dW, BH, N, M,  \
                                       causal, normalize, ws, frag_ws, stream);                                 \
        default:                                                                                                \
            return hipErrorInvalidValue;                                                                        \
    }
    if (dtype == kDtypeF32) {
        MHLA_BWD(float);
    } else {
        MHLA_BWD(uint16_t);
    }
#undef MHLA_BWD
}

size_t backward_workspace_floats(int64_t BH, int64_t N, int D, int64_t M, bool causal) {
    return (size_t)bwd_layout(BH, N, D, M, causal).total;
}

}  // namespace mhla
