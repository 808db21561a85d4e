// backward.hip -- gradients of the MHLA forward pass ("MHLA: Restoring Expressivity
// of Linear Attention via Token-Level Multi-Head", §4.1 steps, App. C causal form;
// the coefficient matrix M_c is learned end to end, §4.2).  For L = sum(dY * Y):
//
//   num_t = phi(q_t) A_t, den_t = phi(q_t).a_t + 1e-6, A_t = S~_i (+ W_ii P_t causal),
//   a_t = z~_i (+ W_ii p_t causal); dnum_t = dy_t / den_t, dden_t = -(dy_t . num_t) / den_t^2
//   d phi(q_t) = A_t dnum_t + dden_t a_t
//   dS~_i = sum_{t in i} phi(q_t) dnum_t^T,  dz~_i = sum_{t in i} dden_t phi(q_t)
//   dS_b = sum_i W[i,b] dS~_i (causal: i > b),  dW[i,b] = sum_pairs <dS~_i | dz~_i, S_b | z_b>
//   d phi(k_j) = dS_b v_j + dz_b,  dv_j = dS_b^T phi(k_j)          (j in block b)
//   causal, keys j of block i: with R_j = sum_{t in i, t >= j} phi(q_t) dnum_t^T and
//   r_j = sum_{t >= j} dden_t phi(q_t):  d phi(k_j) += W_ii (R_j v_j + r_j),
//   dv_j += W_ii R_j^T phi(k_j),  dW[i,i] += sum_j phi(k_j)^T R_j v_j + phi(k_j) . r_j
//   dq = d phi(q) * phi'(q), dk = d phi(k) * phi'(k), phi'(x) = 1 (x > 0) or exp(x).
//
// Every step is float32 arithmetic on the exact input values (phi with the
// full-precision exp).  Summaries here use the plain layout, [r][c] row-major then
// z: the backward recomputes S_b (bwd_summary_kernel) and S~_i (the mixing GEMM),
// then runs one workgroup per (pair, block) over 16-token tiles staged in LDS:
// bwd_query_kernel (dq, dS~, dz~; causal: a second, reverse pass over the block
// for the within-block terms of dk, dv, dW_ii), the mixing GEMM with the
// transposed W (dS), bwd_key_kernel (dk, dv), and a two-step deterministic
// reduction for dW.
#include "common.hpp"
#include "kernels.hpp"

namespace mhla {

namespace {

constexpr int kTile = 16;  // tokens per LDS tile

template <typename T>
__device__ __forceinline__ float in_val(const T* p, int64_t i);
template <>
__device__ __forceinline__ float in_val<uint16_t>(const uint16_t* p, int64_t i) {
    return bf16_to_f32(p[i]);
}
template <>
__device__ __forceinline__ float in_val<float>(const float* p, int64_t i) {
    return p[i];
}

__device__ __forceinline__ float dphi(float x) { return x > 0.f ? 1.f : expf(x); }

}  // namespace

// S_b, z_b in float32, plain layout: one workgroup per (pair, block).
template <int D, typename T>
__global__ __launch_bounds__(256) void bwd_summary_kernel(const T* __restrict__ K, const T* __restrict__ V,
                                                          float* __restrict__ S, int64_t BH, int N, int M) {
    constexpr int L = D * D + D;
    constexpr int EPT = (L + 255) / 256;  // entries per thread
    __shared__ float fk[kTile][D], vv[kTile][D];
    const int tid = threadIdx.x;
    const int64_t unit = blockIdx.x;  // pair * M + block
    const int64_t pair = unit / M;
    const int blk = (int)(unit % M);
    const int C = N / M;
    const T* Kp = K + (pair * N + (int64_t)blk * C) * D;
    const T* Vp = V + (pair * N + (int64_t)blk * C) * D;
    float acc[EPT];
#pragma unroll
    for (int u = 0; u < EPT; ++u) acc[u] = 0.f;
    for (int t0 = 0; t0 < C; t0 += kTile) {
        for (int x = tid; x < kTile * D; x += 256) {
            const int t = x / D, r = x % D;
            const bool ok = t0 + t < C;
            fk[t][r] = ok ? phi_precise(in_val<T>(Kp, (int64_t)(t0 + t) * D + r)) : 0.f;
            vv[t][r] = ok ? in_val<T>(Vp, (int64_t)(t0 + t) * D + r) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            const int e = tid + 256 * u;
            if (e < D * D) {
                const int r = e / D, c = e % D;
                for (int t = 0; t < kTile; ++t) acc[u] = fmaf(fk[t][r], vv[t][c], acc[u]);
            } else if (e < L) {
                for (int t = 0; t < kTile; ++t) acc[u] += fk[t][e - D * D];
            }
        }
        __syncthreads();
    }
    float* out = S + ((int64_t)blk * BH + pair) * L;
#pragma unroll
    for (int u = 0; u < EPT; ++u) {
        const int e = tid + 256 * u;
        if (e < L) out[e] = acc[u];
    }
}

// dq, dS~_i, dz~_i for one (pair, query block i); causal also the within-block
// terms of dk, dv (written to dk, dv as d phi(k) and dv partials) and dW_ii.
template <int D, typename T, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_query_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                        const T* __restrict__ V, const float* __restrict__ dY,
                                                        const float* __restrict__ W, const float* __restrict__ St,
                                                        float* __restrict__ dSt, float* __restrict__ G,
                                                        float* __restrict__ dQ, float* __restrict__ dK,
                                                        float* __restrict__ dV, float* __restrict__ dWdiag,
                                                        int64_t BH, int N, int M) {
    constexpr int L = D * D + D;
    constexpr int EPT = (L + 255) / 256;
    constexpr int OPT = kTile * D / 256;  // (token, column) outputs per thread
    __shared__ float A[L];  // S~_i (+ W_ii P of the earlier tiles) and z~_i (+ W_ii p); reverse pass: R, r
    __shared__ float fq[kTile][D], fk[kTile][D], vv[kTile][D], dyv[kTile][D], nm[kTile][D];
    __shared__ float sc[kTile][kTile], gg[kTile][kTile], den[kTile], dd[kTile], red[kTile];
    const int tid = threadIdx.x;
    const int64_t unit = blockIdx.x;
    const int64_t pair = unit / M;
    const int blk = (int)(unit % M);
    const int C = N / M;
    const int64_t base = pair * N + (int64_t)blk * C;  // first token row of the block
    const float wii = CAUSAL ? W[(int64_t)blk * M + blk] : 0.f;
    const float* Sv = St + ((int64_t)blk * BH + pair) * L;
    for (int e = tid; e < L; e += 256) A[e] = Sv[e];
    float acc[EPT];  // dS~_i, dz~_i entries tid + 256u
#pragma unroll
    for (int u = 0; u < EPT; ++u) acc[u] = 0.f;
    __syncthreads();

    for (int t0 = 0; t0 < C; t0 += kTile) {
        for (int x = tid; x < kTile * D; x += 256) {
            const int t = x / D, r = x % D;
            const bool ok = t0 + t < C;
            const int64_t row = (base + t0 + t) * D + r;
            fq[t][r] = ok ? phi_precise(in_val<T>(Q, row)) : 0.f;
            dyv[t][r] = ok ? dY[row] : 0.f;
            if constexpr (CAUSAL) {
                fk[t][r] = ok ? phi_precise(in_val<T>(K, row)) : 0.f;
                vv[t][r] = ok ? in_val<T>(V, row) : 0.f;
            }
        }
        __syncthreads();
        if constexpr (CAUSAL) {  // in-tile scores phi(q_t).phi(k_j)
            const int t = tid / kTile, j = tid % kTile;
            float s = 0.f;
            for (int r = 0; r < D; ++r) s = fmaf(fq[t][r], fk[j][r], s);
            sc[t][j] = s;
            __syncthreads();
        }
        // numerator and denominator (A holds S~_i + W_ii P of the earlier tiles)
#pragma unroll
        for (int o = 0; o < OPT; ++o) {
            const int x = tid + 256 * o, t = x / D, c = x % D;
            float s = 0.f;
            for (int r = 0; r < D; ++r) s = fmaf(fq[t][r], A[r * D + c], s);
            if constexpr (CAUSAL)
                for (int j = 0; j <= t; ++j) s = fmaf(wii * sc[t][j], vv[j][c], s);
            nm[t][c] = s;
        }
        if (tid < kTile) {
            const int t = tid;
            float s = 0.f;
            for (int r = 0; r < D; ++r) s = fmaf(fq[t][r], A[D * D + r], s);
            if constexpr (CAUSAL)
                for (int j = 0; j <= t; ++j) s = fmaf(wii, sc[t][j], s);
            den[t] = s + kEps;
        }
        __syncthreads();
        if (tid < kTile) {
            const int t = tid;
            float s = 0.f;
            for (int c = 0; c < D; ++c) s = fmaf(dyv[t][c], nm[t][c], s);
            dd[t] = t0 + t < C ? -s / (den[t] * den[t]) : 0.f;
        }
        __syncthreads();
        for (int x = tid; x < kTile * D; x += 256) {  // nm becomes dnum
            const int t = x / D, c = x % D;
            nm[t][c] = t0 + t < C ? dyv[t][c] / den[t] : 0.f;
        }
        __syncthreads();
        if constexpr (CAUSAL) {  // g[t][j] = v_j . dnum_t + dden_t
            const int t = tid / kTile, j = tid % kTile;
            float s = dd[t];
            for (int c = 0; c < D; ++c) s = fmaf(vv[j][c], nm[t][c], s);
            gg[t][j] = s;
            __syncthreads();
        }
        // d phi(q_t) = A dnum_t + dden_t a (+ W_ii sum_{j <= t in tile} g[t][j] phi(k_j)) -> dq
#pragma unroll
        for (int o = 0; o < OPT; ++o) {
            const int x = tid + 256 * o, t = x / D, r = x % D;
            float s = dd[t] * A[D * D + r];
            for (int c = 0; c < D; ++c) s = fmaf(A[r * D + c], nm[t][c], s);
            if constexpr (CAUSAL)
                for (int j = 0; j <= t; ++j) s = fmaf(wii * gg[t][j], fk[j][r], s);
            if (t0 + t < C) {
                const int64_t row = (base + t0 + t) * D + r;
                dQ[row] = s * dphi(in_val<T>(Q, row));
            }
        }
        // dS~_i += phi(q_t) dnum_t^T, dz~_i += dden_t phi(q_t)
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            const int e = tid + 256 * u;
            if (e < D * D) {
                const int r = e / D, c = e % D;
                for (int t = 0; t < kTile; ++t) acc[u] = fmaf(fq[t][r], nm[t][c], acc[u]);
            } else if (e < L) {
                for (int t = 0; t < kTile; ++t) acc[u] = fmaf(dd[t], fq[t][e - D * D], acc[u]);
            }
        }
        if constexpr (CAUSAL) {
            // keep dnum, dden for the reverse pass
            for (int x = tid; x < kTile * (D + 1); x += 256) {
                const int t = x / (D + 1), c = x % (D + 1);
                if (t0 + t < C) G[(base + t0 + t) * (D + 1) + c] = c < D ? nm[t][c] : dd[t];
            }
            __syncthreads();
            // fold this tile's summary, times W_ii, into A
            for (int e = tid; e < L; e += 256) {
                float s = 0.f;
                if (e < D * D) {
                    const int r = e / D, c = e % D;
                    for (int j = 0; j < kTile; ++j) s = fmaf(fk[j][r], vv[j][c], s);
                } else {
                    for (int j = 0; j < kTile; ++j) s += fk[j][e - D * D];
                }
                A[e] = fmaf(wii, s, A[e]);
            }
        }
        __syncthreads();
    }
    float* out = dSt + ((int64_t)blk * BH + pair) * L;
#pragma unroll
    for (int u = 0; u < EPT; ++u) {
        const int e = tid + 256 * u;
        if (e < L) out[e] = acc[u];
    }
    if constexpr (!CAUSAL) return;

    // ---- reverse pass over the block: R_j, r_j for keys j (later queries first) ----
    for (int e = tid; e < L; e += 256) A[e] = 0.f;  // A now holds R (after the current tile), r
    float dw = 0.f;
    __syncthreads();
    const int ntiles = (C + kTile - 1) / kTile;
    for (int ti = ntiles - 1; ti >= 0; --ti) {
        const int t0 = ti * kTile;
        for (int x = tid; x < kTile * D; x += 256) {
            const int t = x / D, r = x % D;
            const bool ok = t0 + t < C;
            const int64_t row = (base + t0 + t) * D + r;
            fq[t][r] = ok ? phi_precise(in_val<T>(Q, row)) : 0.f;
            fk[t][r] = ok ? phi_precise(in_val<T>(K, row)) : 0.f;
            vv[t][r] = ok ? in_val<T>(V, row) : 0.f;
            nm[t][r] = ok ? G[(base + t0 + t) * (D + 1) + r] : 0.f;
        }
        if (tid < kTile) dd[tid] = t0 + tid < C ? G[(base + t0 + tid) * (D + 1) + D] : 0.f;
        __syncthreads();
        {  // sc[t][j] = phi(q_t).phi(k_j), gg[t][j] = v_j . dnum_t + dden_t
            const int t = tid / kTile, j = tid % kTile;
            float s = 0.f, u = dd[t];
            for (int r = 0; r < D; ++r) {
                s = fmaf(fq[t][r], fk[j][r], s);
                u = fmaf(vv[j][r], nm[t][r], u);
            }
            sc[t][j] = s;
            gg[t][j] = u;
        }
        __syncthreads();
        // d phi(k_j) += W_ii (R v_j + r + sum_{t >= j in tile} g[t][j] phi(q_t)); dv_j += W_ii (R^T phi(k_j) + ...)
        float dwp = 0.f;
#pragma unroll
        for (int o = 0; o < OPT; ++o) {
            const int x = tid + 256 * o, j = x / D, r = x % D;
            float s = A[D * D + r], sv = 0.f;
            for (int c = 0; c < D; ++c) {
                s = fmaf(A[r * D + c], vv[j][c], s);
                sv = fmaf(A[c * D + r], fk[j][c], sv);
            }
            // phi(k_j)^T R v_j + phi(k_j) . r, summed over r by the reduction below
            dwp = fmaf(fk[j][r], s, dwp);
            for (int t = j; t < kTile; ++t) {
                s = fmaf(gg[t][j], fq[t][r], s);
                sv = fmaf(sc[t][j], nm[t][r], sv);
            }
            if (t0 + j < C) {
                const int64_t row = (base + t0 + j) * D + r;
                dK[row] = wii * s;
                dV[row] = wii * sv;
            }
        }
        if (tid < kTile * kTile) {  // in-tile part of dW_ii: sum_{t >= j} sc[t][j] g[t][j]
            const int t = tid / kTile, j = tid % kTile;
            if (t >= j) dwp = fmaf(sc[t][j], gg[t][j], dwp);
        }
        dw += dwp;
        __syncthreads();
        // R += sum_t phi(q_t) dnum_t^T, r += sum_t dden_t phi(q_t)
        for (int e = tid; e < L; e += 256) {
            float s = 0.f;
            if (e < D * D) {
                const int r = e / D, c = e % D;
                for (int t = 0; t < kTile; ++t) s = fmaf(fq[t][r], nm[t][c], s);
            } else {
                for (int t = 0; t < kTile; ++t) s = fmaf(dd[t], fq[t][e - D * D], s);
            }
            A[e] += s;
        }
        __syncthreads();
    }
    // dW_ii of this (pair, block): fixed-order sum of the threads' partials
    dw = sum_over_groups(dw);
    dw += __shfl_xor(dw, 1, 64);
    dw += __shfl_xor(dw, 2, 64);
    dw += __shfl_xor(dw, 4, 64);
    dw += __shfl_xor(dw, 8, 64);
    if ((tid & 63) == 0) red[tid >> 6] = dw;
    __syncthreads();
    if (tid == 0) dWdiag[pair * M + blk] = red[0] + red[1] + red[2] + red[3];
}

// Wt[b][i] = W[i][b] for the summaries that block b feeds (causal: i > b), else 0.
__global__ __launch_bounds__(256) void bwd_wt_kernel(const float* __restrict__ W, float* __restrict__ Wt, int M,
                                                     int causal) {
    const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= (int64_t)M * M) return;
    const int b = (int)(x / M), i = (int)(x % M);
    Wt[x] = (!causal || i > b) ? W[(int64_t)i * M + b] : 0.f;
}

// dk, dv for one (pair, key block b) from dS_b, dz_b (causal: added to the
// within-block partials the query kernel left in dK, dV).
template <int D, typename T, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_key_kernel(const T* __restrict__ K, const T* __restrict__ V,
                                                      const float* __restrict__ dS, float* __restrict__ dK,
                                                      float* __restrict__ dV, int64_t BH, int N, int M) {
    constexpr int L = D * D + D;
    constexpr int OPT = kTile * D / 256;
    __shared__ float G[L], fk[kTile][D], vv[kTile][D];
    const int tid = threadIdx.x;
    const int64_t unit = blockIdx.x;
    const int64_t pair = unit / M;
    const int blk = (int)(unit % M);
    const int C = N / M;
    const int64_t base = pair * N + (int64_t)blk * C;
    const float* g = dS + ((int64_t)blk * BH + pair) * L;
    for (int e = tid; e < L; e += 256) G[e] = g[e];
    __syncthreads();
    for (int t0 = 0; t0 < C; t0 += kTile) {
        for (int x = tid; x < kTile * D; x += 256) {
            const int t = x / D, r = x % D;
            const bool ok = t0 + t < C;
            const int64_t row = (base + t0 + t) * D + r;
            fk[t][r] = ok ? phi_precise(in_val<T>(K, row)) : 0.f;
            vv[t][r] = ok ? in_val<T>(V, row) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int o = 0; o < OPT; ++o) {
            const int x = tid + 256 * o, j = x / D, r = x % D;
            float s = G[D * D + r], sv = 0.f;
            for (int c = 0; c < D; ++c) {
                s = fmaf(G[r * D + c], vv[j][c], s);
                sv = fmaf(G[c * D + r], fk[j][c], sv);
            }
            if (t0 + j < C) {
                const int64_t row = (base + t0 + j) * D + r;
                if constexpr (CAUSAL) {
                    s += dK[row];
                    sv += dV[row];
                }
                dK[row] = s * dphi(in_val<T>(K, row));
                dV[row] = sv;
            }
        }
        __syncthreads();
    }
}

// dW partials: workgroup (tile of 16 x 16 (i, b), column chunk) sums dSt[i][col] S[b][col].
__global__ __launch_bounds__(256) void bwd_dw_partial_kernel(const float* __restrict__ dSt,
                                                             const float* __restrict__ S, float* __restrict__ part,
                                                             int64_t ncols, int M, int64_t chunk, int ntiles) {
    __shared__ float a[16][65], b[16][65];
    const int tid = threadIdx.x;
    const int tile = (int)(blockIdx.x % ntiles);
    const int64_t ch = blockIdx.x / ntiles;
    const int tpr = (M + 15) / 16;
    const int i0 = 16 * (tile / tpr), b0 = 16 * (tile % tpr);
    const int il = tid / 16, bl = tid % 16;
    const int64_t c0 = ch * chunk, c1 = min(ncols, c0 + chunk);
    float s = 0.f;
    for (int64_t c = c0; c < c1; c += 64) {
        for (int x = tid; x < 16 * 64; x += 256) {
            const int rr = x / 64, cc = x % 64;
            const int64_t col = c + cc;
            a[rr][cc] = (i0 + rr < M && col < c1) ? dSt[(int64_t)(i0 + rr) * ncols + col] : 0.f;
            b[rr][cc] = (b0 + rr < M && col < c1) ? S[(int64_t)(b0 + rr) * ncols + col] : 0.f;
        }
        __syncthreads();
        for (int cc = 0; cc < 64; ++cc) s = fmaf(a[il][cc], b[bl][cc], s);
        __syncthreads();
    }
    if (i0 + il < M && b0 + bl < M) part[(ch * M + i0 + il) * (int64_t)M + b0 + bl] = s;
}

// dW[i][b] = sum over chunks (fixed order); causal: b < i only, plus the diagonal
// from the within-block partials of every pair.
__global__ __launch_bounds__(256) void bwd_dw_reduce_kernel(const float* __restrict__ part,
                                                            const float* __restrict__ dWdiag, float* __restrict__ dW,
                                                            int M, int64_t nchunks, int64_t BH, int causal) {
    const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= (int64_t)M * M) return;
    const int i = (int)(x / M), b = (int)(x % M);
    float s = 0.f;
    if (!causal || b < i)
        for (int64_t ch = 0; ch < nchunks; ++ch) s += part[ch * M * M + x];
    if (causal && b == i)
        for (int64_t p = 0; p < BH; ++p) s += dWdiag[p * M + i];
    dW[x] = s;
}

size_t backward_dw_chunk(int64_t ncols) { return ncols >= (1 << 16) ? 4096 : 1024; }

hipError_t launch_backward(int dtype, const void* q, const void* k, const void* v, const float* W, const float* dy,
                           float* dq, float* dk, float* dv, float* dW, int64_t BH, int64_t N, int D, int64_t M,
                           bool causal, float* ws, void* frag_ws, hipStream_t stream) {
    const int64_t L = (int64_t)D * D + D;
    const int64_t arr = M * BH * L;
    float* S = ws;
    float* St = S + arr;
    float* dSt = St + arr;
    float* dS = dSt + arr;
    float* Wt = dS + arr;
    float* G = Wt + M * M;                        // causal: dnum, dden per token
    float* dWdiag = G + (causal ? BH * N * (D + 1) : 0);
    float* part = dWdiag + BH * M;
    const int64_t ncols = BH * L;
    const int64_t chunk = (int64_t)backward_dw_chunk(ncols);
    const int64_t nchunks = (ncols + chunk - 1) / chunk;
    const int ntiles = (int)(((M + 15) / 16) * ((M + 15) / 16));
    const dim3 units((unsigned)(BH * M)), block(256);
    hipError_t e;
#define MHLA_BWD_D(T, DD)                                                                                        \
    do {                                                                                                         \
        const T* qq = (const T*)q;                                                                               \
        const T* kk = (const T*)k;                                                                               \
        const T* vv = (const T*)v;                                                                               \
        bwd_summary_kernel<DD, T><<<units, block, 0, stream>>>(kk, vv, S, BH, (int)N, (int)M);                  \
        if ((e = hipGetLastError()) != hipSuccess) return e;                                                     \
        if ((e = launch_mix(S, W, St, BH, DD, M, causal, false, 0, frag_ws, stream)) != hipSuccess) return e;       \
        if (causal)                                                                                              \
            bwd_query_kernel<DD, T, true><<<units, block, 0, stream>>>(qq, kk, vv, dy, W, St, dSt, G, dq, dk, dv, \
                                                                       dWdiag, BH, (int)N, (int)M);              \
        else                                                                                                     \
            bwd_query_kernel<DD, T, false><<<units, block, 0, stream>>>(qq, kk, vv, dy, W, St, dSt, G, dq, dk,    \
                                                                        dv, dWdiag, BH, (int)N, (int)M);         \
        if ((e = hipGetLastError()) != hipSuccess) return e;                                                     \
        bwd_wt_kernel<<<dim3((unsigned)((M * M + 255) / 256)), block, 0, stream>>>(W, Wt, (int)M, causal);      \
        if ((e = hipGetLastError()) != hipSuccess) return e;                                                     \
        if ((e = launch_mix(dSt, Wt, dS, BH, DD, M, false, false, 0, frag_ws, stream)) != hipSuccess) return e;     \
        if (causal)                                                                                              \
            bwd_key_kernel<DD, T, true><<<units, block, 0, stream>>>(kk, vv, dS, dk, dv, BH, (int)N, (int)M);   \
        else                                                                                                     \
            bwd_key_kernel<DD, T, false><<<units, block, 0, stream>>>(kk, vv, dS, dk, dv, BH, (int)N, (int)M);  \
        if ((e = hipGetLastError()) != hipSuccess) return e;                                                     \
    } while (0)
#define MHLA_BWD(T)                         \
    switch (D) {                            \
        case 16: MHLA_BWD_D(T, 16); break;  \
        case 32: MHLA_BWD_D(T, 32); break;  \
        case 64: MHLA_BWD_D(T, 64); break;  \
        default: return hipErrorInvalidValue; \
    }
    if (dtype == kDtypeF32) {
        MHLA_BWD(float);
    } else {
        MHLA_BWD(uint16_t);
    }
#undef MHLA_BWD
#undef MHLA_BWD_D
    bwd_dw_partial_kernel<<<dim3((unsigned)(nchunks * ntiles)), block, 0, stream>>>(dSt, S, part, ncols, (int)M, chunk,
                                                                                    ntiles);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    bwd_dw_reduce_kernel<<<dim3((unsigned)((M * M + 255) / 256)), block, 0, stream>>>(part, dWdiag, dW, (int)M, nchunks,
                                                                                      BH, causal ? 1 : 0);
    return hipGetLastError();
}

size_t backward_workspace_floats(int64_t BH, int64_t N, int D, int64_t M, bool causal) {
    const int64_t L = (int64_t)D * D + D;
    const int64_t ncols = BH * L;
    const int64_t chunk = (int64_t)backward_dw_chunk(ncols);
    const int64_t nchunks = (ncols + chunk - 1) / chunk;
    return (size_t)(4 * M * BH * L + M * M + (causal ? BH * N * (D + 1) : 0) + BH * M + nchunks * M * M);
}

}  // namespace mhla
