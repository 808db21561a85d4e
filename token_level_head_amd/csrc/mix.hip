// mix.hip -- stage 2 of the MHLA forward pass: multi-head mixing of the block
// summaries ("MHLA: Restoring Expressivity of Linear Attention via Token-Level
// Multi-Head", §4.1: S~_i = sum_b m_{i,b} S_b and z~_i = sum_b m_{i,b} z_b, done
// as one GEMM with the coefficient matrix M_c; App. C: causal mixing over b < i).
//
// With the summaries stored block-major, S[b][pair][d*d + d], all pairs share
// one GEMM:  St (M x ncols) = W (M x M) * S (M x ncols),  ncols = BH * (d*d + d).
// The reduction depth is M (16 to 256) and ncols is large, so each wave owns a
// 64-column strip and up to 64 output rows.  The S strip is read with 16-byte
// loads (four columns per lane; MFMA j of the four uses column 4n + j), split
// into bf16 hi + lo parts, and multiplied on 16x16x32 bf16 MFMA as
// W_hi S_hi + W_hi S_lo + W_lo S_hi with float32 accumulation (about 16
// significant bits per operand, well inside the float32 summaries' needs).
// The float32 path uses plain float32 FMAs instead.
#include "common.hpp"
#include "kernels.hpp"

namespace mhla {

template <bool CAUSAL>
__global__ __launch_bounds__(256) void mix_split_kernel(const float* __restrict__ S, const float* __restrict__ W,
                                                        float* __restrict__ St, int64_t ncols, int M, int RG,
                                                        int64_t ntiles) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, n = lane & 15;
    const int64_t w = (int64_t)blockIdx.x * 4 + wave;
    const int rg = (int)(w % RG);
    const int64_t ct = w / RG;
    if (ct >= ntiles) return;  // whole wave; no barriers in this kernel

    const int64_t col = ct * 64 + 4 * n;
    const bool colok = col < ncols;
    const int i0 = rg * 64;
    const int imax = min(M, i0 + 64);        // rows [i0, imax)
    const int kend = CAUSAL ? imax - 1 : M;  // causal rows use b < i <= imax - 1

    f32x4 acc[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[r][j] = zero4();

    for (int kb = 0; kb < kend; kb += 32) {
        f32x4 sv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int b = kb + 8 * g + e;
            sv[e] = (b < kend && colok) ? *reinterpret_cast<const f32x4*>(S + (int64_t)b * ncols + col) : zero4();
        }
        bf16x8 bh[4], bl[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const bf16pair h = split_bf16(sv[e][j]);
                bh[j][e] = h.hi;
                bl[j][e] = h.lo;
            }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ibase = i0 + 16 * r;
            if (ibase < imax) {  // uniform across the wave
                const int i = ibase + n;
                bf16x8 ah, al;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int b = kb + 8 * g + e;
                    const bool use = i < M && b < kend && (!CAUSAL || b < i);
                    const bf16pair h = split_bf16(use ? W[(int64_t)i * M + b] : 0.f);
                    ah[e] = h.hi;
                    al[e] = h.lo;
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc[r][j] = mfma32(ah, bh[j], acc[r][j]);
                    acc[r][j] = mfma32(ah, bl[j], acc[r][j]);
                    acc[r][j] = mfma32(al, bh[j], acc[r][j]);
                }
            }
        }
    }
    if (!colok) return;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = i0 + 16 * r + 4 * g + i;
            if (row < imax)
                *reinterpret_cast<f32x4*>(St + (int64_t)row * ncols + col) =
                    f32x4{acc[r][0][i], acc[r][1][i], acc[r][2][i], acc[r][3][i]};
        }
    }
}

// float32 path: one thread per four columns, float32 FMAs in a fixed order.
__global__ __launch_bounds__(256) void mix_f32_kernel(const float* __restrict__ S, const float* __restrict__ W,
                                                      float* __restrict__ St, int64_t ncols, int M, int causal) {
    const int64_t col = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (col >= ncols) return;
    for (int i = 0; i < M; ++i) {
        f32x4 acc = zero4();
        const int bend = causal ? i : M;
        for (int b = 0; b < bend; ++b) {
            const float wv = W[(int64_t)i * M + b];
            const f32x4 s = *reinterpret_cast<const f32x4*>(S + (int64_t)b * ncols + col);
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] = fmaf(wv, s[c], acc[c]);
        }
        *reinterpret_cast<f32x4*>(St + (int64_t)i * ncols + col) = acc;
    }
}

hipError_t launch_mix(const float* S, const float* W, float* St, int64_t BH, int D, int64_t M, bool causal,
                      bool precise, hipStream_t stream) {
    const int64_t ncols = BH * (int64_t)(D * D + D);
    if (precise) {
        const int64_t threads = ncols / 4;
        mix_f32_kernel<<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream>>>(S, W, St, ncols, (int)M,
                                                                                        causal ? 1 : 0);
        return hipGetLastError();
    }
    const int64_t ntiles = (ncols + 63) / 64;
    const int RG = (int)((M + 63) / 64);
    const int64_t waves = ntiles * RG;
    const dim3 grid((unsigned)((waves + 3) / 4));
    if (causal)
        mix_split_kernel<true><<<grid, dim3(256), 0, stream>>>(S, W, St, ncols, (int)M, RG, ntiles);
    else
        mix_split_kernel<false><<<grid, dim3(256), 0, stream>>>(S, W, St, ncols, (int)M, RG, ntiles);
    return hipGetLastError();
}

}  // namespace mhla
