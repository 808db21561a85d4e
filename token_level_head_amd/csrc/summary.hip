// summary.hip -- stage 1 of the MHLA forward pass: phi(K) fused with the
// per-block KV summaries ("MHLA: Restoring Expressivity of Linear Attention via
// Token-Level Multi-Head", §4.1: S_b = sum_{j in b} phi(k_j) v_j^T, z_b = sum phi(k_j)).
//
// bf16 path.  S_b = phi(K_b)^T V_b is a d x d product whose reduction runs over
// tokens, while K and V are stored token-major.  Instead of transposing tiles
// through LDS, each lane loads P = d/16 consecutive features of 8 tokens (one
// 8-byte load per token for d = 64; 16 lanes cover a whole 128-byte row) and
// repacks them in registers: MFMA (ia, ib) of the P x P set treats its row m as
// feature P*m + ia and its column n as value column P*n + ib.  The accumulators
// then hold S in the packed layout of common.hpp, which is written with
// full-wave 1 KiB stores.  phi(k) is rounded to bf16 once; the same rounded
// values feed both S_b and z_b so numerator and denominator stay consistent.
// Accumulation is float32 in the MFMA accumulators.
//
// A block of C tokens may be split over `wpb` waves of one workgroup
// (wpb in {1, 2, 4}); their partial sums are added in LDS in a fixed order, so
// results do not depend on scheduling.
#include "common.hpp"
#include "kernels.hpp"

namespace mhla {

template <int P>
__device__ __forceinline__ void load_feat(const uint16_t* p, bool ok, const uint16_t* safe, uint16_t (&out)[P]) {
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

template <int D>
__global__ __launch_bounds__(256) void summaries_bf16_kernel(const uint16_t* __restrict__ K,
                                                             const uint16_t* __restrict__ V,
                                                             float* __restrict__ S, int64_t BH, int64_t N,
                                                             int64_t M, int wpb) {
    constexpr int P = D / 16;
    constexpr int L = D * D + D;
    extern __shared__ float red[];  // (4 - 4/wpb) partial results of 64 lanes x (4P^2 + P) floats

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, n = lane & 15;
    const int per_wg = 4 / wpb;
    const int64_t unit = (int64_t)blockIdx.x * per_wg + wave / wpb;  // unit = pair * M + block
    const int seg = wave % wpb;
    const bool active = unit < BH * M;
    const int64_t C = N / M;

    f32x4 acc[P][P];
#pragma unroll
    for (int a = 0; a < P; ++a)
#pragma unroll
        for (int b = 0; b < P; ++b) acc[a][b] = zero4();
    float zacc[P];
#pragma unroll
    for (int a = 0; a < P; ++a) zacc[a] = 0.f;

    int64_t pair = 0, blk = 0;
    if (active) {
        pair = unit / M;
        blk = unit % M;
        const int64_t seg_len = ((C + wpb - 1) / wpb + 31) / 32 * 32;
        const int64_t t_beg = blk * C + seg * seg_len;
        const int64_t t_end = min(blk * C + C, t_beg + seg_len);
        const uint16_t* Kp = K + pair * N * D + P * n;
        const uint16_t* Vp = V + pair * N * D + P * n;
        for (int64_t t = t_beg; t < t_end; t += 32) {
            uint16_t kr[8][P], vr[8][P];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int64_t tok = t + 8 * g + e;
                const bool ok = tok < t_end;
                load_feat<P>(Kp + tok * D, ok, K, kr[e]);
                load_feat<P>(Vp + tok * D, ok, V, vr[e]);
            }
            issue_fence();
            bf16x8 a[P], b[P];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const bool ok = t + 8 * g + e < t_end;
#pragma unroll
                for (int f = 0; f < P; ++f) {
                    const __bf16 ph = (__bf16)(ok ? phi_fast(bf16_to_f32(kr[e][f])) : 0.f);
                    a[f][e] = ph;
                    zacc[f] += bf16v_to_f32(ph);
                    b[f][e] = bits_to_bf16(vr[e][f]);
                }
            }
#pragma unroll
            for (int ia = 0; ia < P; ++ia)
#pragma unroll
                for (int ib = 0; ib < P; ++ib) acc[ia][ib] = mfma32(a[ia], b[ib], acc[ia][ib]);
        }
    }
    // z: sum the four token groups; lanes (., n) then hold z[P*n + f].
#pragma unroll
    for (int f = 0; f < P; ++f) zacc[f] = sum_over_groups(zacc[f]);

    if (wpb > 1) {
        constexpr int PER_LANE = 4 * P * P + P;
        const int unit_in_wg = wave / wpb;
        if (seg > 0) {
            float* dst = red + ((size_t)(unit_in_wg * (wpb - 1) + seg - 1) * 64 + lane) * PER_LANE;
#pragma unroll
            for (int a = 0; a < P; ++a)
#pragma unroll
                for (int b = 0; b < P; ++b)
#pragma unroll
                    for (int i = 0; i < 4; ++i) dst[(a * P + b) * 4 + i] = acc[a][b][i];
#pragma unroll
            for (int f = 0; f < P; ++f) dst[4 * P * P + f] = zacc[f];
        }
        __syncthreads();
        if (seg == 0) {
            for (int s = 1; s < wpb; ++s) {
                const float* src = red + ((size_t)(unit_in_wg * (wpb - 1) + s - 1) * 64 + lane) * PER_LANE;
#pragma unroll
                for (int a = 0; a < P; ++a)
#pragma unroll
                    for (int b = 0; b < P; ++b)
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[a][b][i] += src[(a * P + b) * 4 + i];
#pragma unroll
                for (int f = 0; f < P; ++f) zacc[f] += src[4 * P * P + f];
            }
        }
    }
    if (!active || seg != 0) return;

    float* out = S + (blk * BH + pair) * (int64_t)L;
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
                                                            int64_t M, int D) {
    const int64_t unit = blockIdx.x;  // pair * M + block
    const int64_t pair = unit / M, blk = unit % M;
    const int64_t C = N / M;
    const int P = D / 16, L = D * D + D;
    const float* Kp = K + (pair * N + blk * C) * D;
    const float* Vp = V + (pair * N + blk * C) * D;
    float* out = S + (blk * BH + pair) * (int64_t)L;
    for (int e = threadIdx.x; e < L; e += blockDim.x) {
        float acc = 0.f;
        if (e < D * D) {
            const int chunk = e / 256, rem = e % 256, ln = rem / 4, i = rem % 4;
            const int ia = chunk / P, ib = chunk % P;
            const int r = P * (4 * (ln / 16) + i) + ia, c = P * (ln % 16) + ib;
            for (int64_t j = 0; j < C; ++j) acc = fmaf(phi_precise(Kp[j * D + r]), Vp[j * D + c], acc);
        } else {
            const int r = e - D * D;
            for (int64_t j = 0; j < C; ++j) acc += phi_precise(Kp[j * D + r]);
        }
        out[e] = acc;
    }
}

hipError_t launch_summaries(int dtype, const void* k, const void* v, float* S, int64_t BH, int64_t N,
                            int D, int64_t M, hipStream_t stream) {
    const int64_t units = BH * M;
    if (dtype == kDtypeF32) {
        summaries_f32_kernel<<<dim3((unsigned)units), dim3(256), 0, stream>>>(
            (const float*)k, (const float*)v, S, BH, N, M, D);
        return hipGetLastError();
    }
    const int64_t C = N / M;
    const int wpb = C >= 256 ? 4 : (C >= 128 ? 2 : 1);
    const int per_wg = 4 / wpb;
    const int64_t grid = (units + per_wg - 1) / per_wg;
    const int P = D / 16;
    const size_t lds = wpb > 1 ? (size_t)(4 - per_wg) * 64 * (4 * P * P + P) * sizeof(float) : 0;
    const uint16_t* kk = (const uint16_t*)k;
    const uint16_t* vv = (const uint16_t*)v;
    switch (D) {
        case 16: summaries_bf16_kernel<16><<<dim3((unsigned)grid), dim3(256), lds, stream>>>(kk, vv, S, BH, N, M, wpb); break;
        case 32: summaries_bf16_kernel<32><<<dim3((unsigned)grid), dim3(256), lds, stream>>>(kk, vv, S, BH, N, M, wpb); break;
        case 64: summaries_bf16_kernel<64><<<dim3((unsigned)grid), dim3(256), lds, stream>>>(kk, vv, S, BH, N, M, wpb); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace mhla
