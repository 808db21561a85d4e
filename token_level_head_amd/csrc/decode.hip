// decode.hip -- streaming causal decoding, one token per call ("MHLA: Restoring
// Expressivity of Linear Attention via Token-Level Multi-Head", App. C inference:
// fold token t into its block's running summary, re-mix, read out; the running
// sum is the recurrence of "Linear Attention 笔记" §4, guard as in §4/§5).
//
// State per (batch, head) pair, float32, each vector d*d + d long (S[r][c] with
// S[r][c] = sum phi(k)[r] v[c], stored by 16-column groups as described at the
// token kernel, then z[r]):
//   St    mixed summary of the current block's predecessors, S~_i and z~_i
//   P     running summary of the current block up to the last token (P, p)
//   p2    a second copy of p: token t reads p from P when t is even and from p2
//         when t is odd and writes the other one, so the d/16 workgroups of a
//         pair never read a p that another of them has already updated
//   hist  summaries of the completed blocks 0 .. M-2
// Token t belongs to block i = t / C.  When t % C == 0 the step first closes block
// i - 1 (P goes to hist[i-1] and is reset) and forms St = sum_{b<i} W[i,b] hist[b];
// then every token adds phi(k_t) v_t^T to P and writes
//   y_t = phi(q_t)(St + W[i,i] P) / (phi(q_t)(z~ + W[i,i] p) + 1e-6),
// which is row t of the causal forward pass (without the normaliser, §4.1's remark
// on the output: the numerator alone).  W may be one matrix per head.  All arithmetic is float32 (phi with
// the full-precision exp), in a fixed order: results are bit-reproducible.
#include "common.hpp"
#include "kernels.hpp"

namespace mhla {

namespace {

template <typename T>
__device__ __forceinline__ float load_in(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_in<uint16_t>(const uint16_t* p, int64_t i) {
    return bf16_to_f32(p[i]);
}
template <>
__device__ __forceinline__ float load_in<float>(const float* p, int64_t i) {
    return p[i];
}

}  // namespace

// Closing block i - 1 and mixing for block i: one thread per (pair, entry).
__global__ __launch_bounds__(256) void decode_advance_kernel(const float* __restrict__ W, float* __restrict__ state,
                                                             int64_t BH, int D, int M, int i, int first, int odd,
                                                             int heads) {
    const int64_t L = (int64_t)D * D + D;
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // pair * L + entry
    if (e >= BH * L) return;
    float* St = state;
    float* P = state + BH * L;
    float* p2 = state + 2 * BH * L;
    float* hist = p2 + BH * D;
    const int64_t pair = e / L, ent = e % L;
    if (heads > 0) W += (pair % heads) * M * M;  // one matrix per head
    // p of an odd token index lives in p2 (see the state description above)
    float* src = (odd && ent >= (int64_t)D * D) ? p2 + pair * D + (ent - (int64_t)D * D) : P + e;
    float x = 0.f;
    if (!first) {
        x = *src;
        hist[(int64_t)(i - 1) * BH * L + e] = x;
    }
    *src = 0.f;
    float acc = 0.f;
    for (int b = 0; b + 1 < i; ++b) acc = fmaf(W[(int64_t)i * M + b], hist[(int64_t)b * BH * L + e], acc);
    if (i >= 1) acc = fmaf(W[(int64_t)i * M + i - 1], x, acc);
    St[e] = acc;
}

// One token.  The d x d part of each state vector is stored by groups of 16 value
// columns, [c / 16][r][c % 16], so that the workgroup owning one column group of
// one pair reads and writes one contiguous span; z follows in plain order.  The
// d/16 workgroups of a pair are numbered to run on one XCD (they all read the
// pair's q, k, z~ and p).  Thread (c, rg) owns column c of the group and rows
// rg*RPT .. rg*RPT + RPT - 1.
template <int D, typename T>
__global__ __launch_bounds__(256) void decode_token_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                           const T* __restrict__ v, const float* __restrict__ W,
                                                           float* __restrict__ state, float* __restrict__ out,
                                                           int64_t BH, int M, int i, int odd, int norm, int heads) {
    constexpr int L = D * D + D;
    constexpr int CG = D / 16;  // column groups (workgroups) per pair
    constexpr int RPT = D / 16; // rows per thread: 16 row groups of 16 threads
    __shared__ float fq[D], fk[D], fv[16], part[4][16], sden;
    const int tid = threadIdx.x;
    const int64_t bid = blockIdx.x;
    const int cg = (int)((bid >> 3) % CG);
    const int64_t pair = ((bid >> 3) / CG) * 8 + (bid & 7);
    if (pair >= BH) return;  // uniform over the workgroup
    float* St = state + pair * L;
    float* P = state + BH * L + pair * L;
    float* p2 = state + 2 * BH * L + pair * D;
    const float* pin = odd ? p2 : P + D * D;  // p after the previous token
    float* pout = odd ? P + D * D : p2;       // p after this one
    if (heads > 0) W += (pair % heads) * M * M;  // one matrix per head
    const float wii = W[(int64_t)i * M + i];

    // The state this thread updates and reads, loaded before the token's features so
    // that both loads are in flight together (the state does not depend on them).
    const int c = tid & 15, rg = tid >> 4;
    const int base = cg * 16 * D;  // this column group's span
    float pv[RPT], sv[RPT];
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) {
        const int e = base + (rg * RPT + rr) * 16 + c;
        pv[rr] = P[e];
        sv[rr] = St[e];
    }
    float zv = 0.f, pz0 = 0.f;
    if (tid < D) {
        zv = St[D * D + tid];
        pz0 = pin[tid];
    }
    if (tid < D) {
        fq[tid] = phi_precise(load_in<T>(q, pair * D + tid));
        fk[tid] = phi_precise(load_in<T>(k, pair * D + tid));
    } else if (tid < D + 16) {
        fv[tid - D] = load_in<T>(v, pair * D + 16 * cg + tid - D);
    }
    __syncthreads();

    float num = 0.f;
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) {
        const int r = rg * RPT + rr;
        const int e = base + r * 16 + c;
        const float pn = fmaf(fk[r], fv[c], pv[rr]);
        P[e] = pn;
        num = fmaf(fq[r], fmaf(wii, pn, sv[rr]), num);
    }
    // numerator of column c: the four row groups of each wave by lane exchange, then the
    // four waves' parts in wave order
    num += __shfl_xor(num, 16, 64);
    num += __shfl_xor(num, 32, 64);
    if ((tid & 63) < 16) part[tid >> 6][c] = num;
    if (tid < 64) {  // normaliser: p[r] + phi(k)[r]; den = sum_r phi(q)[r] (z~[r] + W[i,i] p[r])
        float dp = 0.f;
        if (tid < D) {
            const float pz = pz0 + fk[tid];
            if (cg == 0) pout[tid] = pz;
            dp = fq[tid] * fmaf(wii, pz, zv);
        }
#pragma unroll
        for (int m = 1; m < 64; m *= 2) dp += __shfl_xor(dp, m, 64);
        if (tid == 0) sden = dp;
    }
    __syncthreads();
    if (tid < 16) {
        const float n = (part[0][tid] + part[1][tid]) + (part[2][tid] + part[3][tid]);
        out[pair * D + 16 * cg + tid] = norm ? n / (sden + kEps) : n;  // without the normaliser: the numerator
    }
}

hipError_t launch_decode_step(int dtype, const void* q, const void* k, const void* v, const float* W, float* state,
                              float* out, int64_t BH, int D, int64_t M, int64_t C, int64_t t, bool normalize,
                              int heads, hipStream_t stream) {
    const int64_t L = (int64_t)D * D + D;
    const int i = (int)(t / C);
    if (t % C == 0) {
        const int64_t total = BH * L;
        decode_advance_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream>>>(
            W, state, BH, D, (int)M, i, t == 0 ? 1 : 0, (int)(t & 1), heads);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const dim3 grid((unsigned)(((BH + 7) / 8) * 8 * (D / 16))), block(256);
#define MHLA_DECODE(DD, TT)                                                                                \
    decode_token_kernel<DD, TT><<<grid, block, 0, stream>>>((const TT*)q, (const TT*)k, (const TT*)v, W, state, \
                                                            out, BH, (int)M, i, (int)(t & 1), normalize ? 1 : 0, heads)
    if (dtype == kDtypeF32) {
        switch (D) {
            case 16: MHLA_DECODE(16, float); break;
            case 32: MHLA_DECODE(32, float); break;
            case 64: MHLA_DECODE(64, float); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (D) {
            case 16: MHLA_DECODE(16, uint16_t); break;
            case 32: MHLA_DECODE(32, uint16_t); break;
            case 64: MHLA_DECODE(64, uint16_t); break;
            default: return hipErrorInvalidValue;
        }
    }
#undef MHLA_DECODE
    return hipGetLastError();
}

}  // namespace mhla
