// common.hpp -- device helpers shared by the MHLA kernels (gfx950, wave64).
//
// MFMA operand layouts used throughout (lane l of a 64-lane wave, g = l / 16,
// n = l % 16; verified on gfx950):
//   v_mfma_f32_16x16x32_bf16 : A[m = n][k = 8g + e], B[k = 8g + e][col = n], e = 0..7
//   v_mfma_f32_16x16x16_bf16 : A[m = n][k = 4g + e], B[k = 4g + e][col = n], e = 0..3
//   result (both)            : C[row = 4g + i][col = n], i = 0..3
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"  // OutSpec

namespace mhla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kEps = 1e-6f;  // denominator guard ("Linear Attention 笔记" §4/§5)

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ __bf16 bits_to_bf16(uint16_t b) { return __builtin_bit_cast(__bf16, b); }

__device__ __forceinline__ float bf16v_to_f32(__bf16 b) {
    return __uint_as_float((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// phi(x) = ELU(x) + 1 ("Linear Attention 笔记" §2) = max(x, 0) + exp(min(x, 0)),
// formed as m + exp(x - m) with m = max(x, 0): x - m is exactly min(x, 0) for every
// finite x (x - x = 0 above zero, x - 0 = x below), and a NaN input stays NaN through
// the subtraction, where a min (IEEE maxNum/minNum: max(NaN, 0) = 0) would turn it
// into phi = 1.  For x > 0 the result is x + 1 rounded once.  No step is a product
// feeding an add, so floating-point contraction cannot fuse any two of them (fusing
// x*log2(e) into a subtraction of its own rounded value would leave that product's
// rounding error inside the exponential).
// phi_fast is for results rounded to bfloat16 afterwards: the exponential is the
// hardware exp2 of (x - m) log2(e): a max, a subtract, a multiply, exp2 and an add.
// phi_precise keeps float32 accuracy.  Both give NaN for x = NaN and x = +inf.
//
// relu0(x) = max(x, 0) as the single v_max_f32.  Written through fmaxf, the compiler
// first quiets x (a second v_max_f32 x, x) whenever x is not the result of arithmetic
// -- here it is usually a bf16 value widened by a shift -- since IEEE maxNum must not
// see a signalling NaN.  phi needs no quieting: whatever the max returns for a NaN
// (0, or a quiet NaN), the subtraction x - m is NaN and so is phi.
__device__ __forceinline__ float relu0(float x) {
    float m;
    asm("v_max_f32 %0, 0, %1" : "=v"(m) : "v"(x));
    return m;
}
__device__ __forceinline__ float phi_fast(float x) {
    const float m = relu0(x);
    return m + __builtin_amdgcn_exp2f((x - m) * 1.44269504088896341f);
}
__device__ __forceinline__ float phi_precise(float x) {
    const float m = relu0(x);
    return m + expf(x - m);
}

// Hardware reciprocal (about 1 ulp).  Every denominator here is >= 1e-6 and finite.
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi), both round-to-nearest-even:
// hi*y + lo*y carries about 16 significant bits of x into a bf16 product.
struct bf16pair {
    __bf16 hi, lo;
};
__device__ __forceinline__ bf16pair split_bf16(float x) {
    const __bf16 hi = (__bf16)x;
    return {hi, (__bf16)(x - bf16v_to_f32(hi))};
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats to packed bf16 (round-to-nearest-even), a in the low half: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// split_bf16 of two values at once, packed: hi = bf16(a) | bf16(b) << 16, lo likewise
// from a - hi_a and b - hi_b.  Each difference is exact in float32 and is formed
// by one bf16 dot product (hi . (-1, 0) + a), so the split costs two conversions
// and two dot products per pair.  The (-1, 0) and (0, -1) operands are kept in
// registers: folded to the inline constant -1.0, the packed bf16 operand reads as
// the float32 bit pattern of -1.0, i.e. (0, -1), and the wrong half is subtracted.
__device__ __forceinline__ void split2_bf16(float a, float b, uint32_t& hi, uint32_t& lo) {
    hi = pack_bf16(a, b);
    const bf16x2 h = __builtin_bit_cast(bf16x2, hi);
    uint32_t m0 = 0x0000bf80u, m1 = 0xbf800000u;  // (-1, 0), (0, -1) as packed bf16
    asm("" : "+v"(m0), "+v"(m1));
    lo = pack_bf16(__builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2, m0), a, false),
                   __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2, m1), b, false));
}

__device__ __forceinline__ f32x4 mfma32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// Factor applied to a row's numerator: 1 / (phi(q)^T z~ + eps), or 1 without the
// normaliser.  `guarded_den` already includes eps.
__device__ __forceinline__ float out_scale(const OutSpec& o, float guarded_den) {
    return o.norm ? fast_rcp(guarded_den) : 1.f;
}

// Stores of Y (element offset e), which nothing later in the pass reads: marked
// non-temporal, so that the output stream does not evict the block summaries that
// the next stage reads back from the caches.
__device__ __forceinline__ void store_out(const OutSpec& o, int64_t e, f32x4 v) {
    if (o.bf16) {
        const u32x2 w = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(static_cast<uint16_t*>(o.y) + e));
    } else {
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(static_cast<float*>(o.y) + e));
    }
}
__device__ __forceinline__ void store_out(const OutSpec& o, int64_t e, f32x2 v) {
    if (o.bf16)
        __builtin_nontemporal_store(pack_bf16(v[0], v[1]), reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(o.y) + e));
    else
        __builtin_nontemporal_store(v, reinterpret_cast<f32x2*>(static_cast<float*>(o.y) + e));
}
__device__ __forceinline__ void store_out(const OutSpec& o, int64_t e, float v) {
    if (o.bf16)
        __builtin_nontemporal_store(__builtin_bit_cast(uint16_t, (__bf16)v), static_cast<uint16_t*>(o.y) + e);
    else
        __builtin_nontemporal_store(v, static_cast<float*>(o.y) + e);
}

// Per-head mixing (heads > 0: one M x M matrix per head).  The summary arrays are
// then head-major, row head * B + batch for pair = batch * H + head, so that one
// head's summaries form a contiguous column block of the mixing GEMM; heads == 0
// means one shared matrix and batch-major rows (row = pair).
__device__ __forceinline__ int64_t summary_row(int64_t pair, int heads, int64_t BH) {
    return heads > 0 ? (pair % heads) * (BH / heads) + pair / heads : pair;
}
// The mixing matrix a (batch, head) pair uses.
__device__ __forceinline__ const float* pair_w(const float* W, int64_t pair, int heads, int64_t M) {
    return heads > 0 ? W + (pair % heads) * M * M : W;
}

// Token range [beg, end) of block b in the block layout's token list.
__device__ __forceinline__ void block_range(const BlockLayout& lay, int64_t b, int N, int64_t M, int& beg,
                                            int& end) {
    if (lay.offsets) {
        beg = min(max(lay.offsets[b], 0), N);
        end = min(max(lay.offsets[b + 1], beg), N);
    } else {
        const int C = (int)(N / M);
        beg = (int)b * C;
        end = beg + C;
    }
}
// Sequence position of list entry i of a block layout (i < N), or -1 for an entry
// outside [0, N).  Identity without a token list.
__device__ __forceinline__ int token_row(const BlockLayout& lay, int i, int N) {
    if (!lay.order) return i;
    const int r = lay.order[i];
    return (unsigned)r < (unsigned)N ? r : -1;
}

// Workgroup barrier ordering LDS accesses only.  __syncthreads() is a fence over all
// memory, which on gfx9 waits for every outstanding global load and store of the wave
// (vmcnt(0)) before the barrier; with fences scoped to LDS ("local"), only the wave's
// LDS operations are awaited, and prefetched loads and output stores stay in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Masked load without a branch: the address falls back to `safe` (any valid,
// suitably aligned element) when !ok and the bits are then cleared with an
// integer mask.  A select on the loaded value would let the compiler sink the
// load into an exec-masked branch with its own wait; this form keeps every load
// unconditional, so a whole batch is issued before the first wait.
template <int BYTES>
struct MaskBits;
template <>
struct MaskBits<2> { typedef uint16_t type; };
template <>
struct MaskBits<4> { typedef uint32_t type; };
template <>
struct MaskBits<8> { typedef uint32_t type __attribute__((ext_vector_type(2))); };
template <>
struct MaskBits<16> { typedef uint32_t type __attribute__((ext_vector_type(4))); };

// Raw buffer access (gfx9 family): a scalar resource descriptor over `bytes` bytes
// from `base`, addressed with 32-bit byte offsets in a vector register.  A load
// whose offset lies at or beyond `bytes` returns zero and touches no memory, so
// masked loads need neither a branch nor a select, and no 64-bit address
// arithmetic is spent per lane.  Word 3 = 0x00020000 selects untyped 32-bit
// data (no swizzle, no per-lane index).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;  // any offset at or past the end reads zero

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint32_t off_if(bool ok, uint32_t byte_off) { return ok ? byte_off : kOutOfRange; }

// NT selects the non-temporal policy (for token inputs streamed once; see
// stream_token_inputs in kernels.hpp).
template <bool NT = false>
__device__ __forceinline__ uint16_t buf_load16(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, NT ? 2 : 0);
}
template <bool NT = false>
__device__ __forceinline__ uint32_t buf_load32(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, NT ? 2 : 0);
}
template <bool NT = false>
__device__ __forceinline__ u32x2 buf_load64(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, NT ? 2 : 0));
}
template <bool NT = false>
__device__ __forceinline__ u32x4 buf_load128(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, NT ? 2 : 0));
}

// Keeps the scheduler from moving instructions across this point; placed after a
// batch of loads so that the whole batch is issued before its consumers run
// (otherwise the scheduler may serialise the loads to save registers).
__device__ __forceinline__ void issue_fence() { __builtin_amdgcn_sched_barrier(0); }

template <typename T>
__device__ __forceinline__ T load_or_zero(const T* p, bool ok, const T* safe) {
    using U = typename MaskBits<sizeof(T)>::type;
    const U v = __builtin_bit_cast(U, *(ok ? p : safe));
    return __builtin_bit_cast(T, (U)(v & (U)(ok ? ~0u : 0u)));
}
// The same for token inputs (Q, K, V); NT as for the buffer loads.
template <bool NT, typename T>
__device__ __forceinline__ T load_token_or_zero(const T* p, bool ok, const T* safe) {
    using U = typename MaskBits<sizeof(T)>::type;
    const U* q = reinterpret_cast<const U*>(ok ? p : safe);
    const U v = NT ? __builtin_nontemporal_load(q) : *q;
    return __builtin_bit_cast(T, (U)(v & (U)(ok ? ~0u : 0u)));
}

// Sum over the four 16-lane groups (lanes n, n+16, n+32, n+48).
__device__ __forceinline__ float sum_over_groups(float x) {
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    return x;
}

// Packed summary layout (shared by all three kernels).  For d = 16P the d x d part
// of a summary vector is stored as P*P chunks of 64 lanes x 4 floats: chunk
// (ia, ib) of lane l = 16g + n holds S[P*(4g + i) + ia][P*n + ib] for i = 0..3 at
// float offset (ia*P + ib)*256 + l*4 + i.  This is exactly the result layout of
// the summary MFMAs, and also exactly the B-operand set the output kernel needs
// in the same lane, so neither kernel moves data across lanes.  z follows at
// offset d*d in plain order.
__host__ __device__ __forceinline__ int64_t packed_index(int P, int r, int c) {
    const int ia = r % P, q = r / P, g = q / 4, i = q % 4;
    const int n = c / P, ib = c % P;
    return (int64_t)(ia * P + ib) * 256 + (int64_t)(16 * g + n) * 4 + i;
}

}  // namespace mhla
