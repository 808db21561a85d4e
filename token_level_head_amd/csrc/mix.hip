// mix.hip -- stage 2 of the MHLA forward pass: multi-head mixing of the block
// summaries ("MHLA: Restoring Expressivity of Linear Attention via Token-Level
// Multi-Head", §4.1: S~_i = sum_b m_{i,b} S_b and z~_i = sum_b m_{i,b} z_b, done
// as one GEMM with the coefficient matrix M_c; App. C: causal mixing over b < i).
//
// With the summaries stored block-major, S[b][pair][d*d + d], all pairs share
// one GEMM:  St (M x ncols) = W (M x M) * S (M x ncols),  ncols = BH * (d*d + d).
// The reduction depth is M and ncols is large, so each wave owns a strip of
// 16*J columns (J = 2 or 4 consecutive columns per lane, read with 8- or
// 16-byte loads; MFMA j uses column J*n + j) and 16*RT output rows.  Both
// operands are split into bf16 hi + lo parts and multiplied on bf16 MFMA as
// W_hi S_hi + W_hi S_lo + W_lo S_hi with float32 accumulation (about 16
// significant bits per operand, well inside the float32 summaries' needs).
//
// W is split into per-lane MFMA fragments (causal mask applied there).  For
// M <= 64 each workgroup does that itself into LDS; for 64 < M <= 256 each wave
// splits its rows of W in registers as it streams them from L2 (the strip of S
// is what lives in LDS); for larger M a small kernel does it once per call and
// the mixing waves read their fragments as coalesced 16-byte loads that stay in
// L2, prefetched one k-chunk ahead together with S.
// In both kernels the next k-chunk of S is loaded while the current one is
// multiplied.  A single block (M = 1) is a plain float32 scale.  Workgroups that share a column strip (different row groups) are
// numbered so that they land on the same XCD and share its L2.  The float32
// path uses plain float32 FMAs instead.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace mhla {

namespace {

constexpr int64_t kMaxFragM = 1024;  // larger M uses the fragment-free fallback kernel
constexpr int kWideMaxNT = 8;        // 64 < M <= 256 kernel: column tiles of 16 per workgroup
constexpr int kWideMaxKC = 8;        // ... k-chunks of 32 (M <= 256)
constexpr int kWideTasks = 2;        // ... strip-load tasks per thread: 16 * KC * NT / 512
constexpr int kWideRT = 2;           // ... row tiles of 16 per wave (8 waves: 256 rows)
constexpr int kWalkPerCU = 2;       // 32 < M <= 64 kernel: persistent workgroups of four waves per CU
constexpr int kWalkJ = 4;           // ... columns per lane (a wave's tile: 16 J columns)

template <int KSTEP>
struct MixOps;
template <>
struct MixOps<32> {
    typedef bf16x8 frag;
    static constexpr int E = 8;
    static __device__ __forceinline__ f32x4 mma(const frag& a, const frag& b, const f32x4& c) { return mfma32(a, b, c); }
};
template <>
struct MixOps<16> {
    typedef bf16x4 frag;
    static constexpr int E = 4;
    static __device__ __forceinline__ f32x4 mma(const frag& a, const frag& b, const f32x4& c) { return mfma16(a, b, c); }
};

}  // namespace

size_t mix_fragment_bytes(int64_t M) {
    if (M <= 256 || M > kMaxFragM) return 0;  // M <= 256 splits W in LDS or registers; huge M in every wave
    const int64_t RG = (M + 63) / 64, KC = (M + 31) / 32;  // RT = 4, 32-deep k-chunks
    return (size_t)(RG * 4 * KC * 64 * 2) * 16;
}

// One thread per (row group, row tile, k-chunk, lane) slot: the hi and lo
// fragments of W that lane feeds to the MFMA A operand.
template <int KSTEP, int RT, bool CAUSAL>
__global__ __launch_bounds__(256) void wsplit_kernel(const float* __restrict__ W,
                                                     typename MixOps<KSTEP>::frag* __restrict__ frags, int M,
                                                     int RG, int KC) {
    using frag = typename MixOps<KSTEP>::frag;
    constexpr int E = MixOps<KSTEP>::E;
    W += (int64_t)blockIdx.y * M * M;  // grid row y: one head's W and fragments
    frags += (int64_t)blockIdx.y * 2 * RG * RT * KC * 64;
    const int64_t slot = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (slot >= (int64_t)RG * RT * KC * 64) return;
    const int ln = (int)(slot & 63);
    const int64_t t = slot >> 6;
    const int kc = (int)(t % KC);
    const int rrt = (int)(t / KC);  // rg * RT + rt
    const int i = 16 * rrt + (ln & 15);
    const int b0 = kc * KSTEP + E * (ln >> 4);
    frag h, l;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int b = b0 + e;
        const bool use = i < M && b < M && (!CAUSAL || b < i);
        const bf16pair p = split_bf16(load_or_zero(W + (int64_t)i * M + b, use, W));
        h[e] = p.hi;
        l[e] = p.lo;
    }
    frags[2 * slot] = h;
    frags[2 * slot + 1] = l;
}

template <int J>
__device__ __forceinline__ void load_cols(const float* p, bool ok, const float* safe, float (&v)[J]) {
    if constexpr (J == 4) {
        const f32x4 x = load_or_zero(reinterpret_cast<const f32x4*>(p), ok, reinterpret_cast<const f32x4*>(safe));
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = x[j];
    } else {
        const float2 x = load_or_zero(reinterpret_cast<const float2*>(p), ok, reinterpret_cast<const float2*>(safe));
        v[0] = x.x;
        v[1] = x.y;
    }
}

template <int KSTEP, int RT, int J, bool CAUSAL>
__global__ __launch_bounds__(256) void mix_frag_kernel(const float* __restrict__ S,
                                                       const typename MixOps<KSTEP>::frag* __restrict__ frags,
                                                       float* __restrict__ St, int64_t ncols, int64_t ld, int M, int RG,
                                                       int64_t ntiles, int KC) {
    // Grid row y: one head's contiguous column block (head-major summaries) and its W.
    S += (int64_t)blockIdx.y * ncols;
    St += (int64_t)blockIdx.y * ncols;
    frags += (int64_t)blockIdx.y * 2 * RG * RT * KC * 64;  // hi and lo per slot
    using Ops = MixOps<KSTEP>;
    using frag = typename Ops::frag;
    constexpr int E = Ops::E;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, n = lane & 15;
    // Workgroup b runs on XCD b % 8; the RG workgroups of one column group share that XCD.
    const int64_t b = blockIdx.x;
    const int rg = (int)((b >> 3) % RG);
    const int64_t ctg = ((b >> 3) / RG) * 8 + (b & 7);
    const int64_t ct = ctg * 4 + wave;
    if (ct >= ntiles) return;  // whole wave; no barriers in this kernel

    const int i0 = rg * 16 * RT;
    const int imax = min(M, i0 + 16 * RT);
    const int kend = CAUSAL ? imax - 1 : M;  // causal rows use b < i <= imax - 1
    const int kcn = (kend + KSTEP - 1) / KSTEP;
    const int64_t col = ct * 16 * J + J * n;
    const bool colok = col < ncols;
    const frag* fr = frags + (int64_t)rg * RT * KC * 64 * 2;

    f32x4 acc[RT][J];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int j = 0; j < J; ++j) acc[r][j] = zero4();

    // One k-chunk of operands: S (E rows x J columns per lane) and this lane's W
    // fragments for every row tile, loaded together so both are in flight at once.
    struct Chunk {
        float sv[E][J];
        frag wh[RT], wl[RT];
    };
    auto load = [&](int kc, Chunk& ch) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int bb = kc * KSTEP + E * g + e;
            load_cols<J>(S + (int64_t)bb * ld + col, colok && bb < kend, S, ch.sv[e]);
        }
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            if (i0 + 16 * r < imax) {  // uniform
                const frag* f = fr + ((int64_t)(r * KC + kc) * 64 + lane) * 2;
                ch.wh[r] = f[0];
                ch.wl[r] = f[1];
            }
        }
    };
    auto compute = [&](const Chunk& ch) {
        frag bh[J], bl[J];
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const bf16pair p = split_bf16(ch.sv[e][j]);
                bh[j][e] = p.hi;
                bl[j][e] = p.lo;
            }
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            if (i0 + 16 * r < imax) {  // uniform
#pragma unroll
                for (int j = 0; j < J; ++j) {
                    acc[r][j] = Ops::mma(ch.wh[r], bh[j], acc[r][j]);
                    acc[r][j] = Ops::mma(ch.wh[r], bl[j], acc[r][j]);
                    acc[r][j] = Ops::mma(ch.wl[r], bh[j], acc[r][j]);
                }
            }
        }
    };

    {  // the next k-chunk is in flight while this one is multiplied
        Chunk ca, cb;
        if (kcn > 0) load(0, ca);
        for (int kc = 0; kc < kcn; kc += 2) {
            if (kc + 1 < kcn) load(kc + 1, cb);
            issue_fence();
            compute(ca);
            if (kc + 1 < kcn) {
                if (kc + 2 < kcn) load(kc + 2, ca);
                issue_fence();
                compute(cb);
            }
        }
    }

    if (!colok) return;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = i0 + 16 * r + 4 * g + i;
            if (row < imax) {
                float* dst = St + (int64_t)row * ld + col;
                if constexpr (J == 4)
                    *reinterpret_cast<f32x4*>(dst) = f32x4{acc[r][0][i], acc[r][1][i], acc[r][2][i], acc[r][3][i]};
                else
                    *reinterpret_cast<float2*>(dst) = make_float2(acc[r][0][i], acc[r][1][i]);
            }
        }
    }
}


// 64 < M <= 256: one workgroup per strip of 16*NT columns (NT <= 8) and all M rows.
// The strip of S (M x 16*NT floats) is read from HBM once, split into bf16 hi + lo
// once and kept in LDS transposed to [column][block] (about 135 KiB: one
// workgroup of eight waves per CU), so that each MFMA B operand (8 consecutive
// blocks of one column) is one 16-byte LDS read.  Wave w owns rows 32w .. 32w + 31 and reads its
// rows of W as float32 straight from L2 (W is at most 256 KiB), two k-chunks ahead,
// splitting them into hi + lo A operands in registers; every A operand then serves
// the NT column tiles of the strip.
template <int NT, bool CAUSAL>
__global__ __launch_bounds__(512) void mix_wide_kernel(const float* __restrict__ S, const float* __restrict__ W,
                                                       float* __restrict__ St, int64_t ncols, int64_t ld, int M, int KC) {
    // Grid row y: one head's contiguous column block (head-major summaries) and its W.
    S += (int64_t)blockIdx.y * ncols;
    St += (int64_t)blockIdx.y * ncols;
    W += (int64_t)blockIdx.y * M * M;
    __shared__ __align__(16) uint4 strip[2 * 16 * kWideMaxNT * (4 * kWideMaxKC + 1)];  // hi then lo
    const int RS4 = 4 * KC + 1;  // 32*KC bf16 of one column, + 16 bytes against bank conflicts
    uint4* const sh = strip;
    uint4* const sl = strip + 16 * NT * RS4;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, n = lane & 15;
    const int64_t col0 = (int64_t)blockIdx.x * 16 * NT;

    // 1. strip -> LDS: task (8-block group bg, 4-column group cg), blocks 8bg .. 8bg+7;
    //    a thread's (at most kWideTasks) tasks issue all their loads before any is used.
    const int ntask = 4 * KC * 4 * NT;
    f32x4 x[kWideTasks][8];
#pragma unroll
    for (int q = 0; q < kWideTasks; ++q) {
        const int task = threadIdx.x + 512 * q;
        const int bg = task / (4 * NT), cg = task % (4 * NT);
        const int64_t c = col0 + 4 * cg;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int b = 8 * bg + r;
            x[q][r] = load_or_zero(reinterpret_cast<const f32x4*>(S + (int64_t)b * ld + c),
                                   task < ntask && b < M && c < ncols, reinterpret_cast<const f32x4*>(S));
        }
    }
    issue_fence();
#pragma unroll
    for (int q = 0; q < kWideTasks; ++q) {
        const int task = threadIdx.x + 512 * q;
        if (task < ntask) {
            const int bg = task / (4 * NT), cg = task % (4 * NT);
#pragma unroll
            for (int xx = 0; xx < 4; ++xx) {
                uint32_t h[4], l[4];
#pragma unroll
                for (int r2 = 0; r2 < 4; ++r2) split2_bf16(x[q][2 * r2][xx], x[q][2 * r2 + 1][xx], h[r2], l[r2]);
                sh[(4 * cg + xx) * RS4 + bg] = uint4{h[0], h[1], h[2], h[3]};
                sl[(4 * cg + xx) * RS4 + bg] = uint4{l[0], l[1], l[2], l[3]};
            }
        }
    }
    __syncthreads();

    // 2. this wave's rows (no barriers below)
    const int i0 = 16 * kWideRT * wave;
    if (i0 >= M) return;
    const int rows = min(16 * kWideRT, M - i0);
    const int nrt = (rows + 15) / 16;
    const int kend = CAUSAL ? min(M, i0 + rows - 1) : M;  // causal rows use b < i <= i0 + rows - 1
    const int kcn = (kend + 31) / 32;
    const bool vec = (M & 3) == 0;  // rows of W 16-byte aligned

    f32x4 acc[kWideRT][NT];
#pragma unroll
    for (int r = 0; r < kWideRT; ++r)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[r][t] = zero4();

    // A operands of k-chunk kc: lane (g, n) row tile r holds W[i0 + 16r + n][32kc + 8g + e], e < 8.
    auto load_w = [&](int kc, f32x4 (&w)[kWideRT][2]) {
#pragma unroll
        for (int r = 0; r < kWideRT; ++r) {
            const int i = i0 + 16 * r + n;
            const int b0 = 32 * kc + 8 * g;
            if (vec) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    w[r][h] = load_or_zero(reinterpret_cast<const f32x4*>(W + (int64_t)i * M + b0 + 4 * h),
                                           i < M && b0 + 4 * h < M, reinterpret_cast<const f32x4*>(W));
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    w[r][e / 4][e % 4] = load_or_zero(W + (int64_t)i * M + b0 + e, i < M && b0 + e < M, W);
            }
        }
    };
    auto compute = [&](int kc, const f32x4 (&w)[kWideRT][2]) {
        // Entries past M were loaded as zero; causal rows also drop b >= i.
        bf16x8 ah[kWideRT], al[kWideRT];
#pragma unroll
        for (int r = 0; r < kWideRT; ++r) {
            const int i = i0 + 16 * r + n;
            uint32_t h[4], l[4];
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                float x0 = w[r][e2 / 2][(2 * e2) % 4], x1 = w[r][e2 / 2][(2 * e2 + 1) % 4];
                if constexpr (CAUSAL) {
                    const int b = 32 * kc + 8 * g + 2 * e2;
                    x0 = b < i ? x0 : 0.f;
                    x1 = b + 1 < i ? x1 : 0.f;
                }
                split2_bf16(x0, x1, h[e2], l[e2]);
            }
            ah[r] = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
            al[r] = __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], l[2], l[3]});
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const bf16x8 bh = __builtin_bit_cast(bf16x8, sh[(16 * t + n) * RS4 + 4 * kc + g]);
            const bf16x8 bl = __builtin_bit_cast(bf16x8, sl[(16 * t + n) * RS4 + 4 * kc + g]);
#pragma unroll
            for (int r = 0; r < kWideRT; ++r) {
                if (r < nrt) {  // uniform
                    acc[r][t] = mfma32(ah[r], bh, acc[r][t]);
                    acc[r][t] = mfma32(ah[r], bl, acc[r][t]);
                    acc[r][t] = mfma32(al[r], bh, acc[r][t]);
                }
            }
        }
    };
    {
        // W two k-chunks ahead (ring of three; the chunk loop is unrolled, at most kWideMaxKC)
        f32x4 wr[3][kWideRT][2];
        if (kcn > 0) load_w(0, wr[0]);
        if (kcn > 1) load_w(1, wr[1]);
#pragma unroll
        for (int kc = 0; kc < kWideMaxKC; ++kc) {
            if (kc < kcn) {  // uniform
                if (kc + 2 < kcn) load_w(kc + 2, wr[(kc + 2) % 3]);
                issue_fence();
                compute(kc, wr[kc % 3]);
            }
        }
    }

#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int64_t col = col0 + 16 * t + n;
        if (col >= ncols) continue;
#pragma unroll
        for (int r = 0; r < kWideRT; ++r) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int row = 16 * r + 4 * g + ii;
                if (row < rows) St[(int64_t)(i0 + row) * ld + col] = acc[r][t][ii];
            }
        }
    }
}

// Small M (<= 64): the workgroup splits its rows of W into MFMA fragments in LDS
// itself (at most 16 KiB), which costs less than a separate launch.
// 64 < M <= 256, persistent: one workgroup of eight waves per CU walks the 16-column
// tiles blockIdx.x, blockIdx.x + gridDim.x, ...  Wave w owns rows 32w .. 32w + 31 and
// keeps its rows of W resident in registers as bf16 hi + lo MFMA operands (128
// VGPRs), split once.  Each tile of S (M x 16 floats) is loaded into registers two
// tiles ahead of its use, split into hi + lo and written to LDS transposed to
// [column][block] (double-buffered, one barrier per tile), so that loads, MFMAs and
// stores of different tiles overlap.  The MFMA takes the S tile as its A operand and
// W as its B operand, so each lane ends with 4 consecutive columns of one output row
// and writes them with one 16-byte store.
constexpr int kStreamRS = 256 + 8;  // bf16 per LDS column (M <= 256 blocks, padded)
constexpr int kStreamKC = 8;        // 32-deep k-chunks for M <= 256

template <bool CAUSAL, bool FULL>  // FULL: M == 256, non-causal (every wave: 32 rows, 8 k-chunks)
__global__ __launch_bounds__(512) void mix_stream_kernel(const float* __restrict__ S, const float* __restrict__ W,
                                                         float* __restrict__ St, int64_t ncols, int64_t ld, int M,
                                                         int64_t ntiles) {
    // Grid row y: one head's contiguous column block (head-major summaries) and its W.
    S += (int64_t)blockIdx.y * ncols;
    St += (int64_t)blockIdx.y * ncols;
    W += (int64_t)blockIdx.y * M * M;
    __shared__ __align__(16) uint32_t tile[2][2][16 * kStreamRS / 2];  // [buffer][hi, lo][column][block pair]

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, n = lane & 15;
    // Wave w owns rows 32((w + blockIdx.x) mod 8) ..: neighbouring workgroups read
    // different rows of W at any moment instead of all the same L2 lines.
    const int i0 = 32 * ((wave + (int)blockIdx.x) & 7);
    const int rows = FULL ? 32 : max(0, min(32, M - i0));
    const int nrt = FULL ? 2 : (rows + 15) / 16;
    const int kend = CAUSAL ? min(M, i0 + rows - 1) : M;  // causal rows use b < i <= i0 + rows - 1
    const int kcn = FULL ? kStreamKC : max(0, (kend + 31) / 32);

    bf16x8 wh[2][kStreamKC], wl[2][kStreamKC];  // this wave's rows of W (B operands), filled below

    // Tile loads: thread -> blocks 2bp, 2bp + 1 (bp < 128) and columns 4cg .. 4cg + 3.
    const int bp = threadIdx.x >> 2, cg = threadIdx.x & 3;
    const int64_t my_tiles = ntiles > blockIdx.x ? (ntiles - 1 - blockIdx.x) / gridDim.x + 1 : 0;
    // S through a buffer descriptor (the caller guarantees M * ld * 4 < 2^32): 32-bit
    // offsets, an offset past the end reads zero, and the loads stay where they are
    // written, two tiles ahead of their use.
    const rsrc_t rS = make_rsrc(S, (uint32_t)((int64_t)M * ld * 4));
    const uint32_t soff0 = (uint32_t)(((int64_t)(2 * bp) * ld + 4 * cg) * 4);
    // Column tile of this workgroup's j-th step.  In whole rounds of 256 workgroups the
    // tiles are permuted so that the two 16-column tiles sharing each 128-byte line of S
    // go to workgroups on one XCD (ids congruent mod 8): the line is fetched into one L2.
    auto tile_col = [&](int64_t j) -> int64_t {
        const int64_t t = blockIdx.x + j * gridDim.x;
        if (gridDim.x != 256 || t >= ntiles / 256 * 256) return t;
        const int b = (int)(t % 256);
        return t - b + 2 * (b % 8 + 8 * (b / 16)) + (b / 8) % 2;
    };
    auto load_tile = [&](int64_t j, f32x4 (&x)[2]) {
        const uint32_t col = (uint32_t)(tile_col(j) * 16);
        const bool ok = j < my_tiles;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const bool okh = ok && 2 * bp + h < M;
            x[h] = __builtin_bit_cast(f32x4, buf_load128(rS, off_if(okh, soff0 + (uint32_t)(h * ld + col) * 4)));
        }
    };
    auto store_lds = [&](int buf, const f32x4 (&x)[2]) {
#pragma unroll
        for (int xx = 0; xx < 4; ++xx) {
            uint32_t hi, lo;
            split2_bf16(x[0][xx], x[1][xx], hi, lo);
            tile[buf][0][((4 * cg + xx) * kStreamRS) / 2 + bp] = hi;
            tile[buf][1][((4 * cg + xx) * kStreamRS) / 2 + bp] = lo;
        }
    };
    // One tile: products from LDS buffer buf, 16-byte stores, then tile j + 1 (registers
    // xn) into the other buffer, whose last readers passed the previous barrier, and the
    // loads of tile j + 3 into the registers xf just freed.
    auto step = [&](int64_t j, int buf, const f32x4 (&xn)[2], f32x4 (&xf)[2]) {
        f32x4 acc[2] = {zero4(), zero4()};
        const uint32_t* th = &tile[buf][0][(n * kStreamRS) / 2];
        const uint32_t* tl = &tile[buf][1][(n * kStreamRS) / 2];
#pragma unroll
        for (int kc = 0; kc < kStreamKC; ++kc) {
            if (kc < kcn) {  // uniform
                const bf16x8 ah = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(th + 16 * kc + 4 * g));
                const bf16x8 al = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(tl + 16 * kc + 4 * g));
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    if (r < nrt) {  // uniform
                        acc[r] = mfma32(ah, wh[r][kc], acc[r]);
                        acc[r] = mfma32(al, wh[r][kc], acc[r]);
                        acc[r] = mfma32(ah, wl[r][kc], acc[r]);
                    }
                }
            }
        }
        const int64_t col0 = tile_col(j) * 16;
#pragma unroll
        for (int r = 0; r < 2; ++r) {  // lane (g, n): row i0 + 16r + n, columns 4g .. 4g + 3
            const int row = 16 * r + n;
            if (row < rows) *reinterpret_cast<f32x4*>(St + (int64_t)(i0 + row) * ld + col0 + 4 * g) = acc[r];
        }
        store_lds(buf ^ 1, xn);
        load_tile(j + 3, xf);
        lds_barrier();
    };

    f32x4 p0[2], p1[2], p2[2];  // ring of three tiles in flight
    load_tile(0, p0);  // (the first tile loads while W is read from L2)
    // W rows of this wave, split once: B operand of k-chunk kc, row tile r:
    // lane (g, n) holds W[i0 + 16r + n][32kc + 8g + e], e < 8 (zero past M; causal b < i).
    // W (at most 256 KiB) is read through a buffer descriptor: 32-bit offsets, and an
    // offset past the end reads zero.
    // M = 256 (FULL): each load instruction reads 8 whole 128-byte lines (lane l: row
    // 8h + l / 8 of the row tile, floats 32kc + 4 (l % 8) .. + 3), and the k-chunk's 16 rows
    // are turned into the operand layout through a 2 KiB slice of the second tile buffer
    // per wave, which no wave uses before the first barrier (16-byte pieces swizzled by
    // row: conflict-free writes, two-way reads).  Loads of the operand layout itself touch
    // 16 half lines per instruction, and every CU reading all of W that way took twice as
    // long on cold inputs.
    uint32_t* const wslot = &tile[1][0][0] + 512 * wave;
    const rsrc_t rW = make_rsrc(W, (uint32_t)M * M * 4);
#pragma unroll
    for (int r = 0; r < 2; ++r) {  // one row tile at a time: all its loads, then the splits
        const int i = i0 + 16 * r + n;
        f32x4 x[kStreamKC][2];
#pragma unroll
        for (int kc = 0; kc < kStreamKC; ++kc)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int b = 32 * kc + 8 * g + 4 * h;
                if constexpr (FULL) {
                    const int row = i0 + 16 * r + 8 * h + (lane >> 3);
                    x[kc][h] = __builtin_bit_cast(f32x4,
                                                  buf_load128(rW, (uint32_t)(row * M + 32 * kc + 4 * (lane & 7)) * 4));
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        x[kc][h][e] = __uint_as_float(buf_load32(rW, off_if(i < M && b + e < M, (uint32_t)(i * M + b + e) * 4)));
                }
            }
        issue_fence();
#pragma unroll
        for (int kc = 0; kc < kStreamKC; ++kc) {
            if constexpr (FULL) {  // rows 8h + l / 8, piece l % 8 -> lane (g, n): row n, pieces 2g, 2g + 1
                asm volatile("" ::: "memory");  // the previous k-chunk's reads come first
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int row = 8 * h + (lane >> 3);
                    *reinterpret_cast<f32x4*>(wslot + 32 * row + 4 * ((lane & 7) ^ (row & 7))) = x[kc][h];
                }
                asm volatile("" ::: "memory");
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    x[kc][h] = *reinterpret_cast<const f32x4*>(wslot + 32 * n + 4 * ((2 * g + h) ^ (n & 7)));
            }
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const int b = 32 * kc + 8 * g + 2 * e2;
                float x0 = x[kc][e2 / 2][(2 * e2) % 4], x1 = x[kc][e2 / 2][(2 * e2 + 1) % 4];
                if constexpr (CAUSAL) {
                    x0 = b < i ? x0 : 0.f;
                    x1 = b + 1 < i ? x1 : 0.f;
                }
                split2_bf16(x0, x1, hw[e2], lw[e2]);
            }
            wh[r][kc] = __builtin_bit_cast(bf16x8, u32x4{hw[0], hw[1], hw[2], hw[3]});
            wl[r][kc] = __builtin_bit_cast(bf16x8, u32x4{lw[0], lw[1], lw[2], lw[3]});
        }
    }

    load_tile(1, p1);
    load_tile(2, p2);
    store_lds(0, p0);
    lds_barrier();
    for (int64_t j = 0; j < my_tiles; j += 3) {  // unrolled by the ring length (uniform exits);
        step(j, (int)(j & 1), p1, p0);           // tile j sits in LDS buffer j & 1
        if (j + 1 >= my_tiles) break;
        step(j + 1, (int)((j + 1) & 1), p2, p1);
        if (j + 2 >= my_tiles) break;
        step(j + 2, (int)((j + 2) & 1), p0, p2);
    }
}

template <int KSTEP, int RT, int J, bool PIPE, bool CAUSAL>
__global__ __launch_bounds__(256) void mix_lds_kernel(const float* __restrict__ S, const float* __restrict__ W,
                                                      float* __restrict__ St, int64_t ncols, int64_t ld, int M,
                                                      int64_t ntiles, int kc_cap) {
    // Grid row y: one head's contiguous column block (head-major summaries) and its W.
    S += (int64_t)blockIdx.y * ncols;
    St += (int64_t)blockIdx.y * ncols;
    W += (int64_t)blockIdx.y * M * M;
    using Ops = MixOps<KSTEP>;
    using frag = typename Ops::frag;
    constexpr int E = Ops::E;
    extern __shared__ __align__(16) unsigned char smem[];
    frag* wf = reinterpret_cast<frag*>(smem);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, n = lane & 15;
    const int imax = min(M, 16 * RT);        // a single row group
    const int kend = CAUSAL ? imax - 1 : M;  // causal rows use b < i <= imax - 1
    const int kcn = (kend + KSTEP - 1) / KSTEP;

    for (int slot = threadIdx.x; slot < RT * kcn * 64; slot += blockDim.x) {
        const int ln = slot & 63, t = slot >> 6;
        const int kc = t % kcn, rt = t / kcn;
        const int i = 16 * rt + (ln & 15);
        const int b0 = kc * KSTEP + E * (ln >> 4);
        frag h, l;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int b = b0 + e;
            const bool use = i < M && b < kend && (!CAUSAL || b < i);
            const bf16pair p = split_bf16(load_or_zero(W + (int64_t)i * M + b, use, W));
            h[e] = p.hi;
            l[e] = p.lo;
        }
        wf[((rt * kc_cap + kc) * 64 + ln) * 2] = h;
        wf[((rt * kc_cap + kc) * 64 + ln) * 2 + 1] = l;
    }
    __syncthreads();

    const int64_t ct = (int64_t)blockIdx.x * 4 + wave;
    if (ct >= ntiles) return;  // no barriers below
    const int64_t col = ct * 16 * J + J * n;
    const bool colok = col < ncols;

    f32x4 acc[RT][J];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int j = 0; j < J; ++j) acc[r][j] = zero4();

    auto load = [&](int kc, float (&sv)[E][J]) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int b = kc * KSTEP + E * g + e;
            load_cols<J>(S + (int64_t)b * ld + col, colok && b < kend, S, sv[e]);
        }
    };
    auto compute = [&](int kc, const float (&sv)[E][J]) {
        frag bh[J], bl[J];
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const bf16pair p = split_bf16(sv[e][j]);
                bh[j][e] = p.hi;
                bl[j][e] = p.lo;
            }
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            if (16 * r < imax) {  // uniform
                const frag ah = wf[((r * kc_cap + kc) * 64 + lane) * 2];
                const frag al = wf[((r * kc_cap + kc) * 64 + lane) * 2 + 1];
#pragma unroll
                for (int j = 0; j < J; ++j) {
                    acc[r][j] = Ops::mma(ah, bh[j], acc[r][j]);
                    acc[r][j] = Ops::mma(ah, bl[j], acc[r][j]);
                    acc[r][j] = Ops::mma(al, bh[j], acc[r][j]);
                }
            }
        }
    };

    if constexpr (PIPE) {  // next k-chunk in flight while this one is multiplied
        float sa[E][J], sb[E][J];
        if (kcn > 0) load(0, sa);
        for (int kc = 0; kc < kcn; kc += 2) {
            if (kc + 1 < kcn) load(kc + 1, sb);
            issue_fence();
            compute(kc, sa);
            if (kc + 1 < kcn) {
                if (kc + 2 < kcn) load(kc + 2, sa);
                issue_fence();
                compute(kc + 1, sb);
            }
        }
    } else {
        for (int kc = 0; kc < kcn; ++kc) {
            float sa[E][J];
            load(kc, sa);
            issue_fence();
            compute(kc, sa);
        }
    }

    if (!colok) return;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * r + 4 * g + i;
            if (row < imax) {
                float* dst = St + (int64_t)row * ld + col;
                if constexpr (J == 4)
                    *reinterpret_cast<f32x4*>(dst) = f32x4{acc[r][0][i], acc[r][1][i], acc[r][2][i], acc[r][3][i]};
                else
                    *reinterpret_cast<float2*>(dst) = make_float2(acc[r][0][i], acc[r][1][i]);
            }
        }
    }
}

// 32 < M <= 64 (two 32-deep k-chunks, RT = 4 row tiles, J columns per lane): the kernel above made
// persistent.  Each workgroup splits W into LDS once; its waves then walk column tiles
// 4 blockIdx.x + wave, plus multiples of 4 gridDim.x, with the S loads one k-chunk
// ahead across tile boundaries, so the next tile's first chunk is in flight while the
// current tile's last chunk is multiplied and its rows are stored.  S and St are
// addressed through buffer descriptors: a load past a valid row or column reads zero
// and a store there is dropped, so every wave issues the same loads and stores on
// every tile (the wait counts stay exact) and the last prefetch needs no branch.
template <int J, bool CAUSAL>
__global__ __launch_bounds__(256) void mix_walk_kernel(const float* __restrict__ S, const float* __restrict__ W,
                                                       float* __restrict__ St, int64_t ncols, int64_t ld, int M,
                                                       int64_t ntiles, int kc_cap) {
    constexpr int KSTEP = 32, RT = 4;
    using colv = typename std::conditional<J == 4, f32x4, f32x2>::type;
    S += (int64_t)blockIdx.y * ncols;
    St += (int64_t)blockIdx.y * ncols;
    W += (int64_t)blockIdx.y * M * M;
    using Ops = MixOps<KSTEP>;
    using frag = typename Ops::frag;
    constexpr int E = Ops::E;
    extern __shared__ __align__(16) unsigned char smem[];
    frag* wf = reinterpret_cast<frag*>(smem);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, n = lane & 15;
    const int imax = min(M, 16 * RT);
    const int kend = CAUSAL ? imax - 1 : M;
    const int kcn = 2;  // 32 < kend <= 64
    const uint32_t span = (uint32_t)((int64_t)(M - 1) * ld + ncols) * 4;  // rows 0 .. M-1 of this column block
    const rsrc_t rS = make_rsrc(S, span), rT = make_rsrc(St, span);
    const int64_t stride = 4 * (int64_t)gridDim.x;
    int64_t ct = (int64_t)blockIdx.x * 4 + wave;

    auto load = [&](int64_t t, int kc, colv (&sv)[E]) {
        const int64_t col = t * 16 * J + J * n;
        const bool ok = t < ntiles && col < ncols;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int b = kc * KSTEP + E * g + e;
            const uint32_t off = off_if(ok && b < kend, (uint32_t)(b * ld + col) * 4);
            if constexpr (J == 4)
                sv[e] = __builtin_bit_cast(f32x4, buf_load128(rS, off));
            else
                sv[e] = __builtin_bit_cast(f32x2, buf_load64(rS, off));
        }
    };
    auto compute = [&](int kc, const colv (&sv)[E], f32x4 (&acc)[RT][J]) {
        // W fragments are read from LDS here on every chunk rather than kept in
        // registers across the walk (which would cost 64 VGPRs and halve the waves
        // that keep loads in flight)
        asm volatile("" ::: "memory");
        frag bh[J], bl[J];
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const bf16pair p = split_bf16(sv[e][j]);
                bh[j][e] = p.hi;
                bl[j][e] = p.lo;
            }
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            if (16 * r < imax) {  // uniform
                const frag ah = wf[((r * kc_cap + kc) * 64 + lane) * 2];
                const frag al = wf[((r * kc_cap + kc) * 64 + lane) * 2 + 1];
#pragma unroll
                for (int j = 0; j < J; ++j) {
                    acc[r][j] = Ops::mma(ah, bh[j], acc[r][j]);
                    acc[r][j] = Ops::mma(ah, bl[j], acc[r][j]);
                    acc[r][j] = Ops::mma(al, bh[j], acc[r][j]);
                }
            }
        }
    };
    auto store = [&](int64_t t, f32x4 (&acc)[RT][J]) {
        const int64_t col = t * 16 * J + J * n;
        const bool colok = t < ntiles && col < ncols;
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * r + 4 * g + i;
                const int off = (int)off_if(colok && row < imax, (uint32_t)(row * ld + col) * 4);
                if constexpr (J == 4) {
                    const f32x4 v = f32x4{acc[r][0][i], acc[r][1][i], acc[r][2][i], acc[r][3][i]};
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rT, off, 0, 0);
                } else {
                    const u32x2 v = u32x2{__float_as_uint(acc[r][0][i]), __float_as_uint(acc[r][1][i])};
                    __builtin_amdgcn_raw_buffer_store_b64(v, rT, off, 0, 0);
                }
#pragma unroll
                for (int j = 0; j < J; ++j) acc[r][j][i] = 0.f;
            }
    };

    colv sa[E], sb[E];
    load(ct, 0, sa);  // in flight while W is split
    for (int slot = threadIdx.x; slot < RT * kcn * 64; slot += blockDim.x) {
        const int ln = slot & 63, t = slot >> 6;
        const int kc = t % kcn, rt = t / kcn;
        const int i = 16 * rt + (ln & 15);
        const int b0 = kc * KSTEP + E * (ln >> 4);
        frag h, l;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int b = b0 + e;
            const bool use = i < M && b < kend && (!CAUSAL || b < i);
            const bf16pair p = split_bf16(load_or_zero(W + (int64_t)i * M + b, use, W));
            h[e] = p.hi;
            l[e] = p.lo;
        }
        wf[((rt * kc_cap + kc) * 64 + ln) * 2] = h;
        wf[((rt * kc_cap + kc) * 64 + ln) * 2 + 1] = l;
    }
    __syncthreads();
    if (ct >= ntiles) return;  // no barriers below

    f32x4 acc[RT][J];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int j = 0; j < J; ++j) acc[r][j] = zero4();
    while (true) {
        load(ct, 1, sb);
        issue_fence();
        compute(0, sa, acc);
        issue_fence();  // sa is free before its next loads are issued
        const int64_t nt = ct + stride;
        load(nt, 0, sa);  // past the last tile: reads nothing
        issue_fence();
        compute(1, sb, acc);
        store(ct, acc);
        if (nt >= ntiles) break;
        ct = nt;
    }
}

// M = 1: the mixing is a single scale, St = W[0][0] S (causal: no earlier block, St = 0),
// done as a streaming float32 multiply (exact products, HBM-bound).
template <bool CAUSAL>
__global__ __launch_bounds__(256) void mix_scale_kernel(const f32x4* __restrict__ S, const float* __restrict__ W,
                                                        f32x4* __restrict__ St, int64_t n4) {
    S += (int64_t)blockIdx.y * n4;  // grid row y: one head's column block and its 1 x 1 W
    St += (int64_t)blockIdx.y * n4;
    const float w = CAUSAL ? 0.f : W[blockIdx.y];
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
        const f32x4 x = S[i];
        St[i] = CAUSAL ? zero4() : f32x4{w * x[0], w * x[1], w * x[2], w * x[3]};
    }
}

// Fallback for M > kMaxFragM: each wave splits its W fragments itself.
template <bool CAUSAL>
__global__ __launch_bounds__(256) void mix_split_kernel(const float* __restrict__ S, const float* __restrict__ W,
                                                        float* __restrict__ St, int64_t ncols, int64_t ld, int M, int RG,
                                                        int64_t ntiles) {
    // Grid row y: one head's contiguous column block (head-major summaries) and its W.
    S += (int64_t)blockIdx.y * ncols;
    St += (int64_t)blockIdx.y * ncols;
    W += (int64_t)blockIdx.y * M * M;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, n = lane & 15;
    const int64_t w = (int64_t)blockIdx.x * 4 + wave;
    const int rg = (int)(w % RG);
    const int64_t ct = w / RG;
    if (ct >= ntiles) return;  // whole wave; no barriers in this kernel

    const int64_t col = ct * 64 + 4 * n;
    const bool colok = col < ncols;
    const int i0 = rg * 64;
    const int imax = min(M, i0 + 64);
    const int kend = CAUSAL ? imax - 1 : M;

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
            sv[e] = load_or_zero(reinterpret_cast<const f32x4*>(S + (int64_t)b * ld + col), b < kend && colok,
                                 reinterpret_cast<const f32x4*>(S));
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
                    const bf16pair h = split_bf16(load_or_zero(W + (int64_t)i * M + b, use, W));
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
                *reinterpret_cast<f32x4*>(St + (int64_t)row * ld + col) =
                    f32x4{acc[r][0][i], acc[r][1][i], acc[r][2][i], acc[r][3][i]};
        }
    }
}

// float32 path: one thread per four columns, float32 FMAs in a fixed order.
__global__ __launch_bounds__(256) void mix_f32_kernel(const float* __restrict__ S, const float* __restrict__ W,
                                                      float* __restrict__ St, int64_t ncols, int64_t ld, int M, int causal) {
    // Grid row y: one head's contiguous column block (head-major summaries) and its W.
    S += (int64_t)blockIdx.y * ncols;
    St += (int64_t)blockIdx.y * ncols;
    W += (int64_t)blockIdx.y * M * M;
    const int64_t col = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (col >= ncols) return;
    for (int i = 0; i < M; ++i) {
        f32x4 acc = zero4();
        const int bend = causal ? i : M;
        for (int b = 0; b < bend; ++b) {
            const float wv = W[(int64_t)i * M + b];
            const f32x4 s = *reinterpret_cast<const f32x4*>(S + (int64_t)b * ld + col);
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] = fmaf(wv, s[c], acc[c]);
        }
        *reinterpret_cast<f32x4*>(St + (int64_t)i * ld + col) = acc;
    }
}

hipError_t launch_mix(const float* S, const float* W, float* St, int64_t BH, int D, int64_t M, bool causal,
                      bool precise, int heads, void* frag_ws, hipStream_t stream) {
    // heads > 0: W holds one M x M matrix per head and the summaries are head-major,
    // so that head h owns columns [h*ncols, (h+1)*ncols); grid row y runs head y.
    const int64_t ld = BH * (int64_t)(D * D + D);
    const unsigned gy = heads > 0 ? (unsigned)heads : 1u;
    const int64_t ncols = ld / gy;
    if (precise) {
        const int64_t threads = ncols / 4;
        mix_f32_kernel<<<dim3((unsigned)((threads + 255) / 256), gy), dim3(256), 0, stream>>>(S, W, St, ncols, ld,
                                                                                            (int)M, causal ? 1 : 0);
        return hipGetLastError();
    }
    if (M == 1) {
        const int64_t n4 = ncols / 4;  // d*d + d is a multiple of 4
        const dim3 grid((unsigned)std::min<int64_t>((n4 + 255) / 256, 256 * 8), gy);
        if (causal)
            mix_scale_kernel<true><<<grid, dim3(256), 0, stream>>>(reinterpret_cast<const f32x4*>(S), W,
                                                                   reinterpret_cast<f32x4*>(St), n4);
        else
            mix_scale_kernel<false><<<grid, dim3(256), 0, stream>>>(reinterpret_cast<const f32x4*>(S), W,
                                                                    reinterpret_cast<f32x4*>(St), n4);
        return hipGetLastError();
    }
    using I16 = std::integral_constant<int, 16>;
    using I32 = std::integral_constant<int, 32>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I4 = std::integral_constant<int, 4>;
    if (M <= 64) {
        auto run = [&](auto kstep_c, auto rt_c, auto j_c) {
            constexpr int KSTEP = decltype(kstep_c)::value, RT = decltype(rt_c)::value, J = decltype(j_c)::value;
            constexpr bool PIPE = KSTEP == 32;  // the 16-deep variant serves M <= 16: a single k-chunk
            const int KC = (int)((M + KSTEP - 1) / KSTEP);
            const size_t lds = (size_t)RT * KC * 64 * 2 * (KSTEP == 32 ? 16 : 8);
            const int64_t ntiles = (ncols + 16 * J - 1) / (16 * J);
            const dim3 grid((unsigned)((ntiles + 3) / 4), gy);
            if (causal)
                mix_lds_kernel<KSTEP, RT, J, PIPE, true><<<grid, dim3(256), lds, stream>>>(S, W, St, ncols, ld,
                                                                                          (int)M, ntiles, KC);
            else
                mix_lds_kernel<KSTEP, RT, J, PIPE, false><<<grid, dim3(256), lds, stream>>>(S, W, St, ncols, ld,
                                                                                           (int)M, ntiles, KC);
        };
        if (M <= 16) {
            run(I16{}, I1{}, I4{});
        } else if (M <= 32) {
            run(I32{}, I2{}, I4{});
        } else if (M > 32 + (causal ? 1 : 0) && (M * ld + 64) * 4 < (int64_t(1) << 32)) {  // two k-chunks;
            //                                                                    32-bit buffer offsets
            const int KC = (int)((M + 31) / 32);
            const size_t lds = (size_t)4 * KC * 64 * 2 * 16;
            const int64_t ntiles = (ncols + 16 * kWalkJ - 1) / (16 * kWalkJ);
            // kWalkPerCU workgroups of four waves per CU, shared out over the heads
            const int64_t per_head = std::max<int64_t>(1, (int64_t)device_cu_count() * kWalkPerCU / gy);
            const dim3 grid((unsigned)std::min<int64_t>((ntiles + 3) / 4, per_head), gy);
            if (causal)
                mix_walk_kernel<kWalkJ, true><<<grid, dim3(256), lds, stream>>>(S, W, St, ncols, ld, (int)M, ntiles, KC);
            else
                mix_walk_kernel<kWalkJ, false><<<grid, dim3(256), lds, stream>>>(S, W, St, ncols, ld, (int)M, ntiles, KC);
        } else {
            run(I32{}, I4{}, I4{});
        }
        return hipGetLastError();
    }
    if (M <= 256 && M * ld * 4 < (int64_t(1) << 32) - 64) {  // 64 < M <= 256: persistent tile walk
        const int64_t ntiles = ncols / 16;  // d*d + d is a multiple of 16
        const int cus = device_cu_count();
        const dim3 grid((unsigned)std::max<int64_t>(1, std::min<int64_t>(ntiles, cus)), gy);
        if (causal)
            mix_stream_kernel<true, false><<<grid, dim3(512), 0, stream>>>(S, W, St, ncols, ld, (int)M, ntiles);
        else if (M == 256)
            mix_stream_kernel<false, true><<<grid, dim3(512), 0, stream>>>(S, W, St, ncols, ld, (int)M, ntiles);
        else
            mix_stream_kernel<false, false><<<grid, dim3(512), 0, stream>>>(S, W, St, ncols, ld, (int)M, ntiles);
        return hipGetLastError();
    }
    if (M <= 256) {  // 64 < M <= 256 with S of 4 GiB or more: wide strips, W split per wave
        const int KC = (int)((M + 31) / 32);
        const int64_t tiles16 = (ncols + 15) / 16;
        // strips of NT column tiles: one strip per CU when that takes at most kWideMaxNT tiles
        const int nt = (int)std::min<int64_t>(kWideMaxNT, std::max<int64_t>(1, (tiles16 + 255) / 256));
        const dim3 grid((unsigned)((tiles16 + nt - 1) / nt), gy);
        auto run = [&](auto nt_c) {
            constexpr int NT = decltype(nt_c)::value;
            if (causal)
                mix_wide_kernel<NT, true><<<grid, dim3(512), 0, stream>>>(S, W, St, ncols, ld, (int)M, KC);
            else
                mix_wide_kernel<NT, false><<<grid, dim3(512), 0, stream>>>(S, W, St, ncols, ld, (int)M, KC);
        };
        switch (nt) {
            case 1: run(std::integral_constant<int, 1>{}); break;
            case 2: run(std::integral_constant<int, 2>{}); break;
            case 3: run(std::integral_constant<int, 3>{}); break;
            case 4: run(std::integral_constant<int, 4>{}); break;
            case 5: run(std::integral_constant<int, 5>{}); break;
            case 6: run(std::integral_constant<int, 6>{}); break;
            case 7: run(std::integral_constant<int, 7>{}); break;
            default: run(std::integral_constant<int, 8>{}); break;
        }
        return hipGetLastError();
    }
    if (M <= kMaxFragM) {
        if (!frag_ws) return hipErrorInvalidValue;
        constexpr int KSTEP = 32, RT = 4, J = 2;
        using frag = typename MixOps<KSTEP>::frag;
        frag* frags = static_cast<frag*>(frag_ws);
        const int KC = (int)((M + KSTEP - 1) / KSTEP);
        const int RG = (int)((M + 16 * RT - 1) / (16 * RT));
        const int64_t slots = (int64_t)RG * RT * KC * 64;
        const dim3 sgrid((unsigned)((slots + 255) / 256), gy);
        if (causal)
            wsplit_kernel<KSTEP, RT, true><<<sgrid, dim3(256), 0, stream>>>(W, frags, (int)M, RG, KC);
        else
            wsplit_kernel<KSTEP, RT, false><<<sgrid, dim3(256), 0, stream>>>(W, frags, (int)M, RG, KC);
        const int64_t ntiles = (ncols + 16 * J - 1) / (16 * J);
        const int64_t nctg = (ntiles + 3) / 4;
        const dim3 grid((unsigned)(((nctg + 7) / 8) * 8 * RG), gy);
        if (causal)
            mix_frag_kernel<KSTEP, RT, J, true><<<grid, dim3(256), 0, stream>>>(S, frags, St, ncols, ld, (int)M, RG,
                                                                                ntiles, KC);
        else
            mix_frag_kernel<KSTEP, RT, J, false><<<grid, dim3(256), 0, stream>>>(S, frags, St, ncols, ld, (int)M, RG,
                                                                                 ntiles, KC);
        return hipGetLastError();
    }
    const int64_t ntiles = (ncols + 63) / 64;
    const int RG = (int)((M + 63) / 64);
    const int64_t waves = ntiles * RG;
    const dim3 grid((unsigned)((waves + 3) / 4), gy);
    if (causal)
        mix_split_kernel<true><<<grid, dim3(256), 0, stream>>>(S, W, St, ncols, ld, (int)M, RG, ntiles);
    else
        mix_split_kernel<false><<<grid, dim3(256), 0, stream>>>(S, W, St, ncols, ld, (int)M, RG, ntiles);
    return hipGetLastError();
}

}  // namespace mhla
