// pair.hip -- the whole MHLA forward pass for sequences of moderate length (256 < N
// <= 8192 tokens in at most 16 blocks of a multiple of 32 tokens, non-causal, bf16),
// one (batch, head) pair per workgroup, in the summary form of "MHLA: Restoring
// Expressivity of Linear Attention via Token-Level Multi-Head" (§4.1) with every
// summary kept on chip:
//
//   phase 1  K and V stream through LDS in chunks of 128 tokens (loads two chunks
//            ahead).  Each wave owns the same 16 x 16 tiles of every summary: it forms
//            S_b = phi(K_b)^T V_b of the current block b on bf16 MFMA with float32
//            accumulation and, when the block ends, adds W[i,b] S_b into its tiles of
//            S~_i for every query block i (the mixing of §4.1, done as the summaries
//            complete, in registers, with no exchange between waves); z_b = sum over
//            the block of phi(k) is the product of phi(K)^T with an indicator of the
//            block (column b of one 16 x 16 tile per 16 features).
//   phase 2  z~_i = sum_b W[i,b] z_b of every block to LDS; then Q streams through LDS
//            in the same 128-token chunks (loads two chunks ahead).  Wave w takes query
//            tile w of every chunk (16 queries) and all of its outputs,
//                y_t = phi(q_t)^T S~_i / (phi(q_t) . z~_i + 1e-6)
//            ("Linear Attention 笔记" §4/§5 guard), as Y^T = S~_i^T phi(Q)^T on MFMA
//            with S~_i^T split into bf16 hi and lo parts, and the normaliser as the
//            same product with z~_i's hi and lo parts as two rows.  S~_i of the blocks a
//            chunk meets are copied from the registers that hold them into a ring of
//            four LDS buffers when the chunk first needs them.
//
// HBM traffic is Q, K, V once and Y once: the block summaries, which the staged
// kernels write and read back (16 (d^2 + d) / C bytes per token-head against about
// 10 d for the tokens), never leave the CU.  Blocks of a multiple of 32 tokens keep
// every 32-token product step inside one block.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"
#include "lds_tiles.hpp"

namespace mhla {

namespace {

constexpr int kPW = 8;          // waves per workgroup
constexpr int kPChunk = 128;    // tokens per streamed chunk
constexpr int kPMaxB = 16;      // blocks
constexpr int kPRowsW = kPChunk / kPW;  // K and V rows each wave stages per chunk

template <int D>
struct PairCfg {
    static constexpr int P = D / 16;                    // 16-wide tiles per dimension
    static constexpr int KS = D / 32;                   // 32-deep feature steps
    static constexpr int T = P * P;                     // tiles of one S_b
    static constexpr int TW = (T + kPW - 1) / kPW;      // tiles of one S_b a wave owns (at most)
    static constexpr int CPR = D / 8;                   // 16-byte pieces per row
    static constexpr int LPR = D / 8;                   // staging lanes per row
    static constexpr int NL = (kPRowsW * LPR + 63) / 64;  // row pieces per lane
    // LDS, phase 1: two chunk slots of phi(K) and V [kPChunk][D] bf16; z of every
    // block float [D][16]; z~_i hi and lo [2][D] bf16 of every block; W [M][M] float.
    // Phase 2 reuses the chunk slots for a ring of four S~_i^T hi and lo buffers
    // [D value][D feature] bf16 and the area after z for the Q chunk [kPChunk][D] bf16.
    static constexpr int kRows = kPChunk * D * 2;
    static constexpr int kSlot = 2 * kRows;
    static constexpr int kStBuf = 2 * D * D * 2;
    static constexpr int kZ = 2 * kSlot;
    static constexpr int kQ = kZ + D * kPMaxB * 4;
    static constexpr int kZt = kQ + kRows;
    static constexpr int kZtBuf = 2 * D * 2;
    static constexpr int kW = kZt + kPMaxB * kZtBuf;
    static constexpr int kBytes = kW + kPMaxB * kPMaxB * 4;
    static_assert(4 * kStBuf <= kZ, "the S~ ring fits in the chunk slots");
};

struct PairShape {
    int N, M, C, nchunks, heads;
};

// The wave's tiles of S~_i for every block i: element e of tile j of block i is lane
// element (j * 16 + i) of vector e, so that a block picked at run time is read with
// one indexed register move per element.
template <int D>
struct Mixed {
    typedef float vec __attribute__((ext_vector_type(16 * PairCfg<D>::TW)));
    vec v[4];
};

// The row pieces one wave loads for a chunk of one [N][D] matrix: rows kPRowsW * wave
// .. + kPRowsW - 1 of the chunk, 16 bytes per lane and piece; rows past N (and chunks
// past the end) read zero.
template <int D>
struct PairRows {
    u32x4 x[PairCfg<D>::NL];
};

template <int D>
__device__ __forceinline__ void pair_rows_load(const rsrc_t& r, int chunk, const PairShape& sh, int wave, int lane,
                                               PairRows<D>& L) {
    constexpr int LPR = PairCfg<D>::LPR;
#pragma unroll
    for (int u = 0; u < PairCfg<D>::NL; ++u) {
        const int rr = kPRowsW * wave + 64 / LPR * u + lane / LPR;  // row in the chunk
        const int tok = kPChunk * chunk + rr;
        const bool ok = tok < sh.N && 64 / LPR * u + lane / LPR < kPRowsW;
        L.x[u] = buf_load128(r, off_if(ok, ((uint32_t)tok * D + 8 * (lane % LPR)) * 2));
    }
}

// phi of loaded rows into an LDS array [kPChunk][D] bf16, row-major with swizzled
// 16-byte pieces (raw copies when PHI is false).
template <int D, bool PHI>
__device__ __forceinline__ void pair_rows_stage(const PairRows<D>& L, unsigned char* arr, int wave, int lane) {
    constexpr int LPR = PairCfg<D>::LPR, CPR = PairCfg<D>::CPR;
#pragma unroll
    for (int u = 0; u < PairCfg<D>::NL; ++u) {
        if (64 / LPR * u + lane / LPR >= kPRowsW) continue;
        const int rr = kPRowsW * wave + 64 / LPR * u + lane / LPR;
        const u32x4 w = L.x[u];
        *reinterpret_cast<u32x4*>(arr + 16 * swz(rr, lane % LPR, CPR)) =
            PHI ? u32x4{phi_pair(w[0]), phi_pair(w[1]), phi_pair(w[2]), phi_pair(w[3])} : w;
    }
}

template <int D>
struct PairLoads {
    PairRows<D> k, v;
};

template <int D>
__device__ __forceinline__ void pair_loads(const rsrc_t& rK, const rsrc_t& rV, int chunk, const PairShape& sh,
                                           int wave, int lane, PairLoads<D>& L) {
    pair_rows_load<D>(rK, chunk, sh, wave, lane, L.k);
    pair_rows_load<D>(rV, chunk, sh, wave, lane, L.v);
}

// phi(K) and V of a chunk into an LDS slot.
template <int D>
__device__ __forceinline__ void pair_stage(const PairLoads<D>& L, unsigned char* slot, int wave, int lane) {
    pair_rows_stage<D, true>(L.k, slot, wave, lane);
    pair_rows_stage<D, false>(L.v, slot + PairCfg<D>::kRows, wave, lane);
}

// Mixing of a finished block b into the wave's tiles of every S~_i: S~_i += W[i,b] S_b.
// wt is W^T in LDS, zero-padded to 16 x 16 (the rows i >= M mix zeros into registers
// that are never read), so the column of W comes in four reads and no branch.
template <int D>
__device__ __forceinline__ void pair_flush(const float* wt, int b, f32x4 (&cur)[PairCfg<D>::TW],
                                           Mixed<D>& mix) {
    f32x4 wc[kPMaxB / 4];
#pragma unroll
    for (int r = 0; r < kPMaxB / 4; ++r) wc[r] = reinterpret_cast<const f32x4*>(wt + kPMaxB * b)[r];
#pragma unroll
    for (int i = 0; i < kPMaxB; ++i) {
        const float w = wc[i / 4][i % 4];
#pragma unroll
        for (int j = 0; j < PairCfg<D>::TW; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) mix.v[e][16 * j + i] = fmaf(w, cur[j][e], mix.v[e][16 * j + i]);
    }
#pragma unroll
    for (int j = 0; j < PairCfg<D>::TW; ++j) cur[j] = zero4();
}

// The summaries of one chunk: for each 32-token step (one block), the wave's tiles of
// S_b += phi(K)^T V (flushed into S~ when the block changes) and, for waves below P,
// z tile fi = wave += phi(K)^T [blk == column].
template <int D>
__device__ __forceinline__ void pair_accumulate(const unsigned char* slot, int chunk, const PairShape& sh,
                                                const float* wt, int wave, int g, int n, int& curblk,
                                                f32x4 (&cur)[PairCfg<D>::TW], Mixed<D>& mix,
                                                f32x4& zacc) {
    constexpr int P = PairCfg<D>::P, T = PairCfg<D>::T, TW = PairCfg<D>::TW, CPR = PairCfg<D>::CPR;
    const unsigned char* const fk = slot;
    const unsigned char* const fv = slot + PairCfg<D>::kRows;
#pragma unroll
    for (int S = 0; S < kPChunk / 32; ++S) {
        const int tok0 = kPChunk * chunk + 32 * S;
        if (tok0 >= sh.N) break;
        const int blk = tok0 / sh.C;  // every token of the step is in this block (uniform)
        if (blk != curblk) {
            if (curblk >= 0) pair_flush<D>(wt, curblk, cur, mix);
            curblk = blk;
        }
#pragma unroll
        for (int j = 0; j < TW; ++j) {
            const int t = wave + kPW * j;
            if (t < T) {
                const bf16x8 a = lds_operand_t(fk, 32 * S, 16 * (t / P), CPR, g, n);  // phi(K)^T: features 16 fi + n
                const bf16x8 b = lds_operand_t(fv, 32 * S, 16 * (t % P), CPR, g, n);  // V^T as B: values 16 ci + n
                cur[j] = mfma32(a, b, cur[j]);
            }
        }
        if (wave < P) {
            const bf16x8 az = lds_operand_t(fk, 32 * S, 16 * wave, CPR, g, n);
            const __bf16 one = (__bf16)(n == blk ? 1.f : 0.f);
            const bf16x8 ind = {one, one, one, one, one, one, one, one};
            zacc = mfma32(az, ind, zacc);
        }
    }
}

// S~_i of one block to its ring buffer as S~^T[c][f], split into bf16 hi + lo: lane
// (g, n) of the wave's tile (fi, ci) holds features 16 fi + 4g .. +3 of value 16 ci + n.
template <int D>
__device__ __forceinline__ void pair_stage_block(unsigned char* st, const f32x4 (&tiles)[PairCfg<D>::TW], int wave,
                                                 int g, int n) {
    constexpr int P = PairCfg<D>::P, T = PairCfg<D>::T, TW = PairCfg<D>::TW, CPR = PairCfg<D>::CPR;
#pragma unroll
    for (int j = 0; j < TW; ++j) {
        const int t = wave + kPW * j;
        if (t >= T) continue;
        const f32x4 s = tiles[j];
        uint32_t h0, l0, h1, l1;
        split2_bf16(s[0], s[1], h0, l0);
        split2_bf16(s[2], s[3], h1, l1);
        const int f = 16 * (t / P) + 4 * g, c = 16 * (t % P) + n;
        const int off = 16 * swz(c, f >> 3, CPR) + 2 * (f & 7);
        *reinterpret_cast<u32x2*>(st + off) = u32x2{h0, h1};
        *reinterpret_cast<u32x2*>(st + D * D * 2 + off) = u32x2{l0, l1};
    }
}

// S~_i of blocks first .. last to the ring (buffer i % 4); block i's tiles are read
// with indexed register moves.
template <int D>
__device__ __forceinline__ void pair_stage_mixed(unsigned char* ring, const Mixed<D>& mix,
                                                 int first, int last, int wave, int g, int n) {
    constexpr int TW = PairCfg<D>::TW;
    for (int i = first; i <= last; ++i) {
        f32x4 tiles[TW];
#pragma unroll
        for (int j = 0; j < TW; ++j)
            tiles[j] = f32x4{mix.v[0][16 * j + i], mix.v[1][16 * j + i], mix.v[2][16 * j + i], mix.v[3][16 * j + i]};
        pair_stage_block<D>(ring + (i & 3) * PairCfg<D>::kStBuf, tiles, wave, g, n);
    }
}

// Y of the wave's query tile of a chunk (rows 16 wave .. +15 of the chunk in LDS, phi
// applied), every value tile: the same number of stores on every wave and chunk; the
// stores of rows past N fall outside the output's range and are dropped.  OUT16:
// bfloat16 output.
template <int D, bool OUT16>
__device__ __forceinline__ void pair_outputs(const unsigned char* lds, const rsrc_t& rY, const OutSpec& o,
                                             const PairShape& sh, int chunk, int wave, int g, int n) {
    using Cfg = PairCfg<D>;
    constexpr int P = Cfg::P, KS = Cfg::KS, CPR = Cfg::CPR;
    const int row0 = kPChunk * chunk + 16 * wave;  // first query of the tile
    const bool valid = row0 < sh.N;
    const int i = valid ? row0 / sh.C : 0;
    const unsigned char* const qa = lds + Cfg::kQ;
    const unsigned char* const st = lds + (i & 3) * Cfg::kStBuf;
    const unsigned char* const zt = lds + Cfg::kZt + i * Cfg::kZtBuf;
    bf16x8 bq[KS];  // phi(Q) as B: query n, features 32 ks + 8 g .. +7
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        bq[ks] = *reinterpret_cast<const bf16x8*>(qa + 16 * swz(16 * wave + n, 4 * ks + g, CPR));
    // normaliser: rows 0 and 1 of the A operand are z~ hi and lo
    f32x4 dacc = zero4();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        bf16x8 az = {};
        if (n < 2) az = *reinterpret_cast<const bf16x8*>(zt + 2 * (n * D + 32 * ks + 8 * g));
        dacc = mfma32(az, bq[ks], dacc);
    }
    const float den = __shfl(dacc[0] + dacc[1], n, 64);  // lane (0, n): rows 0 and 1 of column n
    const float rden = out_scale(o, den + kEps);
    auto tile = [&](int c) {  // value tile c of the 16 queries, normalised
        f32x4 y = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int off = 16 * swz(16 * c + n, 4 * ks + g, CPR);  // S~^T[16c + n][32ks + 8g ..]
            const bf16x8 ah = *reinterpret_cast<const bf16x8*>(st + off);
            const bf16x8 al = *reinterpret_cast<const bf16x8*>(st + D * D * 2 + off);
            y = mfma32(ah, bq[ks], y);
            y = mfma32(al, bq[ks], y);
        }
        // lane (g, n): values 16c + 4g .. +3 of query row0 + n
        return f32x4{y[0] * rden, y[1] * rden, y[2] * rden, y[3] * rden};
    };
    if constexpr (OUT16) {
#pragma unroll
        for (int c = 0; c < P; ++c) {
            const f32x4 v = tile(c);
            const uint32_t off = off_if(valid, ((uint32_t)(row0 + n) * D + 16 * c + 4 * g) * 2);
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])}, rY, (int)off, 0, 2);
        }
    } else {
        // tiles c, c + 1 fill the 128-byte lines of their rows: two stores of whole lines
#pragma unroll
        for (int c = 0; c < P; c += 2) {
            const f32x4 y0 = tile(c), y1 = tile(c + 1);
            f32x4 top, bottom;
            whole_lines(y0, y1, n, top, bottom);
            const uint32_t col = 16 * (c + n / 8) + 4 * g, r = row0 + n % 8;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, top), rY,
                                                   (int)off_if(valid, (r * D + col) * 4), 0, 2);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, bottom), rY,
                                                   (int)off_if(valid, ((r + 8) * D + col) * 4), 0, 2);
        }
    }
}

// One Q chunk of phase 2: (after a barrier, when not the first) phi(Q) of chunk c
// from R to LDS and R refilled with chunk c + 2; S~ of the blocks the chunk meets first
// to the ring; barrier; the wave's outputs.  Every wave is done with the previous
// chunk's Q area and ring buffers at the leading barrier.  A chunk meets at most four
// blocks (blocks hold at least 32 tokens), so the ring holds every block it reads.
template <int D, bool OUT16>
__device__ __forceinline__ void pair_q_chunk(unsigned char* lds, const Mixed<D>& mix,
                                             PairRows<D>& R, const rsrc_t& rQ, const rsrc_t& rY, const OutSpec& o,
                                             const PairShape& sh, int c, int& staged, int wave, int lane) {
    const int g = lane >> 4, n = lane & 15;
    if (c > 0) lds_barrier();
    pair_rows_stage<D, true>(R, lds + PairCfg<D>::kQ, wave, lane);
    pair_rows_load<D>(rQ, c + 2, sh, wave, lane, R);
    const int last = min(sh.M - 1, (kPChunk * c + kPChunk - 1) / sh.C);
    pair_stage_mixed<D>(lds, mix, staged + 1, last, wave, g, n);
    staged = last;
    lds_barrier();
    pair_outputs<D, OUT16>(lds, rY, o, sh, c, wave, g, n);
}

template <int D, bool OUT16>
__global__ __launch_bounds__(64 * kPW) void pair_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                       const uint16_t* __restrict__ V, const float* __restrict__ W,
                                                       OutSpec o, PairShape sh) {
    using Cfg = PairCfg<D>;
    constexpr int P = Cfg::P, TW = Cfg::TW;
    static_assert(kPChunk == 16 * kPW, "one query tile per wave and chunk");
    __shared__ __align__(16) unsigned char lds[Cfg::kBytes];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, n = lane & 15;
    const int64_t pair = blockIdx.x;
    const uint32_t pair_bytes = (uint32_t)sh.N * D * 2;
    const rsrc_t rQ = make_rsrc(Q + pair * sh.N * D, pair_bytes);
    const rsrc_t rK = make_rsrc(K + pair * sh.N * D, pair_bytes);
    const rsrc_t rV = make_rsrc(V + pair * sh.N * D, pair_bytes);
    constexpr int esz = OUT16 ? 2 : 4;
    const rsrc_t rY = make_rsrc(static_cast<unsigned char*>(o.y) + pair * sh.N * D * esz, (uint32_t)sh.N * D * esz);
    if (sh.heads > 0) W += (pair % sh.heads) * sh.M * sh.M;  // one matrix per head
    float* const wt = reinterpret_cast<float*>(lds + Cfg::kW);  // W^T, zero-padded to 16 x 16
    if (threadIdx.x < kPMaxB * kPMaxB) {  // read after the first barrier
        const int b = threadIdx.x / kPMaxB, i = threadIdx.x % kPMaxB;
        wt[threadIdx.x] = i < sh.M && b < sh.M ? W[i * sh.M + b] : 0.f;
    }

    // ---- phase 1: summaries, mixed into S~ as each block completes ----
    Mixed<D> mix;  // the wave's tiles of S~_i for every i
    f32x4 cur[TW];  // of S_b for the current block
#pragma unroll
    for (int e = 0; e < 4; ++e) mix.v[e] = 0.f;
#pragma unroll
    for (int j = 0; j < TW; ++j) cur[j] = zero4();
    f32x4 zacc = zero4();
    int curblk = -1;
    unsigned char* const slot0 = lds;
    unsigned char* const slot1 = lds + Cfg::kSlot;
    {
        PairLoads<D> A, B;
        pair_loads<D>(rK, rV, 0, sh, wave, lane, A);
        pair_loads<D>(rK, rV, 1, sh, wave, lane, B);
        pair_stage<D>(A, slot0, wave, lane);
        pair_loads<D>(rK, rV, 2, sh, wave, lane, A);
        lds_barrier();
        for (int c = 0;; c += 2) {
            // chunk c in slot 0 (A holds c + 2), chunk c + 1 in B
            pair_accumulate<D>(slot0, c, sh, wt, wave, g, n, curblk, cur, mix, zacc);
            if (c + 1 >= sh.nchunks) break;
            pair_stage<D>(B, slot1, wave, lane);  // slot 1 was last read before the barrier passed
            pair_loads<D>(rK, rV, c + 3, sh, wave, lane, B);
            lds_barrier();
            pair_accumulate<D>(slot1, c + 1, sh, wt, wave, g, n, curblk, cur, mix, zacc);
            if (c + 2 >= sh.nchunks) break;
            pair_stage<D>(A, slot0, wave, lane);
            pair_loads<D>(rK, rV, c + 4, sh, wave, lane, A);
            lds_barrier();
        }
    }
    // Q of the first two chunks, in flight while the last block is mixed (chunk 1
    // first: the loop below then finds as many later loads and stores after chunk c's
    // loads on its first pass as on the others, and waits for chunk c's loads only)
    PairRows<D> QA, QB;
    pair_rows_load<D>(rQ, 1, sh, wave, lane, QB);
    pair_rows_load<D>(rQ, 0, sh, wave, lane, QA);
    pair_flush<D>(wt, curblk, cur, mix);  // the last block
    // z of every block to LDS: lane (g, n) of wave w < P holds z_n[16w + 4g + e]
    float* const zall = reinterpret_cast<float*>(lds + Cfg::kZ);
    if (wave < P) {
#pragma unroll
        for (int e = 0; e < 4; ++e) zall[(16 * wave + 4 * g + e) * kPMaxB + n] = zacc[e];
    }
    lds_barrier();  // also: every wave is done with the chunk slots (the S~ ring below)

    // ---- phase 2: z~ of every block, then Q chunk by chunk ----
    for (int t = threadIdx.x; t < sh.M * D; t += 64 * kPW) {
        const int i = t / D, f = t % D;
        float z = 0.f;
        for (int bb = 0; bb < sh.M; ++bb) z = fmaf(wt[kPMaxB * bb + i], zall[f * kPMaxB + bb], z);
        const bf16pair p = split_bf16(z);
        __bf16* const zt = reinterpret_cast<__bf16*>(lds + Cfg::kZt + i * Cfg::kZtBuf);
        zt[f] = p.hi;
        zt[D + f] = p.lo;
    }
    // Per chunk: Q to LDS and the S~ of blocks it meets first to the ring, barrier,
    // outputs, barrier (the Q area and ring buffers are then free again).  A chunk
    // meets at most four blocks (blocks hold at least 32 tokens), so the ring's four
    // buffers hold every block a chunk reads.
    int staged = -1;  // the last block whose S~ is in the ring
    pair_q_chunk<D, OUT16>(lds, mix, QA, rQ, rY, o, sh, 0, staged, wave, lane);
    int c = 1;
    for (; c + 1 < sh.nchunks; c += 2) {
        pair_q_chunk<D, OUT16>(lds, mix, QB, rQ, rY, o, sh, c, staged, wave, lane);
        pair_q_chunk<D, OUT16>(lds, mix, QA, rQ, rY, o, sh, c + 1, staged, wave, lane);
    }
    if (c < sh.nchunks) pair_q_chunk<D, OUT16>(lds, mix, QB, rQ, rY, o, sh, c, staged, wave, lane);
}

}  // namespace

bool pair_applicable(int D, int64_t BH, int64_t N, int64_t M) {
    // Summaries on chip for moderate lengths: blocks of whole 32-token steps, at most
    // 16 of them, enough pairs to fill the GPU with one workgroup each (shorter
    // sequences take the token-level kernel, longer ones or few pairs the staged
    // kernels).
    if (D != 32 && D != 64) return false;
    if (M > kPMaxB || N % M || (N / M) % 32 || N <= 256 || N > 8192) return false;
    return BH >= 256;
}

hipError_t launch_pair(const void* q, const void* k, const void* v, const float* W, const OutSpec& out, int64_t BH,
                       int64_t N, int D, int64_t M, int heads, hipStream_t stream) {
    PairShape sh;
    sh.N = (int)N;
    sh.M = (int)M;
    sh.C = (int)(N / M);
    sh.nchunks = (int)((N + kPChunk - 1) / kPChunk);
    sh.heads = heads;
    const dim3 grid((unsigned)BH), block(64 * kPW);
    const uint16_t* qq = static_cast<const uint16_t*>(q);
    const uint16_t* kk = static_cast<const uint16_t*>(k);
    const uint16_t* vv = static_cast<const uint16_t*>(v);
    const bool b16 = out.bf16;
    switch (D) {
        case 32:
            if (b16) pair_kernel<32, true><<<grid, block, 0, stream>>>(qq, kk, vv, W, out, sh);
            else pair_kernel<32, false><<<grid, block, 0, stream>>>(qq, kk, vv, W, out, sh);
            break;
        case 64:
            if (b16) pair_kernel<64, true><<<grid, block, 0, stream>>>(qq, kk, vv, W, out, sh);
            else pair_kernel<64, false><<<grid, block, 0, stream>>>(qq, kk, vv, W, out, sh);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace mhla
