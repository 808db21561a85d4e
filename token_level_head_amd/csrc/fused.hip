// fused.hip -- the whole MHLA forward pass for short sequences (N <= 256, M <= 16
// blocks, non-causal, bf16) in one kernel, in the token-level form of "MHLA:
// Restoring Expressivity of Linear Attention via Token-Level Multi-Head" (§4.2,
// Eq. 5): with blk(t) the block of token t,
//
//   A[t, j] = W[blk(t), blk(j)] * phi(q_t) . phi(k_j),
//   y_t     = sum_j A[t, j] v_j / (sum_j A[t, j] + 1e-6)      (guard: "Linear Attention 笔记" §4/§5)
//
// which is exactly the four steps of §4.1 regrouped (S~_i = sum_b W[i,b] phi(K_b)^T V_b,
// so phi(q_t) S~_i = sum_j A[t, j] v_j, and likewise for the normaliser), with phi =
// ELU + 1 ("Linear Attention 笔记" §2).
//
// Why this form here: for blocks shorter than d (DiT-S/2 at 256x256: 16 tokens, d = 64)
// the d x d summaries are four times larger than the tokens they summarise, and
// forming, mixing and reading them needs float32 operands split into bf16 hi + lo
// at every stage.  The token-level form needs no summaries: two bf16 products per
// 16 x 16 tile of A, with only A split into hi + lo.
//
// Work is split by 16-query tiles: one persistent workgroup of eight waves (two per
// SIMD) per CU takes an equal contiguous share of the B*H*ceil(N/16) query tiles
// (DiT-S/2 at 256: 24 tiles, one and a half pairs, on each of 256 CUs) and walks it
// in jobs of up to 16 tiles -- two per wave -- of one pair, or of several short
// sequences whose keys together fill at most 256 rows.  Each job's keys stream
// through LDS in chunks of 128 rows, a three-stage pipeline per chunk:
//   loads    V rows and (at a job's first chunk) the job's Q tiles are copied from
//            global memory straight into LDS (buffer loads with the LDS flag, no
//            registers); K rows and the chunk's factors W[i, blk(key)] go to registers;
//            issued two chunks ahead, before the barrier that ends the chunk before;
//   staging  half-way through the computation of the previous chunk: phi(K) and the
//            factors are written into the other K slot, and phi(Q) of the wave's
//            tiles is formed in place in the Q area (read into registers when the job
//            starts);
//   compute  each wave walks the chunk 32 keys at a time, for its two tiles:
//     scores  (16 keys x 16 queries, per key tile): phi(K) phi(Q)^T on MFMA, float32;
//     weights A = score * W[blk(query), blk(key)] (factors from LDS), split into
//             bf16 hi + lo;
//     output  Y^T += V^T A^T for each 16-column value tile (hi and lo), and the
//             normaliser as the same product with a row of ones, so numerator and
//             denominator use identical rounded weights.
//            The (step, tile) units form a software pipeline: a unit's split runs while
//            the previous unit's output products and the next unit's score products are
//            in the matrix cores.
// The score MFMA leaves lane (g, n) with keys 4g..4g+3 of two key tiles for query n,
// which is the B operand of the 16x16x32 V^T A^T product when k-slot 8g + 4h + i stands
// for key 16h + 4g + i; V row-major in LDS is read in that order with the gfx950
// transposing LDS read (ds_read_b64_tr_b16), four rows of four columns per 16-lane
// group.  The output MFMA leaves lane (g, n) with value columns 16c + 4g .. +3 of
// query n: one reciprocal per query and 16-byte stores.
// A pair whose tiles fall into two workgroups' shares is staged by both; neighbouring
// shares go to workgroups 8 apart, which the round-robin dispatch puts on one XCD,
// so the second reads that pair from the XCD's L2.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"
#include "lds_tiles.hpp"

namespace mhla {

namespace {

constexpr int kWaves = 8;        // one workgroup per CU, two waves per SIMD
constexpr int kMaxBlocks = 16;   // M: rows of the factor tables
constexpr int kMaxTokens = 256;  // N
constexpr int kJobKeys = 256;    // key rows of a job: its pairs' keys, each pair padded to 32
constexpr int kJobTiles = 2 * kWaves;  // query tiles of a job: two per wave
constexpr int kChunk = 128;      // key rows staged per pipeline step
constexpr int kWaveRows = kChunk / kWaves;  // key rows each wave loads and stages per chunk
constexpr int kStageAt = 4;      // eighths of a chunk's computation done when the next chunk is staged

// LDS: two K slots, each phi(K) bf16 [kChunk keys][D] (row-major, swizzled 16-byte
// pieces) and the chunk's factors, float [block][kChunk keys] (blocks that are not
// whole 16-token tiles) or [block][kChunk / 16 key tiles] (blocks of whole tiles);
// three V slots, V bf16 [kChunk keys][D] in the same layout, copied straight from
// global memory; and the Q area, the query tiles of the next job, [wave][2 tiles][16
// rows][D] likewise.  Chunk c is computed from K slot c % 2 and V slot c % 3 while
// chunk c + 1 is staged into K slot (c + 1) % 2 and chunk c + 2's V is in flight to V
// slot (c + 2) % 3.
template <int D>
struct FusedLds {
    static constexpr int kK = kChunk * D * 2;
    static constexpr int kTab = kMaxBlocks * kChunk * 4;
    static constexpr int kKSlot = kK + kTab;
    static constexpr int kV = kChunk * D * 2;
    static constexpr int kVBase = 2 * kKSlot;
    static constexpr int kTileQ = 16 * D * 2;  // one query tile
    static constexpr int kQBase = kVBase + 3 * kV;
    static constexpr int kBytes = kQBase + kJobTiles * kTileQ;
};

// Global -> LDS copy of 16 bytes per lane (no registers): lane i writes LDS bytes
// dst + 16 i .. +15 (dst wave-uniform) with 16 bytes of buffer r at byte offset off
// (zeros at or past the end of the buffer).  Counted by vmcnt; the data is read only
// after a barrier whose release fence waits for it.
__device__ __forceinline__ void buf_to_lds16(rsrc_t r, unsigned char* dst, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, 0);
}

// Score operand types: 16x16x32 (8 bf16 per lane) for d >= 32, 16x16x16 (4) for d = 16.
template <int D>
struct Op {
    typedef bf16x8 type;
};
template <>
struct Op<16> {
    typedef bf16x4 type;
};
template <int D>
struct RawT {
    typedef u32x4 type;
};
template <>
struct RawT<16> {
    typedef u32x2 type;
};

template <int D>
__device__ __forceinline__ f32x4 score_mfma(const typename Op<D>::type& a, const typename Op<D>::type& b, f32x4 c) {
    if constexpr (D == 16)
        return mfma16(a, b, c);
    else
        return mfma32(a, b, c);
}

template <int D>
__device__ __forceinline__ typename RawT<D>::type load_raw(rsrc_t r, uint32_t off) {
    if constexpr (D >= 32)
        return buf_load128(r, off);
    else
        return buf_load64(r, off);
}

template <int D>
__device__ __forceinline__ typename Op<D>::type phi_op(const typename RawT<D>::type& w) {
    if constexpr (D >= 32)
        return __builtin_bit_cast(bf16x8, u32x4{phi_pair(w[0]), phi_pair(w[1]), phi_pair(w[2]), phi_pair(w[3])});
    else
        return __builtin_bit_cast(bf16x4, u32x2{phi_pair(w[0]), phi_pair(w[1])});
}

// Makes x's value needed here (an empty instruction reading it).
template <typename T>
__device__ __forceinline__ void consume(const T& x) {
    asm volatile("" ::"v"(x));
}

// x / d for 0 <= x < 2^20 / d, with m = ceil(2^20 / d) computed on the host.
__device__ __forceinline__ int divm(int x, int m) { return (int)(((uint32_t)x * (uint32_t)m) >> 20); }

}  // namespace

// Sizes of a fused launch, with host-computed reciprocals (m*) for every division the
// kernel makes.  NP: N padded to 32; KTP = NP / 16 key tiles per pair, KTN of which hold
// tokens; CT: 16-token tiles per block (blocks of whole tiles); pps: pairs per job.
struct FusedShape {
    int N, M, C, NP, QT, KTP, KTN, CT, pps, heads;
    int mNP, mQT, mKTP, mC, mCT;
    int64_t tiles_per;  // query tiles per workgroup (floor), and
    int tiles_rem;      // the remainder spread over the first workgroups
};

namespace {

// A job: `len` query tiles starting at tile q of pair p, from np consecutive pairs whose
// keys form rows = np * NP key rows (len <= kJobTiles, rows <= kJobKeys).  head: the
// head of pair p (per-head mixing matrices).
struct Job {
    int64_t p;
    int q, len, np, rows, head;
};
__device__ __forceinline__ Job make_job(int64_t p, int q, int head, int64_t remaining, const FusedShape& sh) {
    Job j;
    j.p = p;
    j.q = q;
    j.head = head;
    j.len = (int)min<int64_t>(remaining, (int64_t)(sh.pps * sh.QT - q));
    j.np = divm(q + j.len - 1, sh.mQT) + 1;
    j.rows = j.np * sh.NP;
    return j;
}
// head of pair p + slot, from the head of pair p
__device__ __forceinline__ int head_at(const Job& j, int slot, const FusedShape& sh) {
    if (sh.heads <= 0) return 0;
    int h = j.head + slot;
    while (h >= sh.heads) h -= sh.heads;
    return h;
}

// Position in a stream of chunks: chunk k (key rows kChunk k .. kChunk (k + 1) - 1) of
// job `job`; `left` counts the query tiles of the workgroup's range after this job.
struct Cursor {
    Job job;
    int k;
    int64_t left;
    bool valid;
};
__device__ __forceinline__ void advance(Cursor& c, const FusedShape& sh) {
    if (!c.valid) return;
    if (kChunk * (c.k + 1) < c.job.rows) {
        ++c.k;
        return;
    }
    if (c.left <= 0) {
        c.valid = false;
        return;
    }
    const int qn = c.job.q + c.job.len, dp = divm(qn, sh.mQT);
    c.job = make_job(c.job.p + dp, qn - dp * sh.QT, head_at(c.job, dp, sh), c.left, sh);
    c.left -= c.job.len;
    c.k = 0;
}

// What one wave loads for a chunk: into registers, the 16-byte pieces of its
// kWaveRows K rows (NL per lane; phi is applied when they are staged) and its thread's
// factor entries; directly into LDS, its V rows (into the chunk's slot) and, at a
// job's first chunk, the job's query tiles wave and wave + 8 (into the Q area).
template <int D, bool TILED>
struct ChunkLoads {
    static constexpr int LPR = D / 8;                              // lanes per key row
    static constexpr int NL = (kWaveRows * LPR + 63) / 64;         // row pieces per lane
    static constexpr int NW = TILED ? 1 : kMaxBlocks * kChunk / (64 * kWaves);  // factor entries per thread
    static constexpr int NV = (kWaveRows * D / 8 + 63) / 64;        // V copy instructions per wave
    static constexpr int NQ = 2 * ((16 * D / 8 + 63) / 64);         // Q copy instructions per wave (a job's first chunk)
    static constexpr int kLoads = NV + NL + NW;                     // loads every chunk issues, and NQ more at a job's first
    u32x4 k[NL];
    float w[NW];
    Cursor at;
};

// Workgroup barrier after which the LDS writes of every wave before it are visible,
// including its copies into LDS except the `newer` loads issued last, which may still
// be in flight (the release fence of an ordinary barrier would wait for them too).
// Loads complete in order, so waiting until at most `newer` are outstanding completes
// every older one.
template <int newer>
__device__ __forceinline__ void dma_barrier() {
    static_assert(newer < 64, "vmcnt field");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((newer & 15) | ((newer >> 4) << 14) | 0x0070);  // vmcnt(newer) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Copies rows of the [N][D] bf16 matrix of pair `pair` into LDS units L0 .. L0 + 64 n - 1
// of a swizzled [rows][D] array (row 0 of the array = global row `grow0`; rows at or past
// `nvalid` are written as zeros): n = rows * D * 2 / 1024 instructions of 64 lanes (half
// a wave for 512 bytes).  The rows of one instruction lie in one pair.
template <int D>
__device__ __forceinline__ void rows_to_lds(const uint16_t* __restrict__ X, int64_t pair, int N, int grow0, int nvalid,
                                            unsigned char* arr, int L0, int nunits, int lane) {
    constexpr int CPR = D / 8;
    const rsrc_t r = make_rsrc(X + pair * N * D, (uint32_t)N * D * 2);
#pragma unroll
    for (int u = 0; u * 64 < nunits; ++u) {
        const int L = L0 + 64 * u + lane;
        int row, piece;
        unswz(L, CPR, row, piece);
        const bool ok = row < nvalid;
        if (64 * u + lane < nunits)
            buf_to_lds16(r, arr + 16 * (L0 + 64 * u), off_if(ok, (uint32_t)((grow0 + row) * D + 8 * piece) * 2));
    }
}

template <int D, bool TILED>
__device__ __forceinline__ void chunk_loads(const Cursor& at, const FusedShape& sh, const uint16_t* __restrict__ Q,
                                            const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                            const rsrc_t& rW, unsigned char* vslot, unsigned char* qarea, int wave,
                                            int lane, ChunkLoads<D, TILED>& L) {
    // Issue order: V copies, K loads, factor loads, Q copies (a job's first chunk only).
    // Loads complete in order, so the wait for the K registers at staging covers V.
    constexpr int LPR = ChunkLoads<D, TILED>::LPR, NL = ChunkLoads<D, TILED>::NL, CPR = D / 8;
    L.at = at;
    const Job& jb = at.job;
    // V rows kWaveRows * wave .. + kWaveRows - 1 of the chunk, 8 rows (one pair) per
    // instruction; issued for every chunk (rows past the job or the sequence, or an
    // exhausted cursor, read as zeros and are never used), so that every chunk issues
    // the same number of copies before its K and factor loads
    {
        const int rr0 = kWaveRows * wave;                   // first row in the chunk
        const int kr0 = kChunk * at.k + rr0;                // first row in the job
        const bool live = at.valid && kr0 < jb.rows;
        const int slot_ = live ? divm(kr0, sh.mNP) : 0, key0 = kr0 - slot_ * sh.NP;
        rows_to_lds<D>(V, live ? jb.p + slot_ : 0, sh.N, key0 - rr0, live ? sh.N - (key0 - rr0) : 0, vslot,
                       rr0 * CPR, kWaveRows * CPR, lane);
    }
    const uint32_t pair_bytes = (uint32_t)sh.N * D * 2;
    // K rows kWaveRows * wave .. + kWaveRows - 1 of the chunk, 64 / LPR rows at a time
#pragma unroll
    for (int u = 0; u < NL; ++u) {
        const int kr0 = kChunk * at.k + kWaveRows * wave + 64 / LPR * u;  // first row of the piece in the job
        const bool live = at.valid && kr0 < jb.rows;
        const int slot_ = live ? divm(kr0, sh.mNP) : 0;
        const int64_t pair = live ? jb.p + slot_ : 0;
        const rsrc_t rK = make_rsrc(K + pair * sh.N * D, pair_bytes);
        const int key = kr0 - slot_ * sh.NP + lane / LPR;  // keys past N read zero
        const bool ok = live && 64 / LPR * u + lane / LPR < kWaveRows;
        L.k[u] = buf_load128(rK, off_if(ok, ((uint32_t)key * D + 8 * (lane % LPR)) * 2));
    }
    // factor entries (rW: the whole W array, [M][M] or [H][M][M])
    if constexpr (TILED) {
        // [block qb][key tile kt of the chunk], thread qb * (kChunk / 16) + kt
        constexpr int KTC = kChunk / 16;
        const int qb = threadIdx.x / KTC, kt = kChunk / 16 * at.k + threadIdx.x % KTC;  // key tile in the job
        const int slot_ = divm(kt, sh.mKTP), ktp = kt - slot_ * sh.KTP;               // key tile in its pair
        const bool ok = at.valid && qb < sh.M && kt < jb.np * sh.KTP && ktp < sh.KTN;
        const int head = head_at(jb, slot_, sh);
        L.w[0] = __uint_as_float(
            buf_load32(rW, off_if(ok, (uint32_t)((head * sh.M + qb) * sh.M + divm(ktp, sh.mCT)) * 4)));
    } else {
        // [block threadIdx.x / kChunk + (64 kWaves / kChunk) r][key threadIdx.x % kChunk of the chunk]
        const int kr = kChunk * at.k + (threadIdx.x % kChunk);
        const int slot_ = divm(kr, sh.mNP), key = kr - slot_ * sh.NP;
        const bool live = at.valid && kr < jb.rows && key < sh.N;
        const int head = head_at(jb, slot_, sh);
        const int b = divm(key, sh.mC);
#pragma unroll
        for (int r = 0; r < ChunkLoads<D, TILED>::NW; ++r) {
            const int qb = (int)(threadIdx.x / kChunk) + 64 * kWaves / kChunk * r;
            L.w[r] = __uint_as_float(
                buf_load32(rW, off_if(live && qb < sh.M, (uint32_t)((head * sh.M + qb) * sh.M + b) * 4)));
        }
    }
    // last: the query tiles wave, wave + 8 of a new job, 16 rows each
    if (at.valid && at.k == 0) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int ti = jb.q + wave + kWaves * r, po = divm(ti, sh.mQT), qt = ti - po * sh.QT;
            const bool live = wave + kWaves * r < jb.len;
            rows_to_lds<D>(Q, jb.p + po, sh.N, 16 * qt, live ? sh.N - 16 * qt : 0,
                           qarea + (2 * wave + r) * FusedLds<D>::kTileQ, 0, 16 * CPR, lane);
        }
    }
}

// Per-wave state of the current job: its query tiles (wave and wave + 8 of the job)
// and their accumulators.
template <int D>
struct JobTiles {
    static constexpr int FS = D >= 32 ? D / 32 : 1;
    static constexpr int VT = D / 16;
    typename Op<D>::type bq[2][FS];  // phi(Q) as the score MFMA's B operand
    f32x4 oacc[2][VT], dacc[2];
    int slot[2], qb[2], tq[2];       // pair slot (uniform), query block and row of the lane's query
    int64_t yrow[2];
    bool live[2];
};

// Stages chunk L.at into K slot `buf`: phi(K) row-major with swizzled 16-byte pieces
// and the factors (its V is copied separately); at a job's first chunk also phi(Q) of
// the wave's tiles, in place in the wave's part of the Q area.  Runs while the
// previous chunk is being computed from the other K slot.
template <int D, bool TILED>
__device__ __forceinline__ void stage_chunk(const ChunkLoads<D, TILED>& L, const FusedShape& sh, unsigned char* buf,
                                            unsigned char* qarea, int wave, int lane) {
    constexpr int LPR = ChunkLoads<D, TILED>::LPR, NL = ChunkLoads<D, TILED>::NL;
    constexpr int CPR = D / 8;
    // Take every loaded register here, on every path: a load left pending on some path
    // makes the compiler wait for it (and, loads and stores completing in order, for
    // everything issued before it) wherever that register is next reused.
#pragma unroll
    for (int u = 0; u < NL; ++u) consume(L.k[u]);
#pragma unroll
    for (int r = 0; r < ChunkLoads<D, TILED>::NW; ++r) consume(L.w[r]);
    if (!L.at.valid) return;
    unsigned char* const fk = buf;
    float* const tab = reinterpret_cast<float*>(buf + FusedLds<D>::kK);
    const Job& jb = L.at.job;
#pragma unroll
    for (int u = 0; u < NL; ++u) {
        const int rr = kWaveRows * wave + 64 / LPR * u + lane / LPR;  // row in the chunk
        if (kChunk * L.at.k + kWaveRows * wave + 64 / LPR * u >= jb.rows || 64 / LPR * u + lane / LPR >= kWaveRows)
            continue;
        const u32x4 w = L.k[u];
        *reinterpret_cast<u32x4*>(fk + 16 * swz(rr, lane % LPR, CPR)) =
            u32x4{phi_pair(w[0]), phi_pair(w[1]), phi_pair(w[2]), phi_pair(w[3])};
    }
    if constexpr (TILED) {
        if ((int)threadIdx.x < kMaxBlocks * kChunk / 16) tab[threadIdx.x] = L.w[0];
    } else {
#pragma unroll
        for (int r = 0; r < ChunkLoads<D, TILED>::NW; ++r) {
            const int qb = (int)(threadIdx.x / kChunk) + 64 * kWaves / kChunk * r;
            if (qb < sh.M) tab[qb * kChunk + (threadIdx.x % kChunk)] = L.w[r];
        }
    }
    if (L.at.k == 0) {
        // the wave's copies of its query tiles have landed (an explicit wait: the
        // compiler does not relate these reads to the copies); phi in place, each lane
        // converting whole 16-byte units of the wave's region
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        asm volatile("" ::: "memory");
        unsigned char* const qw = qarea + 2 * wave * FusedLds<D>::kTileQ;
#pragma unroll
        for (int u = 0; u < 2 * FusedLds<D>::kTileQ / 16 / 64; ++u) {
            u32x4* const p = reinterpret_cast<u32x4*>(qw + 16 * (64 * u + lane));
            const u32x4 w = *p;
            *p = u32x4{phi_pair(w[0]), phi_pair(w[1]), phi_pair(w[2]), phi_pair(w[3])};
        }
    }
}

// The wave's tiles of job jb (tiles wave and wave + 8): pair slot, query row, block,
// output row.
template <int D>
__device__ __forceinline__ void job_header(const Job& jb, const FusedShape& sh, int wave, int n, JobTiles<D>& jt) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        jt.live[r] = wave + kWaves * r < jb.len;
        const int ti = jb.q + wave + kWaves * r, po = divm(ti, sh.mQT), qt = ti - po * sh.QT;
        jt.slot[r] = po;
        jt.tq[r] = 16 * qt + n;
        jt.qb[r] = divm(min(jt.tq[r], sh.N - 1), sh.mC);  // queries past N: any valid row (not stored)
        jt.yrow[r] = ((jb.p + po) * sh.N + jt.tq[r]) * D;
    }
}

// phi(Q) of the wave's tiles from the Q area as the score MFMA's B operand (lane
// (g, n): query n, features 32 f + 8 g .. +7; d = 16: 4 g .. 4 g + 3).
template <int D>
__device__ __forceinline__ void load_bq(const unsigned char* qarea, int wave, int g, int n, JobTiles<D>& jt) {
    constexpr int CPR = D / 8;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const unsigned char* const qt = qarea + (2 * wave + r) * FusedLds<D>::kTileQ;
#pragma unroll
        for (int f = 0; f < JobTiles<D>::FS; ++f) {
            if constexpr (D >= 32)
                jt.bq[r][f] = *reinterpret_cast<const bf16x8*>(qt + 16 * swz(n, 4 * f + g, CPR));
            else
                jt.bq[r][f] = *reinterpret_cast<const bf16x4*>(qt + 16 * swz(n, g >> 1, CPR) + 8 * (g & 1));
        }
    }
}

// Operands of one 32-key step read from LDS: phi(K) of key tiles 2S, 2S + 1 as the
// score MFMA's A operand (key n, features 32 f + 8 g .. +7; d = 16: 4 g .. 4 g + 3), and
// V as the output MFMA's A operand, read transposed: lane (g, n) of value tile c gets
// V[key 32S + 16hh + 4g + e][16c + n] as k-slot 8g + 4hh + e (it addresses key
// 32S + 16hh + 4g + n / 4, columns 16c + 4 (n % 4) .. +3).
template <int D>
struct StepOps {
    static constexpr int FS = D >= 32 ? D / 32 : 1;
    static constexpr int VT = D / 16;
    typename Op<D>::type ak[2][FS];
    bf16x8 av[VT];
};

template <int D>
__device__ __forceinline__ void step_ak(const unsigned char* buf, int S, int g, int n, StepOps<D>& o) {
    constexpr int FS = StepOps<D>::FS, CPR = D / 8;
    const unsigned char* const fk = buf;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int key = 32 * S + 16 * h + n;
#pragma unroll
        for (int f = 0; f < FS; ++f) {
            if constexpr (D >= 32)
                o.ak[h][f] = *reinterpret_cast<const bf16x8*>(fk + 16 * swz(key, 4 * f + g, CPR));
            else
                o.ak[h][f] = *reinterpret_cast<const bf16x4*>(fk + 16 * swz(key, g >> 1, CPR) + 8 * (g & 1));
        }
    }
}

template <int D>
__device__ __forceinline__ void step_av(const unsigned char* vbuf, int S, int g, int n, StepOps<D>& o) {
#pragma unroll
    for (int c = 0; c < StepOps<D>::VT; ++c) o.av[c] = lds_operand_t(vbuf, 32 * S, 16 * c, D / 8, g, n);
}

template <int D>
__device__ __forceinline__ void step_ops(const unsigned char* kbuf, const unsigned char* vbuf, int S, int g, int n,
                                         StepOps<D>& o) {
    step_ak<D>(kbuf, S, g, n, o);
    step_av<D>(vbuf, S, g, n, o);
}

// Factors of step S for the lane's query block qb: fac[h][i] multiplies the score of
// key 32S + 16h + 4g + i.  Blocks of whole 16-token tiles keep one factor per key tile.
template <bool TILED>
__device__ __forceinline__ void step_factors(const float* tab, int S, int qb, int g, f32x4 (&fac)[2]) {
    if constexpr (TILED) {
        const f32x2 f2 = *reinterpret_cast<const f32x2*>(tab + kChunk / 16 * qb + 2 * S);
        fac[0] = f32x4{f2[0], f2[0], f2[0], f2[0]};
        fac[1] = f32x4{f2[1], f2[1], f2[1], f2[1]};
    } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) fac[h] = *reinterpret_cast<const f32x4*>(tab + qb * kChunk + 32 * S + 16 * h + 4 * g);
    }
}

// Scores of one tile against the step's 32 keys, times the factors, split into bf16
// hi + lo halves laid out as the output MFMA's B operand (k-slot 8g + 4h + i: key
// 32S + 16h + 4g + i; column n: query n of the tile).
template <int D>
__device__ __forceinline__ void step_scores(const StepOps<D>& o, const typename Op<D>::type (&bq)[StepOps<D>::FS],
                                            const f32x4 (&fac)[2], bf16x8& ah, bf16x8& al) {
    constexpr int FS = StepOps<D>::FS;
    f32x4 sc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        sc[h] = zero4();
#pragma unroll
        for (int f = 0; f < FS; ++f) sc[h] = score_mfma<D>(o.ak[h][f], bq[f], sc[h]);
    }
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        split2_bf16(sc[h][0] * fac[h][0], sc[h][1] * fac[h][1], hw[2 * h], lw[2 * h]);
        split2_bf16(sc[h][2] * fac[h][2], sc[h][3] * fac[h][3], hw[2 * h + 1], lw[2 * h + 1]);
    }
    ah = __builtin_bit_cast(bf16x8, u32x4{hw[0], hw[1], hw[2], hw[3]});
    al = __builtin_bit_cast(bf16x8, u32x4{lw[0], lw[1], lw[2], lw[3]});
}

// Accumulates one tile's step: numerator V^T P (hi and lo) and the denominator as the
// column sums of P (a ones operand).
template <int D>
__device__ __forceinline__ void step_accumulate(const StepOps<D>& o, const bf16x8& ah, const bf16x8& al,
                                                f32x4 (&oacc)[StepOps<D>::VT], f32x4& dacc) {
    const bf16x8 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                         (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
#pragma unroll
    for (int c = 0; c < StepOps<D>::VT; ++c) {
        oacc[c] = mfma32(o.av[c], ah, oacc[c]);
        oacc[c] = mfma32(o.av[c], al, oacc[c]);
    }
    dacc = mfma32(ones, ah, dacc);
    dacc = mfma32(ones, al, dacc);
}

// One 32-key step (step S of the chunk in slot `buf`) for both tiles of the wave; a
// tile whose keys are not these (mask false) gets zero factors, so it adds nothing.
template <int D, bool TILED>
__device__ __forceinline__ void step_masked(const unsigned char* kbuf, const unsigned char* vbuf, int S,
                                            const bool (&mask)[2], JobTiles<D>& jt, int g, int n) {
    const float* const tab = reinterpret_cast<const float*>(kbuf + FusedLds<D>::kK);
    StepOps<D> o;
    step_ops<D>(kbuf, vbuf, S, g, n, o);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        f32x4 fac[2];
        step_factors<TILED>(tab, S, jt.qb[t], g, fac);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) fac[h][i] = mask[t] ? fac[h][i] : 0.f;
        bf16x8 ah, al;
        step_scores<D>(o, jt.bq[t], fac, ah, al);
        step_accumulate<D>(o, ah, al, jt.oacc[t], jt.dacc[t]);
    }
}

// A whole chunk of one pair against NT tiles that all belong to that pair, as a
// software pipeline over the units u = (step S, tile j) in that order: unit u splits
// its own scores while the output products of unit u - 1 and the score products of
// unit u + 1 (independent of the split) keep the matrix cores busy.  phi(K) of a step
// is read from LDS two units before its first score product, V at its first unit (one
// unit before its first output product).  `mid` (the staging of the next chunk) runs
// half-way, its vector work interleaving with the products still in flight.
template <int D, int NT, bool TILED, typename Hook>
__device__ __forceinline__ void chunk_tiles(const unsigned char* buf, const unsigned char* vbuf, const int (&ti)[2],
                                            JobTiles<D>& jt, int g, int n, const Hook& hook) {
    constexpr int NS = kChunk / 32, NU = NS * NT, FS = StepOps<D>::FS;
    const float* const tab = reinterpret_cast<const float*>(buf + FusedLds<D>::kK);
    StepOps<D> o[2];
    hook(-1, 0);
    step_ak<D>(buf, 0, g, n, o[0]);
    if constexpr (NT == 1) step_ak<D>(buf, 1, g, n, o[1]);
    // raw scores of unit 0
    f32x4 scn[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        scn[h] = zero4();
#pragma unroll
        for (int f = 0; f < FS; ++f) scn[h] = score_mfma<D>(o[0].ak[h][f], jt.bq[ti[0]][f], scn[h]);
    }
    bf16x8 ahp, alp;  // split weights of unit u - 1
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int S = u / NT, j = u % NT, t = ti[j];
        if (u + 2 < NU && (u + 2) % NT == 0) step_ak<D>(buf, (u + 2) / NT, g, n, o[((u + 2) / NT) & 1]);
        if (j == 0) step_av<D>(vbuf, S, g, n, o[S & 1]);
        // split unit u
        const f32x4 sc0 = scn[0], sc1 = scn[1];
        f32x4 fac[2];
        step_factors<TILED>(tab, S, jt.qb[t], g, fac);
        uint32_t hw[4], lw[4];
        split2_bf16(sc0[0] * fac[0][0], sc0[1] * fac[0][1], hw[0], lw[0]);
        split2_bf16(sc0[2] * fac[0][2], sc0[3] * fac[0][3], hw[1], lw[1]);
        split2_bf16(sc1[0] * fac[1][0], sc1[1] * fac[1][1], hw[2], lw[2]);
        split2_bf16(sc1[2] * fac[1][2], sc1[3] * fac[1][3], hw[3], lw[3]);
        const bf16x8 ah = __builtin_bit_cast(bf16x8, u32x4{hw[0], hw[1], hw[2], hw[3]});
        const bf16x8 al = __builtin_bit_cast(bf16x8, u32x4{lw[0], lw[1], lw[2], lw[3]});
        // output products of unit u - 1
        if (u > 0) {
            const int Sp = (u - 1) / NT, tp = ti[(u - 1) % NT];
            step_accumulate<D>(o[Sp & 1], ahp, alp, jt.oacc[tp], jt.dacc[tp]);
        }
        // score products of unit u + 1
        if (u + 1 < NU) {
            const int Sn = (u + 1) / NT, tn = ti[(u + 1) % NT];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                scn[h] = zero4();
#pragma unroll
                for (int f = 0; f < FS; ++f) scn[h] = score_mfma<D>(o[Sn & 1].ak[h][f], jt.bq[tn][f], scn[h]);
            }
        }
        ahp = ah;
        alp = al;
        hook(8 * u / NU, 8 * (u + 1) / NU);
    }
    step_accumulate<D>(o[(NU - 1) / NT & 1], ahp, alp, jt.oacc[ti[(NU - 1) % NT]], jt.dacc[ti[(NU - 1) % NT]]);
}

// The chunk in K slot `buf` and V slot `vbuf` (cursor at) against the wave's tiles,
// calling hook(p0, p1) as the work done goes from p0 to p1 eighths; at the job's last
// chunk the tiles' rows of Y are written.
template <int D, bool TILED, typename Hook>
__device__ __forceinline__ void chunk_compute(const Cursor& at, const FusedShape& sh, const unsigned char* buf,
                                              const unsigned char* vbuf, const OutSpec& o, int g, int n, JobTiles<D>& jt,
                                              const Hook& hook) {
    constexpr int VT = JobTiles<D>::VT;
    const Job& jb = at.job;
    if (at.k == 0) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            jt.dacc[r] = zero4();
#pragma unroll
            for (int c = 0; c < VT; ++c) jt.oacc[r][c] = zero4();
        }
    }
    const int row0 = kChunk * at.k;
    const bool fast = row0 + kChunk <= jb.rows && sh.NP % kChunk == 0 && divm(row0, sh.mNP) == jt.slot[0] &&
                      jt.live[0] && (!jt.live[1] || jt.slot[1] == jt.slot[0]);
    if (fast) {
        // every key of the chunk is in the pair of the wave's live tiles
        if (jt.live[1]) {
            const int ti[2] = {0, 1};
            chunk_tiles<D, 2, TILED>(buf, vbuf, ti, jt, g, n, hook);
        } else {
            const int ti[2] = {0, 0};
            chunk_tiles<D, 1, TILED>(buf, vbuf, ti, jt, g, n, hook);
        }
    } else {
        for (int S = 0; S < kChunk / 32; ++S) {
            const int r0 = row0 + 32 * S;
            if (r0 >= jb.rows) break;
            const int ss = divm(r0, sh.mNP);  // the pair slot of these keys
            const bool mask[2] = {jt.live[0] && jt.slot[0] == ss, jt.live[1] && jt.slot[1] == ss};
            if (mask[0] || mask[1]) step_masked<D, TILED>(buf, vbuf, S, mask, jt, g, n);
        }
        hook(-1, 8);
    }
    if (kChunk * (at.k + 1) >= jb.rows) {
        // lane (g, n): value columns 16c + 4g .. +3 of query n
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            if (!jt.live[r] || jt.tq[r] >= sh.N) continue;
            const float rden = out_scale(o, jt.dacc[r][0] + kEps);
#pragma unroll
            for (int c = 0; c < VT; ++c) {
                const f32x4 a = jt.oacc[r][c];
                store_out(o, jt.yrow[r] + 16 * c + 4 * g, f32x4{a[0] * rden, a[1] * rden, a[2] * rden, a[3] * rden});
            }
        }
    }
}

// Persistent: workgroup w takes an equal contiguous range of the B*H*QT query tiles
// (pair-major; neighbouring ranges go to workgroups 8 apart, which share an XCD, so a
// pair split between two ranges is read from HBM once) and walks it as jobs of up to
// 16 query tiles, streaming each job's keys through LDS in chunks of kChunk rows.
// Iteration c computes chunk c, staging chunk c + 1 (loaded during iteration c - 1)
// half-way through, then issues the loads of chunk c + 2 and meets the others at a
// barrier.  A slot is rewritten only after the barrier that follows the last
// computation reading it.  The single Q area is safe because every job but a range's
// last spans at least two chunks (its rows, pairs of NP keys each, exceed kChunk), so
// the next job's Q copies are issued only after this job's phi(Q) was read.
template <int D, bool TILED>
__global__ __launch_bounds__(64 * kWaves) void fused_token_kernel(const uint16_t* __restrict__ Q,
                                                                 const uint16_t* __restrict__ K,
                                                                 const uint16_t* __restrict__ V,
                                                                 const float* __restrict__ W, OutSpec o,
                                                                 FusedShape sh) {
    __shared__ __align__(16) unsigned char lds[FusedLds<D>::kBytes];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, n = lane & 15;

    const int G = gridDim.x, w = blockIdx.x;
    const int wk = (G & 7) == 0 ? (w & 7) * (G >> 3) + (w >> 3) : w;
    const int64_t tbeg = sh.tiles_per * wk + (int64_t)sh.tiles_rem * wk / G;
    const int64_t tend = sh.tiles_per * (wk + 1) + (int64_t)sh.tiles_rem * (wk + 1) / G;
    if (tbeg >= tend) return;

    Cursor pf;  // the next chunk to load
    {
        const int64_t p = tbeg / sh.QT;
        const int head = sh.heads > 0 ? (int)(p % sh.heads) : 0;
        pf.job = make_job(p, (int)(tbeg - p * sh.QT), head, tend - tbeg, sh);
        pf.left = tend - tbeg - pf.job.len;
        pf.k = 0;
        pf.valid = true;
    }
    ChunkLoads<D, TILED> L;
    JobTiles<D> jt;
    unsigned char* const qarea = lds + FusedLds<D>::kQBase;
    auto kslot = [&](int i) { return lds + i * FusedLds<D>::kKSlot; };
    auto vslot = [&](int i) { return lds + FusedLds<D>::kVBase + i * FusedLds<D>::kV; };
    const rsrc_t rW = make_rsrc(W, (uint32_t)((sh.heads > 0 ? sh.heads : 1) * sh.M * sh.M) * 4);
    chunk_loads<D, TILED>(pf, sh, Q, K, V, rW, vslot(0), qarea, wave, lane, L);
    advance(pf, sh);
    Cursor cur = L.at;  // the chunk in K slot ks and V slot vs
    int ks = 0, vs = 0;
    stage_chunk<D, TILED>(L, sh, kslot(0), qarea, wave, lane);
    job_header<D>(cur.job, sh, wave, n, jt);
    chunk_loads<D, TILED>(pf, sh, Q, K, V, rW, vslot(1), qarea, wave, lane, L);
    advance(pf, sh);
    if (L.at.valid && L.at.k == 0)
        dma_barrier<ChunkLoads<D, TILED>::kLoads + ChunkLoads<D, TILED>::NQ>();
    else
        dma_barrier<ChunkLoads<D, TILED>::kLoads>();
    for (;;) {
        if (cur.k == 0) {
            // phi(Q) of the new job to registers (the next job's Q copies come at the
            // earliest after this job's first chunk is computed)
            load_bq<D>(qarea, wave, g, n, jt);
        }
        // L holds chunk c + 1: staged into the other K slot half-way through chunk c
        unsigned char* const knext = kslot(ks ^ 1);
        chunk_compute<D, TILED>(cur, sh, kslot(ks), vslot(vs), o, g, n, jt, [&](int p0, int p1) {
            if (p0 < kStageAt && kStageAt <= p1) stage_chunk<D, TILED>(L, sh, knext, qarea, wave, lane);
        });
        if (!L.at.valid) break;
        cur = L.at;
        ks ^= 1;
        vs = vs == 2 ? 0 : vs + 1;
        if (cur.k == 0) job_header<D>(cur.job, sh, wave, n, jt);
        // chunk c + 2: its V slot was last read by chunk c - 1, before the last barrier
        chunk_loads<D, TILED>(pf, sh, Q, K, V, rW, vslot(vs == 2 ? 0 : vs + 1), qarea, wave, lane, L);
        advance(pf, sh);
        if (L.at.valid && L.at.k == 0)
            dma_barrier<ChunkLoads<D, TILED>::kLoads + ChunkLoads<D, TILED>::NQ>();
        else
            dma_barrier<ChunkLoads<D, TILED>::kLoads>();
    }
}

}  // namespace

bool fused_applicable(int D, int64_t BH, int64_t N, int64_t M) {
    (void)D;
    (void)BH;
    // The token-level form costs N d per token (against d^2 + ... for the summaries):
    // it pays for short sequences, where the summaries would be large next to the
    // tokens.  At most 16 blocks (rows of the factor table) and 256 tokens (keys and
    // their transpose in LDS).
    return N <= kMaxTokens && M <= kMaxBlocks;
}

hipError_t launch_fused(const void* q, const void* k, const void* v, const float* W, const OutSpec& out,
                        int64_t BH, int64_t N, int D, int64_t M, int heads, hipStream_t stream) {
    const uint16_t* qq = (const uint16_t*)q;
    const uint16_t* kk = (const uint16_t*)k;
    const uint16_t* vv = (const uint16_t*)v;
    FusedShape sh;
    sh.N = (int)N;
    sh.M = (int)M;
    sh.C = (int)(N / M);
    sh.NP = (int)((N + 31) / 32 * 32);
    sh.QT = (int)((N + 15) / 16);
    sh.KTN = sh.QT;
    const bool tiled = sh.C % 16 == 0;  // blocks of whole 16-token tiles: one factor per tile
    sh.CT = tiled ? sh.C / 16 : 1;
    sh.KTP = sh.NP / 16;
    sh.pps = std::min(kJobTiles / sh.QT, kJobKeys / sh.NP);
    sh.heads = heads;
    auto recip = [](int d) { return (int)(((1 << 20) + d - 1) / d); };  // exact below 2^20 / d (dividends here < 256)
    sh.mNP = recip(sh.NP);
    sh.mQT = recip(sh.QT);
    sh.mKTP = recip(sh.KTP);
    sh.mC = recip(sh.C);
    sh.mCT = recip(sh.CT);
    // One persistent workgroup per CU, each with an equal share of the query tiles
    // (at least 8 of them).
    const int64_t T = BH * sh.QT;
    const int64_t G = std::max<int64_t>(1, std::min<int64_t>(device_cu_count(), (T + 7) / 8));
    sh.tiles_per = T / G;
    sh.tiles_rem = (int)(T % G);
    const dim3 grid((unsigned)G), block(64 * kWaves);
#define MHLA_FUSED_CASE(DD)                                                                          \
    case DD:                                                                                         \
        if (tiled)                                                                                   \
            fused_token_kernel<DD, true><<<grid, block, 0, stream>>>(qq, kk, vv, W, out, sh);      \
        else                                                                                         \
            fused_token_kernel<DD, false><<<grid, block, 0, stream>>>(qq, kk, vv, W, out, sh);     \
        break;
    switch (D) {
        MHLA_FUSED_CASE(16)
        MHLA_FUSED_CASE(32)
        MHLA_FUSED_CASE(64)
        default: return hipErrorInvalidValue;
    }
#undef MHLA_FUSED_CASE
    return hipGetLastError();
}

}  // namespace mhla
