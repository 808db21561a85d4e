// kernels.hpp -- internal launchers of the three MHLA stages (not part of the C ABI).
// Each launcher enqueues its kernel(s) on `stream` and returns hipGetLastError();
// the caller has already validated every size and pointer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mhla {

// Compute units of the current device (cached per device, safe to call from several
// host threads at once; 256 if the query fails).  Launchers size persistent grids and
// work splits with it.
int device_cu_count();

constexpr int kDtypeBF16 = 0;
constexpr int kDtypeF32 = 1;

// Which tokens form each block.  Null pointers: M equal contiguous blocks of N / M
// tokens.  Otherwise block b is the token list order[offsets[b]] .. order[offsets[b+1]-1]
// (positions in the sequence, the same for every (batch, head) pair): blocks of any
// sizes and shapes (2D/3D tiles of a raster-ordered grid).  Kernels clamp offsets to
// [0, N] and skip list entries outside [0, N), so any array contents are memory-safe.
struct BlockLayout {
    const int32_t* order;    // [N] device
    const int32_t* offsets;  // [M + 1] device
};

// Where and how a kernel writes the attention output Y ([pair][N][d], row-major).
struct OutSpec {
    void* y;   // float32 values, or bfloat16 bit patterns when bf16 != 0
    int bf16;  // 1: each value rounded to bfloat16, nearest even
    int norm;  // 0: the numerator phi(q)^T S~ alone, without the normaliser
};

// Token inputs (Q, K, V together) larger than the 256 MiB Infinity Cache are read
// with the non-temporal policy, so that streaming them does not evict the block
// summaries that the next stage reads back.  Smaller inputs are read normally: they
// may be cache-resident (just written by whatever produced them) and stay so.
constexpr int64_t kInfinityCacheBytes = int64_t(256) << 20;
inline bool stream_token_inputs(int64_t BH, int64_t N, int D, int esize) {
    return 3 * BH * N * D * esize > kInfinityCacheBytes;
}

// `heads` (every launcher): 0 for one mixing matrix shared by all (batch, head)
// pairs; H for one M x M matrix per head (W is [H][M][M]), with head-major rows in
// the summary arrays (summary_row in common.hpp).
//
// Stage 1: S[b][row][d*d + d] (packed) from K, V [pair][N][d].  Long blocks on few
// (batch, head) pairs are cut into token segments whose partial summaries go to
// `partial` (summary_partial_bytes() bytes, 16-byte aligned; may be null when that
// is 0) and are then added into S.
// `cmax` bounds the block length (N / M without a token list) and plans the split.
size_t summary_partial_bytes(int dtype, int64_t BH, int64_t cmax, int D, int64_t M);
// The transposed summaries S_b^T, z_b of equal contiguous bf16 blocks for the backward
// pass (packed layout, [M][BH][d*d + d]); summaries_t_fits() says whether one pass
// without token segments covers the shape (else launch_summaries_t refuses it).
bool summaries_t_fits(int64_t BH, int64_t N, int D, int64_t M);
hipError_t launch_summaries_t(const uint16_t* k, const uint16_t* v, float* St, int64_t BH, int64_t N, int D,
                              int64_t M, hipStream_t stream);
hipError_t launch_summaries(int dtype, const void* k, const void* v, float* S, int64_t BH, int64_t N,
                            int D, int64_t M, int heads, const BlockLayout& lay, int64_t cmax, float* partial,
                            hipStream_t stream);

// Stage 2: St[i][col] = sum_b W[i,b] S[b][col] (causal: b < i), col < BH * (d*d + d).
// The bf16 path needs mix_fragment_bytes(M) bytes of device scratch at frag_ws
// (16-byte aligned) for the split W; 0 bytes means it needs none.
size_t mix_fragment_bytes(int64_t M);
hipError_t launch_mix(const float* S, const float* W, float* St, int64_t BH, int D, int64_t M, bool causal,
                      bool precise, int heads, void* frag_ws, hipStream_t stream);

// Stage 3: Y [pair][N][d] from Q and St (causal also K, V and W[i,i]), written as `out` says.
hipError_t launch_output(int dtype, const void* q, const void* k, const void* v, const float* St,
                         const float* W, const OutSpec& out, int64_t BH, int64_t N, int D, int64_t M, bool causal,
                         int heads, const BlockLayout& lay, int64_t cmax, hipStream_t stream);

// Causal bf16 output for blocks of at most 256 tokens: the within-block prefix as one
// masked C x C product per block (used by launch_output when applicable).
bool causal_quad_applicable(int64_t C);
hipError_t launch_causal_quad(const void* q, const void* k, const void* v, const float* St, const float* W,
                              const OutSpec& out, int64_t BH, int64_t N, int D, int64_t M, int heads,
                              hipStream_t stream);

// Streaming causal decoding of token t (state layout in decode.hip).
hipError_t launch_decode_step(int dtype, const void* q, const void* k, const void* v, const float* W, float* state,
                              float* out, int64_t BH, int D, int64_t M, int64_t C, int64_t t, bool normalize,
                              int heads, hipStream_t stream);

// Backward pass (float32 arithmetic): dq, dk, dv [pair][N][d] and dW [M][M] from dy.
// ws holds backward_workspace_floats() floats; frag_ws mix_fragment_bytes(M) bytes.
size_t backward_workspace_floats(int64_t BH, int64_t N, int D, int64_t M, bool causal);
// Token-level backward for short sequences (bwd_fused.hip); launch_backward takes it
// when it applies, with BH * M * M floats of ws for the per-pair dW partials.
bool bwd_fused_applicable(int dtype, int D, int64_t N, int64_t M, bool causal);
hipError_t launch_bwd_fused(const void* q, const void* k, const void* v, const float* W, const float* dy, float* dq,
                            float* dk, float* dv, float* dW, int64_t BH, int64_t N, int D, int64_t M, bool normalize,
                            float* ws, hipStream_t stream);
hipError_t launch_backward(int dtype, const void* q, const void* k, const void* v, const float* W, const float* dy,
                           float* dq, float* dk, float* dv, float* dW, int64_t BH, int64_t N, int D, int64_t M,
                           bool causal, bool normalize, float* ws, void* frag_ws, hipStream_t stream);

// Pair path (non-causal bf16, 256 < N <= 8192, at most 16 blocks of a multiple of 32
// tokens, at least 256 pairs): the whole pass in one kernel per (batch, head) pair,
// every block summary on chip; needs no workspace.
bool pair_applicable(int D, int64_t BH, int64_t N, int64_t M);
hipError_t launch_pair(const void* q, const void* k, const void* v, const float* W, const OutSpec& out, int64_t BH,
                       int64_t N, int D, int64_t M, int heads, hipStream_t stream);

// Fused path (non-causal bf16, short blocks): the whole pass in one kernel with
// the summaries in LDS; needs no workspace.
bool fused_applicable(int D, int64_t BH, int64_t N, int64_t M);
hipError_t launch_fused(const void* q, const void* k, const void* v, const float* W, const OutSpec& out,
                        int64_t BH, int64_t N, int D, int64_t M, int heads, hipStream_t stream);

}  // namespace mhla
