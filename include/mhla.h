/*
 * mhla.h -- C ABI of the MI355X (gfx950) MHLA forward library, libmhla.so.
 *
 * MHLA, "MHLA: Restoring Expressivity of Linear Attention via Token-Level
 * Multi-Head" (§4.1, §4.2, App. C), computes for every (batch, head) pair:
 *
 *   phi(x)  = ELU(x) + 1                                  ("Linear Attention 笔记" §2)
 *   S_b     = sum_{j in block b} phi(k_j) v_j^T   (d x d)  z_b = sum_{j in b} phi(k_j)   (§4.1)
 *   S~_i    = sum_b W[i,b] S_b,                            z~_i = sum_b W[i,b] z_b       (§4.1, §4.2)
 *   y_t     = phi(q_t)^T S~_i / (phi(q_t)^T z~_i + 1e-6)   for t in query block i    (§4.1; guard as in
 *                                                          "Linear Attention 笔记" §4/§5)
 *
 * Causal variant (App. C, chunkwise form of §4.2): S~_i mixes only earlier
 * blocks b < i, and token t of block i adds W[i,i] times the running summary of
 * its own block up to and including t:
 *   y_t = phi(q_t)^T (S~_i + W[i,i] P_t) / (phi(q_t)^T (z~_i + W[i,i] p_t) + 1e-6),
 *   P_t = sum_{j in i, j <= t} phi(k_j) v_j^T,  p_t = sum_{j in i, j <= t} phi(k_j).
 * Entries of W above the diagonal are never read in the causal variant.
 *
 * Common conventions
 *   - Pointers named q, k, v, W, out, S, St are DEVICE pointers on the current
 *     HIP device; the caller allocates and owns them.  The library keeps no
 *     pointer after a call returns, except inside work already enqueued on
 *     `stream`: keep the buffers alive until that work completes.
 *   - Layouts are row-major and contiguous: q, k, v, out are [B][H][N][d];
 *     W is [M][M] float32 with W[i*M + b] the weight of block b's summary for
 *     query block i.  One W is shared by every batch element and head.
 *   - Blocks are contiguous: block b holds tokens [b*C, (b+1)*C), C = N / M.
 *     Spatial (2D/3D) blocks are expressed by storing tokens block-major.
 *   - Supported sizes: B, H, N, M >= 1, N % M == 0, d in {16, 32, 64},
 *     N*d <= 2^30, M <= 65536 and B*H*M <= 2^29 (else MHLA_ERR_UNSUPPORTED).
 *     bf16 inputs are IEEE bfloat16 bit patterns (uint16 per element).
 *   - Pointers must be 16-byte aligned; `out` must not overlap any input.
 *   - Every call validates its arguments on the host before enqueueing
 *     anything; a non-zero status means nothing was enqueued, except
 *     MHLA_ERR_HIP, which reports a failed HIP call or launch (the stream
 *     may then hold part of the work).  No call synchronises the device,
 *     throws, or aborts.  mhla_last_error() returns a thread-local message
 *     describing the last failure on the calling thread.
 *   - Preconditions not checked on the device: W finite and >= 0 with every
 *     used row non-zero (§4.2: rows of M_c are nonnegative and normalised).
 *     NaN inputs give NaN outputs.
 *   - Identical inputs give bit-identical outputs (no floating-point atomics).
 */
#ifndef MHLA_H
#define MHLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
/* The same type as hipStream_t; NULL means the device's null stream. */
typedef struct ihipStream_t* mhla_stream_t;

enum {
    MHLA_OK = 0,
    MHLA_ERR_INVALID_ARG = -1, /* null or misaligned pointer, bad sizes, N % M != 0, overlap */
    MHLA_ERR_UNSUPPORTED = -2, /* valid but not implemented here (e.g. d not in {16,32,64}) */
    MHLA_ERR_NO_MEMORY = -3,   /* workspace allocation failed */
    MHLA_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed */
};

/* Input element type for the stage-level calls. */
enum { MHLA_DTYPE_BF16 = 0, MHLA_DTYPE_F32 = 1 };

/* The kernels mhla_forward runs (see mhla_forward_path). */
enum { MHLA_PATH_STAGED = 0, MHLA_PATH_FUSED = 1, MHLA_PATH_PAIR = 2 };

/*
 * Full forward pass, bfloat16 q/k/v (float32 accumulation, float32 W and out).
 * causal != 0 selects the causal variant.  Two execution paths compute the same
 * four steps:
 *   - staged: the three stage kernels below (block summaries, mixing, output)
 *     through a workspace of mhla_workspace_bytes() bytes.  The library keeps
 *     one workspace per (device, stream) handle, shared by all calls on that
 *     stream (they run in order) and grown from a library-owned memory pool when
 *     a call needs more (the outgrown one is freed in stream order).  A call that
 *     needs no growth allocates nothing and does not wait for the device.  A call
 *     made while its stream is being captured into a HIP graph takes its own
 *     workspace from the pool and frees it at its end, both in stream order, so
 *     the graph owns that memory and never shares the stream's workspace.  Host
 *     threads that issue calls on one stream must serialise those calls (the
 *     workspace relies on their order on the stream);
 *   - fused (non-causal, bf16; N <= 256 tokens in M <= 16 blocks): one kernel in
 *     the token-level form of §4.2 Eq. 5, keys streamed through LDS; no workspace;
 *   - pair (non-causal, bf16; 256 < N <= 8192 tokens in M <= 16 blocks of a
 *     multiple of 32 tokens, d in {32, 64}, B*H >= 256): one workgroup per (batch,
 *     head) pair that keeps every block summary and its mix in registers (§4.1's
 *     four steps without a workspace round trip); no workspace.
 * mhla_forward_path() reports which one a call with given sizes uses.
 */
int mhla_forward(const void* q, const void* k, const void* v, const float* W, float* out,
                 int64_t B, int64_t H, int64_t N, int64_t d, int64_t M, int causal,
                 mhla_stream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): mhla_forward whose staged path
 * takes its workspace from a fixed scratch array that the library keeps on each device
 * (MHLA_NOALLOC_SCRATCH_BYTES bytes, held from the moment the library's code is
 * loaded on that device until the process ends) instead of allocating one.  The call
 * makes no allocation and no free.  Arguments, paths and results are those of
 * mhla_forward, bit for bit; the caller still provides q, k, v, W and out.  Sizes whose
 * workspace (mhla_workspace_bytes) exceeds MHLA_NOALLOC_SCRATCH_BYTES give
 * MHLA_ERR_UNSUPPORTED with nothing enqueued (the fused path needs no workspace and has
 * no such limit).  The first call on a device looks up that device's array address
 * (a host-side lookup, not a stream operation).
 *
 * Every call on one device uses that device's one array, which keeps the last call's
 * contents (no stage reads anything it has not written in the same call, so nothing
 * needs clearing).  Calls that overlap in time on one device -- on different streams,
 * or from several host threads -- race on it and give wrong results: serialise them.
 */
#define MHLA_NOALLOC_SCRATCH_BYTES ((int64_t)256 << 20)
int mhla_forward_noalloc(const void* q, const void* k, const void* v, const float* W, float* out,
                         int64_t B, int64_t H, int64_t N, int64_t d, int64_t M, int causal,
                         mhla_stream_t stream);

/* Same as mhla_forward with float32 q/k/v; every step runs in float32. */
int mhla_forward_f32(const float* q, const float* k, const float* v, const float* W, float* out,
                     int64_t B, int64_t H, int64_t N, int64_t d, int64_t M, int causal,
                     mhla_stream_t stream);

/* Options of mhla_forward_ex (bit flags, combined with |). */
enum {
    MHLA_OPT_CAUSAL = 1,        /* the causal variant (as causal != 0 above) */
    MHLA_OPT_NO_NORMALIZER = 2, /* y_t = phi(q_t)^T S~_i (plus, causal, W[i,i] phi(q_t)^T P_t), with
                                   no division by phi(q_t)^T z~_i + 1e-6: the form §4.1 allows for
                                   long sequences (its remark on the output), for training stability */
    MHLA_OPT_OUT_BF16 = 4,      /* out holds bfloat16 bit patterns, each value rounded to nearest
                                   even, instead of float32; the arithmetic is unchanged */
    MHLA_OPT_W_PER_HEAD = 8     /* W is [H][M][M]: head h (of every batch element) mixes with its
                                   own matrix W + h*M*M (§4.1/§4.2 applied per head; the pages
                                   describe one M_c shared by all heads) */
};

/*
 * The forward pass with options.  dtype (MHLA_DTYPE_BF16 or _F32) describes q, k
 * and v; out is [B][H][N][d] float32, or bfloat16 with MHLA_OPT_OUT_BF16.
 * mhla_forward(..., causal, ...) and mhla_forward_ex(..., MHLA_DTYPE_BF16, ...,
 * causal ? MHLA_OPT_CAUSAL : 0, ...) give bit-identical results (likewise
 * mhla_forward_f32 with MHLA_DTYPE_F32).  Unknown option bits give
 * MHLA_ERR_INVALID_ARG.  Paths, workspace and all other conventions as for
 * mhla_forward; mhla_forward_path() applies unchanged (the options do not change
 * the path).  With MHLA_OPT_W_PER_HEAD the staged path's workspace holds one
 * split copy of W per head when 256 < M <= 1024: H times the split-W bytes that
 * mhla_workspace_bytes() counts once.  The summary arrays are then ordered head-major
 * inside the workspace, so that each head's mix is one contiguous GEMM.
 */
int mhla_forward_ex(const void* q, const void* k, const void* v, int dtype, const float* W, void* out,
                    int64_t B, int64_t H, int64_t N, int64_t d, int64_t M, unsigned options,
                    mhla_stream_t stream);

/*
 * The forward pass over blocks given as token lists (§4.1: blocks are defined along
 * spatial or spatio-temporal axes, "N_b tokens" each, of any sizes; App. E pads a
 * 224 grid to 256 only so that equal blocks divide it).  Block b holds the tokens
 * order[offsets[b]] .. order[offsets[b+1] - 1] -- positions 0 .. N-1 of the sequence,
 * the same for every (batch, head) pair -- so 2D/3D tiles of a raster-ordered grid,
 * ragged edge tiles included, need no reordering of q, k, v or out.
 *
 * order: device int32 [N], a permutation of 0 .. N-1; offsets: device int32 [M + 1],
 * non-decreasing, offsets[0] = 0, offsets[M] = N (blocks may differ in size; an empty
 * block has S_b = 0).  Both 4-byte aligned and not written by the call.  max_block:
 * an upper bound of offsets[b+1] - offsets[b] (1 <= max_block <= N) used to plan the
 * launches.  These preconditions are not checked on the device: the kernels clamp
 * offsets to [0, N] and skip entries outside [0, N), so other contents give wrong
 * results but no out-of-bounds access, and rows of out missing from `order` are not
 * written.  N need not be a multiple of M.
 *
 * Non-causal only (MHLA_OPT_CAUSAL gives MHLA_ERR_UNSUPPORTED); the other options of
 * mhla_forward_ex apply.  Always the staged path; with offsets[b] = b*N/M and the
 * identity order it gives mhla_forward_ex's staged results.  Workspace: as
 * mhla_workspace_bytes() with blocks of max_block tokens.
 */
int mhla_forward_blocks(const void* q, const void* k, const void* v, int dtype, const float* W, void* out,
                        int64_t B, int64_t H, int64_t N, int64_t d, int64_t M, const int32_t* order,
                        const int32_t* offsets, int64_t max_block, unsigned options, mhla_stream_t stream);

/* Which path mhla_forward (dtype MHLA_DTYPE_BF16) or mhla_forward_f32
 * (MHLA_DTYPE_F32; always staged) takes for these sizes: MHLA_PATH_STAGED,
 * MHLA_PATH_FUSED or MHLA_PATH_PAIR; -1 for invalid sizes or dtype. */
int mhla_forward_path(int64_t B, int64_t H, int64_t N, int64_t d, int64_t M, int causal, int dtype);

/* Bytes of device workspace one staged bf16 forward call uses (the fused path uses none): the S and
 * S~ summary arrays (2 * M * B*H * (d*d + d) floats), the bf16 hi/lo split of W
 * for the mixing kernel when 256 < M <= 1024 (4 * M * M bytes, rounded up to
 * whole 64 x 32 MFMA tiles, then to 256 bytes; none otherwise), and, when
 * blocks are long and B*H*M small (global linear attention over a long
 * sequence), the partial summaries of the token segments each block is cut
 * into (nseg * M * B*H * (d*d + d) floats); -1 for invalid sizes. */
int64_t mhla_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int64_t M, int causal);

/* Floats in one packed summary vector: d*d + d (S_b followed by z_b). */
int64_t mhla_summary_floats(int64_t d);

/*
 * Stage 1 (§4.1, local KV summaries): phi(K) and the per-block reductions.
 * Writes S[b][p][0 .. d*d+d) for every block b < M and pair p = batch*H + head:
 * a packed summary vector holding S_b (d*d floats, in the MFMA-native order
 * decoded by mhla_unpack_summaries) followed by z_b (d floats, plain order).
 * S must hold M * B*H * (d*d + d) floats.  dtype is MHLA_DTYPE_BF16 or _F32
 * and describes k and v.
 */
int mhla_block_summaries(const void* k, const void* v, int dtype, float* S,
                         int64_t B, int64_t H, int64_t N, int64_t d, int64_t M,
                         mhla_stream_t stream);

/*
 * Stage 2 (§4.1 multi-head mixing, done as one GEMM with the coefficient
 * matrix as §4.1 describes): St[i][p][:] = sum_b W[i,b] S[b][p][:] over all
 * b (causal == 0) or over b < i (causal != 0; row 0 becomes zero).  S and St
 * use the packed layout of mhla_block_summaries; `precise` selects float32
 * products (used by the float32 path) instead of the bfloat16 hi/lo split
 * (three bfloat16 products per term, float32 accumulation).  The split W
 * fragments go to the stream's workspace (as for mhla_forward).
 */
int mhla_mix_summaries(const float* S, const float* W, float* St, int64_t BH, int64_t d, int64_t M,
                       int causal, int precise, mhla_stream_t stream);

/*
 * Stage 3 (§4.1 output ratio; App. C for causal): y_t from phi(q_t) and the
 * mixed summaries St of stage 2.  k and v are read only when causal != 0 (the
 * within-block running summary and W[i,i]); W is read only when causal != 0.
 * Writes out [B][H][N][d] float32.
 */
int mhla_output(const void* q, const void* k, const void* v, int dtype, const float* St,
                const float* W, float* out, int64_t B, int64_t H, int64_t N, int64_t d, int64_t M,
                int causal, mhla_stream_t stream);

/*
 * Backward pass: gradients of L = sum(dy * Y), Y = the forward pass of these
 * inputs (same sizes and causal flag), with respect to q, k, v and W (the
 * coefficient matrix M_c is learned end to end, §4.2).  The chain rule runs
 * through the four steps of §4.1 (App. C running summary when causal): it
 * recomputes S_b and S~_i, then forms dq and the gradients of S~, maps them
 * back through W^T to the summaries' gradients, and from those dk and dv; dW
 * sums <dS~_i, S_b> over every batch element and head.  Causal: entries of W
 * above the diagonal get zero gradient.
 *
 * q, k, v: [B][H][N][d] (dtype MHLA_DTYPE_BF16 or _F32); W [M][M] float32;
 * dy, dq, dk, dv: [B][H][N][d] float32; dW: [M][M] float32.  Outputs are
 * overwritten (not accumulated).  Every product runs on bf16 matrix cores with
 * both operands split into bf16 hi + lo parts (about 16 significant bits each;
 * exact bf16 inputs enter unsplit), accumulated in float32 in a fixed order
 * (bit-reproducible); phi uses the hardware exp2.  Workspace of
 * mhla_backward_workspace_bytes() bytes comes from the stream's workspace, as
 * for mhla_forward.  Outputs must not overlap each other or an input.
 */
int64_t mhla_backward_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int64_t M, int causal);

int mhla_backward(const void* q, const void* k, const void* v, int dtype, const float* W, const float* dy,
                  float* dq, float* dk, float* dv, float* dW, int64_t B, int64_t H, int64_t N, int64_t d,
                  int64_t M, int causal, mhla_stream_t stream);

/*
 * The backward pass with options: MHLA_OPT_CAUSAL (as causal != 0 above) and
 * MHLA_OPT_NO_NORMALIZER, the gradients of the forward form without the normaliser
 * (y_t = phi(q_t)^T S~_i, causal plus W[i,i] phi(q_t)^T P_t; §4.1, remark on the
 * output), where the den terms of the chain rule vanish and dnum_t = dy_t.
 * MHLA_OPT_OUT_BF16 and MHLA_OPT_W_PER_HEAD give MHLA_ERR_UNSUPPORTED, unknown bits
 * MHLA_ERR_INVALID_ARG.  mhla_backward(..., causal, ...) is mhla_backward_ex(...,
 * causal ? MHLA_OPT_CAUSAL : 0, ...).  Everything else as for mhla_backward.
 */
int mhla_backward_ex(const void* q, const void* k, const void* v, int dtype, const float* W, const float* dy,
                     float* dq, float* dk, float* dv, float* dW, int64_t B, int64_t H, int64_t N, int64_t d,
                     int64_t M, unsigned options, mhla_stream_t stream);

/*
 * Streaming causal decoding (App. C inference: fold the new token into its
 * block's running summary, re-mix, read out; the running sum is the recurrence of
 * "Linear Attention 笔记" §4).  One call produces y_t for token t of every
 * (batch, head) pair with O(d^2) work per pair, equal up to rounding to row t of
 * mhla_forward(causal = 1) on the tokens 0 .. t of the sequence.
 *
 * `state` is a caller-owned device buffer of mhla_decode_state_bytes(B, H, d, M)
 * = ((M + 1) * (d*d + d) + d) * B*H * 4 bytes (float32, 16-byte aligned): per
 * pair the mixed summary of the current block's predecessors, the running
 * summary of the current block (with a second copy of its normaliser) and the
 * summaries of the completed blocks.  Calls on one state must come in order
 * t = 0, 1, 2, ... on one stream; t = 0 starts a new sequence (no clearing
 * needed beforehand).  Token t belongs to block i = t / C (blocks of C tokens,
 * i < M, else MHLA_ERR_INVALID_ARG); at the first token of a block the call
 * first closes the previous block and mixes the completed ones with W[i, b],
 * b < i.  W[i, i] weights the running summary; entries above the diagonal are
 * never read.
 *
 * q, k, v: [B][H][d] for token t (dtype MHLA_DTYPE_BF16 or _F32); out: [B][H][d]
 * float32.  All arithmetic is float32 in a fixed order (bit-reproducible).
 * Sizes as for the forward pass with N = M*C; out must not overlap anything,
 * and state must not overlap q, k, v or W.
 */
int64_t mhla_decode_state_bytes(int64_t B, int64_t H, int64_t d, int64_t M);

int mhla_decode_step(const void* q, const void* k, const void* v, int dtype, const float* W, float* state,
                     float* out, int64_t B, int64_t H, int64_t d, int64_t M, int64_t C, int64_t t,
                     mhla_stream_t stream);

/*
 * Decoding with options (the stream of calls as for mhla_decode_step; the decode is
 * always causal, MHLA_OPT_CAUSAL may be given or not): MHLA_OPT_NO_NORMALIZER writes
 * the numerator phi(q_t)^T (S~_i + W[i,i] P_t) alone (§4.1, remark on the output, the
 * form meant for long sequences), equal up to rounding to row t of mhla_forward_ex
 * with MHLA_OPT_CAUSAL | MHLA_OPT_NO_NORMALIZER; MHLA_OPT_W_PER_HEAD takes W as
 * [H][M][M], head h mixing with W + h*M*M.  MHLA_OPT_OUT_BF16 gives
 * MHLA_ERR_UNSUPPORTED, unknown bits MHLA_ERR_INVALID_ARG.  mhla_decode_step is
 * mhla_decode_step_ex(..., MHLA_OPT_CAUSAL, ...).  A state must be driven with the
 * same options from t = 0 on.
 */
int mhla_decode_step_ex(const void* q, const void* k, const void* v, int dtype, const float* W, float* state,
                        float* out, int64_t B, int64_t H, int64_t d, int64_t M, int64_t C, int64_t t,
                        unsigned options, mhla_stream_t stream);

/*
 * Host-only helper (no HIP calls): decodes `count` packed summary vectors in
 * HOST memory into row-major S [count][d][d] (S[r][c] = sum phi(k)[r] v[c])
 * and z [count][d].  Returns MHLA_OK or MHLA_ERR_INVALID_ARG.
 */
int mhla_unpack_summaries(const float* packed, int64_t count, int64_t d, float* S, float* z);

/*
 * Frees the workspace the library keeps for `stream` on the current device (the
 * buffer that staged mhla_forward* calls, mhla_block_summaries,
 * mhla_mix_summaries and mhla_backward share on that stream), in stream order:
 * work already enqueued on the stream that uses it completes first.  Call it
 * before destroying a stream that the library was called on: the cache is keyed
 * by the stream handle, and a stream created later may receive the same handle.
 * A later call on the stream takes a new workspace.  Returns MHLA_OK also when
 * no workspace was held; MHLA_ERR_HIP if the free could not be enqueued.
 */
int mhla_release_workspace(mhla_stream_t stream);

/*
 * Test hook for the allocation-failure path: the next `count` calls that need
 * workspace memory (staged forward, stage calls that use it, backward) return
 * MHLA_ERR_NO_MEMORY before making any HIP call, so nothing is enqueued, exactly
 * as when the allocation itself fails.  count <= 0 switches it off.  Not meant
 * for production use.
 */
void mhla_debug_fail_workspace(int count);

/* Human-readable name of a status code (static storage). */
const char* mhla_status_string(int status);

/* Thread-local description of the last failing call on this thread ("" if none). */
const char* mhla_last_error(void);

/* Library version string (static storage). */
const char* mhla_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MHLA_H */
