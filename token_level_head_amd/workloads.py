"""Seeded synthetic workloads for the MHLA forward pass.

This module only draws inputs; it holds none of the method's arithmetic, so the
GPU library's tests and the CPU oracle can both take their inputs from it.

Each workload mirrors a shape the MHLA paper's experiments use ("MHLA: Restoring
Expressivity of Linear Attention via Token-Level Multi-Head", §5.2 image
generation with DiT-S/2 at 256, 512 and 4096 resolution, SANA-style text-to-image,
§5.4 causal language modelling), with random data in place of trained
projections: Q, K, V ~ N(0, 1) * scale and each row of W a softmax of N(0, 1) *
wscale logits (nonnegative rows summing to one, as §4.2 asks of M_c).  For the
causal workload each row's softmax runs over b <= i and the entries above the
diagonal are zero.

Spatial blocks (4x4 or 16x16 tiles of a latent grid) are realised by storing
tokens block-major, so block b is always the contiguous token range
[b*C, (b+1)*C) with C = N / M.

Recipe: ``numpy.random.default_rng(seed)`` (PCG64), draws in the order Q, K, V
(``standard_normal`` float32, shape [B, H, N, d]) then the [M, M] logits
(float64); bf16 workloads round Q, K, V to bfloat16 with round-to-nearest-even
and keep them as the exactly equal float32 values.
"""
from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    key: str
    description: str
    B: int
    H: int
    N: int
    d: int
    M: int
    causal: bool
    dtype: str  # "f32" or "bf16": the type of q, k, v (W and the output are always float32)
    scale: float
    wscale: float
    seed: int

    @property
    def C(self):
        return self.N // self.M

    @property
    def tokens(self):
        return self.B * self.N

    def shrink(self, **kw):
        """The same recipe at other sizes (used for fast CPU-side checks)."""
        return replace(self, **kw)


WORKLOADS = {
    w.key: w
    for w in [
        Workload("tiny_f32", "tiny fp32 check: 256 tokens in 4 contiguous blocks of 64",
                 B=1, H=1, N=256, d=16, M=4, causal=False, dtype="f32", scale=1.0, wscale=1.0, seed=1001),
        Workload("dit_s2_256", "DiT-S/2 at 256x256: 16x16 latent grid, 16 blocks of 4x4 tokens",
                 B=64, H=6, N=256, d=64, M=16, causal=False, dtype="bf16", scale=1.0, wscale=1.0, seed=1002),
        Workload("dit_s2_512", "DiT-S/2 at 512x512: 32x32 latent grid, 16 blocks of 8x8 tokens",
                 B=64, H=6, N=1024, d=64, M=16, causal=False, dtype="bf16", scale=1.0, wscale=1.0, seed=1006),
        Workload("dit_s2_4096", "DiT-S/2 at 4096x4096: 256x256 latent grid, 256 blocks of 16x16 tokens",
                 B=1, H=6, N=65536, d=64, M=256, causal=False, dtype="bf16", scale=1.0, wscale=1.0, seed=1003),
        Workload("sana_128", "SANA-like 128x128 grid, 70 heads of 32, 64 blocks of 16x16 tokens",
                 B=4, H=70, N=16384, d=32, M=64, causal=False, dtype="bf16", scale=0.5, wscale=2.0, seed=1004),
        Workload("lm_causal_8k", "causal LM: 8192 tokens, 64 contiguous blocks of 128",
                 B=8, H=16, N=8192, d=64, M=64, causal=True, dtype="bf16", scale=1.0, wscale=1.0, seed=1005),
    ]
}


def round_bf16(x):
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def mixing_weights(logits, causal):
    """Row-softmax of the logits (over b <= i when causal, zeros above)."""
    logits = np.asarray(logits, dtype=np.float64)
    M = logits.shape[0]
    allowed = np.tril(np.ones((M, M), dtype=bool)) if causal else np.ones((M, M), dtype=bool)
    z = np.where(allowed, logits, -np.inf)
    z = z - z.max(axis=1, keepdims=True)
    e = np.where(allowed, np.exp(z), 0.0)
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def per_head_weights(w: Workload, seed=None):
    """[H, M, M] float32: one mixing matrix per head, drawn like W from a stream of
    its own (seed + 7919), for the per-head option."""
    rng = np.random.default_rng((w.seed if seed is None else seed) + 7919)
    return np.stack([mixing_weights(rng.standard_normal((w.M, w.M)) * w.wscale, w.causal) for _ in range(w.H)])


def grid_blocks(dims, tile):
    """Blocks as token lists for a raster-ordered grid of `dims` (e.g. (h, w) or (t, h, w))
    cut into tiles of `tile` (edge tiles are smaller when a side does not divide).
    Returns order [N] int32 (tokens block by block, raster order inside a tile),
    offsets [M + 1] int32 and blk [N] (each token's block)."""
    dims, tile = tuple(dims), tuple(tile)
    N = int(np.prod(dims))
    coords = np.stack(np.unravel_index(np.arange(N), dims), axis=1)
    ntile = [(a + b - 1) // b for a, b in zip(dims, tile)]
    blk = np.ravel_multi_index(tuple((coords // np.array(tile)).T), ntile)
    order = np.argsort(blk, kind="stable").astype(np.int32)
    M = int(np.prod(ntile))
    offsets = np.concatenate([[0], np.cumsum(np.bincount(blk, minlength=M))]).astype(np.int32)
    return order, offsets, blk.astype(np.int32)


def random_blocks(N, M, seed):
    """An unequal partition of N tokens into M blocks (some possibly empty), each block's
    tokens scattered over the sequence: order, offsets, blk as grid_blocks returns."""
    rng = np.random.default_rng(seed)
    blk = rng.integers(0, M, N)
    order = np.argsort(blk, kind="stable").astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(np.bincount(blk, minlength=M))]).astype(np.int32)
    return order, offsets, blk.astype(np.int32)


def make_inputs(w: Workload, seed=None):
    """q, k, v [B, H, N, d] float32 (bf16-exact for bf16 workloads) and W [M, M] float32."""
    if w.N % w.M:
        raise ValueError("N must be a multiple of M")
    rng = np.random.default_rng(w.seed if seed is None else seed)
    shape = (w.B, w.H, w.N, w.d)
    q, k, v = (rng.standard_normal(shape, dtype=np.float32) * np.float32(w.scale) for _ in range(3))
    W = mixing_weights(rng.standard_normal((w.M, w.M)) * w.wscale, w.causal)
    if w.dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return q, k, v, W
