"""GPU parity of the backward pass against the float64 backward oracle.

mhla_backward forms every product on bf16 MFMA with both operands split into
hi + lo parts (about 16 significant bits per operand) and float32 accumulation,
so the bar is max|dX - dX_ref| / max|dX_ref| <= 1e-4 for every gradient; the oracle (oracle/backward.py) is pinned by finite
differences of the explicit O(N^2) definition.
"""
import sys

import numpy as np
import pytest
import torch

import token_level_head_amd as mh
from oracle.backward import backward as oracle_backward
from token_level_head_amd.workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

TOL = 1e-4

BACKWARD = [  # (B, H, N, d, M, causal, dtype)
    (2, 2, 64, 16, 4, False, "bf16"),
    (1, 2, 96, 32, 6, True, "bf16"),    # C = 16: one tile per block
    (1, 1, 128, 64, 4, True, "f32"),    # C = 32: two tiles per block
    (2, 1, 64, 64, 16, False, "bf16"),  # C = 4: partial tiles
    (1, 1, 100, 32, 5, True, "bf16"),   # C = 20: ragged second tile
    (1, 2, 48, 16, 48, True, "f32"),    # one token per block
    (1, 1, 256, 64, 1, True, "bf16"),   # one block of 16 tiles: the plain recurrence
    (1, 1, 640, 16, 80, False, "bf16"), # M = 80: mixing through split-W fragments
    (1, 2, 1024, 64, 4, False, "bf16"), # C = 256: a block's tiles over 4 waves, partials added in LDS
    (1, 3, 512, 32, 16, False, "f32"),  # C = 32: 2 waves per block, float32 inputs
    (1, 1, 512, 16, 32, True, "bf16"),  # M = 32: two column tiles per dW block
    (1, 1, 8192, 64, 64, True, "bf16"),    # the causal LM shape: 64 blocks of 128 tokens (8 tiles each)
    (1, 1, 16384, 64, 256, False, "bf16"), # M = 256: streaming mixing GEMM, 4 x 4 dW output blocks
]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_backward(q, k, v, W, dy, causal, dtype, normalize=True):
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    qd, kd, vd = (torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dt) for a in (q, k, v))
    Wd = torch.from_numpy(W).cuda()
    dyd = torch.from_numpy(dy.astype(np.float32)).cuda()
    dq, dk, dv = (torch.full(q.shape, float("nan"), device="cuda") for _ in range(3))
    dW = torch.full(W.shape, float("nan"), device="cuda")
    if normalize:
        mh.mhla_backward(qd, kd, vd, Wd, dyd, dq, dk, dv, dW, causal=causal)
    else:
        mh.mhla_backward_ex(qd, kd, vd, Wd, dyd, dq, dk, dv, dW, causal=causal, normalize=False)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (dq, dk, dv, dW)]


@pytest.mark.parametrize("case", BACKWARD, ids=lambda c: "B{}H{}N{}d{}M{}{}{}".format(*c[:5], "c" if c[5] else "", c[6]))
def test_backward_matches_oracle(case):
    B, H, N, d, M, causal, dtype = case
    w = WORKLOADS["lm_causal_8k"].shrink(B=B, H=H, N=N, d=d, M=M, causal=causal, dtype=dtype,
                                         seed=6000 + BACKWARD.index(case))
    q, k, v, W = make_inputs(w)
    dy = np.random.default_rng(6100 + BACKWARD.index(case)).standard_normal(q.shape).astype(np.float32)
    say(f"[backward] B={B} H={H} N={N} d={d} M={M} causal={causal} dtype={dtype}")
    got = gpu_backward(q, k, v, W, dy, causal, dtype)
    ref = oracle_backward(q, k, v, W, dy, causal=causal)
    for name, g, r in zip(("dq", "dk", "dv", "dW"), got, ref):
        assert np.all(np.isfinite(g)), name
        err = float(np.max(np.abs(g.astype(np.float64) - r)))
        if name == "dW" and M == 1:
            # One block: Y depends on a positive W only through the 1e-6 guard, so the exact
            # dW is ~1e-9 and float32 evaluates it as a cancelling sum of O(1) terms.
            say(f"[backward]   dW (M = 1): |d| = {err:.2e}, |ref| = {np.max(np.abs(r)):.2e}")
            assert err <= 1e-5, err
            continue
        e = err / float(np.max(np.abs(r)))
        say(f"[backward]   {name}: max|d|/max|ref| = {e:.2e}")
        assert e <= TOL, (name, e)
    if causal:
        assert np.all(np.triu(got[3], 1) == 0)


def test_backward_is_deterministic():
    w = WORKLOADS["lm_causal_8k"].shrink(B=2, H=2, N=256, M=8, seed=6200)
    q, k, v, W = make_inputs(w)
    dy = np.random.default_rng(6201).standard_normal(q.shape).astype(np.float32)
    a = gpu_backward(q, k, v, W, dy, True, "bf16")
    b = gpu_backward(q, k, v, W, dy, True, "bf16")
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


NO_NORMALISER = [BACKWARD[i] for i in (0, 1, 2, 3, 7, 9, 11)]


@pytest.mark.parametrize("case", NO_NORMALISER,
                         ids=lambda c: "B{}H{}N{}d{}M{}{}{}".format(*c[:5], "c" if c[5] else "", c[6]))
def test_backward_without_normaliser_matches_oracle(case):
    # the gradients of y = A V, the form without the normaliser ("MHLA" §4.1, remark on
    # the output); the same 1e-4 bar
    B, H, N, d, M, causal, dtype = case
    w = WORKLOADS["lm_causal_8k"].shrink(B=B, H=H, N=N, d=d, M=M, causal=causal, dtype=dtype,
                                         seed=6300 + NO_NORMALISER.index(case))
    q, k, v, W = make_inputs(w)
    dy = np.random.default_rng(6400 + NO_NORMALISER.index(case)).standard_normal(q.shape).astype(np.float32)
    say(f"[backward, no normaliser] B={B} H={H} N={N} d={d} M={M} causal={causal} dtype={dtype}")
    got = gpu_backward(q, k, v, W, dy, causal, dtype, normalize=False)
    ref = oracle_backward(q, k, v, W, dy, causal=causal, normalize=False)
    for name, g, r in zip(("dq", "dk", "dv", "dW"), got, ref):
        assert np.all(np.isfinite(g)), name
        e = float(np.max(np.abs(g.astype(np.float64) - r)) / np.max(np.abs(r)))
        say(f"[backward, no normaliser]   {name}: max|d|/max|ref| = {e:.2e}")
        assert e <= TOL, (name, e)
    if causal:
        assert np.all(np.triu(got[3], 1) == 0)


TOKEN_LEVEL = [  # (B, H, N, d, M): shapes the token-level backward takes (bf16, non-causal,
    #               N <= 256 in blocks of whole 16-token tiles, an even number of tiles)
    (2, 2, 256, 64, 16),  # DiT-S/2 at 256: blocks of 16 tokens
    (1, 3, 256, 64, 4),   # blocks of 64 tokens
    (2, 1, 128, 32, 8),   # d = 32
    (1, 2, 64, 64, 1),    # one block (global linear attention)
    (3, 1, 96, 32, 3),    # blocks of 32 tokens, 6 tiles
    (1, 1, 32, 64, 2),    # two tiles
    (1, 2, 160, 64, 5),   # 10 tiles: waves 2 .. 7 own one query and one key tile
    (64, 6, 256, 64, 16), # the full DiT-S/2 256 batch (between one and two workgroups per CU:
    #                       some pairs split into halves)
    (40, 8, 256, 32, 16), # 320 pairs, d = 32: 192 of them in halves
    (33, 9, 256, 64, 4),  # 297 pairs: 208 in halves, 89 whole
]


CAUSAL_QUERIES = [  # (B, H, N, d, M): causal bf16 shapes whose query side runs in the token-level form
    #                  (blocks of an even number of 16-token tiles, at most 256 tokens)
    (2, 2, 256, 64, 8),   # blocks of 32 tokens: two tiles
    (1, 3, 384, 32, 6),   # 64 tokens, d = 32
    (1, 2, 768, 64, 4),   # 192 tokens: 12 tiles, the larger LDS variant, snake slots partly empty
    (1, 1, 1024, 64, 4),  # 256 tokens: 16 tiles, four per wave
    (2, 2, 1024, 32, 8),  # 128 tokens at d = 32
]


@pytest.mark.parametrize("normalize", [True, False], ids=["norm", "nonorm"])
@pytest.mark.parametrize("case", CAUSAL_QUERIES, ids=lambda c: "B{}H{}N{}d{}M{}".format(*c))
def test_causal_token_level_queries_match_oracle(case, normalize):
    """Causal backward whose query side (dq, dS~, dz~, dW[i,i], per-token den) takes masked
    query x key products over the block instead of a running state, against the backward
    oracle at the same 1e-4 bar, with and without the normaliser."""
    B, H, N, d, M = case
    idx = CAUSAL_QUERIES.index(case)
    w = WORKLOADS["lm_causal_8k"].shrink(B=B, H=H, N=N, d=d, M=M, causal=True, dtype="bf16", seed=6800 + idx)
    q, k, v, W = make_inputs(w)
    dy = np.random.default_rng(6900 + idx).standard_normal(q.shape).astype(np.float32)
    say(f"[backward, causal queries] B={B} H={H} N={N} d={d} M={M} normalize={normalize}")
    got = gpu_backward(q, k, v, W, dy, True, "bf16", normalize=normalize)
    ref = oracle_backward(q, k, v, W, dy, causal=True, normalize=normalize)
    for name, g, r in zip(("dq", "dk", "dv", "dW"), got, ref):
        assert np.all(np.isfinite(g)), name
        e = float(np.max(np.abs(g.astype(np.float64) - r))) / float(np.max(np.abs(r)))
        say(f"[backward, causal queries]   {name}: max|d|/max|ref| = {e:.2e}")
        assert e <= TOL, (name, e)
    assert np.all(np.triu(got[3], 1) == 0)


def test_causal_token_level_queries_deterministic():
    w = WORKLOADS["lm_causal_8k"].shrink(B=2, H=2, N=1024, M=8, seed=6950)
    q, k, v, W = make_inputs(w)
    dy = np.random.default_rng(6951).standard_normal(q.shape).astype(np.float32)
    a = gpu_backward(q, k, v, W, dy, True, "bf16")
    b = gpu_backward(q, k, v, W, dy, True, "bf16")
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("normalize", [True, False], ids=["norm", "nonorm"])
@pytest.mark.parametrize("case", TOKEN_LEVEL, ids=lambda c: "B{}H{}N{}d{}M{}".format(*c))
def test_token_level_backward_matches_oracle(case, normalize):
    """The token-level backward (scores of each pair on chip, no summaries) against the
    backward oracle, to the same 1e-4 bar, with and without the normaliser."""
    B, H, N, d, M = case
    w = WORKLOADS["dit_s2_256"].shrink(B=B, H=H, N=N, d=d, M=M, seed=6500 + TOKEN_LEVEL.index(case))
    q, k, v, W = make_inputs(w)
    dy = np.random.default_rng(6600 + TOKEN_LEVEL.index(case)).standard_normal(q.shape).astype(np.float32)
    say(f"[backward, token level] B={B} H={H} N={N} d={d} M={M} normalize={normalize}")
    got = gpu_backward(q, k, v, W, dy, False, "bf16", normalize=normalize)
    ref = oracle_backward(q, k, v, W, dy, normalize=normalize)
    for name, g, r in zip(("dq", "dk", "dv", "dW"), got, ref):
        assert np.all(np.isfinite(g)), name
        err = float(np.max(np.abs(g.astype(np.float64) - r)))
        if name == "dW" and M == 1 and normalize:
            # as above: the exact dW of one block is ~1e-9, a cancelling sum in float32
            say(f"[backward, token level]   dW (M = 1): |d| = {err:.2e}, |ref| = {np.max(np.abs(r)):.2e}")
            assert err <= 1e-5, err
            continue
        e = err / float(np.max(np.abs(r)))
        say(f"[backward, token level]   {name}: max|d|/max|ref| = {e:.2e}")
        assert e <= TOL, (name, e)


def test_token_level_backward_is_deterministic():
    w = WORKLOADS["dit_s2_256"].shrink(B=50, H=6, seed=6700)  # 300 pairs: whole and split
    q, k, v, W = make_inputs(w)
    dy = np.random.default_rng(6701).standard_normal(q.shape).astype(np.float32)
    a = gpu_backward(q, k, v, W, dy, False, "bf16")
    b = gpu_backward(q, k, v, W, dy, False, "bf16")
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
def test_streaming_backward_matches_split_batch(causal):
    """Token inputs larger than the 256 MiB Infinity Cache are summarised with streaming
    (non-temporal) loads; the same pairs run as two half batches below that size take the
    cached loads, whose results the oracle cases above pin.  The per-pair gradients of the
    two runs agree to rounding (the reduction order may follow the batch size) and dW of
    the whole batch is the sum of the halves' dW."""
    B, H, N, d, M = 4, 2, 98304, 64, 256  # C = 384: one pass without token segments
    assert 3 * B * H * N * d * 2 > 256 << 20 >= 3 * (B // 2) * H * N * d * 2
    say(f"[backward streaming] B={B} H={H} N={N} d={d} M={M} causal={causal}")
    g = torch.Generator(device="cuda").manual_seed(7100 + causal)
    q, k, v = (torch.randn((B, H, N, d), generator=g, device="cuda").to(torch.bfloat16) for _ in range(3))
    W = torch.rand((M, M), generator=g, device="cuda") + 0.05
    dy = torch.randn((B, H, N, d), generator=g, device="cuda")

    def run(lo, hi):
        grads = [torch.empty((hi - lo, H, N, d), device="cuda") for _ in range(3)]
        dW = torch.empty((M, M), device="cuda")
        mh.mhla_backward(q[lo:hi].contiguous(), k[lo:hi].contiguous(), v[lo:hi].contiguous(), W,
                         dy[lo:hi].contiguous(), *grads, dW, causal=causal)
        return grads, dW

    whole, dW = run(0, B)
    first, dW0 = run(0, B // 2)
    second, dW1 = run(B // 2, B)
    torch.cuda.synchronize()
    for name, a, b0, b1 in zip(("dq", "dk", "dv"), whole, first, second):
        ref = torch.cat([b0, b1])
        assert torch.isfinite(a).all(), name
        e = float((a - ref).abs().max() / ref.abs().max())
        say(f"[backward streaming]   {name}: {e:.2e}")
        assert e <= 1e-5, (name, e)
    e = float((dW - (dW0 + dW1)).abs().max() / dW.abs().max())
    say(f"[backward streaming]   dW: {e:.2e}")
    assert e <= 1e-5, e
