"""GPU parity at the size limits of the C ABI.

* One sequence of N = 2^24 tokens at d = 64 (N*d = 2^30, the largest the ABI accepts:
  byte offsets inside a (batch, head) pair reach 2^31) in M = 4096 blocks, with the
  identity as mixing matrix, so that each block is independent linear attention over
  its own 4096 tokens ("MHLA ..." §4.1 with M_c = I; causal: the running summary of
  App. C restarted at each block).  Sampled blocks (first, middle, last) are compared
  with the oracle run on those blocks alone (one block, W = [[1]]); the whole output
  must be finite.
* 65536 (batch, head) pairs on the fused path (grid of 65536 workgroups; the pair's
  base offset pair * N * d leaves 32 bits), sampled pairs against the oracle.

Inputs are drawn on the device from seeded generators; only the sampled slices are
copied to the host.
"""
import os
import sys

import numpy as np
import pytest
import torch

import token_level_head_amd as mh

pytestmark = pytest.mark.gpu

TOL = 3e-3
NTHREADS = min(16, os.cpu_count() or 1)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "these tests need the MI355X"
    mh.load_library()
    yield


def rel(y, ref):
    return float(np.max(np.abs(y.astype(np.float64) - ref)) / np.max(np.abs(ref)))


def draw(shape, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
def test_longest_sequence_identity_mixing(orc, causal):
    N, d, M = 1 << 24, 64, 4096
    C = N // M
    say(f"[limits] N={N} d={d} M={M} causal={causal}: inputs on the device")
    q, k, v = (draw((1, 1, N, d), 7100 + i) for i in range(3))
    W = torch.eye(M, dtype=torch.float32, device="cuda")
    out = torch.empty((1, 1, N, d), dtype=torch.float32, device="cuda")
    mh.mhla_forward(q, k, v, W, out, causal=causal)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    one = np.ones((1, 1), dtype=np.float32)
    for blk in (0, M // 2, M - 1):
        s = slice(blk * C, (blk + 1) * C)
        qb, kb, vb = (t[:, :, s].float().cpu().numpy() for t in (q, k, v))
        ref = orc.forward(qb, kb, vb, one, causal=causal, nthreads=NTHREADS)
        e = rel(out[:, :, s].cpu().numpy(), ref)
        say(f"[limits]   block {blk}: {e:.3e}")
        assert e <= TOL, (blk, e)
    del q, k, v, out, W
    torch.cuda.empty_cache()


def test_many_pairs_fused(orc):
    B, H, N, d, M = 16384, 4, 16, 64, 1
    assert mh.mhla_forward_path(B, H, N, d, M) == mh.MHLA_PATH_FUSED
    say(f"[limits] B*H={B * H} pairs, N={N}, fused path")
    q, k, v = (draw((B, H, N, d), 7200 + i) for i in range(3))
    W = torch.ones((1, 1), dtype=torch.float32, device="cuda")
    out = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
    mh.mhla_forward(q, k, v, W, out)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    for b in (0, B // 2 + 3, B - 1):
        qb, kb, vb = (t[b:b + 1].float().cpu().numpy() for t in (q, k, v))
        ref = orc.forward(qb, kb, vb, W.cpu().numpy(), nthreads=NTHREADS)
        e = rel(out[b:b + 1].cpu().numpy(), ref)
        say(f"[limits]   batch {b}: {e:.3e}")
        assert e <= TOL, (b, e)
