"""GPU parity of the per-pair kernel: mhla_forward for moderate lengths (256 < N <= 8192,
blocks of whole 32-token steps, M <= 16, at least 256 (batch, head) pairs).

One workgroup per (batch, head) pair forms the block summaries S_b, z_b of
"MHLA: Restoring Expressivity of Linear Attention via Token-Level Multi-Head"
§4.1 in registers, mixes them with W without a round trip through HBM, and
writes every output of the pair.  Each case is compared with the oracle over the
whole output to the bfloat16-input bar (3e-3 of max|Y|); the options (no
normaliser, bfloat16 output, one W per head) are checked as in the other paths:
the bfloat16 output is the float32 output rounded to nearest even, bit for bit.
"""
import os
import sys

import numpy as np
import pytest
import torch

import token_level_head_amd as mh
from token_level_head_amd.workloads import WORKLOADS, make_inputs, per_head_weights

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


def round_bf16_bits(x):
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


PAIR = [  # (B, H, N, d, M)
    (64, 4, 1024, 64, 16),   # blocks of 64 tokens: two 32-token steps each
    (32, 8, 512, 32, 16),    # blocks of one 32-token step
    (16, 16, 1024, 64, 4),   # blocks of 256 tokens: two 128-token chunks each
    (2, 128, 2048, 64, 1),   # one block (global linear attention)
    (128, 2, 384, 64, 12),   # 12 blocks, N not a multiple of the 128-token chunk
    (64, 4, 320, 32, 5),     # 5 blocks of 64 tokens, a half chunk at the end
    (32, 8, 768, 64, 3),     # 3 blocks of 256 tokens
    (300, 1, 1024, 32, 16),  # 300 pairs
    (257, 1, 4096, 32, 8),   # blocks of 512 tokens
    (256, 1, 8192, 64, 16),  # the longest sequences the kernel takes
]


def inputs(case, seed):
    B, H, N, d, M = case
    w = WORKLOADS["dit_s2_256"].shrink(B=B, H=H, N=N, d=d, M=M, seed=seed)
    q, k, v, W = make_inputs(w)
    return w, (q, k, v, W)


@pytest.mark.parametrize("case", PAIR, ids=lambda c: "B{}H{}N{}d{}M{}".format(*c))
def test_pair_path(orc, case):
    B, H, N, d, M = case
    assert mh.mhla_forward_path(B, H, N, d, M) == mh.MHLA_PATH_PAIR
    w, (q, k, v, W) = inputs(case, 8000 + PAIR.index(case))
    say(f"[pair] B={B} H={H} N={N} d={d} M={M}")
    qd, kd, vd = (torch.from_numpy(a).to("cuda", torch.bfloat16) for a in (q, k, v))
    y = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    mh.mhla_forward(qd, kd, vd, torch.from_numpy(W).cuda(), y)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    assert np.all(np.isfinite(y))
    ref = orc.forward(q, k, v, W, nthreads=NTHREADS)
    e = rel(y, ref)
    say(f"[pair]   max|dY|/max|Y| = {e:.3e} (tol {TOL:.0e})")
    assert e <= TOL, e


OPTION_CASES = [PAIR[0], PAIR[1], PAIR[4], PAIR[5]]


@pytest.mark.parametrize("case", OPTION_CASES, ids=lambda c: "B{}H{}N{}d{}M{}".format(*c))
def test_pair_options(orc, case):
    """No normaliser and bfloat16 output through the per-pair kernel."""
    B, H, N, d, M = case
    w, (q, k, v, W) = inputs(case, 8100 + OPTION_CASES.index(case))
    qd, kd, vd = (torch.from_numpy(a).to("cuda", torch.bfloat16) for a in (q, k, v))
    Wd = torch.from_numpy(W).cuda()
    say(f"[pair options] B={B} H={H} N={N} d={d} M={M}")
    for normalize in (True, False):
        y32 = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
        y16 = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        mh.mhla_forward_ex(qd, kd, vd, Wd, y32, normalize=normalize)
        mh.mhla_forward_ex(qd, kd, vd, Wd, y16, normalize=normalize)
        torch.cuda.synchronize()
        a32 = y32.cpu().numpy()
        b16 = y16.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.all(np.isfinite(a32))
        assert np.array_equal(b16, round_bf16_bits(a32)), "bf16 output is not the rounded float32 output"
        ref = orc.forward(q, k, v, W, nthreads=NTHREADS, normalize=normalize)
        e32 = rel(a32, ref)
        e16 = rel((b16.astype(np.uint32) << 16).view(np.float32), ref)
        say(f"[pair options]   normalize={normalize}: f32 out {e32:.3e}, bf16 out {e16:.3e}")
        assert e32 <= TOL, (normalize, e32)
        assert e16 <= TOL + 2.0 ** -8, (normalize, e16)


@pytest.mark.parametrize("case", [PAIR[0], PAIR[6]], ids=lambda c: "B{}H{}N{}d{}M{}".format(*c))
def test_pair_per_head(orc, case):
    """W [H, M, M]: against the oracle; equal matrices give the shared pass's bits."""
    B, H, N, d, M = case
    w, (q, k, v, W) = inputs(case, 8200 + N)
    Wh = per_head_weights(w)
    qd, kd, vd = (torch.from_numpy(a).to("cuda", torch.bfloat16) for a in (q, k, v))
    say(f"[pair per-head] B={B} H={H} N={N} d={d} M={M}")
    y = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    mh.mhla_forward_ex(qd, kd, vd, torch.from_numpy(Wh).cuda(), y)
    Wd = torch.from_numpy(W).cuda()
    shared = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    same = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    mh.mhla_forward_ex(qd, kd, vd, Wd, shared)
    mh.mhla_forward_ex(qd, kd, vd, Wd.unsqueeze(0).repeat(H, 1, 1).contiguous(), same)
    torch.cuda.synchronize()
    assert torch.equal(same, shared), "per-head mixing with equal matrices differs from the shared pass"
    e = rel(y.cpu().numpy(), orc.forward(q, k, v, Wh, nthreads=NTHREADS))
    say(f"[pair per-head]   max|dY|/max|Y| = {e:.3e}")
    assert e <= TOL, e


def test_pair_matches_staged_path():
    """The same sums through the staged kernels (the identity token list takes them):
    the two paths round differently, so they agree to the bfloat16 bar, not bit for bit."""
    case = (64, 4, 1024, 64, 16)
    w, (q, k, v, W) = inputs(case, 8300)
    qd, kd, vd = (torch.from_numpy(a).to("cuda", torch.bfloat16) for a in (q, k, v))
    Wd = torch.from_numpy(W).cuda()
    a = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    mh.mhla_forward(qd, kd, vd, Wd, a)
    order = torch.arange(1024, dtype=torch.int32, device="cuda")
    offsets = torch.arange(0, 1025, 64, dtype=torch.int32, device="cuda")
    mh.mhla_forward_blocks(qd, kd, vd, Wd, b, order, offsets, 64)
    torch.cuda.synchronize()
    e = float((a - b).abs().max() / b.abs().max())
    say(f"[pair vs staged] {e:.3e}")
    assert e <= TOL, e
