"""GPU parity of mhla_forward_ex: the form without the normaliser and the bfloat16 output.

The form without the normaliser (MHLA §4.1, the remark on the output for long
sequences) is compared with the oracle's own option on the same seeded inputs,
to the bars of the plain pass (1e-5 for float32 inputs, 3e-3 for bfloat16).  The
bfloat16 output must equal the float32 output of the same call rounded to
nearest even, bit for bit, and so lies within the plain bar plus the bfloat16
unit roundoff (half an ulp: at most 2^-8 of |y|, so of max|Y|) of the oracle.
Every case also checks that mhla_forward_ex without options gives
mhla_forward's bits.
"""
import os
import sys

import numpy as np
import pytest
import torch

import token_level_head_amd as mh
from token_level_head_amd.workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 3e-3}
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


CASES = [  # (B, H, N, d, M, causal, dtype): one per kernel the options pass through
    (4, 2, 256, 64, 16, False, "bf16"),   # fused path
    (1, 2, 120, 32, 10, False, "bf16"),   # fused path, blocks of 12 tokens
    (2, 2, 256, 64, 4, False, "bf16"),    # fused path over tiles: blocks of 64 tokens
    (2, 1, 1024, 32, 16, False, "bf16"),  # staged, non-causal output kernel
    (1, 2, 500, 64, 4, True, "bf16"),     # causal, one masked product per block
    (1, 2, 1536, 32, 3, True, "bf16"),    # causal, running-state output kernel (C = 512)
    (2, 3, 128, 64, 8, True, "f32"),      # float32 path
    (2, 1, 160, 16, 10, False, "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}N{}d{}M{}{}{}".format(*c[:5], "c" if c[5] else "", c[6]))
def test_options(orc, case):
    B, H, N, d, M, causal, dtype = case
    w = WORKLOADS["tiny_f32"].shrink(B=B, H=H, N=N, d=d, M=M, causal=causal, dtype=dtype, seed=900 + N + M)
    q, k, v, W = make_inputs(w)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    qd, kd, vd = (torch.from_numpy(a).to("cuda", tdt) for a in (q, k, v))
    Wd = torch.from_numpy(W).cuda()
    say(f"[variants] B={B} H={H} N={N} d={d} M={M} causal={causal} dtype={dtype}")

    plain = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    (mh.mhla_forward if dtype == "bf16" else mh.mhla_forward_f32)(qd, kd, vd, Wd, plain, causal=causal)
    ex = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    mh.mhla_forward_ex(qd, kd, vd, Wd, ex, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(plain, ex), "mhla_forward_ex without options differs from mhla_forward"

    for normalize in (True, False):
        y32 = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
        y16 = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        mh.mhla_forward_ex(qd, kd, vd, Wd, y32, causal=causal, normalize=normalize)
        mh.mhla_forward_ex(qd, kd, vd, Wd, y16, causal=causal, normalize=normalize)
        torch.cuda.synchronize()
        a32 = y32.cpu().numpy()
        b16 = y16.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.all(np.isfinite(a32))
        assert np.array_equal(b16, round_bf16_bits(a32)), "bf16 output is not the rounded float32 output"
        ref = orc.forward(q, k, v, W, causal=causal, nthreads=NTHREADS, normalize=normalize)
        e32 = rel(a32, ref)
        e16 = rel((b16.astype(np.uint32) << 16).view(np.float32), ref)
        say(f"[variants]   normalize={normalize}: f32 out {e32:.3e}, bf16 out {e16:.3e}")
        assert e32 <= TOL[dtype], (normalize, e32)
        assert e16 <= TOL[dtype] + 2.0 ** -8, (normalize, e16)


def test_options_full_size_dit(orc):
    """The 256 x 256 DiT-S/2 workload without the normaliser, bfloat16 output."""
    w = WORKLOADS["dit_s2_256"]
    q, k, v, W = make_inputs(w)
    qd, kd, vd = (torch.from_numpy(a).to("cuda", torch.bfloat16) for a in (q, k, v))
    Wd = torch.from_numpy(W).cuda()
    y16 = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    mh.mhla_forward_ex(qd, kd, vd, Wd, y16, normalize=False)
    torch.cuda.synchronize()
    y = y16.float().cpu().numpy()
    ref = orc.forward(q, k, v, W, nthreads=NTHREADS, normalize=False)
    e = rel(y, ref)
    say(f"[variants] dit_s2_256 without normaliser, bf16 out: {e:.3e}")
    assert e <= TOL["bf16"] + 2.0 ** -8


def test_unknown_option_rejected():
    q = torch.zeros((1, 1, 16, 16), dtype=torch.bfloat16, device="cuda")
    W = torch.ones((1, 1), dtype=torch.float32, device="cuda")
    out = torch.zeros((1, 1, 16, 16), dtype=torch.float32, device="cuda")
    lib = mh.load_library()
    import ctypes
    st = lib.mhla_forward_ex(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(q.data_ptr()),
                             ctypes.c_void_p(q.data_ptr()), 0, ctypes.c_void_p(W.data_ptr()),
                             ctypes.c_void_p(out.data_ptr()), 1, 1, 16, 16, 1, 1 << 10, None)
    assert st == mh.MHLA_ERR_INVALID_ARG


PER_HEAD = [  # (B, H, N, d, M, causal, dtype): one per mixing kernel and output kernel
    (2, 3, 256, 64, 16, False, "bf16"),   # fused path
    (4, 3, 256, 32, 4, False, "bf16"),    # fused path over 16-token tiles (blocks of 64 tokens)
    (2, 3, 2048, 32, 1, False, "bf16"),   # M = 1 (token segments in the summaries)
    (2, 2, 1024, 16, 32, True, "bf16"),   # M <= 64 mixing, causal masked products
    (1, 3, 1024, 32, 64, False, "bf16"),
    (2, 70, 256, 32, 64, False, "bf16"),  # 70 heads: the persistent M <= 64 walk with a grid row per head
    (1, 6, 960, 16, 48, True, "bf16"),    # causal 32 < M <= 64 walk, per head
    (1, 2, 2560, 16, 160, True, "bf16"),  # 64 < M <= 256 mixing
    (1, 2, 4096, 64, 256, False, "bf16"),  # M = 256 walk, one grid row per head
    (1, 2, 600, 32, 300, False, "bf16"),  # split-W fragments, one copy per head
    (1, 2, 2048, 16, 2048, False, "bf16"),  # M > 1024 mixing
    (1, 2, 1536, 32, 3, True, "bf16"),    # running-state causal output kernel
    (2, 3, 128, 64, 8, True, "f32"),      # float32 path
]


@pytest.mark.parametrize("case", PER_HEAD, ids=lambda c: "B{}H{}N{}d{}M{}{}{}".format(*c[:5], "c" if c[5] else "", c[6]))
def test_per_head_mixing(orc, case):
    """W [H, M, M]: against the oracle with per-head matrices; equal matrices give the shared pass's bits."""
    from token_level_head_amd.workloads import per_head_weights
    B, H, N, d, M, causal, dtype = case
    w = WORKLOADS["tiny_f32"].shrink(B=B, H=H, N=N, d=d, M=M, causal=causal, dtype=dtype, seed=950 + N + M)
    q, k, v, W = make_inputs(w)
    Wh = per_head_weights(w)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    qd, kd, vd = (torch.from_numpy(a).to("cuda", tdt) for a in (q, k, v))
    say(f"[per-head] B={B} H={H} N={N} d={d} M={M} causal={causal} dtype={dtype}")
    y = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    mh.mhla_forward_ex(qd, kd, vd, torch.from_numpy(Wh).cuda(), y, causal=causal)
    shared = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    same = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    Wd = torch.from_numpy(W).cuda()
    mh.mhla_forward_ex(qd, kd, vd, Wd, shared, causal=causal)
    mh.mhla_forward_ex(qd, kd, vd, Wd.unsqueeze(0).repeat(H, 1, 1).contiguous(), same, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(same, shared), "per-head mixing with equal matrices differs from the shared pass"
    ref = orc.forward(q, k, v, Wh, causal=causal, nthreads=NTHREADS)
    e = rel(y.cpu().numpy(), ref)
    say(f"[per-head]   max|dY|/max|Y| = {e:.3e}")
    assert e <= TOL[dtype], e


TOKEN_LISTS = [  # (B, H, grid, tile, d, dtype, per_head): raster grids cut into tiles, ragged edges
    (2, 2, (16, 16), (4, 4), 64, "bf16", False),    # equal 4 x 4 tiles (C = 16)
    (1, 3, (14, 14), (4, 4), 64, "bf16", False),    # 224 / 16 without padding: 2-wide edge tiles
    (1, 2, (40, 48), (16, 16), 32, "bf16", True),   # 16 x 16 tiles, ragged bottom row, per-head W
    (2, 1, (8, 12, 12), (2, 8, 8), 16, "bf16", False),  # 3D (time, h, w) tiles
    (1, 2, (20, 30), (16, 16), 32, "f32", False),   # float32 path
]


@pytest.mark.parametrize("case", TOKEN_LISTS, ids=lambda c: "B{}H{}g{}t{}d{}{}{}".format(
    c[0], c[1], "x".join(map(str, c[2])), "x".join(map(str, c[3])), c[4], c[5], "ph" if c[6] else ""))
def test_token_list_blocks(orc, case):
    """Raster-ordered grids cut into tiles, given as token lists, against the oracle's block assignment."""
    from token_level_head_amd.workloads import grid_blocks, per_head_weights, mixing_weights
    B, H, grid, tile, d, dtype, per_head = case
    order, offsets, blk = grid_blocks(grid, tile)
    N, M = len(order), len(offsets) - 1
    w = WORKLOADS["tiny_f32"].shrink(B=B, H=H, N=N, d=d, M=1, dtype=dtype, seed=970 + N)
    q, k, v, _ = make_inputs(w)
    W = (per_head_weights(w.shrink(M=M)) if per_head
         else mixing_weights(np.random.default_rng(971 + N).standard_normal((M, M)), False))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    qd, kd, vd = (torch.from_numpy(a).to("cuda", tdt) for a in (q, k, v))
    Wd = torch.from_numpy(W).cuda()
    od, fd = torch.from_numpy(order).cuda(), torch.from_numpy(offsets).cuda()
    say(f"[token lists] B={B} H={H} grid={grid} tile={tile} N={N} M={M} d={d} dtype={dtype} per_head={per_head}")
    for normalize in (True, False):
        y = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
        mh.mhla_forward_blocks(qd, kd, vd, Wd, y, od, fd, int(np.diff(offsets).max()), normalize=normalize)
        torch.cuda.synchronize()
        ref = orc.forward(q, k, v, W, nthreads=NTHREADS, normalize=normalize, blk=blk)
        e = rel(y.cpu().numpy(), ref)
        say(f"[token lists]   normalize={normalize}: {e:.3e}")
        assert e <= TOL[dtype], (normalize, e)


def test_token_list_identity_is_staged_path():
    """Equal contiguous blocks as a token list give the staged path's bits."""
    w = WORKLOADS["tiny_f32"].shrink(B=2, H=2, N=1024, d=32, M=16, dtype="bf16", seed=980)
    q, k, v, W = make_inputs(w)
    qd, kd, vd = (torch.from_numpy(a).to("cuda", torch.bfloat16) for a in (q, k, v))
    Wd = torch.from_numpy(W).cuda()
    order = torch.arange(1024, dtype=torch.int32, device="cuda")
    offsets = torch.arange(0, 1025, 64, dtype=torch.int32, device="cuda")
    a = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    assert mh.mhla_forward_path(2, 2, 1024, 32, 16) == mh.MHLA_PATH_STAGED
    mh.mhla_forward(qd, kd, vd, Wd, a)
    mh.mhla_forward_blocks(qd, kd, vd, Wd, b, order, offsets, 64)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_token_list_rejects_causal():
    q = torch.zeros((1, 1, 16, 16), dtype=torch.bfloat16, device="cuda")
    W = torch.ones((1, 1), dtype=torch.float32, device="cuda")
    out = torch.zeros((1, 1, 16, 16), dtype=torch.float32, device="cuda")
    order = torch.arange(16, dtype=torch.int32, device="cuda")
    offsets = torch.tensor([0, 16], dtype=torch.int32, device="cuda")
    import ctypes
    st = mh.load_library().mhla_forward_blocks(*(ctypes.c_void_p(t.data_ptr()) for t in (q, q, q)), 0,
                                               ctypes.c_void_p(W.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                               1, 1, 16, 16, 1, ctypes.c_void_p(order.data_ptr()),
                                               ctypes.c_void_p(offsets.data_ptr()), 16, mh.MHLA_OPT_CAUSAL, None)
    assert st == mh.MHLA_ERR_UNSUPPORTED
