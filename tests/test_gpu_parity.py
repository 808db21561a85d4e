"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

The bar is max|dY| / max|Y_oracle| <= 1e-5 for float32 inputs and <= 3e-3 for
bfloat16 inputs (float32 accumulation).  Every comparison is over the whole
output tensor; the oracle is linear in N, so it runs the full workloads too.
Intermediate results (block summaries, mixed summaries) are compared against
the oracle's own stages.
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
    mh.load_library()  # raises if libmhla.so is missing
    yield


def to_dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)


def gpu_forward(q, k, v, W, causal, dtype):
    qd, kd, vd = (to_dev(a, dtype) for a in (q, k, v))
    Wd = torch.from_numpy(W).cuda()
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    fwd = mh.mhla_forward if dtype == "bf16" else mh.mhla_forward_f32
    fwd(qd, kd, vd, Wd, out, causal=causal)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def rel(y, ref):
    return float(np.max(np.abs(y.astype(np.float64) - ref)) / np.max(np.abs(ref)))


def check(w, q, k, v, W, orc, label):
    say(f"[parity] {label}: B={w.B} H={w.H} N={w.N} d={w.d} M={w.M} causal={w.causal} dtype={w.dtype}")
    y = gpu_forward(q, k, v, W, w.causal, w.dtype)
    ref = orc.forward(q, k, v, W, causal=w.causal, nthreads=NTHREADS)
    assert np.all(np.isfinite(y))
    e = rel(y, ref)
    say(f"[parity] {label}: max|dY|/max|Y| = {e:.3e} (tol {TOL[w.dtype]:.0e})")
    assert e <= TOL[w.dtype], (label, e)
    return y, ref


@pytest.mark.parametrize("key", list(WORKLOADS))
def test_workload_full_size(orc, key):
    """Every workload at its full size, compared element by element."""
    w = WORKLOADS[key]
    q, k, v, W = make_inputs(w)
    check(w, q, k, v, W, orc, key)


SWEEP = [  # (B, H, N, d, M, causal, dtype)
    (1, 1, 256, 16, 4, False, "bf16"),
    (1, 1, 256, 16, 4, True, "bf16"),
    (1, 1, 256, 16, 4, True, "f32"),
    (2, 3, 128, 32, 8, False, "f32"),
    (2, 3, 128, 64, 8, True, "f32"),
    (1, 2, 96, 64, 6, False, "bf16"),   # C = 16
    (1, 2, 96, 64, 6, True, "bf16"),
    (2, 1, 170, 32, 10, False, "bf16"),  # C = 17: ragged tiles
    (2, 1, 170, 32, 10, True, "bf16"),
    (1, 2, 500, 64, 4, False, "bf16"),  # C = 125
    (1, 2, 500, 64, 4, True, "bf16"),
    (1, 1, 1024, 64, 1, False, "bf16"),  # one block: global linear attention
    (1, 1, 1024, 64, 1, True, "bf16"),
    (1, 1, 64, 64, 64, False, "bf16"),  # one token per block
    (1, 1, 64, 64, 64, True, "bf16"),
    (1, 1, 64, 16, 64, True, "f32"),
    (3, 1, 40, 16, 8, True, "bf16"),    # C = 5
    (1, 1, 4096, 32, 256, False, "bf16"),
    (1, 1, 4096, 64, 256, False, "bf16"),  # M = 256 walk: 260 column tiles, 4 in the last round
    (1, 1, 4096, 64, 256, True, "bf16"),
    (1, 2, 1536, 64, 3, False, "bf16"),  # C = 512: split summaries
    (1, 2, 1536, 64, 3, True, "bf16"),
    (2, 2, 768, 32, 3, True, "bf16"),   # C = 256, d = 32
    (1, 2, 750, 64, 3, True, "bf16"),   # C = 250: 16 causal tiles, ragged last tile
    (1, 2, 1536, 32, 3, True, "bf16"),  # C = 512 causal at d = 32: running-state output kernel
    (1, 1, 1024, 16, 2, True, "bf16"),  # C = 512 causal at d = 16
    (1, 1, 600, 32, 2, True, "bf16"),   # C = 300 causal at d = 32, ragged last tile
    (1, 3, 5000, 32, 2, False, "bf16"),  # long blocks on few pairs: 10 token segments, ragged last one
    (2, 1, 16384, 16, 1, False, "bf16"),  # global linear attention, 64 token segments per block
    (1, 2, 8192, 64, 4, True, "bf16"),   # causal, 8 token segments per block
    (1, 2, 1280, 16, 80, False, "bf16"),   # 64 < M <= 128: strip mixing, two row tiles per wave
    (1, 1, 2560, 32, 160, True, "bf16"),   # M = 160: three row tiles per wave, causal
    (2, 1, 1536, 64, 192, False, "bf16"),  # M = 192, odd number of 32-deep k-chunks
    (1, 1, 784, 32, 98, True, "bf16"),     # M = 98: rows of W not 16-byte aligned
    (1, 1, 300, 64, 300, False, "f32"),  # M > 256: several mixing row groups
    (1, 1, 600, 32, 300, True, "bf16"),
    (1, 1, 2048, 16, 2048, False, "bf16"),  # mixing fragments beyond LDS: global-fragment kernel
    (1, 1, 2048, 16, 2048, True, "bf16"),
    (2, 1, 1024, 64, 32, False, "bf16"),  # M = 32 mixing variant
    (2, 1, 1024, 64, 32, True, "bf16"),
    (1, 3, 768, 16, 48, False, "bf16"),  # 32 < M <= 64, persistent mixing walk: ragged last column tile
    (2, 1, 680, 32, 34, True, "bf16"),   # M = 34 causal: 33 blocks in two k-chunks, the second of one
]


@pytest.mark.parametrize("case", SWEEP, ids=lambda c: "B{}H{}N{}d{}M{}{}{}".format(*c[:5], "c" if c[5] else "", c[6]))
def test_shape_sweep(orc, case):
    B, H, N, d, M, causal, dtype = case
    w = WORKLOADS["tiny_f32"].shrink(B=B, H=H, N=N, d=d, M=M, causal=causal, dtype=dtype,
                                     seed=2000 + SWEEP.index(case))
    q, k, v, W = make_inputs(w)
    check(w, q, k, v, W, orc, "sweep")


FUSED = [  # (B, H, N, d, M): shapes mhla_forward runs through the fused on-chip kernel
    (64, 1, 256, 64, 16),   # DiT-S/2 @256 blocks, one head
    (64, 1, 160, 64, 16),   # 10-token blocks: ragged 16-token k-steps and query tiles
    (32, 2, 16, 64, 1),     # one block of 16 tokens
    (64, 1, 176, 64, 16),   # 11-token blocks
    (96, 4, 256, 64, 16),   # more workgroups than fit at once
    (3, 2, 16, 64, 16),     # one token per block
    (5, 3, 120, 64, 12),    # 12 blocks: waves 4..7 own one block
    (7, 1, 60, 32, 5),      # 5 blocks (not a multiple of 4), 12-token blocks, d = 32
    (128, 1, 48, 32, 16),   # d = 32, 3-token blocks
    (64, 2, 256, 32, 16),   # d = 32, 16-token blocks
    (256, 1, 16, 16, 16),   # d = 16, one token per block
    (16, 3, 256, 16, 16),   # d = 16, 16-token blocks
    (9, 2, 26, 16, 2),      # d = 16, 2 blocks of 13 tokens
    (16, 3, 256, 64, 4),    # blocks of 64 tokens: 4 tiles each
    (8, 2, 192, 32, 4),     # blocks of 48 tokens: 12 tiles, 3 per block
    (16, 1, 128, 16, 2),    # 8 tiles, 4 per block
    (4, 2, 256, 64, 8),     # blocks of 32 tokens
    (100, 3, 256, 32, 16),  # 300 pairs: some run as two halves of their query tiles
    (70, 5, 160, 64, 16),   # 350 pairs, 10-token blocks, halves
    (24, 2, 256, 64, 1),    # one block of 256 tokens (global linear attention)
    (6, 3, 200, 32, 8),     # 25-token blocks: block edges inside 4-key groups, 7 padded keys
    (12, 1, 96, 16, 3),     # blocks of 32 tokens, d = 16, three 32-key steps
    (260, 1, 224, 64, 14),  # 260 pairs (4 in halves), 14 query tiles, 16-token blocks
]


@pytest.mark.parametrize("case", FUSED, ids=lambda c: "B{}H{}N{}d{}M{}".format(*c))
def test_fused_path(orc, case):
    B, H, N, d, M = case
    assert mh.mhla_forward_path(B, H, N, d, M) == mh.MHLA_PATH_FUSED
    w = WORKLOADS["dit_s2_256"].shrink(B=B, H=H, N=N, d=d, M=M, seed=4000 + FUSED.index(case))
    q, k, v, W = make_inputs(w)
    check(w, q, k, v, W, orc, "fused")


GRAPH_CASES = [  # (workload, shrink): one fused and two staged shapes (pool workspace inside the graph)
    ("dit_s2_256", dict(B=8)),
    ("lm_causal_8k", dict(B=1, H=2, N=1024, M=8)),
    ("dit_s2_4096", dict(H=2, N=4096, M=256)),
]


@pytest.mark.parametrize("case", GRAPH_CASES, ids=lambda c: c[0])
def test_graph_replay(orc, case):
    """mhla_forward captured into a HIP graph: every replay, with eager work and
    synchronisations in between, equals the eager result bit for bit."""
    key, kw = case
    w = WORKLOADS[key].shrink(seed=4100 + GRAPH_CASES.index(case), **kw)
    q, k, v, W = make_inputs(w)
    qd, kd, vd = (to_dev(a, "bf16") for a in (q, k, v))
    Wd = torch.from_numpy(W).cuda()
    eager = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    mh.mhla_forward(qd, kd, vd, Wd, eager, causal=w.causal)
    torch.cuda.synchronize()
    ref = orc.forward(q, k, v, W, causal=w.causal, nthreads=NTHREADS)
    assert rel(eager.cpu().numpy(), ref) <= TOL["bf16"]
    out = torch.empty_like(eager)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mh.mhla_forward(qd, kd, vd, Wd, out, causal=w.causal)
    other = torch.empty_like(eager)
    for rep in range(4):
        say(f"[graph] {key} replay {rep}")
        out.fill_(float("nan"))
        mh.mhla_forward(kd, qd, vd, Wd, other, causal=w.causal)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep


def staged_forward(q, k, v, W, causal, dtype):
    """The three stage entry points chained by hand (the staged path end to end)."""
    B, H, N, d = q.shape
    M = W.shape[0]
    qd, kd, vd = (to_dev(a, dtype) for a in (q, k, v))
    Wd = torch.from_numpy(W).cuda()
    L = mh.mhla_summary_floats(d)
    S = torch.empty(M * B * H * L, dtype=torch.float32, device="cuda")
    St = torch.empty_like(S)
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    mh.mhla_block_summaries(kd, vd, S, M)
    mh.mhla_mix_summaries(S, Wd, St, B * H, d, causal=causal, precise=(dtype == "f32"))
    mh.mhla_output(qd, kd, vd, St, Wd, out, causal=causal)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("key", ["dit_s2_256", "tiny_f32"])
def test_staged_path_end_to_end(orc, key):
    """The staged kernels on shapes where mhla_forward would take the fused path."""
    w = WORKLOADS[key]
    q, k, v, W = make_inputs(w)
    say(f"[parity] staged {key}")
    y = staged_forward(q, k, v, W, w.causal, w.dtype)
    ref = orc.forward(q, k, v, W, causal=w.causal, nthreads=NTHREADS)
    e = rel(y, ref)
    say(f"[parity] staged {key}: max|dY|/max|Y| = {e:.3e}")
    assert e <= TOL[w.dtype], e


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [16, 32, 64])
def test_stage_summaries_and_mix(orc, dtype, d):
    """Stage 1 and stage 2 outputs against the oracle's S_b, z_b, S~_i, z~_i."""
    B, H, N, M = 2, 3, 256, 8
    for causal in (False, True):
        w = WORKLOADS["tiny_f32"].shrink(B=B, H=H, N=N, d=d, M=M, causal=causal, dtype=dtype, seed=3000 + d)
        q, k, v, W = make_inputs(w)
        kd, vd = to_dev(k, dtype), to_dev(v, dtype)
        L = mh.mhla_summary_floats(d)
        S = torch.empty(M * B * H * L, dtype=torch.float32, device="cuda")
        St = torch.empty_like(S)
        mh.mhla_block_summaries(kd, vd, S, M)
        mh.mhla_mix_summaries(S, torch.from_numpy(W).cuda(), St, B * H, d, causal=causal, precise=(dtype == "f32"))
        torch.cuda.synchronize()
        Sg, zg = mh.mhla_unpack_summaries(S.cpu().reshape(M, B, H, L), d)
        Stg, ztg = mh.mhla_unpack_summaries(St.cpu().reshape(M, B, H, L), d)
        S_ref, z_ref = orc.summaries(k, v, M)        # [B, H, M, d, d]
        St_ref, zt_ref = orc.mix(S_ref, z_ref, W, causal=causal)
        tol = 1e-5 if dtype == "f32" else 3e-3
        for got, ref in ((Sg, S_ref), (zg, z_ref), (Stg, St_ref), (ztg, zt_ref)):
            got = np.moveaxis(got.numpy(), 0, 2)  # [M, B, H, ...] -> [B, H, M, ...]
            assert rel(got, ref) <= tol, (dtype, d, causal, rel(got, ref))


def test_deterministic(orc):
    w = WORKLOADS["lm_causal_8k"].shrink(B=2, H=2, N=1024, M=8)
    q, k, v, W = make_inputs(w)
    a = gpu_forward(q, k, v, W, True, "bf16")
    b = gpu_forward(q, k, v, W, True, "bf16")
    assert np.array_equal(a, b)


def test_causality_bitwise():
    """Changing tokens after T leaves output rows up to T bit-identical."""
    w = WORKLOADS["lm_causal_8k"].shrink(B=1, H=2, N=2048, M=16)
    q, k, v, W = make_inputs(w)
    y = gpu_forward(q, k, v, W, True, "bf16")
    for T in (0, 100, 127, 128, 1500):
        q2, k2, v2 = q.copy(), k.copy(), v.copy()
        for a in (q2, k2, v2):
            a[:, :, T + 1:] = -a[:, :, T + 1:] * 0.5
        y2 = gpu_forward(q2, k2, v2, W, True, "bf16")
        assert np.array_equal(y[:, :, : T + 1], y2[:, :, : T + 1]), T
        assert not np.array_equal(y[:, :, T + 1:], y2[:, :, T + 1:]), T


def test_causal_ignores_upper_triangle():
    w = WORKLOADS["lm_causal_8k"].shrink(B=1, H=2, N=1024, M=8)
    q, k, v, W = make_inputs(w)
    Wn = W.copy()
    Wn[np.triu_indices(8, 1)] = np.nan
    y = gpu_forward(q, k, v, W, True, "bf16")
    yn = gpu_forward(q, k, v, Wn, True, "bf16")
    assert np.array_equal(y, yn)


def test_guard_bytes_and_stream(orc):
    """Writes stay inside `out`; a non-default stream works without a device sync."""
    w = WORKLOADS["dit_s2_256"].shrink(B=2)
    q, k, v, W = make_inputs(w)
    qd, kd, vd = (to_dev(a, "bf16") for a in (q, k, v))
    Wd = torch.from_numpy(W).cuda()
    n = q.size
    guard = 4096
    buf = torch.full((n + 2 * guard,), 12345.0, dtype=torch.float32, device="cuda")
    out = buf[guard: guard + n].view(q.shape)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        mh.mhla_forward(qd, kd, vd, Wd, out, causal=False)
    s.synchronize()
    b = buf.cpu().numpy()
    assert np.all(b[:guard] == 12345.0) and np.all(b[guard + n:] == 12345.0)
    ref = orc.forward(q, k, v, W, nthreads=NTHREADS)
    assert rel(out.cpu().numpy(), ref) <= TOL["bf16"]


def test_errors_raise_on_device():
    q = torch.zeros((1, 1, 256, 24), dtype=torch.bfloat16, device="cuda")
    W = torch.ones((4, 4), dtype=torch.float32, device="cuda")
    out = torch.empty((1, 1, 256, 24), dtype=torch.float32, device="cuda")
    with pytest.raises(mh.MhlaError) as e:
        mh.mhla_forward(q, q, q, W, out)
    assert e.value.status == mh.MHLA_ERR_UNSUPPORTED
    q = torch.zeros((1, 1, 250, 64), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((1, 1, 250, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(mh.MhlaError) as e:
        mh.mhla_forward(q, q, q, W, out)
    assert e.value.status == mh.MHLA_ERR_INVALID_ARG
    out = torch.zeros((1, 1, 256, 64), dtype=torch.float32, device="cuda")
    q = out.view(-1).view(torch.bfloat16)[: 256 * 64].view(1, 1, 256, 64)  # the first half of out
    with pytest.raises(mh.MhlaError) as e:  # out overlaps q
        mh.mhla_forward(q, q, q, W, out)
    assert e.value.status == mh.MHLA_ERR_INVALID_ARG
