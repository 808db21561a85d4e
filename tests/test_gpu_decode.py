"""GPU parity of the streaming causal decode step against the oracle.

Decoding a whole sequence one token at a time must reproduce every row of the
causal forward pass (App. C inference equals the causal forward).  The decode
kernels compute in float32 on the exact input values, so the bar is the float32
one, max|dY| / max|Y_oracle| <= 1e-5, for bf16 inputs too.
"""
import os
import sys

import numpy as np
import pytest
import torch

import token_level_head_amd as mh
from token_level_head_amd.workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

NTHREADS = min(16, os.cpu_count() or 1)

DECODE = [  # (B, H, N, d, M, causal inputs dtype)
    (2, 3, 256, 64, 4, "bf16"),   # C = 64
    (1, 2, 128, 32, 8, "f32"),    # C = 16
    (2, 1, 96, 16, 6, "bf16"),    # d = 16
    (1, 1, 64, 64, 64, "bf16"),   # one token per block
    (1, 2, 200, 64, 1, "f32"),    # one block: the plain recurrence
    (1, 1, 150, 32, 10, "bf16"),  # C = 15
]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def decode_sequence(q, k, v, W, C, dtype, normalize=True):
    B, H, N, d = q.shape
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    qd, kd, vd = (torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dt) for a in (q, k, v))
    Wd = torch.from_numpy(np.ascontiguousarray(W)).cuda()
    M = W.shape[-1]
    state = torch.full((mh.mhla_decode_state_bytes(B, H, d, M) // 4,), float("nan"), device="cuda")
    out = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
    yt = torch.empty((B, H, d), dtype=torch.float32, device="cuda")
    for t in range(N):
        if normalize and W.ndim == 2:
            mh.mhla_decode_step(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(), vd[:, :, t].contiguous(), Wd,
                                state, yt, C, t)
        else:
            mh.mhla_decode_step_ex(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(), vd[:, :, t].contiguous(),
                                   Wd, state, yt, C, t, normalize=normalize)
        out[:, :, t].copy_(yt)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("case", DECODE, ids=lambda c: "B{}H{}N{}d{}M{}{}".format(*c))
def test_decode_equals_causal_forward(orc, case):
    B, H, N, d, M, dtype = case
    w = WORKLOADS["lm_causal_8k"].shrink(B=B, H=H, N=N, d=d, M=M, dtype=dtype, seed=5000 + DECODE.index(case))
    q, k, v, W = make_inputs(w)
    say(f"[decode] B={B} H={H} N={N} d={d} M={M} dtype={dtype}")
    y = decode_sequence(q, k, v, W, N // M, dtype)
    ref = orc.forward(q, k, v, W, causal=True, nthreads=NTHREADS)
    assert np.all(np.isfinite(y))
    e = float(np.max(np.abs(y.astype(np.float64) - ref)) / np.max(np.abs(ref)))
    say(f"[decode] max|dY|/max|Y| = {e:.3e}")
    assert e <= 1e-5, e


def test_decode_is_deterministic(orc):
    w = WORKLOADS["lm_causal_8k"].shrink(B=2, H=2, N=128, M=4, seed=5100)
    q, k, v, W = make_inputs(w)
    a = decode_sequence(q, k, v, W, 32, "bf16")
    b = decode_sequence(q, k, v, W, 32, "bf16")
    assert np.array_equal(a, b)


@pytest.mark.parametrize("case", [DECODE[i] for i in (0, 1, 2, 4)], ids=lambda c: "B{}H{}N{}d{}M{}{}".format(*c))
def test_decode_without_normaliser_equals_causal_forward(orc, case):
    # the numerator alone ("MHLA" §4.1, remark on the output): row t of the causal
    # forward pass without the normaliser
    B, H, N, d, M, dtype = case
    w = WORKLOADS["lm_causal_8k"].shrink(B=B, H=H, N=N, d=d, M=M, dtype=dtype, seed=5200 + DECODE.index(case))
    q, k, v, W = make_inputs(w)
    say(f"[decode, no normaliser] B={B} H={H} N={N} d={d} M={M} dtype={dtype}")
    y = decode_sequence(q, k, v, W, N // M, dtype, normalize=False)
    ref = orc.forward(q, k, v, W, causal=True, nthreads=NTHREADS, normalize=False)
    assert np.all(np.isfinite(y))
    e = float(np.max(np.abs(y.astype(np.float64) - ref)) / np.max(np.abs(ref)))
    say(f"[decode, no normaliser] max|dY|/max|Y| = {e:.3e}")
    assert e <= 1e-5, e


@pytest.mark.parametrize("normalize", [True, False])
def test_decode_per_head_w_equals_causal_forward(orc, normalize):
    # one mixing matrix per head: head h decodes with W[h]
    B, H, N, d, M = 2, 3, 128, 32, 8
    w = WORKLOADS["lm_causal_8k"].shrink(B=B, H=H, N=N, d=d, M=M, dtype="bf16", seed=5300 + int(normalize))
    q, k, v, W0 = make_inputs(w)
    rng = np.random.default_rng(5310 + int(normalize))
    W = np.stack([np.tril(np.exp(rng.standard_normal((M, M)))) for _ in range(H)])
    W = (W / W.sum(axis=2, keepdims=True)).astype(np.float32)
    say(f"[decode, W per head] B={B} H={H} N={N} d={d} M={M} normalize={normalize}")
    y = decode_sequence(q, k, v, W, N // M, "bf16", normalize=normalize)
    ref = orc.forward(q, k, v, W, causal=True, nthreads=NTHREADS, normalize=normalize)
    e = float(np.max(np.abs(y.astype(np.float64) - ref)) / np.max(np.abs(ref)))
    say(f"[decode, W per head] max|dY|/max|Y| = {e:.3e}")
    assert e <= 1e-5, e
