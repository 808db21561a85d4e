"""The staged entry points only enqueue work: a call must return without waiting for
the device, also when it needs workspace.

A long run of device work is enqueued first; calls of every entry point that uses
workspace (staged forward, the stage entry points, the backward pass) follow on the
same stream, and the earlier work must still be pending when they have all returned.
"""
import sys

import numpy as np
import torch
import pytest

import token_level_head_amd as mh
from token_level_head_amd.workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "these tests need the MI355X"
    mh.load_library()
    yield


def test_staged_calls_do_not_wait_for_the_device():
    w = WORKLOADS["dit_s2_4096"].shrink(B=1, H=2, N=4096, M=64, seed=7300)  # staged path, M > 16
    assert mh.mhla_forward_path(w.B, w.H, w.N, w.d, w.M) == mh.MHLA_PATH_STAGED
    q, k, v, W = make_inputs(w)
    qd, kd, vd = (torch.from_numpy(a).to("cuda", torch.bfloat16) for a in (q, k, v))
    Wd = torch.from_numpy(W).cuda()
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    L = w.d * w.d + w.d
    S = torch.empty(w.M * w.B * w.H * L, dtype=torch.float32, device="cuda")
    St = torch.empty_like(S)
    dy = torch.ones(q.shape, dtype=torch.float32, device="cuda")
    grads = [torch.empty(q.shape, dtype=torch.float32, device="cuda") for _ in range(3)]
    dW = torch.empty_like(Wd)

    def calls():
        mh.mhla_forward(qd, kd, vd, Wd, out)
        mh.mhla_block_summaries(kd, vd, S, w.M)
        mh.mhla_mix_summaries(S, Wd, St, w.B * w.H, w.d)
        mh.mhla_output(qd, kd, vd, St, Wd, out)
        mh.mhla_backward(qd, kd, vd, Wd, dy, *grads, dW)

    calls()  # first calls size the stream's workspace
    torch.cuda.synchronize()
    busy = torch.ones(1 << 26, dtype=torch.float32, device="cuda")
    say("[async] enqueueing ~0.5 s of device work, then 20 rounds of staged calls")
    for _ in range(10000):
        busy.sum()
    pending = torch.cuda.Event()
    pending.record()
    for _ in range(20):
        calls()
    still_pending = not pending.query()
    torch.cuda.synchronize()
    assert still_pending, "a staged call waited for earlier device work"
    assert np.all(np.isfinite(out.cpu().numpy()))
