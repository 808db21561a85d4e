"""The per-stream workspace of the staged path, against the oracle.

* Two streams running staged forward passes at the same time (each stream has its
  own workspace; the calls interleave on the device).
* Growth: a small call, then a larger one on the same stream (the workspace is
  replaced by a larger one), then the small one again.
* A HIP graph captured on the stream is replayed after the stream's workspace has
  grown: a captured call takes its own workspace inside the graph (allocation and
  free nodes), so the replay does not depend on the stream's workspace.
* Graphs captured, replayed and deleted one after another on the same stream, with
  eager calls of other sizes in between (each graph's workspace ends with it).
"""
import os
import sys

import numpy as np
import pytest
import torch

import token_level_head_amd as mh
from token_level_head_amd.workloads import WORKLOADS, make_inputs

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


def case(B, H, N, M, seed, causal=False):
    w = WORKLOADS["dit_s2_4096"].shrink(B=B, H=H, N=N, M=M, causal=causal, seed=seed)
    assert mh.mhla_forward_path(w.B, w.H, w.N, w.d, w.M, w.causal) == mh.MHLA_PATH_STAGED
    q, k, v, W = make_inputs(w)
    dev = [torch.from_numpy(a).to("cuda", torch.bfloat16) for a in (q, k, v)]
    return w, (q, k, v, W), dev, torch.from_numpy(W).cuda()


def rel(y, ref):
    return float(np.max(np.abs(y.astype(np.float64) - ref)) / np.max(np.abs(ref)))


def check(orc, host, out, causal=False):
    q, k, v, W = host
    bf = [torch.from_numpy(a).to(torch.bfloat16).float().numpy() for a in (q, k, v)]
    ref = orc.forward(*bf, W, causal=causal, nthreads=NTHREADS)
    e = rel(out.cpu().numpy(), ref)
    assert e <= TOL, e
    return e


def test_two_streams_at_once(orc):
    a = case(2, 3, 2048, 32, 7400)
    b = case(1, 4, 4096, 64, 7401, causal=True)
    outs = [torch.empty(x[2][0].shape, dtype=torch.float32, device="cuda") for x in (a, b)]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    say("[workspace] two streams, 10 interleaved staged calls each")
    torch.cuda.synchronize()
    for _ in range(10):
        with torch.cuda.stream(s1):
            mh.mhla_forward(*a[2], a[3], outs[0])
        with torch.cuda.stream(s2):
            mh.mhla_forward(*b[2], b[3], outs[1], causal=True)
    torch.cuda.synchronize()
    say(f"[workspace]   stream 1: {check(orc, a[1], outs[0]):.2e}")
    say(f"[workspace]   stream 2: {check(orc, b[1], outs[1], causal=True):.2e}")


def test_growth_and_graph_across_growth(orc):
    small = case(1, 2, 1024, 16, 7410)
    large = case(4, 8, 8192, 256, 7411)
    s = torch.cuda.Stream()
    out_s = torch.empty(small[2][0].shape, dtype=torch.float32, device="cuda")
    out_l = torch.empty(large[2][0].shape, dtype=torch.float32, device="cuda")
    with torch.cuda.stream(s):
        mh.mhla_forward(*small[2], small[3], out_s)  # sizes this stream's workspace
    s.synchronize()
    say(f"[workspace] small call: {check(orc, small[1], out_s):.2e}")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        mh.mhla_forward(*small[2], small[3], out_s)
    with torch.cuda.stream(s):
        mh.mhla_forward(*large[2], large[3], out_l)  # grows the workspace
    s.synchronize()
    say(f"[workspace] large call after it: {check(orc, large[1], out_l):.2e}")
    for r in range(3):
        out_s.zero_()
        graph.replay()
        torch.cuda.synchronize()
        say(f"[workspace] replay {r} of the graph captured before the growth: {check(orc, small[1], out_s):.2e}")
    out_s.zero_()
    with torch.cuda.stream(s):
        mh.mhla_forward(*small[2], small[3], out_s)
    s.synchronize()
    say(f"[workspace] small call after the growth: {check(orc, small[1], out_s):.2e}")


def test_graphs_deleted_between_captures(orc):
    cases = [case(1, 2, 1024, 16, 7420), case(2, 2, 2048, 64, 7421), case(1, 3, 1024, 32, 7422)]
    s = torch.cuda.Stream()
    outs = [torch.empty(c[2][0].shape, dtype=torch.float32, device="cuda") for c in cases]
    for rnd in range(2):
        for c, out in zip(cases, outs):
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=s):
                mh.mhla_forward(*c[2], c[3], out)
            for _ in range(2):
                out.zero_()
                graph.replay()
            torch.cuda.synchronize()
            say(f"[workspace] round {rnd}, B={c[0].B} N={c[0].N} M={c[0].M}: graph {check(orc, c[1], out):.2e}")
            del graph
            with torch.cuda.stream(s):
                out.zero_()
                mh.mhla_forward(*c[2], c[3], out)
            s.synchronize()
            say(f"[workspace]   eager on the capture stream: {check(orc, c[1], out):.2e}")
