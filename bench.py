#!/usr/bin/env python3
"""Benchmark of the MHLA forward pass on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload sana_128] [--gpus 1]
    python bench.py --sweep          # N x M throughput grid (the paper's scaling study)
    python bench.py --decode         # streaming causal decode step (lm_causal_8k shape)
    python bench.py --backward       # backward pass (dq, dk, dv, dW) on the workload

One step is one full forward pass (phi, block summaries, mixing, output) over
the workload's synthetic batch, with inputs resident in HBM before the timed
region and the caches cold: the K timed calls rotate over copies of the inputs
and outputs that together exceed twice the Infinity Cache, so each call reads
its inputs from HBM.
Prints ONE JSON line with throughput (tokens/s), model TFLOP/s, the HBM roofline
of the dominant kernel (its duration measured with HIP events on the launch
stream: the whole step on the fused path, the stage inside a chain of
summaries -> mixing -> output calls on the staged path) and the CPU oracle timed
on this host's cores.  --warm adds back-to-back steps on cache-resident inputs.
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

import token_level_head_amd as mh
from token_level_head_amd.workloads import WORKLOADS, make_inputs

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
PATH_NAMES = {0: "staged", 1: "fused", 2: "pair"}  # mhla_forward_path() values
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
METRIC = "MHLA fwd tokens/s and TFLOP/s at 1 MI355X; % of HBM/MFMA roofline"


def model_flops(w):
    """Model FLOPs of one forward pass (multiply-add = 2)."""
    BH, N, d, M, C = w.B * w.H, w.N, w.d, w.M, w.C
    nnz = M * (M - 1) // 2 if w.causal else M * M
    per_pair = N * (2 * d * d + d)            # summaries: phi(k) v^T and z
    per_pair += 2 * nnz * (d * d + d)         # mixing GEMM
    per_pair += N * (2 * d * d + 3 * d)       # output: numerator, denominator, divide
    if w.causal:
        per_pair += N * (2 * d * (C + 1) + (C + 1) / 2)  # within-block prefix (average over positions)
    return BH * per_pair


def mix_flops(w):
    """(model, executed) FLOPs of the mixing GEMM: 2 * nnz(W) * (d*d + d) per pair, and the
    bf16 MFMA work that carries it out (three hi/lo products per term)."""
    BH, d, M = w.B * w.H, w.d, w.M
    nnz = M * (M - 1) // 2 if w.causal else M * M
    model = 2 * nnz * (d * d + d) * BH
    return model, (3 * model if w.dtype == "bf16" else model)


def kernel_bytes(w):
    """Algorithmic HBM bytes per launch of each stage (inputs read once, outputs written once)."""
    BH, N, d, M = w.B * w.H, w.N, w.d, w.M
    e = 2 if w.dtype == "bf16" else 4
    L = d * d + d
    summ = BH * M * L * 4
    return {
        "summaries": 2 * BH * N * d * e + summ,
        "mix": 2 * summ + M * M * 4,
        "output": BH * N * d * e + summ + BH * N * d * 4 + (2 * BH * N * d * e + M * 4 if w.causal else 0),
        # one kernel, summaries on chip: q, k, v read once, y written once
        "fused": 3 * BH * N * d * e + BH * N * d * 4 + M * M * 4,
        "pair": 3 * BH * N * d * e + BH * N * d * 4 + M * M * 4,
    }


def measured_traffic(workload, stage):
    """HBM bytes per launch of `stage` from the committed counter summary, or None when
    there is none for this workload or the kernel's source changed since it was taken."""
    from token_level_head_amd.build import kernel_source_digest

    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", f"counters_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        prof = json.load(f)
    prefix = {"fused": "fused_", "pair": "pair_", "summaries": "summaries_", "mix": "mix_", "output": "output_"}[stage]
    for name, k in prof["kernels"].items():
        if name.startswith(prefix):
            if k.get("source_digest") != kernel_source_digest(name):
                return None
            return round(k["traffic_bytes"])
    return None


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def cpu_baseline(w, q, k, v, W, budget_s):
    """The oracle (test infrastructure, never tuned) on this host's cores, on a bounded
    sample of the workload: whole (batch, head) pairs -- the oracle's unit of work, each
    pair the full sequence of N tokens -- taken in [B][H] order, once on one thread and
    once on all the threads this process may use (at most 16, the host share of one
    GPU).  Rates are scaled to the metric's unit: a token of the workload is H
    token-heads, so tokens/s = pairs * N / H / seconds."""
    import oracle  # test infrastructure: used only for this reported baseline

    orc = oracle.default_oracle()
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    threads = max(1, min(avail, 16))
    BH = w.B * w.H
    shape = (1, BH, w.N, w.d)
    qs, ks, vs = (np.ascontiguousarray(a).reshape(shape) for a in (q, k, v))

    def run(pairs, nthreads):
        sl = slice(0, pairs)
        t0 = time.perf_counter()
        orc.forward(qs[:, sl], ks[:, sl], vs[:, sl], W, causal=w.causal, nthreads=nthreads)
        return time.perf_counter() - t0

    def measured(nthreads, unit):
        """Calibrate on `unit` pairs, then time enough pairs (a multiple of unit) for
        about budget_s seconds."""
        t_unit = run(unit, nthreads)
        reps = max(1, min(BH // unit, int(budget_s / max(t_unit, 1e-6))))
        pairs = reps * unit
        dt = run(pairs, nthreads)
        return pairs, dt

    p1, t1 = measured(1, 1)
    unit = min(threads, BH)
    pm, tm = measured(threads, unit)
    rate = lambda pairs, dt: pairs * w.N / w.H / dt  # noqa: E731
    return {
        "value": rate(pm, tm),
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{pm} of the {BH} (batch, head) pairs of {w.key} (each {w.N} tokens, d={w.d}, M={w.M}) "
                  f"in {tm:.2f} s on {threads} threads; tokens/s = pairs * N / H / s",
        "single_thread": {"value": rate(p1, t1), "unit": "tokens/s", "cores": 1,
                          "sample": f"{p1} pairs in {t1:.2f} s on 1 thread"},
        "host": {"nproc": os.cpu_count(), "threads_available": avail, "cpu_model": _cpu_model()},
    }


def decode_bench(args, w):
    """One block of C decode steps starting at the first token of block M/2 (so the
    timed region includes one block boundary: closing a block and mixing M/2
    completed summaries), timed as one HIP graph replay and as eager launches; the
    token kernel alone is timed on the C - 1 steps after the boundary."""
    B, H, d, M, C = w.B, w.H, w.d, w.M, w.C
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    gen = torch.Generator(device="cpu").manual_seed(w.seed)
    q, k, v = (torch.randn((C, B, H, d), generator=gen).to("cuda", dt) for _ in range(3))
    W = torch.from_numpy(make_inputs(w.shrink(B=1, H=1, N=w.M, d=16))[3]).cuda()
    state = torch.zeros(mh.mhla_decode_state_bytes(B, H, d, M) // 4, device="cuda")
    out = torch.empty((B, H, d), dtype=torch.float32, device="cuda")
    t0 = (M // 2) * C
    stream = torch.cuda.current_stream()

    def steps(first, count):
        for j in range(first, first + count):
            mh.mhla_decode_step(q[j], k[j], v[j], W, state, out, C, t0 + j)

    def elapsed_ms(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    def best_ms(first, count):
        steps(first, count)  # warm-up
        eager = elapsed_ms(lambda: steps(first, count)) / count
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            steps(first, count)
        graph.replay()
        return min(eager, elapsed_ms(graph.replay) / count), eager

    ms, eager_ms = best_ms(0, C)
    tok_ms, _ = best_ms(1, C - 1) if C > 1 else (ms, ms)
    L = d * d + d
    e = 2 if w.dtype == "bf16" else 4
    tok_bytes = B * H * (3 * L * 4 + 3 * d * e + d * 4)  # read S~ and P, write P; q, k, v in, y out
    achieved = tok_bytes / (tok_ms * 1e-3) / 1e9
    line = {
        "metric": "MHLA causal decode tokens/s at 1 MI355X (one token per sequence per step)",
        "value": round(B / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": C,
        "warmup": C,
        "ms_per_step": round(ms, 5),
        "eager_ms_per_step": round(eager_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.key + "_decode", "B": B, "H": H, "d": d, "M": M, "C": C, "first_token": t0,
                   "global_batch": B, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "kernel": "decode_token_kernel", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)
    return 0


def backward_bench(args, w):
    """The backward pass (dq, dk, dv, dW of sum(dy * Y)) on the workload's batch: K calls
    timed between HIP events (faster of one HIP-graph replay and eager launches).  Bytes
    per call counted as q, k, v, dy read once and dq, dk, dv written once (float32
    arithmetic; the kernels recompute the summaries and read the inputs more than once)."""
    q, k, v, W = make_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    qd, kd, vd = (torch.from_numpy(a).to("cuda", dt) for a in (q, k, v))
    Wd = torch.from_numpy(W).cuda()
    gen = torch.Generator(device="cuda").manual_seed(w.seed + 1)
    dy = torch.randn(q.shape, generator=gen, device="cuda", dtype=torch.float32)
    dq, dk, dv = (torch.empty(q.shape, dtype=torch.float32, device="cuda") for _ in range(3))
    dW = torch.empty_like(Wd)
    stream = torch.cuda.current_stream()

    def run(n):
        for _ in range(n):
            mh.mhla_backward(qd, kd, vd, Wd, dy, dq, dk, dv, dW, causal=w.causal)

    def elapsed_ms(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    run(args.warmup)
    eager = elapsed_ms(lambda: run(args.steps)) / args.steps
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(args.steps)
    graph.replay()
    gms = elapsed_ms(graph.replay) / args.steps
    ms = min(eager, gms)
    e = 2 if w.dtype == "bf16" else 4
    nbytes = w.B * w.H * w.N * w.d * (3 * e + 4 + 3 * 4)
    achieved = nbytes / (ms * 1e-3) / 1e9
    line = {
        "metric": "MHLA backward (dq, dk, dv, dW) tokens/s at 1 MI355X",
        "value": round(w.tokens / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "graph_ms_per_step": round(gms, 5), "eager_ms_per_step": round(eager, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.key + "_backward", "B": w.B, "H": w.H, "N": w.N, "d": w.d, "M": w.M,
                   "causal": w.causal, "global_batch": w.B, "seq_len": w.N, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "kernel": "backward (all kernels)", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)
    return 0


def sweep_bench(args):
    """Throughput over a grid of sequence lengths N and block counts M at the DiT-S/2 head
    shape (H = 6, d = 64, bf16, non-causal), each point on a batch of about 2^18 tokens,
    relative to M = 1 (global linear attention): the design of the N x M scaling study of
    the MHLA paper (App. F.4, Table 14), whose cost model puts the mixing term M^2 d^2 next
    to N d^2.  Inputs: Q, K, V ~ N(0, 1) drawn on the device from a fixed seed; W rows are
    softmaxes of N(0, 1) logits."""
    H, d = 6, 64
    stream = torch.cuda.current_stream()
    gen = torch.Generator(device="cuda").manual_seed(4242)
    points = []
    for N in (256, 1024, 4096, 16384, 65536):
        B = max(1, (1 << 18) // N)
        q, k, v = (torch.randn((B, H, N, d), generator=gen, device="cuda").to(torch.bfloat16) for _ in range(3))
        out = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
        base = None
        for M in (1, 4, 16, 64, 256):
            if M > N or N % M:
                continue
            W = torch.softmax(torch.randn((M, M), generator=gen, device="cuda", dtype=torch.float64), dim=1).float()
            for _ in range(args.warmup):
                mh.mhla_forward(q, k, v, W, out)
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for _ in range(args.steps):
                    mh.mhla_forward(q, k, v, W, out)
            graph.replay()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.steps
            tok_s = B * N / (ms * 1e-3)
            base = tok_s if M == 1 else base
            path = mh.mhla_forward_path(B, H, N, d, M, False, mh.MHLA_DTYPE_BF16)
            points.append({"N": N, "M": M, "B": B, "M2_lt_N": M * M < N, "ms": round(ms, 5),
                           "tokens_per_s": round(tok_s, 1), "rel_to_M1": round(tok_s / base, 4),
                           "path": PATH_NAMES[path]})
            print(f"N={N} M={M} B={B}: {ms * 1e3:.1f} us, {tok_s:.3e} tokens/s, x{tok_s / base:.3f} of M=1",
                  file=sys.stderr, flush=True)
            del graph
        del q, k, v, out
    line = {"metric": "MHLA fwd tokens/s over an N x M grid at 1 MI355X (DiT-S/2 heads: H=6, d=64, bf16)",
            "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
            "data": "synthetic", "config": {"workload": "nm_sweep", "H": H, "d": d, "tokens_per_point": 1 << 18},
            "points": points}
    print(json.dumps(line), flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="sana_128", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-budget", type=float, default=5.0,
                    help="seconds of oracle wall time for each of the one-thread and all-thread samples")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode", action="store_true",
                    help="time the streaming causal decode step (one token per call) on the workload's "
                         "B, H, d, M, C instead of the forward pass; prints its own JSON line")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (dq, dk, dv, dW) on the workload instead of the forward")
    ap.add_argument("--sweep", action="store_true",
                    help="time mhla_forward over the N x M grid of the paper's scaling study instead of one "
                         "workload; prints its own JSON line")
    ap.add_argument("--warm", action="store_true",
                    help="also time back-to-back steps on cache-resident inputs (reported under `warm`)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device-to-device copy (3x), the reference that scales "
                         "the FETCH_SIZE / WRITE_SIZE counters in counter-collection runs")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path).", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2

    w = WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    mh.load_library()
    if args.decode:
        return decode_bench(args, w)
    if args.backward:
        return backward_bench(args, w)
    if args.sweep:
        return sweep_bench(args)
    q, k, v, W = make_inputs(w)
    dt_in = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    qd, kd, vd = (torch.from_numpy(a).to(device="cuda", dtype=dt_in) for a in (q, k, v))
    Wd = torch.from_numpy(W).cuda()
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    fwd = mh.mhla_forward if w.dtype == "bf16" else mh.mhla_forward_f32
    stream = torch.cuda.current_stream()
    path = mh.mhla_forward_path(w.B, w.H, w.N, w.d, w.M, w.causal,
                                mh.MHLA_DTYPE_BF16 if w.dtype == "bf16" else mh.MHLA_DTYPE_F32)

    def elapsed_ms(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    # ---- whole-pass throughput, cold caches ----
    # The calls rotate over `nbuf` copies of the inputs and outputs, at least 512 MiB in
    # all (twice the Infinity Cache), so each call's buffers were last touched nbuf - 1
    # calls earlier and have been evicted from L2 and the Infinity Cache: every call
    # reads its inputs from HBM.  K back-to-back calls between two HIP events on the
    # launch stream.
    per_call = sum(t.numel() * t.element_size() for t in (qd, kd, vd, out))
    nbuf = int(min(16, max(1, -(-(512 << 20) // per_call))))
    sets = [(qd, kd, vd, out)] + [tuple(t.clone() for t in (qd, kd, vd, out)) for _ in range(nbuf - 1)]

    def run_cold(n, start=0):
        for i in range(n):
            a, b_, c, o = sets[(start + i) % nbuf]
            fwd(a, b_, c, Wd, o, causal=w.causal)

    # A pre-roll of device work (reads, so no dirty lines are left behind) keeps the GPU
    # busy while the host enqueues the timed calls; `pre_done` still pending once they are
    # enqueued shows that the GPU never waited for the host.
    preroll = torch.ones(1 << 26, dtype=torch.float32, device="cuda")
    run_cold(args.warmup)
    torch.cuda.synchronize()
    for _ in range(8 * args.steps):
        preroll.sum()
    pre_done = torch.cuda.Event()
    pre_done.record(stream)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    run_cold(args.steps, args.warmup)
    t1.record(stream)
    steps_gapless = not pre_done.query()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    tokens_s = w.tokens / (ms * 1e-3)
    tflops = model_flops(w) / (ms * 1e-3) / 1e12

    # ---- optional: warm steps (back to back on the same, cache-resident inputs), as one
    # HIP graph replay of K calls and as K eager launches; the replayed output must equal
    # the eager output bit for bit. ----
    warm = None
    if args.warm:
        def run_steps(n):
            for _ in range(n):
                fwd(qd, kd, vd, Wd, out, causal=w.causal)

        run_steps(args.warmup)
        eager_ms = elapsed_ms(lambda: run_steps(args.steps)) / args.steps
        ref = out.clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run_steps(args.steps)
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(out, ref):
            raise RuntimeError("graph replay of the forward pass differs from the eager result")
        graph.replay()
        graph_ms = elapsed_ms(graph.replay) / args.steps
        wms = min(graph_ms, eager_ms)
        warm = {"ms_per_step": round(wms, 5), "value": round(w.tokens / (wms * 1e-3), 1),
                "graph_ms_per_step": round(graph_ms, 5), "eager_ms_per_step": round(eager_ms, 5),
                "timing": "K steps back to back on cache-resident inputs, faster of one HIP graph replay "
                          "and K eager launches"}

    # ---- per-stage durations: K chains of summaries -> mixing -> output (each stage
    # consuming the previous one's result, as inside mhla_forward) over the rotating
    # buffer sets, HIP events between the stages on the launch stream; mean per stage.  When mhla_forward takes the fused path these are reported for reference only
    # (`staged_kernels`); the step itself is the fused kernel. ----
    L = w.d * w.d + w.d
    S = torch.empty(w.M * w.B * w.H * L, dtype=torch.float32, device="cuda")
    St = torch.empty_like(S)
    names = ["summaries", "mix", "output"]

    def chain(i):
        a, b_, c, o = sets[i % nbuf]
        return [
            lambda: mh.mhla_block_summaries(b_, c, S, w.M),
            lambda: mh.mhla_mix_summaries(S, Wd, St, w.B * w.H, w.d, causal=w.causal, precise=(w.dtype == "f32")),
            lambda: mh.mhla_output(a, b_, c, St, Wd, o, causal=w.causal),
        ]

    for i in range(args.warmup):
        for f in chain(i):
            f()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    # A pre-roll of device fills keeps the GPU busy while the host enqueues the timed
    # chains, so no host launch gap falls between two events.  `pre_done` still pending
    # once everything is enqueued shows that the GPU never waited for the host.
    for _ in range(8 * args.steps):
        preroll.sum()
    pre_done = torch.cuda.Event()
    pre_done.record(stream)
    for it in range(args.steps):
        evs[it][0].record(stream)
        for j, f in enumerate(chain(args.warmup + it)):
            f()
            evs[it][j + 1].record(stream)
    gapless = not pre_done.query()
    torch.cuda.synchronize()
    del preroll
    kms = {name: sum(evs[it][j].elapsed_time(evs[it][j + 1]) for it in range(args.steps)) / args.steps
           for j, name in enumerate(names)}
    kb = kernel_bytes(w)

    def entry(name, t_ms):
        return {"ms": round(t_ms, 5), "bytes": kb[name], "GBps": round(kb[name] / (t_ms * 1e-3) / 1e9, 1),
                "hbm_frac": round(kb[name] / (t_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}

    staged = {n: entry(n, kms[n]) for n in names}
    # The mixing GEMM also against the MFMA roofline: model FLOPs, and the bf16 MFMA work
    # executed (hi/lo products) as a fraction of the dense bf16 peak.
    mf_model, mf_exec = mix_flops(w)
    t_mix = kms["mix"] * 1e-3
    staged["mix"]["model_TFLOPs"] = round(mf_model / t_mix / 1e12, 2)
    if w.dtype == "bf16":
        staged["mix"]["mfma_TFLOPs"] = round(mf_exec / t_mix / 1e12, 2)
        staged["mix"]["mfma_frac"] = round(mf_exec / t_mix / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
    if path in (mh.MHLA_PATH_FUSED, mh.MHLA_PATH_PAIR):
        # the step is one kernel: its duration is the step's
        one = PATH_NAMES[path]
        kms[one] = ms
        kernels = {one: entry(one, ms)}
        dom = one
    else:
        kernels = staged
        dom = max(names, key=lambda n: kms[n])
    achieved = kb[dom] / (kms[dom] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(w.key, dom)}

    # Device-copy bandwidth on this GPU (2^28 floats = 1 GiB read and 1 GiB written, far
    # larger than the caches): the practical ceiling of streaming kernels, reported next to
    # the 8 TB/s datasheet figure that `frac` uses.
    csrc = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
    cdst = torch.empty_like(csrc)
    cdst.copy_(csrc)
    copy_ms = elapsed_ms(lambda: [cdst.copy_(csrc) for _ in range(5)]) / 5
    del csrc, cdst
    copy_gbs = 2 * (1 << 30) / (copy_ms * 1e-3) / 1e9
    roofline["copy_GBps"] = round(copy_gbs, 1)
    roofline["copy_frac"] = round(achieved / copy_gbs, 4)

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, q, k, v, W, args.cpu_budget)

    line = {
        "metric": METRIC,
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "timing": "K back-to-back calls rotating over copies of the inputs and outputs that together "
                  "exceed twice the Infinity Cache (each call reads from HBM)",
        "buffer_sets": nbuf,
        "host_gaps": not steps_gapless,
        "warm": warm,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.key, "description": w.description, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "M": w.M, "causal": w.causal, "global_batch": w.B, "seq_len": w.N, "parallelism": "none (1 GPU)"},
        "tflops": round(tflops, 3),
        "path": PATH_NAMES[path],
        "kernels": kernels,
        "staged_kernels": staged,
        "stage_timing": "K chains over the rotating buffer sets; "
                        + ("no host gaps" if gapless else "host gaps possible"),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
