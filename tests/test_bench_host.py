"""Host-side parts of bench.py (no GPU): the one-GPU rule of its command line and the
algorithmic byte counts its roofline figures divide by."""
import os
import subprocess
import sys

import bench
from token_level_head_amd.workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
    assert not r.stdout.strip().startswith("{")  # no result line


def test_fused_bytes_of_the_dit_workload():
    # DiT-S/2 at 256x256: 64 images x 6 heads x 256 tokens x 64 features.  Q, K, V are read
    # once as bf16 (2 bytes), Y written once as float32, W (16 x 16 float32) read once.
    elems = 64 * 6 * 256 * 64
    assert elems == 6291456
    expect = 3 * elems * 2 + elems * 4 + 16 * 16 * 4
    assert expect == 62915584
    assert bench.kernel_bytes(WORKLOADS["dit_s2_256"])["fused"] == expect


def test_staged_bytes_of_the_long_dit_workload():
    # DiT-S/2 at 4096x4096: one image, 6 heads, 65536 tokens, d = 64, 256 blocks.
    # Summaries: 256 blocks x 6 pairs x (64*64 + 64) float32 = 25,559,040 bytes.
    tok = 6 * 65536 * 64 * 2          # one bf16 token tensor
    summ = 256 * 6 * 4160 * 4
    assert summ == 25559040
    b = bench.kernel_bytes(WORKLOADS["dit_s2_4096"])
    assert b["summaries"] == 2 * tok + summ        # K, V in; S out
    assert b["mix"] == 2 * summ + 256 * 256 * 4    # S in, S~ out, W in
    assert b["output"] == tok + summ + 2 * tok     # Q, S~ in; float32 Y out (twice the bf16 size)


def test_default_workload_is_the_largest_single_gpu_config():
    src = open(os.path.join(ROOT, "bench.py")).read()
    assert 'default="sana_128"' in src
    by_bytes = max((w for w in WORKLOADS.values() if w.dtype == "bf16"),
                   key=lambda w: 3 * w.B * w.H * w.N * w.d * 2 + w.B * w.H * w.N * w.d * 4)
    assert by_bytes.key == "sana_128"


def test_staged_bytes_of_the_sana_workload():
    # 4 images x 70 heads x 16384 tokens x 32 features; 64 blocks of 256 tokens.
    tok = 4 * 70 * 16384 * 32 * 2      # one bf16 token tensor: 293,601,280 bytes
    assert tok == 293601280
    summ = 64 * 280 * (32 * 32 + 32) * 4
    assert summ == 75694080
    b = bench.kernel_bytes(WORKLOADS["sana_128"])
    assert b["summaries"] == 2 * tok + summ
    assert b["mix"] == 2 * summ + 64 * 64 * 4
    assert b["output"] == tok + summ + 2 * tok


def test_cpu_baseline_reports_host_and_both_samples():
    from token_level_head_amd.workloads import make_inputs

    w = WORKLOADS["sana_128"].shrink(B=1, H=3, N=1024, M=4)
    q, k, v, W = make_inputs(w)
    cb = bench.cpu_baseline(w, q, k, v, W, 0.05)
    assert cb["kind"] == "oracle" and cb["unit"] == "tokens/s" and cb["value"] > 0
    assert 1 <= cb["cores"] <= 16 and cb["single_thread"]["cores"] == 1 and cb["single_thread"]["value"] > 0
    assert cb["host"]["nproc"] >= 1 and cb["host"]["cpu_model"]


def test_pair_bytes_of_the_dit_512_workload():
    # 64 images x 6 heads x 1024 tokens x 64 features, 16 blocks of 64 tokens: the
    # per-pair kernel reads Q, K, V once and writes the float32 Y once.
    tok = 64 * 6 * 1024 * 64 * 2       # one bf16 token tensor: 50,331,648 bytes
    assert tok == 50331648
    b = bench.kernel_bytes(WORKLOADS["dit_s2_512"])
    assert b["pair"] == 3 * tok + 2 * tok + 16 * 16 * 4
