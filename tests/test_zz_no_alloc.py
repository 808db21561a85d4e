"""mhla_forward_noalloc (the entry point for callers that cannot allocate device memory)
against mhla_forward, through the C ABI: the same kernels on the same inputs, so the
outputs must be bit-identical.  Several calls in a row, each smaller than the one
before (the scratch array keeps the previous call's contents), covering the staged
path's workspace parts: summary arrays, the split-W fragments (256 < M <= 1024) and
the partial summaries of long blocks; plus a fused-path shape (no workspace) and a
size whose workspace exceeds the scratch array (refused, nothing written)."""
import ctypes

import pytest
import torch

import token_level_head_amd as mh

pytestmark = pytest.mark.gpu


def inputs(B, H, N, d, M, causal, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    q, k, v = (torch.randn((B, H, N, d), generator=g, device="cuda").to(torch.bfloat16) for _ in range(3))
    W = torch.softmax(torch.randn((M, M), generator=g, device="cuda", dtype=torch.float64), dim=1)
    if causal:
        W = torch.tril(W)
        W = W / W.sum(dim=1, keepdim=True)
    return q, k, v, W.float()


def abi_call(fn, q, k, v, W, out, causal):
    lib = mh.load_library()
    B, H, N, d = q.shape
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return getattr(lib, fn)(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                            ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(W.data_ptr()),
                            ctypes.c_void_p(out.data_ptr()), B, H, N, d, W.shape[0], int(causal), s)


# each smaller (in workspace bytes) than the one before
CASES = [
    (4, 70, 16384, 32, 64, False),   # the SANA-like shape: 151 MB of summaries
    (1, 6, 65536, 64, 256, False),   # the DiT-S/2 4096x4096 shape: 51 MB
    (2, 4, 8192, 64, 64, True),      # causal
    (2, 3, 4096, 16, 512, False),    # 256 < M <= 1024: split-W fragments in the scratch array
    (1, 2, 65536, 32, 1, False),     # global linear attention: long blocks cut into segments
    (4, 6, 256, 64, 16, False),      # fused path: no workspace
]


def test_noalloc_matches_forward_on_consecutive_calls():
    sizes = [mh.mhla_workspace_bytes(B, H, N, d, M, int(c)) for (B, H, N, d, M, c) in CASES[:-1]]
    assert sizes == sorted(sizes, reverse=True) and sizes[0] <= mh.MHLA_NOALLOC_SCRATCH_BYTES
    for i, (B, H, N, d, M, causal) in enumerate(CASES):
        print(f"noalloc case {i}: B={B} H={H} N={N} d={d} M={M} causal={causal}", flush=True)
        q, k, v, W = inputs(B, H, N, d, M, causal, 100 + i)
        ref = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
        out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
        assert abi_call("mhla_forward", q, k, v, W, ref, causal) == mh.MHLA_OK
        assert abi_call("mhla_forward_noalloc", q, k, v, W, out, causal) == mh.MHLA_OK, mh.mhla_last_error()
        torch.cuda.synchronize()
        assert torch.isfinite(ref).all()
        assert torch.equal(out, ref), f"case {i}: max diff {(out - ref).abs().max().item()}"
        # and once more on the same inputs (the scratch array now holds this call's data)
        out2 = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
        assert abi_call("mhla_forward_noalloc", q, k, v, W, out2, causal) == mh.MHLA_OK
        torch.cuda.synchronize()
        assert torch.equal(out2, ref)


def test_noalloc_refuses_workspace_beyond_the_scratch_array():
    # causal LM shape: 2 * 64 * 128 * (64*64 + 64) * 4 bytes = 273 MB > 256 MiB
    B, H, N, d, M = 8, 16, 8192, 64, 64
    assert mh.mhla_workspace_bytes(B, H, N, d, M, 1) > mh.MHLA_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    W = torch.tril(torch.ones((M, M), device="cuda"))
    out = torch.full(q.shape, 7.0, dtype=torch.float32, device="cuda")
    assert abi_call("mhla_forward_noalloc", q, q, q, W, out, True) == mh.MHLA_ERR_UNSUPPORTED
    assert "scratch" in mh.mhla_last_error()
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    with pytest.raises(mh.MhlaError):
        mh.mhla_forward_noalloc(q, q, q, W, out, causal=True)
