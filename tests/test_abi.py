"""The C ABI on the host: exported symbols, argument validation, host helpers.

No GPU is needed: every call here either fails validation before any HIP call
or is a host-only function.
"""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import token_level_head_amd as mh
from token_level_head_amd.binding import SIGNATURES

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "mhla.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mhla_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_bound_api():
    assert header_functions() == sorted(SIGNATURES)


def test_library_exports_every_declared_symbol(mhla_lib):
    for name in header_functions():
        assert hasattr(mhla_lib, name), name


def test_version_and_sizes(mhla_lib):
    assert mh.mhla_version().startswith("mhla-gfx950")
    for d in (16, 32, 64):
        assert mh.mhla_summary_floats(d) == d * d + d
    # two summary arrays, plus the split-W fragments (4 * M * M bytes) when 256 < M <= 1024
    assert mh.mhla_workspace_bytes(64, 6, 256, 64, 16) == 2 * 16 * 384 * (64 * 64 + 64) * 4
    assert mh.mhla_workspace_bytes(8, 16, 8192, 64, 64, 1) == 2 * 64 * 128 * (64 * 64 + 64) * 4
    assert mh.mhla_workspace_bytes(1, 6, 65536, 64, 256) == 2 * 256 * 6 * (64 * 64 + 64) * 4
    assert mh.mhla_workspace_bytes(1, 1, 512 * 16, 16, 512) == 2 * 512 * (16 * 16 + 16) * 4 + 4 * 512 * 512
    # global linear attention over 65536 tokens on 24 pairs: each block is cut into 43 segments
    # of 1536 tokens whose partial summaries are part of the workspace
    L = 64 * 64 + 64
    assert mh.mhla_workspace_bytes(4, 6, 65536, 64, 1) == 2 * 24 * L * 4 + 43 * 24 * L * 4
    assert mh.mhla_workspace_bytes(1, 1, 250, 64, 16) == -1
    assert mh.mhla_workspace_bytes(1, 1, 256, 24, 16) == -1


FAKE = 1 << 20  # a 16-byte-aligned nonzero address; never dereferenced (validation fails first)


def test_forward_ex_validation(mhla_lib):
    p = [FAKE, FAKE * 2, FAKE * 3]

    def call(dtype=0, opts=0, W=FAKE * 4, out=FAKE * 5, B=1, H=1, N=256, d=16, M=4):
        return mhla_lib.mhla_forward_ex(*p, dtype, W, out, B, H, N, d, M, opts, None)

    assert call(opts=1 << 7) == mh.MHLA_ERR_INVALID_ARG
    assert "option" in mh.mhla_last_error()
    assert call(dtype=5) == mh.MHLA_ERR_INVALID_ARG
    assert call(N=250) == mh.MHLA_ERR_INVALID_ARG
    # a float32 output of B*H*N*d*4 bytes reaches W placed half-way along it
    assert call(W=FAKE * 5 + 256 * 16 * 2, out=FAKE * 5) == mh.MHLA_ERR_INVALID_ARG
    assert "overlap" in mh.mhla_last_error()
    # per-head W spans H * M * M floats: an output right after the first head's matrix overlaps
    assert call(W=FAKE * 5, out=FAKE * 5 + 4 * 4 * 4, H=2, opts=mh.MHLA_OPT_W_PER_HEAD) == mh.MHLA_ERR_INVALID_ARG


def test_forward_blocks_validation(mhla_lib):
    p = [FAKE, FAKE * 2, FAKE * 3]
    order, offsets = FAKE * 6, FAKE * 7

    def call(order=order, offsets=offsets, max_block=64, opts=0, N=250, M=4):
        return mhla_lib.mhla_forward_blocks(*p, 0, FAKE * 4, FAKE * 5, 1, 1, N, 16, M, order, offsets,
                                            max_block, opts, None)

    assert call(order=None) == mh.MHLA_ERR_INVALID_ARG
    assert call(offsets=None) == mh.MHLA_ERR_INVALID_ARG
    assert call(order=FAKE * 6 + 2) == mh.MHLA_ERR_INVALID_ARG
    assert "aligned" in mh.mhla_last_error()
    assert call(max_block=0) == mh.MHLA_ERR_INVALID_ARG
    assert call(max_block=251) == mh.MHLA_ERR_INVALID_ARG
    assert call(opts=mh.MHLA_OPT_CAUSAL) == mh.MHLA_ERR_UNSUPPORTED
    assert call(opts=1 << 9) == mh.MHLA_ERR_INVALID_ARG


@pytest.mark.parametrize("fn", ["mhla_forward", "mhla_forward_f32"])
def test_forward_validation(mhla_lib, fn):
    f = getattr(mhla_lib, fn)
    p = [FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5]

    def call(ptrs=p, B=1, H=1, N=256, d=16, M=4):
        return f(*ptrs, B, H, N, d, M, 0, None)

    assert call(ptrs=[None] + p[1:]) == mh.MHLA_ERR_INVALID_ARG
    assert "q is NULL" in mh.mhla_last_error()
    assert call(ptrs=p[:4] + [None]) == mh.MHLA_ERR_INVALID_ARG
    assert call(ptrs=[FAKE + 2] + p[1:]) == mh.MHLA_ERR_INVALID_ARG
    assert "aligned" in mh.mhla_last_error()
    assert call(N=250) == mh.MHLA_ERR_INVALID_ARG
    assert "multiple" in mh.mhla_last_error()
    assert call(B=0) == mh.MHLA_ERR_INVALID_ARG
    assert call(M=0) == mh.MHLA_ERR_INVALID_ARG
    assert call(d=24) == mh.MHLA_ERR_UNSUPPORTED
    assert call(d=128) == mh.MHLA_ERR_UNSUPPORTED
    assert call(B=1 << 30, H=1 << 30) == mh.MHLA_ERR_INVALID_ARG
    assert call(N=1 << 25, d=64, M=1) == mh.MHLA_ERR_UNSUPPORTED  # N*d beyond 32-bit pair offsets
    # out overlapping q
    assert call(ptrs=[FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE + 64]) == mh.MHLA_ERR_INVALID_ARG
    assert "overlap" in mh.mhla_last_error()


def test_stage_validation(mhla_lib):
    assert mhla_lib.mhla_block_summaries(FAKE, FAKE * 2, 7, FAKE * 3, 1, 1, 256, 16, 4, None) == mh.MHLA_ERR_INVALID_ARG
    assert mhla_lib.mhla_block_summaries(None, FAKE * 2, 0, FAKE * 3, 1, 1, 256, 16, 4, None) == mh.MHLA_ERR_INVALID_ARG
    assert mhla_lib.mhla_mix_summaries(FAKE, FAKE * 2, FAKE, 1, 16, 4, 0, 0, None) == mh.MHLA_ERR_INVALID_ARG
    assert mhla_lib.mhla_mix_summaries(FAKE, FAKE * 2, FAKE * 3, 1, 48, 4, 0, 0, None) == mh.MHLA_ERR_UNSUPPORTED
    # the causal output reads k, v and W; the non-causal one does not need them
    assert mhla_lib.mhla_output(FAKE, None, None, 0, FAKE * 2, None, FAKE * 3, 1, 1, 256, 16, 4, 1, None) == \
        mh.MHLA_ERR_INVALID_ARG


def test_decode_validation(mhla_lib):
    # state: (M + 1) summary vectors and one more normaliser per pair
    assert mh.mhla_decode_state_bytes(8, 16, 64, 64) == (65 * (64 * 64 + 64) + 64) * 8 * 16 * 4
    assert mh.mhla_decode_state_bytes(1, 1, 24, 4) == -1
    f = mhla_lib.mhla_decode_step
    p = [FAKE, FAKE * 2, FAKE * 3]

    def call(q=FAKE, k=FAKE * 2, v=FAKE * 3, dtype=0, W=FAKE * 4, state=FAKE * 8, out=FAKE * 16,
             B=1, H=1, d=16, M=4, C=16, t=0):
        return f(q, k, v, dtype, W, state, out, B, H, d, M, C, t, None)

    assert call(q=None) == mh.MHLA_ERR_INVALID_ARG
    assert call(state=None) == mh.MHLA_ERR_INVALID_ARG
    assert "state is NULL" in mh.mhla_last_error()
    assert call(out=FAKE + 8) == mh.MHLA_ERR_INVALID_ARG
    assert call(dtype=5) == mh.MHLA_ERR_INVALID_ARG
    assert call(d=48) == mh.MHLA_ERR_UNSUPPORTED
    assert call(C=0) == mh.MHLA_ERR_INVALID_ARG
    assert call(t=-1) == mh.MHLA_ERR_INVALID_ARG
    assert call(t=64) == mh.MHLA_ERR_INVALID_ARG  # block 4 of M = 4
    assert "outside" in mh.mhla_last_error()
    assert call(out=FAKE * 8 + 256) == mh.MHLA_ERR_INVALID_ARG  # out inside the state
    assert call(state=FAKE * 4) == mh.MHLA_ERR_INVALID_ARG  # state on top of W
    assert "overlap" in mh.mhla_last_error()


def test_backward_validation(mhla_lib):
    assert mh.mhla_backward_workspace_bytes(1, 1, 250, 64, 16) == -1
    assert mh.mhla_backward_workspace_bytes(2, 3, 256, 64, 16) > 4 * 16 * 6 * (64 * 64 + 64) * 4
    f = mhla_lib.mhla_backward
    base = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, dtype=0, W=FAKE * 4, dy=FAKE * 5, dq=FAKE * 6, dk=FAKE * 7,
                dv=FAKE * 8, dW=FAKE * 9, B=1, H=1, N=256, d=16, M=4, causal=0)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["q"], a["k"], a["v"], a["dtype"], a["W"], a["dy"], a["dq"], a["dk"], a["dv"], a["dW"],
                 a["B"], a["H"], a["N"], a["d"], a["M"], a["causal"], None)

    assert call(dy=None) == mh.MHLA_ERR_INVALID_ARG
    assert "dy is NULL" in mh.mhla_last_error()
    assert call(dtype=3) == mh.MHLA_ERR_INVALID_ARG
    assert call(d=48) == mh.MHLA_ERR_UNSUPPORTED
    assert call(N=250) == mh.MHLA_ERR_INVALID_ARG
    assert call(dq=FAKE * 5 + 64) == mh.MHLA_ERR_INVALID_ARG  # dq inside dy
    assert call(dk=FAKE * 6 + 16) == mh.MHLA_ERR_INVALID_ARG  # dk inside dq
    assert "overlap" in mh.mhla_last_error()


def test_option_entry_points_validate_options(mhla_lib):
    # host-side rejections before any device work (null pointers are never touched)
    b = mhla_lib.mhla_backward_ex
    args = (FAKE, FAKE * 2, FAKE * 3, 0, FAKE * 4, FAKE * 5, FAKE * 6, FAKE * 7, FAKE * 8, FAKE * 9, 1, 1, 256, 16, 4)
    assert b(*args, mh.MHLA_OPT_OUT_BF16, None) == mh.MHLA_ERR_UNSUPPORTED
    assert b(*args, mh.MHLA_OPT_W_PER_HEAD, None) == mh.MHLA_ERR_UNSUPPORTED
    assert b(*args, 64, None) == mh.MHLA_ERR_INVALID_ARG
    assert "unknown option" in mh.mhla_last_error()
    assert b(*args[:5], None, *args[6:], mh.MHLA_OPT_NO_NORMALIZER, None) == mh.MHLA_ERR_INVALID_ARG  # dy NULL
    dstep = mhla_lib.mhla_decode_step_ex
    dargs = (FAKE, FAKE * 2, FAKE * 3, 0, FAKE * 4, FAKE * 5, FAKE * 6, 1, 1, 16, 4, 8, 0)
    assert dstep(*dargs, mh.MHLA_OPT_OUT_BF16, None) == mh.MHLA_ERR_UNSUPPORTED
    assert dstep(*dargs, 64, None) == mh.MHLA_ERR_INVALID_ARG
    assert dstep(*dargs[:-1], 32, mh.MHLA_OPT_NO_NORMALIZER, None) == mh.MHLA_ERR_INVALID_ARG  # t past M * C


def test_forward_path_selection(mhla_lib):
    # non-causal bf16 with at most 256 tokens in at most 16 blocks: fused; otherwise staged
    assert mh.mhla_forward_path(64, 6, 256, 64, 16) == mh.MHLA_PATH_FUSED
    assert mh.mhla_forward_path(64, 6, 256, 64, 16, causal=True) == mh.MHLA_PATH_STAGED
    assert mh.mhla_forward_path(64, 6, 256, 64, 16, dtype=mh.MHLA_DTYPE_F32) == mh.MHLA_PATH_STAGED
    assert mh.mhla_forward_path(1, 6, 65536, 64, 256) == mh.MHLA_PATH_STAGED   # M > 16
    assert mh.mhla_forward_path(4, 70, 16384, 32, 64) == mh.MHLA_PATH_STAGED   # blocks of 256 tokens
    assert mh.mhla_forward_path(1, 6, 256, 64, 16) == mh.MHLA_PATH_FUSED
    assert mh.mhla_forward_path(256, 1, 64, 16, 64) == mh.MHLA_PATH_STAGED     # M > 16
    assert mh.mhla_forward_path(8, 2, 272, 64, 16) == mh.MHLA_PATH_STAGED      # 17-token blocks
    assert mh.mhla_forward_path(8, 2, 60, 32, 5) == mh.MHLA_PATH_FUSED
    assert mh.mhla_forward_path(8, 2, 256, 64, 1) == mh.MHLA_PATH_FUSED       # one block of 256 tokens
    assert mh.mhla_forward_path(8, 2, 200, 32, 8) == mh.MHLA_PATH_FUSED       # 25-token blocks
    assert mh.mhla_forward_path(8, 2, 512, 64, 16) == mh.MHLA_PATH_STAGED     # N > 256
    assert mh.mhla_forward_path(1, 1, 250, 64, 16) == -1


def test_status_strings(mhla_lib):
    assert mh.mhla_status_string(0) == "MHLA_OK"
    assert mh.mhla_status_string(mh.MHLA_ERR_HIP) == "MHLA_ERR_HIP"
    assert mh.mhla_status_string(12345) == "MHLA_ERR_UNKNOWN"


@pytest.mark.parametrize("d", [16, 32, 64])
def test_unpack_is_a_permutation(mhla_lib, d):
    """The packed summary layout stores every S[r][c] exactly once, then z in order."""
    L = d * d + d
    packed = torch.arange(2 * L, dtype=torch.float32).reshape(2, L)
    S, z = mh.mhla_unpack_summaries(packed, d)
    for u in range(2):
        vals = np.sort(S[u].numpy().ravel())
        assert np.array_equal(vals, np.arange(u * L, u * L + d * d, dtype=np.float32))
        assert np.array_equal(z[u].numpy(), np.arange(u * L + d * d, (u + 1) * L, dtype=np.float32))


def test_unpack_validation(mhla_lib):
    buf = np.zeros(16, dtype=np.float32)
    p = buf.ctypes.data_as(ctypes.c_void_p)
    assert mhla_lib.mhla_unpack_summaries(None, 1, 16, p, p) == mh.MHLA_ERR_INVALID_ARG
    assert mhla_lib.mhla_unpack_summaries(p, 1, 20, p, p) == mh.MHLA_ERR_UNSUPPORTED


def test_no_memory_path_enqueues_nothing(mhla_lib):
    """A failed workspace allocation returns MHLA_ERR_NO_MEMORY before any HIP call (the
    test hook fails the request; no device is touched, so this runs without a GPU)."""
    p = [FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5]
    try:
        mh.mhla_debug_fail_workspace(2)
        # staged shapes (the fused path takes no workspace): C3's block count, and the backward pass
        assert mhla_lib.mhla_forward(*p, 1, 2, 4096, 64, 256, 0, None) == mh.MHLA_ERR_NO_MEMORY
        assert "simulated" in mh.mhla_last_error()
        g = [FAKE * 6, FAKE * 7, FAKE * 8, FAKE * 9]
        assert mhla_lib.mhla_backward(FAKE, FAKE * 2, FAKE * 3, 0, FAKE * 4, FAKE * 5, *g, 1, 1, 256, 16, 4, 0,
                                      None) == mh.MHLA_ERR_NO_MEMORY
        # validation still comes first: a bad argument is reported as such, not as memory
        mh.mhla_debug_fail_workspace(1)
        assert mhla_lib.mhla_forward(*p, 1, 2, 4100, 64, 256, 0, None) == mh.MHLA_ERR_INVALID_ARG
    finally:
        mh.mhla_debug_fail_workspace(0)
