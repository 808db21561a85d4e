"""The Python binding rejects arguments that a raw device address cannot describe
(element type, shape, density, device) before it loads or calls the library.

Host-only: every tensor here is a CPU tensor, and every call must raise before
any library call; the last check of each list is the device check, which a CPU
tensor with the right dtype and shape still fails.
"""
import pytest
import torch

import token_level_head_amd as mh
from token_level_head_amd import binding

bf, f32 = torch.bfloat16, torch.float32
SHAPE = (1, 2, 64, 16)
M = 4


@pytest.fixture(autouse=True)
def no_library_calls(monkeypatch):
    """Any attempt to reach the library fails the test."""
    def refuse(*a, **k):
        raise AssertionError("the binding reached the library with invalid arguments")

    monkeypatch.setattr(binding, "load_library", refuse)


def t(shape=SHAPE, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def W(m=M):
    return torch.ones((m, m), dtype=f32)


def raises(exc, match, fn, *a, **k):
    with pytest.raises(exc, match=match):
        fn(*a, **k)


def test_forward_rejects_mismatched_dtypes():
    raises(TypeError, "q must be bfloat16", mh.mhla_forward, t(dtype=f32), t(), t(), W(), t(dtype=f32))
    raises(TypeError, "k must be bfloat16", mh.mhla_forward, t(), t(dtype=f32), t(), W(), t(dtype=f32))
    raises(TypeError, "W must be float32", mh.mhla_forward, t(), t(), t(), W().to(bf), t(dtype=f32))
    # the common mistake of an output like q: 2-byte elements where the kernel writes 4-byte ones
    raises(TypeError, "out must be float32", mh.mhla_forward, t(), t(), t(), W(), t())
    raises(TypeError, "q must be float32", mh.mhla_forward_f32, t(), t(), t(), W(), t(dtype=f32))
    raises(TypeError, "v must be float32", mh.mhla_forward_f32, t(dtype=f32), t(dtype=f32), t(), W(),
           t(dtype=f32))
    # mhla_forward_ex: q decides the dtype, k and v must follow it
    raises(TypeError, "k must be bfloat16", mh.mhla_forward_ex, t(), t(dtype=f32), t(), W(), t(dtype=f32))
    raises(TypeError, "out must be float32 or bfloat16", mh.mhla_forward_ex, t(), t(), t(), W(),
           t(dtype=torch.float16))
    raises(TypeError, "q must be bfloat16 or float32", mh.mhla_forward_ex, t(dtype=torch.float16),
           t(dtype=torch.float16), t(dtype=torch.float16), W(), t(dtype=f32))


def test_forward_rejects_mismatched_shapes():
    out = t(dtype=f32)
    raises(ValueError, "k must have shape", mh.mhla_forward, t(), t((1, 2, 32, 16)), t(), W(), out)
    raises(ValueError, "out must have shape", mh.mhla_forward, t(), t(), t(), W(), t((1, 2, 32, 16), f32))
    raises(ValueError, r"q must be \[B, H, N, d\]", mh.mhla_forward, t((2, 64, 16)), t((2, 64, 16)),
           t((2, 64, 16)), W(), t((2, 64, 16), f32))
    raises(ValueError, "W must have shape", mh.mhla_forward, t(), t(), t(), torch.ones((4, 5)), out)
    raises(ValueError, r"W must be \[M, M\]", mh.mhla_forward, t(), t(), t(), torch.ones(4), out)
    # a per-head W exists only in the options entry points, and must be [H, M, M]
    raises(ValueError, r"W must be \[M, M\]", mh.mhla_forward, t(), t(), t(), torch.ones((2, 4, 4)), out)
    raises(ValueError, "W must have shape", mh.mhla_forward_ex, t(), t(), t(), torch.ones((3, 4, 4)), out)


def test_forward_rejects_non_dense_views():
    out = t(dtype=f32)
    q = t((1, 2, 16, 64)).transpose(2, 3)  # [1, 2, 64, 16] with swapped strides
    raises(ValueError, "q must be contiguous", mh.mhla_forward, q, t(), t(), W(), out)
    k = t((1, 1, 64, 16)).expand(SHAPE)  # stride 0 over heads
    raises(ValueError, "k must be contiguous", mh.mhla_forward, t(), k, t(), W(), out)
    w = torch.ones((8, 8))[::2, ::2]
    raises(ValueError, "W must be contiguous", mh.mhla_forward, t(), t(), t(), w, out)


def test_forward_rejects_host_tensors():
    # right dtypes and shapes, but host memory: the address would be handed to the GPU
    raises(ValueError, "must be on a GPU", mh.mhla_forward, t(), t(), t(), W(), t(dtype=f32))
    raises(ValueError, "must be on a GPU", mh.mhla_forward_f32, t(dtype=f32), t(dtype=f32), t(dtype=f32), W(),
           t(dtype=f32))
    raises(ValueError, "must be on a GPU", mh.mhla_forward_ex, t(), t(), t(), torch.ones((2, 4, 4)), t())


def test_forward_blocks_checks():
    N = SHAPE[2]
    order, offsets = torch.arange(N, dtype=torch.int32), torch.tensor([0, 16, 32, 48, 64], dtype=torch.int32)
    out = t(dtype=f32)
    raises(TypeError, "order must be int32", mh.mhla_forward_blocks, t(), t(), t(), W(), out, order.long(),
           offsets, 16)
    raises(ValueError, "offsets must have shape", mh.mhla_forward_blocks, t(), t(), t(), W(), out, order,
           offsets[:4], 16)
    raises(ValueError, "order must have shape", mh.mhla_forward_blocks, t(), t(), t(), W(), out, order[:10],
           offsets, 16)
    raises(ValueError, "must be on a GPU", mh.mhla_forward_blocks, t(), t(), t(), W(), out, order, offsets, 16)


def test_stage_checks():
    L = 16 * 16 + 16
    S = torch.zeros(M * 2 * L, dtype=f32)
    raises(ValueError, "S must hold at least", mh.mhla_block_summaries, t(), t(), S[:-1], M)
    raises(TypeError, "S must be float32", mh.mhla_block_summaries, t(), t(), S.to(bf), M)
    raises(TypeError, "v must be bfloat16", mh.mhla_block_summaries, t(), t(dtype=f32), S, M)
    raises(ValueError, "must be on a GPU", mh.mhla_block_summaries, t(), t(), S, M)
    raises(ValueError, "St must hold at least", mh.mhla_mix_summaries, S, W(), S[:10], 2, 16)
    raises(ValueError, "must be on a GPU", mh.mhla_mix_summaries, S, W(), S.clone(), 2, 16)
    raises(TypeError, "out must be float32", mh.mhla_output, t(), None, None, S, W(), t())
    raises(ValueError, "St must hold at least", mh.mhla_output, t(), None, None, S[:5], W(), t(dtype=f32))
    raises(TypeError, "k must be bfloat16", mh.mhla_output, t(), t(dtype=f32), t(), S, W(), t(dtype=f32), causal=True)
    raises(ValueError, "must be on a GPU", mh.mhla_output, t(), None, None, S, W(), t(dtype=f32))


def test_backward_checks():
    g = t(dtype=f32)
    dW = torch.zeros((M, M))
    raises(TypeError, "dy must be float32", mh.mhla_backward, t(), t(), t(), W(), t(), g, g, g, dW)
    raises(ValueError, "dv must have shape", mh.mhla_backward, t(), t(), t(), W(), g, g, g, t((1, 2, 64, 32), f32),
           dW)
    raises(ValueError, "dW must have shape", mh.mhla_backward, t(), t(), t(), W(), g, g, g, g, torch.zeros((4, 3)))
    raises(ValueError, "must be on a GPU", mh.mhla_backward, t(), t(), t(), W(), g, g, g, g, dW)


def test_decode_checks():
    B, H, d = 2, 3, 16
    q = t((B, H, d))
    need = ((M + 1) * (d * d + d) + d) * B * H
    state = torch.zeros(need, dtype=f32)
    out = t((B, H, d), f32)
    raises(ValueError, r"q must be \[B, H, d\]", mh.mhla_decode_step, t(), t(), t(), W(), state, out, 16, 0)
    raises(ValueError, "state must hold at least", mh.mhla_decode_step, q, q, q, W(), state[:-1], out, 16, 0)
    raises(TypeError, "state must be float32", mh.mhla_decode_step, q, q, q, W(), state.to(bf), out, 16, 0)
    raises(ValueError, "out must have shape", mh.mhla_decode_step, q, q, q, W(), state, t((B, H, 32), f32), 16, 0)
    raises(ValueError, "must be on a GPU", mh.mhla_decode_step, q, q, q, W(), state, out, 16, 0)


def test_unpack_checks():
    raises(ValueError, "packed must be", mh.mhla_unpack_summaries, torch.zeros((3, 100)), 16)
    raises(TypeError, "packed must be float32", mh.mhla_unpack_summaries, torch.zeros((3, 272), dtype=bf), 16)


def test_not_a_tensor():
    raises(TypeError, "q must be a torch.Tensor", mh.mhla_forward, [[1.0]], t(), t(), W(), t(dtype=f32))
