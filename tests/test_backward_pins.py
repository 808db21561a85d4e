"""Pins for the backward oracle (oracle/backward.py), CPU only.

The gradients are checked against central finite differences of the explicit
O(N^2) definition in oracle/bruteforce.py (independent of both the backward
code and the linear-time oracle), element by element for q, k, v and W, on tiny
shapes covering several blocks, one block, one token per block and the causal
form; and against the degree-0 homogeneity of Y in each row of W
("MHLA: Restoring Expressivity of Linear Attention via Token-Level
Multi-Head", §4.1: the ratio cancels a positive row scale), which makes
sum_b W[i,b] dW[i,b] vanish up to the 1e-6 guard.
"""
import numpy as np
import pytest

from oracle import bruteforce
from oracle.backward import backward
from token_level_head_amd.workloads import WORKLOADS, make_inputs

SHAPES = [  # (B, H, N, d, M, causal)
    (1, 2, 8, 4, 2, False),
    (1, 2, 8, 4, 2, True),
    (1, 1, 12, 4, 3, True),
    (2, 1, 6, 3, 6, False),   # one token per block
    (1, 1, 6, 3, 6, True),
    (1, 1, 8, 4, 1, True),    # one block: the plain recurrence
    (1, 1, 8, 4, 1, False),
]


def _case(shape, seed):
    B, H, N, d, M, causal = shape
    w = WORKLOADS["tiny_f32"].shrink(B=B, H=H, N=N, d=d, M=M, causal=causal, seed=seed)
    q, k, v, W = (np.asarray(a, dtype=np.float64) for a in make_inputs(w))
    dy = np.random.default_rng(seed + 1).standard_normal(q.shape)
    return q, k, v, W, dy


def _loss(q, k, v, W, dy, causal, normalize=True):
    return float(np.sum(dy * bruteforce.forward(q, k, v, W, causal=causal, normalize=normalize)))


def _fd(q, k, v, W, dy, causal, h=1e-5, normalize=True):
    args = [q, k, v, W]
    grads = []
    for a in range(4):
        g = np.zeros_like(args[a])
        for idx in np.ndindex(args[a].shape):
            plus = [x.copy() for x in args]
            minus = [x.copy() for x in args]
            plus[a][idx] += h
            minus[a][idx] -= h
            g[idx] = (_loss(*plus, dy, causal, normalize) - _loss(*minus, dy, causal, normalize)) / (2 * h)
        grads.append(g)
    return grads


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}H{}N{}d{}M{}{}".format(*s[:5], "c" if s[5] else ""))
def test_backward_matches_finite_differences(shape):
    q, k, v, W, dy = _case(shape, 7000 + SHAPES.index(shape))
    causal = shape[5]
    got = backward(q, k, v, W, dy, causal=causal)
    ref = _fd(q, k, v, W, dy, causal)
    for name, g, r in zip(("dq", "dk", "dv", "dW"), got, ref):
        # central differences with h = 1e-5 carry ~1e-11 absolute error; with one
        # block dW is itself ~1e-7 (it acts only through the guard)
        assert np.max(np.abs(g - r)) <= 1e-7 * np.max(np.abs(r)) + 1e-9, name
    if causal:  # entries above the diagonal are never read
        assert np.all(np.triu(got[3], 1) == 0)


def test_backward_row_homogeneity():
    q, k, v, W, dy = _case((2, 2, 32, 8, 4, False), 7100)
    dW = backward(q, k, v, W, dy)[3]
    for i in range(W.shape[0]):
        assert abs(np.dot(W[i], dW[i])) < 1e-5 * np.max(np.abs(dW))


@pytest.mark.parametrize("shape", SHAPES[:5], ids=lambda s: "B{}H{}N{}d{}M{}{}".format(*s[:5], "c" if s[5] else ""))
def test_backward_without_normaliser_matches_finite_differences(shape):
    # the form without the normaliser (MHLA §4.1, remark on the output): y = A V
    q, k, v, W, dy = _case(shape, 7200 + SHAPES.index(shape))
    causal = shape[5]
    got = backward(q, k, v, W, dy, causal=causal, normalize=False)
    ref = _fd(q, k, v, W, dy, causal, normalize=False)
    for name, g, r in zip(("dq", "dk", "dv", "dW"), got, ref):
        assert np.max(np.abs(g - r)) <= 1e-7 * np.max(np.abs(r)) + 1e-9, name


def test_backward_without_normaliser_dv_is_a_transpose_product():
    # y = A V is linear in V, so dv = A^T dy exactly, with A the explicit matrix of
    # MHLA §4.2 Eq. 5 (brute force, independent of the backward code)
    q, k, v, W, dy = _case((1, 2, 12, 4, 3, False), 7300)
    dv = backward(q, k, v, W, dy, normalize=False)[2]
    M, N = W.shape[0], q.shape[2]
    blk = np.arange(N) * M // N
    for h in range(q.shape[1]):
        A = W[np.ix_(blk, blk)] * (bruteforce.phi(q[0, h]) @ bruteforce.phi(k[0, h]).T)
        assert np.allclose(dv[0, h], A.T @ dy[0, h], rtol=1e-12, atol=1e-12)
