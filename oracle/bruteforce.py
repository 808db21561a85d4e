"""The plain O(N^2) definition of the MHLA forward pass -- TEST INFRASTRUCTURE ONLY.

"MHLA: Restoring Expressivity of Linear Attention via Token-Level Multi-Head",
§4.2 (token-level effect of multi-head mixing, Eq. 5) and App. B, writes the
mixed numerator for a query from block i as a sum over every token t:

    phi(q)^T S~_i = sum_t m_{i,b(t)} (phi(q)^T phi(k_t)) v_t^T

and §4.1 divides it by the same weights summed without v_t.  That is ordinary
normalised attention (§3.1, the Sim-weighted average over tokens) with the
explicit weight

    A[t, j] = M_c[b(t), b(j)] * (phi(q_t) . phi(k_j)),

restricted to j <= t for the causal variant (App. C masks the future), and with
the 1e-6 guard of "Linear Attention 笔记" §4/§5 added to the row sum.  This
module builds that matrix explicitly in NumPy binary64 and applies it to V.
It does not use block summaries, so it checks the linear-time oracle in
``mhla_oracle.c`` from an independent direction.
"""
import numpy as np

EPS = 1e-6


def phi(x):
    """ELU(x) + 1 ("Linear Attention 笔记" §2), evaluated in binary64."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def contiguous_blocks(N, M):
    """b(t) for M equal contiguous blocks (block b = tokens [b*C, (b+1)*C))."""
    if N % M:
        raise ValueError("N must be a multiple of M")
    return np.arange(N) // (N // M)


def weight_matrix(q, k, W, blk, causal, rows=None):
    """Explicit A[t, j] for one (batch, head): q, k [N, d]; returns [len(rows), N]."""
    N = k.shape[0]
    rows = np.arange(N) if rows is None else np.asarray(rows)
    sim = phi(q[rows]) @ phi(k).T                       # phi(q_t) . phi(k_j)
    mix = np.asarray(W, dtype=np.float64)[blk[rows]][:, blk]  # M_c[b(t), b(j)]
    if causal:
        allowed = np.arange(N)[None, :] <= rows[:, None]
        # where() rather than a product, so unused (masked) W entries never leak in
        return np.where(allowed, mix * sim, 0.0)
    return mix * sim


def forward(q, k, v, W, causal=False, blk=None, rows=None, normalize=True):
    """Y for q, k, v [B, H, N, d] (any float dtype) and W [M, M] (or [H, M, M]: head h
    mixes with W[h]).

    ``blk`` gives each token's block (default: contiguous equal blocks); ``rows``
    restricts the output to those token indices (same for every (batch, head)).
    ``normalize=False`` returns A V itself, without the row normalisation (the form
    §4.1 of the MHLA page allows for long sequences).  Returns binary64
    [B, H, len(rows), d].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    W = np.asarray(W)
    M = W.shape[-1]
    blk = contiguous_blocks(N, M) if blk is None else np.asarray(blk)
    nrows = N if rows is None else len(rows)
    out = np.empty((B, H, nrows, d), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            A = weight_matrix(q[b, h], k[b, h], W[h] if W.ndim == 3 else W, blk, causal, rows)
            out[b, h] = (A @ v[b, h]) / (A.sum(axis=1, keepdims=True) + EPS) if normalize else A @ v[b, h]
    return out
