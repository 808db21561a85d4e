"""Gradients of the MHLA forward pass -- TEST INFRASTRUCTURE ONLY.

The method is trained end to end, coefficient matrix M_c included ("MHLA:
Restoring Expressivity of Linear Attention via Token-Level Multi-Head", §4.2:
M_c is a learnable parameter).  This module gives, in NumPy binary64, the
gradients of L = sum(dY * Y) with respect to q, k, v and W, written by the
chain rule through the four steps of §4.1 (and App. C's causal form):

    num_t = phi(q_t) A_t,   den_t = phi(q_t) . a_t + 1e-6,   y_t = num_t / den_t
    A_t = S~_i (+ W[i,i] P_t causal),   a_t = z~_i (+ W[i,i] p_t causal)

so that, with dnum_t = dy_t / den_t and dden_t = -(dy_t . y_t) / den_t (without the
normaliser, y_t = num_t: dnum_t = dy_t and dden_t = 0),

    d phi(q_t) = A_t dnum_t + dden_t a_t
    dS~_i      = sum_{t in i} phi(q_t) dnum_t^T,   dz~_i = sum_{t in i} dden_t phi(q_t)
    dS_b       = sum_i W[i,b] dS~_i,               dz_b  = sum_i W[i,b] dz~_i
    dW[i,b]   += <dS~_i, S_b> + dz~_i . z_b        (summed over batch and heads)
    d phi(k_j) = dS_b v_j + dz_b,   dv_j = dS_b^T phi(k_j)     (j in block b)

plus, in the causal form, the within-block running summary P_t, p_t of block i
(dP_t = W[i,i] phi(q_t) dnum_t^T, dp_t = W[i,i] dden_t phi(q_t) reach every
key j <= t of the block, and dW[i,i] += <phi(q_t) dnum_t^T, P_t> + dden_t
phi(q_t) . p_t).  Finally dq = d phi(q) * phi'(q) and dk = d phi(k) * phi'(k)
with phi'(x) = 1 for x > 0 and exp(x) otherwise.  Plain loops over pairs,
blocks and tokens, no fusion: slow and meant to be read against the formulas.
"""
import numpy as np

from .bruteforce import EPS, phi


def dphi(x):
    """Derivative of ELU(x) + 1: 1 for x > 0, exp(x) otherwise."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))


def backward(q, k, v, W, dy, causal=False, normalize=True):
    """(dq, dk, dv, dW) of sum(dy * forward(q, k, v, W)) in binary64.

    q, k, v, dy: [B, H, N, d]; W: [M, M] (causal: entries above the diagonal are
    never used and get zero gradient); blocks are contiguous, C = N / M.
    normalize=False differentiates the form without the normaliser (MHLA §4.1,
    remark on the output), y_t = num_t: then dnum_t = dy_t and the den terms vanish.
    """
    q, k, v, dy = (np.asarray(a, dtype=np.float64) for a in (q, k, v, dy))
    W = np.asarray(W, dtype=np.float64)
    B, H, N, d = q.shape
    M = W.shape[0]
    C = N // M
    fq, fk = phi(q), phi(k)
    dfq = np.zeros_like(q)
    dfk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dW = np.zeros_like(W)
    for bb in range(B):
        for hh in range(H):
            Fq, Fk, V, dY = fq[bb, hh], fk[bb, hh], v[bb, hh], dy[bb, hh]
            S = np.zeros((M, d, d))
            z = np.zeros((M, d))
            for b in range(M):
                for j in range(b * C, (b + 1) * C):
                    S[b] += np.outer(Fk[j], V[j])
                    z[b] += Fk[j]
            dSt = np.zeros((M, d, d))
            dzt = np.zeros((M, d))
            for i in range(M):
                src = range(i) if causal else range(M)
                St = sum((W[i, b] * S[b] for b in src), np.zeros((d, d)))
                zt = sum((W[i, b] * z[b] for b in src), np.zeros(d))
                P = np.zeros((d, d))
                p = np.zeros(d)
                for t in range(i * C, (i + 1) * C):
                    if causal:  # running summary of block i, inclusive of t
                        P = P + np.outer(Fk[t], V[t])
                        p = p + Fk[t]
                        A, a = St + W[i, i] * P, zt + W[i, i] * p
                    else:
                        A, a = St, zt
                    num = Fq[t] @ A
                    if normalize:
                        den = Fq[t] @ a + EPS
                        y = num / den
                        dnum = dY[t] / den
                        dden = -(dY[t] @ y) / den
                    else:
                        dnum = dY[t]
                        dden = 0.0
                    dfq[bb, hh, t] += A @ dnum + dden * a
                    dA = np.outer(Fq[t], dnum)
                    da = dden * Fq[t]
                    dSt[i] += dA
                    dzt[i] += da
                    if causal:
                        dW[i, i] += np.sum(dA * P) + da @ p
                        for j in range(i * C, t + 1):  # keys j <= t of block i, through P_t and p_t
                            dfk[bb, hh, j] += W[i, i] * (dA @ V[j] + da)
                            dv[bb, hh, j] += W[i, i] * (dA.T @ Fk[j])
            for i in range(M):
                for b in (range(i) if causal else range(M)):
                    dW[i, b] += np.sum(dSt[i] * S[b]) + dzt[i] @ z[b]
            for b in range(M):
                users = range(b + 1, M) if causal else range(M)
                dS = sum((W[i, b] * dSt[i] for i in users), np.zeros((d, d)))
                dz = sum((W[i, b] * dzt[i] for i in users), np.zeros(d))
                for j in range(b * C, (b + 1) * C):
                    dfk[bb, hh, j] += dS @ V[j] + dz
                    dv[bb, hh, j] += dS.T @ Fk[j]
    return dfq * dphi(q), dfk * dphi(k), dv, dW
