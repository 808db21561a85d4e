"""The backward pins catch planted mistakes (CPU only).

Each mutant changes one site of oracle/backward.py (a sign, a dropped term, an
off-by-one causal range, a transposed product, a missing phi') in a copy that is
executed in memory; the finite-difference and homogeneity pins must reject it.
"""
import os
import types

import pytest

import test_backward_pins as pins

SRC = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "backward.py")).read()

MUTANTS = [
    ("dden = -(dY[t] @ y) / den", "dden = (dY[t] @ y) / den"),
    ("dfq[bb, hh, t] += A @ dnum + dden * a", "dfq[bb, hh, t] += A @ dnum"),
    ("dfq[bb, hh, t] += A @ dnum + dden * a", "dfq[bb, hh, t] += A.T @ dnum + dden * a"),
    ("for j in range(i * C, t + 1):", "for j in range(i * C, t):"),
    ("dW[i, b] += np.sum(dSt[i] * S[b]) + dzt[i] @ z[b]", "dW[i, b] += np.sum(dSt[i] * S[b])"),
    ("dW[i, b] += np.sum(dSt[i] * S[b]) + dzt[i] @ z[b]", "dW[b, i] += np.sum(dSt[i] * S[b]) + dzt[i] @ z[b]"),
    ("users = range(b + 1, M) if causal else range(M)", "users = range(b, M) if causal else range(M)"),
    ("dv[bb, hh, j] += dS.T @ Fk[j]", "dv[bb, hh, j] += dS @ Fk[j]"),
    ("return dfq * dphi(q), dfk * dphi(k), dv, dW", "return dfq * dphi(q), dfk, dv, dW"),
    ("dW[i, i] += np.sum(dA * P) + da @ p", "dW[i, i] += np.sum(dA * P)"),
    ("dfk[bb, hh, j] += W[i, i] * (dA @ V[j] + da)", "dfk[bb, hh, j] += W[i, i] * dA @ V[j]"),
    ("dnum = dY[t] / den", "dnum = dY[t]"),
    # the form without the normaliser
    ("                        dnum = dY[t]\n                        dden = 0.0",
     "                        dnum = dY[t]\n                        dden = -(dY[t] @ num)"),
    ("                        dnum = dY[t]\n                        dden = 0.0",
     "                        dnum = dY[t] / (Fq[t] @ a + EPS)\n                        dden = 0.0"),
]


@pytest.mark.parametrize("mut", MUTANTS, ids=lambda m: m[1][:40])
def test_mutant_is_caught(mut, monkeypatch):
    old, new = mut
    assert old in SRC
    mod = types.ModuleType("oracle.backward_mutant")
    mod.__package__ = "oracle"
    exec(compile(SRC.replace(old, new), "backward_mutant", "exec"), mod.__dict__)
    monkeypatch.setattr(pins, "backward", mod.backward)
    with pytest.raises(AssertionError):
        for shape in pins.SHAPES:
            pins.test_backward_matches_finite_differences(shape)
        pins.test_backward_row_homogeneity()
        for shape in pins.SHAPES[:5]:
            pins.test_backward_without_normaliser_matches_finite_differences(shape)
        pins.test_backward_without_normaliser_dv_is_a_transpose_product()
