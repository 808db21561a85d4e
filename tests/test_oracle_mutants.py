"""Planted mistakes in the oracle must be caught by its pins.

Each mutant is a one-site textual edit of a temporary copy of
``oracle/mhla_oracle.c`` -- a dropped term, a wrong index, a transposed operand,
a wrong mixing range -- compiled on the CPU and run through every pin of
``tests/oracle_pins.py`` in a child process.  The pins must fail for every
mutant and pass for the unmodified copy.  Nothing here touches a GPU.
"""
import os
import shutil
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = os.path.join(ROOT, "tests", "oracle_pins.py")

MUTANTS = {
    "phi_plain_elu": ("return x > 0.0 ? x + 1.0 : exp(x);", "return x > 0.0 ? x : exp(x) - 1.0;"),
    "phi_relu_plus_one": ("return x > 0.0 ? x + 1.0 : exp(x);", "return x > 0.0 ? x + 1.0 : 1.0;"),
    "summary_transposed": ("Sb[r * d + c] += fk[r] * (double)vj[c];", "Sb[c * d + r] += fk[r] * (double)vj[c];"),
    "summary_block_shift": ("const float* kj = k + (p * N + j) * d;",
                            "const float* kj = k + (p * N + (j + C) % N) * d;"),
    "normaliser_weighted_by_v": ("zb[r] += fk[r];", "zb[r] += fk[r] * (double)vj[r];"),
    "mix_transposed_weights": ("const double w = (double)W[i * M + b];", "const double w = (double)W[b * M + i];"),
    "mix_unweighted_normaliser": ("zi[r] += w * zb[r];", "zi[r] += zb[r];"),
    "causal_mix_includes_diagonal": ("const long bend = causal ? i : M;", "const long bend = causal ? i + 1 : M;"),
    "causal_mix_skips_previous": ("const long bend = causal ? i : M;", "const long bend = causal ? (i > 0 ? i - 1 : 0) : M;"),
    "output_wrong_block": ("const double* Si = St + i * d * d;", "const double* Si = St + ((i + 1) % M) * d * d;"),
    "causal_state_not_reset": ("memset(P, 0, sizeof(double) * d * d);", ";"),
    "causal_prefix_unweighted": ("Si[r * d + c] + wii * P[r * d + c]", "Si[r * d + c] + P[r * d + c]"),
    "causal_den_unweighted": ("zi[r] + wii * pz[r]", "zi[r] + pz[r]"),
    "causal_prefix_dropped": ("Si[r * d + c] + wii * P[r * d + c]", "Si[r * d + c]"),
    "eps_dropped": ("den += MHLA_ORACLE_EPS;", "den += 0.0;"),
    "eps_per_block": ("den += MHLA_ORACLE_EPS;", "den += MHLA_ORACLE_EPS * M;"),
    "query_phi_skipped": ("fq[r] = mhla_oracle_phi((double)q[t * d + r]);", "fq[r] = (double)q[t * d + r] + 1.0;"),
    "causal_key_phi_skipped": ("fk[r] = mhla_oracle_phi((double)k[t * d + r]);", "fk[r] = (double)k[t * d + r];"),
    "no_normaliser_ignored": ("out[t * d + c] = normalise ? num / den : num;", "out[t * d + c] = num / den;"),
    "no_normaliser_always": ("out[t * d + c] = normalise ? num / den : num;", "out[t * d + c] = num;"),
    "no_normaliser_option_ignored": ("const int normalise = (options & MHLA_ORACLE_NO_NORMALISER) == 0;",
                                     "const int normalise = 1;"),
    "per_head_by_batch": ("const float* Wp = per_head ? W + (p % H) * M * M : W;",
                          "const float* Wp = per_head ? W + (p / H) * M * M : W;"),
    "per_head_ignored": ("const float* Wp = per_head ? W + (p % H) * M * M : W;", "const float* Wp = W;"),
    "token_list_output_block_shifted": ("const long i = blk[t];", "const long i = blk[(t + 1) % N];"),
    "token_list_summary_contiguous": ("const long b = blk[j];", "const long b = j * M / N;"),
    "token_list_eps_dropped": ("const double guarded = dot + MHLA_ORACLE_EPS;", "const double guarded = dot;"),
    "token_list_normaliser_ignored": ("out[t * d + c] = normalise ? acc / guarded : acc;",
                                      "out[t * d + c] = acc / guarded;"),
    "token_list_option_ignored": ("const int normalise = !(options & MHLA_ORACLE_NO_NORMALISER);",
                                  "const int normalise = 1;"),
    "token_list_per_head_ignored": ("const float* Wq = per_head ? W + (p % H) * M * M : W;", "const float* Wq = W;"),
}


def _build_copy(tmp_path, name, edit):
    work = tmp_path / name
    work.mkdir()
    src = os.path.join(ROOT, "oracle", "mhla_oracle.c")
    text = open(src).read()
    if edit is not None:
        old, new = edit
        assert text.count(old) == 1, f"mutation site for {name} no longer unique in mhla_oracle.c"
        text = text.replace(old, new)
    (work / "mhla_oracle.c").write_text(text)
    shutil.copy(os.path.join(ROOT, "oracle", "mhla_oracle.h"), work / "mhla_oracle.h")
    return oracle.build(src=str(work / "mhla_oracle.c"), out=str(work / "lib.so"), openmp=False)


def _run_pins(lib):
    return subprocess.run([sys.executable, PINS, "--lib", lib], capture_output=True, text=True, timeout=300)


def test_unmodified_copy_passes(tmp_path):
    r = _run_pins(_build_copy(tmp_path, "control", None))
    assert r.returncode == 0, r.stdout + r.stderr


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    r = _run_pins(_build_copy(tmp_path, name, MUTANTS[name]))
    assert r.returncode != 0, f"mutant {name} survived every pin:\n{r.stdout}{r.stderr}"
