"""CPU oracle for the MHLA forward pass -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it, and it
never imports the GPU library: the two share no code.

Two independent implementations live here:

* ``mhla_oracle.c`` (loaded by :class:`Oracle`): the four steps of
  "MHLA: Restoring Expressivity of Linear Attention via Token-Level
  Multi-Head" §4.1 (and App. C for the causal variant) in plain binary64 loops,
  linear in N.
* :mod:`oracle.bruteforce`: the plain definition, the explicit N x N weight
  matrix of the token-level expansion (same page, §4.2 Eq. 5), applied to V
  and normalised, in NumPy binary64.  Quadratic in N; rows can be sampled.
"""
import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_LIB = os.path.join(HERE, "libmhla_oracle.so")
SOURCE = os.path.join(HERE, "mhla_oracle.c")


def build(src=SOURCE, out=DEFAULT_LIB, openmp=True):
    """Compile the C oracle with gcc (IEEE binary64, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
           src, "-o", out, "-lm"]
    if openmp:
        cmd.insert(1, "-fopenmp")
    subprocess.run(cmd, check=True)
    return out


_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_L = ctypes.c_long


def _ptr(a, kind):
    return a.ctypes.data_as(kind)


class Oracle:
    """ctypes handle on a built copy of ``mhla_oracle.c``."""

    def __init__(self, lib_path=DEFAULT_LIB):
        if not os.path.exists(lib_path):
            raise FileNotFoundError(f"{lib_path} is not built; call oracle.build()")
        self.lib = ctypes.CDLL(lib_path)
        self.lib.mhla_oracle_phi.restype = ctypes.c_double
        self.lib.mhla_oracle_phi.argtypes = [ctypes.c_double]
        self.lib.mhla_oracle_summaries.argtypes = [_f32p, _f32p, _L, _L, _L, _L, _f64p, _f64p]
        self.lib.mhla_oracle_mix.argtypes = [_f64p, _f64p, _f32p, _L, _L, _L, ctypes.c_int, _f64p, _f64p]
        self.lib.mhla_oracle_forward.argtypes = [_f32p, _f32p, _f32p, _f32p, _f64p, _L, _L, _L, _L, _L,
                                                 ctypes.c_int, ctypes.c_int]
        self.lib.mhla_oracle_forward_ex.argtypes = [_f32p, _f32p, _f32p, _f32p, _f64p, _L, _L, _L, _L, _L,
                                                    ctypes.c_int, ctypes.c_int]
        self.lib.mhla_oracle_forward_blocks.argtypes = [_f32p, _f32p, _f32p, _f32p, _f64p, _L, _L, _L, _L, _L,
                                                        ctypes.POINTER(ctypes.c_int), ctypes.c_int, ctypes.c_int]

    def phi(self, x):
        return self.lib.mhla_oracle_phi(float(x))

    @staticmethod
    def _f32(a):
        return np.ascontiguousarray(a, dtype=np.float32)

    def forward(self, q, k, v, W, causal=False, nthreads=1, normalize=True, blk=None):
        """q, k, v: [B, H, N, d] float32; W: [M, M] float32 (or [H, M, M]: one matrix per
        head) -> float64 [B, H, N, d].

        normalize=False drops the normaliser (MHLA §4.1, remark on the output); blk [N]
        assigns token t to block blk[t] (blocks of any sizes; non-causal only)."""
        q, k, v, W = (self._f32(a) for a in (q, k, v, W))
        B, H, N, d = q.shape
        M = W.shape[-1]
        if W.ndim == 3 and W.shape != (H, M, M):
            raise ValueError("a per-head W must be [H, M, M]")
        out = np.empty((B, H, N, d), dtype=np.float64)
        opts = (1 if causal else 0) | (0 if normalize else 2) | (4 if W.ndim == 3 else 0)
        if blk is not None:
            blk = np.ascontiguousarray(blk, dtype=np.intc)
            if causal or blk.shape != (N,):
                raise ValueError("blk must be [N] and the pass non-causal")
            rc = self.lib.mhla_oracle_forward_blocks(
                _ptr(q, _f32p), _ptr(k, _f32p), _ptr(v, _f32p), _ptr(W, _f32p), _ptr(out, _f64p), B, H, N, d, M,
                blk.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), opts, int(nthreads))
            if rc != 0:
                raise ValueError("mhla_oracle_forward_blocks rejected its arguments")
            return out
        rc = self.lib.mhla_oracle_forward_ex(_ptr(q, _f32p), _ptr(k, _f32p), _ptr(v, _f32p), _ptr(W, _f32p),
                                             _ptr(out, _f64p), B, H, N, d, M, opts, int(nthreads))
        if rc != 0:
            raise ValueError("mhla_oracle_forward rejected its arguments")
        return out

    def summaries(self, k, v, M):
        """Per-block S_b [B, H, M, d, d] and z_b [B, H, M, d] (float64)."""
        k, v = self._f32(k), self._f32(v)
        B, H, N, d = k.shape
        S = np.empty((B, H, M, d, d), dtype=np.float64)
        z = np.empty((B, H, M, d), dtype=np.float64)
        rc = self.lib.mhla_oracle_summaries(_ptr(k, _f32p), _ptr(v, _f32p), B * H, N, d, M,
                                            _ptr(S, _f64p), _ptr(z, _f64p))
        if rc != 0:
            raise ValueError("mhla_oracle_summaries rejected its arguments")
        return S, z

    def mix(self, S, z, W, causal=False):
        """Mixed summaries S~_i, z~_i from per-block S_b, z_b."""
        S = np.ascontiguousarray(S, dtype=np.float64)
        z = np.ascontiguousarray(z, dtype=np.float64)
        W = self._f32(W)
        B, H, M, d, _ = S.shape
        St = np.empty_like(S)
        zt = np.empty_like(z)
        rc = self.lib.mhla_oracle_mix(_ptr(S, _f64p), _ptr(z, _f64p), _ptr(W, _f32p), B * H, d, M,
                                      int(bool(causal)), _ptr(St, _f64p), _ptr(zt, _f64p))
        if rc != 0:
            raise ValueError("mhla_oracle_mix rejected its arguments")
        return St, zt


_default = None


def default_oracle():
    """The oracle built in-tree, built first if it is missing."""
    global _default
    if _default is None:
        if not os.path.exists(DEFAULT_LIB):
            build()
        _default = Oracle(DEFAULT_LIB)
    return _default
