"""CPU oracle for the quantized matvec / prefill product / greedy head.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the product
package ``gemm_qgemv_amd`` never does, and shares no code with it.

The arithmetic lives in ``qg_oracle.c`` (plain loops, double accumulation);
this module builds it with gcc and marshals numpy arrays through ctypes. The
one exception is ``Oracle.qgemm_dense``: the weights decoded exactly by
``qg_oracle.c``, then numpy's float64 matrix product as a library step.
Inputs are host numpy arrays in the layouts documented in ``qg_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

I8_ROW, U4_G64, B1_G128, I8_G64 = 1, 2, 3, 4

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qg_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, OpenMP over outputs)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-Wall", "-Werror", src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


class Oracle:
    """ctypes view of one built oracle library (the default one, or another
    build of it such as a planted-mistake copy made by the tests)."""

    def __init__(self, path: str = _LIB):
        if not os.path.exists(path):
            raise RuntimeError(
                f"oracle library {path} is missing: run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        P, I64, I32, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.oracle_decode.argtypes = [I32, P, P, P, I64, I64, P]
        lib.oracle_qgemv.argtypes = [I32, P, P, P, P, I64, I64, I64, P, P]
        lib.oracle_qgemv_sample.argtypes = [I32, P, P, P, P, I64, I64, I64, P, P, I64, P, P]
        lib.oracle_argmax.argtypes = [P, I64, I64, P, P]
        lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_value.restype = D
        lib.oracle_fp16_value.argtypes = [ctypes.c_uint16]
        lib.oracle_fp16_value.restype = D
        lib.oracle_num_threads.restype = I32
        lib.oracle_set_threads.argtypes = [I32]
        lib.oracle_set_threads.restype = None
        lib.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        lib.oracle_f32_to_f16.restype = ctypes.c_uint16
        lib.oracle_embed.argtypes = [P, P, P, P, I64, I64, I64, P]
        lib.oracle_embed.restype = I32
        for f in (lib.oracle_decode, lib.oracle_qgemv, lib.oracle_qgemv_sample,
                  lib.oracle_argmax):
            f.restype = I32
        self.lib = lib
        self.path = path

    # -- helpers --------------------------------------------------------
    @staticmethod
    def _ptr(a):
        return None if a is None else a.ctypes.data

    @staticmethod
    def _check(rc, what):
        if rc != 0:
            raise ValueError(f"oracle {what} rejected its arguments (code {rc})")

    @staticmethod
    def _prep(codes, scales, biases):
        codes = np.ascontiguousarray(codes)
        scales = np.ascontiguousarray(scales)
        biases = None if biases is None else np.ascontiguousarray(biases)
        return codes, scales, biases

    # -- entry points ---------------------------------------------------
    def bf16_value(self, bits: int) -> float:
        return self.lib.oracle_bf16_value(int(bits))

    def fp16_value(self, bits: int) -> float:
        return self.lib.oracle_fp16_value(int(bits))

    def num_threads(self) -> int:
        return self.lib.oracle_num_threads()

    def set_threads(self, n: int) -> None:
        """Threads of the per-output loops from now on."""
        self.lib.oracle_set_threads(int(n))

    def decode(self, fmt, codes, scales, biases, M, K):
        """Exact weights w[M][K] as float64."""
        codes, scales, biases = self._prep(codes, scales, biases)
        w = np.empty((M, K), np.float64)
        self._check(self.lib.oracle_decode(fmt, self._ptr(codes), self._ptr(scales),
                                           self._ptr(biases), M, K, self._ptr(w)),
                    "decode")
        return w

    def qgemv(self, fmt, codes, scales, biases, x, M, K):
        """y[N][M] = sum_k w[m][k] x[n][k] and a[N][M] = sum_k |w x| (float64).
        x is float32 [N][K] (N = batch rows or prefill tokens)."""
        codes, scales, biases = self._prep(codes, scales, biases)
        x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1, K)
        N = x.shape[0]
        y = np.empty((N, M), np.float64)
        a = np.empty((N, M), np.float64)
        self._check(self.lib.oracle_qgemv(fmt, self._ptr(codes), self._ptr(scales),
                                          self._ptr(biases), self._ptr(x), M, K, N,
                                          self._ptr(y), self._ptr(a)), "qgemv")
        return y, a

    def qgemv_sample(self, fmt, codes, scales, biases, x, M, K, n_idx, m_idx):
        """The same outputs at the (n_idx[i], m_idx[i]) pairs only."""
        codes, scales, biases = self._prep(codes, scales, biases)
        x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1, K)
        n_idx = np.ascontiguousarray(n_idx, dtype=np.int64)
        m_idx = np.ascontiguousarray(m_idx, dtype=np.int64)
        y = np.empty(n_idx.shape[0], np.float64)
        a = np.empty(n_idx.shape[0], np.float64)
        self._check(self.lib.oracle_qgemv_sample(
            fmt, self._ptr(codes), self._ptr(scales), self._ptr(biases), self._ptr(x),
            M, K, x.shape[0], self._ptr(n_idx), self._ptr(m_idx), n_idx.shape[0],
            self._ptr(y), self._ptr(a)), "qgemv_sample")
        return y, a

    def qgemm_dense(self, fmt, codes, scales, biases, x, M, K):
        """The same y[N][M] and a[N][M] as ``qgemv``, for products too large
        for the per-output loops: the exact weights from ``decode`` (float64,
        the plain definition of each format) times the activations with
        numpy's float64 matrix product, y = x w^T and a = |x| |w|^T. Every
        term is exact or within one double rounding, so the result differs
        from ``qgemv`` only by the order of the float64 additions (relative
        error about K * 2^-53 of a). (MiniCPM-V-4.6 on a Tesla C2075, section
        3.1 "Prefill projections: dequantize, then call the vendor": the
        prompt's projections expand the codes to float once and hand them to
        a dense matrix product.)"""
        w = self.decode(fmt, codes, scales, biases, M, K)
        xd = np.ascontiguousarray(x, dtype=np.float32).reshape(-1, K).astype(np.float64)
        y = xd @ w.T
        np.abs(w, out=w)
        np.abs(xd, out=xd)
        a = xd @ w.T
        return y, a

    def f32_to_f16(self, v: float) -> int:
        """IEEE binary16 bits of float32 v, rounded to nearest even."""
        return int(self.lib.oracle_f32_to_f16(v))

    def embed(self, codes, scales, biases, ids, M, K):
        """Embedding rows e[t][k] of the 4-bit format (float32 [n][K])."""
        c, s, b = self._prep(codes, scales, biases)
        ids = np.ascontiguousarray(ids, np.int32)
        out = np.empty((len(ids), K), np.float32)
        self._check(self.lib.oracle_embed(self._ptr(c), self._ptr(s), self._ptr(b), self._ptr(ids),
                                           M, K, len(ids), self._ptr(out)), "embed")
        return out

    def argmax(self, y):
        """Lowest index of the row maximum, and the top-2 gap, per row."""
        y = np.ascontiguousarray(y, dtype=np.float64)
        y2 = y.reshape(-1, y.shape[-1])
        idx = np.empty(y2.shape[0], np.int32)
        gap = np.empty(y2.shape[0], np.float64)
        self._check(self.lib.oracle_argmax(self._ptr(y2), y2.shape[1], y2.shape[0],
                                           self._ptr(idx), self._ptr(gap)), "argmax")
        return idx, gap


_default = None


def get() -> Oracle:
    """The oracle built from qg_oracle.c in this directory."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
