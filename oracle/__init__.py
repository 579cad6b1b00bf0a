"""fp64 CPU oracle for the no-KV-cache multi-head attention forward.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product
library (``head_attention_no_amd``) never imports it, and the two share no
code: the oracle is plain C (``oracle_fp64.c``) built with the host compiler,
plus the NumPy recurrences in ``online_softmax.py``.

The definition it follows is the "FlashAttentionGPU" API page
(max.modular.com), section "execute", Steps 0-4 and the grouped-attention
Step -1: scores = Q @ K^T, times ``scale``, mask functor, row softmax, @ V,
with Q/K/V/answer in BSHD (K/V may have fewer heads, BShD). The C file's
header lists the readings taken where the page is silent.

Arrays are NumPy; they are widened to float64 (exact for bf16/fp16/fp32
values) before the call.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

MASK_NONE = 0
MASK_CAUSAL = 1
MASK_SLIDING_WINDOW = 2

_MASKS = {"none": MASK_NONE, "causal": MASK_CAUSAL, "sliding_window": MASK_SLIDING_WINDOW,
          "window": MASK_SLIDING_WINDOW}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_fp64.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    """Compile ``oracle_fp64.c`` into ``liboracle.so`` with gcc and OpenMP."""
    return compile_library(_SRC, _LIB, verbose=verbose)


def compile_library(src: str, out: str, verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", src, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def mask_code(mask) -> int:
    if isinstance(mask, str):
        return _MASKS[mask]
    return int(mask)


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # a torch tensor: widen on the CPU, exactly
        import torch

        x = x.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be rank 4 (BSHD / BShD)")
    B, S, H, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[1] != S or k.shape[3] != D:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    return B, S, H, k.shape[2], D


class Oracle:
    """One loaded build of ``oracle_fp64.c`` (the default one, or a test's variant)."""

    def __init__(self, path: str = _LIB):
        if path == _LIB and not os.path.exists(path):
            build()
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        i = ctypes.c_int
        lib.fa355_oracle_attention.argtypes = [dp, dp, dp, dp, i, i, i, i, i, ctypes.c_double, i,
                                               i, i]
        lib.fa355_oracle_attention.restype = i
        lib.fa355_oracle_rows.argtypes = [dp, dp, dp, i, i, i, i, i, ctypes.c_double, i, i,
                                          ctypes.POINTER(ctypes.c_int64), ctypes.c_int64, dp, i]
        lib.fa355_oracle_rows.restype = i
        lib.fa355_oracle_probs.argtypes = [dp, dp, i, i, i, i, i, ctypes.c_double, i, i, i, i, i,
                                           dp]
        lib.fa355_oracle_probs.restype = i
        lib.fa355_oracle_visible_pairs.argtypes = [i, i, i]
        lib.fa355_oracle_visible_pairs.restype = ctypes.c_int64
        lib.fa355_oracle_threads.argtypes = []
        lib.fa355_oracle_threads.restype = i
        self.lib = lib
        self.path = path

    def attention(self, q, k, v, scale: float, mask="none", window: int = -1,
                  threads: int = 0) -> np.ndarray:
        """Whole operator in fp64; returns the answer in BSHD like ``q``."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, S, H, Hkv, D = _shapes(q, k, v)
        out = np.empty_like(q)
        rc = self.lib.fa355_oracle_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, S, H, Hkv,
                                             D, float(scale), mask_code(mask), int(window),
                                             int(threads))
        if rc != 0:
            raise ValueError(f"oracle rejected the arguments (status {rc})")
        return out

    def attention_rows(self, q, k, v, scale: float, mask, window: int, rows,
                       threads: int = 0) -> np.ndarray:
        """Output rows O[b, i, h, :] for each (b, h, i) in ``rows``; returns (n, D)."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, S, H, Hkv, D = _shapes(q, k, v)
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
        out = np.empty((r.shape[0], D), dtype=np.float64)
        rc = self.lib.fa355_oracle_rows(_ptr(q), _ptr(k), _ptr(v), B, S, H, Hkv, D, float(scale),
                                        mask_code(mask), int(window),
                                        r.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                        r.shape[0], _ptr(out), int(threads))
        if rc != 0:
            raise ValueError(f"oracle rejected the arguments (status {rc})")
        return out

    def probs(self, q, k, scale: float, mask, window: int, b: int, h: int, i: int) -> np.ndarray:
        """Row i of the softmaxed attention matrix of batch b, head h (length S)."""
        q, k = _f64(q), _f64(k)
        B, S, H, D = q.shape
        p = np.empty(S, dtype=np.float64)
        rc = self.lib.fa355_oracle_probs(_ptr(q), _ptr(k), B, S, H, k.shape[2], D, float(scale),
                                         mask_code(mask), int(window), int(b), int(h), int(i),
                                         _ptr(p))
        if rc != 0:
            raise ValueError(f"oracle rejected the arguments (status {rc})")
        return p

    def threads(self) -> int:
        """Number of threads the oracle's parallel loops use."""
        return int(self.lib.fa355_oracle_threads())

    def visible_pairs(self, S: int, mask, window: int = -1) -> int:
        """Count of (query, key) pairs the mask leaves visible in one head."""
        return int(self.lib.fa355_oracle_visible_pairs(int(S), mask_code(mask), int(window)))


_default: Oracle | None = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def attention(q, k, v, scale: float, mask="none", window: int = -1, threads: int = 0):
    return default().attention(q, k, v, scale, mask, window, threads)


def attention_rows(q, k, v, scale: float, mask, window: int, rows, threads: int = 0):
    return default().attention_rows(q, k, v, scale, mask, window, rows, threads)


def probs(q, k, scale: float, mask, window: int, b: int, h: int, i: int):
    return default().probs(q, k, scale, mask, window, b, h, i)


def visible_pairs(S: int, mask, window: int = -1) -> int:
    return default().visible_pairs(S, mask, window)
