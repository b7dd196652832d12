"""fp64 CPU oracle of the self-conditioning soft embedding -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does; the two
share no code.  The arithmetic lives in ``softembed_oracle.c`` (plain C, fp64,
sequential sums); this file only builds it with gcc and marshals numpy arrays.

Functions
---------
row_stats(logits)                      -> dict(max, argmax, lse, entropy)  (fp64 / int32)
soft_embed(logits, s, e, w, gamma, ..) -> ndarray [rows, d] fp64
soft_embed_ranges(logits, bounds, w, gamma, ..) -> the same, range by range (one-read form)
round_bf16(x)                          -> fp64 values rounded to bfloat16 (RNE)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "softembed_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, strict IEEE: no -ffast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_row_stats.argtypes = [p, i64, i64, i64, p, p, p, p]
        lib.oracle_row_stats.restype = ctypes.c_int
        lib.oracle_soft_embed.argtypes = [p, i64, i64, i64, i64, i64, p, p, i64, i64,
                                          ctypes.c_double, ctypes.c_int, p, i64]
        lib.oracle_soft_embed.restype = ctypes.c_int
        lib.oracle_soft_embed_ranges.argtypes = [p, i64, i64, i64, i64, i64, p, i64, p, p, i64,
                                                 i64, ctypes.c_double, ctypes.c_int, p, i64]
        lib.oracle_soft_embed_ranges.restype = ctypes.c_int
        lib.oracle_round_bf16.argtypes = [ctypes.c_double]
        lib.oracle_round_bf16.restype = ctypes.c_double
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _rows(logits: np.ndarray) -> np.ndarray:
    a = np.asarray(logits)
    if a.dtype != np.float32 or a.ndim != 2:
        raise TypeError("logits must be a 2-D float32 array")
    if a.strides[1] != 4 or a.strides[0] % 4:
        a = np.ascontiguousarray(a)
    return a


def row_stats(logits: np.ndarray) -> dict:
    x = _rows(logits)
    n, v = x.shape
    ld = x.strides[0] // 4
    out = {"max": np.empty(n), "argmax": np.empty(n, np.int32),
           "lse": np.empty(n), "entropy": np.empty(n)}
    rc = _load().oracle_row_stats(_ptr(x), ld, n, v, _ptr(out["max"]), _ptr(out["argmax"]),
                                  _ptr(out["lse"]), _ptr(out["entropy"]))
    if rc:
        raise ValueError("oracle_row_stats: non-finite logits")
    return out


def soft_embed(logits: np.ndarray, vocab_start: int, vocab_end: int, w: np.ndarray,
               gamma: float, round_p_bf16: bool = False) -> np.ndarray:
    """gamma * softmax(logits)[:, s:e] @ w[: e - s].

    ``w`` is the local shard (row 0 = vocab id ``vocab_start``): either float32
    values or uint16 bfloat16 bit patterns.  ``gamma`` is widened exactly from
    the float32 value the GPU receives.
    """
    x = _rows(logits)
    n, v = x.shape
    w = np.asarray(w)
    if w.ndim != 2 or w.strides[1] != w.itemsize:
        w = np.ascontiguousarray(w)
    if w.shape[0] < vocab_end - vocab_start:
        raise ValueError("table shard shorter than the slice")
    d = w.shape[1]
    ldw = w.strides[0] // w.itemsize
    out = np.empty((n, d))
    g = float(np.float32(gamma))
    if w.dtype == np.float32:
        wf, wb = _ptr(w), None
    elif w.dtype == np.uint16:
        wf, wb = None, _ptr(w)
    else:
        raise TypeError("table must be float32 or uint16 (bf16 bits)")
    rc = _load().oracle_soft_embed(_ptr(x), x.strides[0] // 4, n, v, vocab_start, vocab_end,
                                   wf, wb, ldw, d, g, int(bool(round_p_bf16)), _ptr(out), d)
    if rc:
        raise ValueError(f"oracle_soft_embed failed ({rc})")
    return out


def soft_embed_ranges(logits: np.ndarray, bounds, w: np.ndarray, gamma: float,
                      round_q_bf16: bool = False) -> np.ndarray:
    """gamma * softmax(logits)[:, s:e] @ w[: e - s] formed range by range: ``bounds`` =
    [s, b_1, ..., e] (vocab ids); range r's probabilities are e^(l - m_r) against the
    range's own maximum m_r (optionally rounded to bf16), rescaled by e^(m_r - lse)."""
    x = _rows(logits)
    n, v = x.shape
    b = np.ascontiguousarray(np.asarray(bounds, dtype=np.int64))
    s, e = int(b[0]), int(b[-1])
    w = np.asarray(w)
    if w.ndim != 2 or w.strides[1] != w.itemsize:
        w = np.ascontiguousarray(w)
    if w.shape[0] < e - s:
        raise ValueError("table shard shorter than the slice")
    d = w.shape[1]
    out = np.empty((n, d))
    g = float(np.float32(gamma))
    if w.dtype == np.float32:
        wf, wb = _ptr(w), None
    elif w.dtype == np.uint16:
        wf, wb = None, _ptr(w)
    else:
        raise TypeError("table must be float32 or uint16 (bf16 bits)")
    rc = _load().oracle_soft_embed_ranges(_ptr(x), x.strides[0] // 4, n, v, s, e, _ptr(b),
                                          b.size - 1, wf, wb, w.strides[0] // w.itemsize, d, g,
                                          int(bool(round_q_bf16)), _ptr(out), d)
    if rc:
        raise ValueError(f"oracle_soft_embed_ranges failed ({rc})")
    return out


def round_bf16(x) -> np.ndarray:
    f = _load().oracle_round_bf16
    a = np.asarray(x, dtype=np.float64)
    return np.vectorize(f, otypes=[np.float64])(a)
