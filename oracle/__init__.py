"""ORACLE -- test infrastructure only.

Plain CPU causal grouped-query attention (oracle/oracle.c, built with gcc in
fp64 and fp32) used to check the HIP path.  Only tests/, the smoke check and
the bench's CPU-baseline leg may import it; the library never does, and the
two share no code.

Inputs are bf16 bit patterns (numpy uint16): q [B, Hq, q_len, D] and
k/v [B, Hkv, kv_capacity, D].  Query row r sits at position
kv_len - q_len + r and attends to keys 0..pos of KV head h // (Hq // Hkv).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIBS = {
    "f64": os.path.join(_HERE, "liboracle_f64.so"),
    "f32": os.path.join(_HERE, "liboracle_f32.so"),
}
_REAL = {"f64": "double", "f32": "float"}
_loaded: dict = {}


def build() -> None:
    """Compile both precisions of the oracle (always recompiles)."""
    for prec, path in _LIBS.items():
        cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               "-pthread", f"-DKBO_REAL={_REAL[prec]}", f"-DKBO_SUFFIX=_{prec}", _SRC,
               "-o", path + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(path + ".tmp", path)


def bind(path: str, prec: str):
    """(attention, weights, backward, backward_dq_rows) C entry points of an
    oracle build at `path`."""
    lib = ctypes.CDLL(path)
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    f = getattr(lib, f"kbo_attention_{prec}")
    f.argtypes = [P] * 3 + [I64] * 7 + [ctypes.c_double, P, I64, P, P, ctypes.c_int]
    f.restype = ctypes.c_int
    w = getattr(lib, f"kbo_weights_{prec}")
    w.argtypes = [P] * 3 + [I64] * 7 + [ctypes.c_double, I64, P]
    w.restype = ctypes.c_int
    bw = getattr(lib, f"kbo_backward_{prec}")
    bw.argtypes = [P] * 4 + [I64] * 5 + [ctypes.c_double, I64] + [P] * 6 + [ctypes.c_int]
    bw.restype = ctypes.c_int
    br = getattr(lib, f"kbo_backward_dq_rows_{prec}")
    br.argtypes = [P] * 4 + [I64] * 5 + [ctypes.c_double, P, I64, P, P, ctypes.c_int]
    br.restype = ctypes.c_int
    return f, w, bw, br


def _lib(prec: str):
    if prec not in _loaded:
        if not os.path.exists(_LIBS[prec]):
            build()
        _loaded[prec] = bind(_LIBS[prec], prec)
    return _loaded[prec]


def _threads(n):
    if n:
        return int(n)
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _check(q, k, v):
    for name, x in (("q", q), ("k", k), ("v", v)):
        if x.dtype != np.uint16 or x.ndim != 4 or not x.flags.c_contiguous:
            raise ValueError(f"{name} must be a contiguous 4-D uint16 (bf16 bits) array")
    if k.shape != v.shape or q.shape[0] != k.shape[0] or q.shape[3] != k.shape[3]:
        raise ValueError("shape mismatch")


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, kv_len: int | None = None,
              scale: float | None = None, rows=None, precision: str = "f64",
              threads: int | None = None, entry=None) -> np.ndarray:
    """Attention output as float64.

    Without rows: shape [B, Hq, q_len, D].  With rows (flat ids
    b*Hq*q_len + h*q_len + r): shape [len(rows), D].
    """
    out, _ = _forward(q, k, v, kv_len, scale, rows, precision, threads, entry, want_lse=False)
    return out


def lse(q: np.ndarray, k: np.ndarray, v: np.ndarray, kv_len: int | None = None,
        scale: float | None = None, rows=None, precision: str = "f64",
        threads: int | None = None, entry=None) -> np.ndarray:
    """Per-row log-sum-exp, log(sum_j exp(scale <q, k_j>)) over the visible
    keys, as float64: shape [B, Hq, q_len], or [len(rows)] with rows."""
    _, l = _forward(q, k, v, kv_len, scale, rows, precision, threads, entry, want_lse=True)
    return l


def _forward(q, k, v, kv_len, scale, rows, precision, threads, entry, want_lse):
    _check(q, k, v)
    B, Hq, q_len, D = q.shape
    Hkv, cap = k.shape[1], k.shape[2]
    kv_len = cap if kv_len is None else int(kv_len)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    f = (entry if entry is not None else _lib(precision))[0]
    if rows is None:
        out = np.empty((B, Hq, q_len, D), dtype=np.float64)
        rows_ptr, n = None, B * Hq * q_len
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        out = np.empty((rows.size, D), dtype=np.float64)
        rows_ptr, n = rows.ctypes.data, rows.size
    lse_out = np.empty(out.shape[:-1], dtype=np.float64) if want_lse else None
    rc = f(q.ctypes.data, k.ctypes.data, v.ctypes.data, B, Hq, Hkv, q_len, kv_len, cap, D, scale,
           rows_ptr, n, out.ctypes.data, lse_out.ctypes.data if want_lse else None, _threads(threads))
    if rc != 0:
        raise ValueError(f"oracle rejected the problem (code {rc})")
    return out, lse_out


def weights(q, k, v, row: int, kv_len: int | None = None, scale: float | None = None,
            precision: str = "f64", entry=None) -> np.ndarray:
    """Normalised softmax weights of one row (flat id), length pos + 1."""
    _check(q, k, v)
    B, Hq, q_len, D = q.shape
    Hkv, cap = k.shape[1], k.shape[2]
    kv_len = cap if kv_len is None else int(kv_len)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    r = row % q_len
    pos = kv_len - q_len + r
    out = np.empty(pos + 1, dtype=np.float64)
    w = (entry if entry is not None else _lib(precision))[1]
    rc = w(q.ctypes.data, k.ctypes.data, v.ctypes.data, B, Hq, Hkv, q_len, kv_len, cap, D, scale, row,
           out.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle rejected the problem (code {rc})")
    return out


def _check_bwd(q, k, v, dout):
    _check(q, k, v)
    if dout.dtype != np.uint16 or dout.shape != q.shape or not dout.flags.c_contiguous:
        raise ValueError("dout must be a contiguous uint16 (bf16 bits) array shaped like q")
    if q.shape[2] != k.shape[2]:
        raise ValueError("the backward covers full sequences: q and k must have the same length")


def backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray, scale: float | None = None,
             row_from: int = 0, budgets: bool = False, precision: str = "f64",
             threads: int | None = None, entry=None) -> dict:
    """Gradients of the full causal forward for upstream gradient dout.

    Returns {"dq", "dk", "dv"} as float64 (dq shaped like q, dk/dv like k),
    plus {"eq", "ek", "ev"} error budgets when budgets is set.  With
    row_from > 0 only rows >= row_from are visited: dq is valid for those
    rows and dk/dv for keys >= row_from (the rest is zero or partial).
    """
    _check_bwd(q, k, v, dout)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    bw = (entry if entry is not None else _lib(precision))[2]
    out = {"dq": np.zeros(q.shape), "dk": np.zeros(k.shape), "dv": np.zeros(k.shape)}
    if budgets:
        out.update(eq=np.zeros(q.shape), ek=np.zeros(k.shape), ev=np.zeros(k.shape))
    ptr = lambda name: out[name].ctypes.data if name in out else None
    rc = bw(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data, B, Hq, Hkv, S, D, scale,
            int(row_from), ptr("dq"), ptr("dk"), ptr("dv"), ptr("eq"), ptr("ek"), ptr("ev"),
            min(_threads(threads), B * Hkv))
    if rc != 0:
        raise ValueError(f"oracle rejected the problem (code {rc})")
    return out


def backward_dq_rows(q, k, v, dout, rows, scale: float | None = None, budgets: bool = False,
                     precision: str = "f64", threads: int | None = None, entry=None):
    """dq of the listed flat rows (b*Hq*S + h*S + i): [len(rows), D] float64,
    and its error budget (or None)."""
    _check_bwd(q, k, v, dout)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    br = (entry if entry is not None else _lib(precision))[3]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    dq = np.zeros((rows.size, D))
    eq = np.zeros((rows.size, D)) if budgets else None
    rc = br(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data, B, Hq, Hkv, S, D, scale,
            rows.ctypes.data, rows.size, dq.ctypes.data, eq.ctypes.data if budgets else None,
            _threads(threads))
    if rc != 0:
        raise ValueError(f"oracle rejected the problem (code {rc})")
    return dq, eq
