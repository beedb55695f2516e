"""Seeded synthetic inputs for the attention tests, the bench and the smoke check.

The generator is counter based (SplitMix64 stream, Box-Muller, round to bf16),
so a tensor depends only on (seed, tensor id, shape) and not on the thread
split or the host.  It holds none of the attention arithmetic; the oracle and
the HIP path both consume its output as raw bf16 bit patterns (numpy uint16).

Workload recipe (shapes and distributions of the pages' workloads, see the
KernelBraid README, "Features" and "Usage"):
  Q [B, Hq, S, D], K/V [B, Hkv, S, D], bf16 ~ N(0, 1), Hq=32, Hkv=8, D=128.
  The stress case adds 4 seeded outlier channels scaled by 8 in Q and K.
"""
from __future__ import annotations

import ctypes
import hashlib
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libkb_gen.so")

# tensor ids inside one seed's namespace
TID_Q, TID_K, TID_V = 1, 2, 3

_lib = None


def build() -> str:
    """Compile the generator into kb_gen/libkb_gen.so (always recompiles)."""
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
           _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.kbg_normal_bf16.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                        ctypes.c_void_p, ctypes.c_int]
        lib.kbg_normal_bf16.restype = ctypes.c_int
        lib.kbg_normal_bf16_at.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64]
        lib.kbg_normal_bf16_at.restype = ctypes.c_uint16
        lib.kbg_outlier_channels.argtypes = [ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        lib.kbg_outlier_channels.restype = ctypes.c_int
        lib.kbg_scale_channels.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int,
                                           ctypes.c_void_p, ctypes.c_int, ctypes.c_int]
        lib.kbg_scale_channels.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def normal_bf16(seed: int, tensor_id: int, shape, threads: int | None = None) -> np.ndarray:
    """bf16 N(0,1) bit patterns (uint16) of the given shape."""
    lib = _load()
    out = np.empty(shape, dtype=np.uint16)
    rc = lib.kbg_normal_bf16(seed, tensor_id, out.size, out.ctypes.data,
                             threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"kbg_normal_bf16 failed ({rc})")
    return out


def normal_bf16_at(seed: int, tensor_id: int, index: int) -> int:
    return int(_load().kbg_normal_bf16_at(seed, tensor_id, index))


def outlier_channels(seed: int, n: int = 4, head_dim: int = 128) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    if _load().kbg_outlier_channels(seed, n, head_dim, out.ctypes.data) != 0:
        raise ValueError("bad outlier request")
    return out


def scale_channels(x: np.ndarray, channels: np.ndarray, log2_factor: int = 3) -> np.ndarray:
    """In place: multiply the given last-axis channels of x (uint16 bf16 bits) by 2**log2_factor."""
    assert x.dtype == np.uint16 and x.flags.c_contiguous
    ch = np.ascontiguousarray(channels, dtype=np.int32)
    rows = x.size // x.shape[-1]
    if _load().kbg_scale_channels(x.ctypes.data, rows, x.shape[-1], ch.ctypes.data, ch.size,
                                  log2_factor) != 0:
        raise ValueError("bad channel scaling")
    return x


def attention_inputs(seed: int, batch: int, seq: int, n_q_heads: int = 32, n_kv_heads: int = 8,
                     head_dim: int = 128, kv_seq: int | None = None, q_seq: int | None = None,
                     outliers: int = 0, threads: int | None = None):
    """(q, k, v) as uint16 bf16 bits: q [B,Hq,q_seq,D], k/v [B,Hkv,kv_seq,D].

    With outliers > 0, that many seeded channels of q and k are scaled by 8.
    """
    kv_seq = seq if kv_seq is None else kv_seq
    q_seq = seq if q_seq is None else q_seq
    q = normal_bf16(seed, TID_Q, (batch, n_q_heads, q_seq, head_dim), threads)
    k = normal_bf16(seed, TID_K, (batch, n_kv_heads, kv_seq, head_dim), threads)
    v = normal_bf16(seed, TID_V, (batch, n_kv_heads, kv_seq, head_dim), threads)
    if outliers:
        ch = outlier_channels(seed, outliers, head_dim)
        scale_channels(q, ch)
        scale_channels(k, ch)
    return q, k, v


def bf16_bits_to_f32(x: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (bits << 16)."""
    return (x.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even narrowing of float32 to bf16 bit patterns (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def sha256(x: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(x).view(np.uint8)).hexdigest()
