"""Bitwise-aligned causal grouped-query attention for AMD MI355X (gfx950).

Thin Python binding over the C-ABI library libkb_attn.so (include/kb_attn.h).
It only marshals arguments: every step of the attention runs in the HIP
kernels.  PyTorch supplies device memory and the current stream.  There is no
fallback: if the library is missing or the tensors are not on the GPU, the
calls raise.

Entry points (KernelBraid / AReaL-TIK README, "Usage" and "Method"):
  prefill(q, k, v)                          causal full-sequence forward
  partitioned(q, k_cache, v_cache, kv_len)  a chunk of rows against cached KV
  decode(q, k_cache, v_cache, kv_len)       one query token
  unified_prefill / unified_decode          the README's call shapes
All three give bitwise-identical rows for the same inputs and context.
"""
from __future__ import annotations

import ctypes
import math
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkb_attn.so")

HEAD_DIM = 128
GROUP = 4


class KBAttnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"kb_attn error {code}: {message}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C-ABI library (raises when it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it with __graft_entry__.build() "
                              "or python -m bitwise_aligned_causal_amd._build")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
        L.kb_attn_prefill.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, i32, f32, vp]
        L.kb_attn_prefill.restype = ctypes.c_int
        L.kb_attn_partitioned.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, i32, f32, vp]
        L.kb_attn_partitioned.restype = ctypes.c_int
        L.kb_attn_decode.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, f32, vp, ctypes.c_size_t,
                                     vp]
        L.kb_attn_decode.restype = ctypes.c_int
        L.kb_attn_decode_workspace_bytes.argtypes = [i64, i64, i32, i32]
        L.kb_attn_decode_workspace_bytes.restype = ctypes.c_size_t
        L.kb_attn_strerror.argtypes = [ctypes.c_int]
        L.kb_attn_strerror.restype = ctypes.c_char_p
        L.kb_attn_contract.argtypes = [ctypes.POINTER(i32)] * 3
        L.kb_attn_contract.restype = None
        _lib = L
    return _lib


def check(code: int) -> None:
    if code != 0:
        raise KBAttnError(code, lib().kb_attn_strerror(code).decode())


def contract() -> dict:
    t, c, ver = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    lib().kb_attn_contract(ctypes.byref(t), ctypes.byref(c), ctypes.byref(ver))
    return {"kv_tile": t.value, "kv_chunk": c.value, "version": ver.value,
            "mfma": "v_mfma_f32_32x32x16_bf16"}


def decode_workspace_bytes(batch: int, kv_len: int, n_q_heads: int = 32, head_dim: int = HEAD_DIM) -> int:
    return int(lib().kb_attn_decode_workspace_bytes(batch, kv_len, n_q_heads, head_dim))


def _torch():
    import torch
    return torch


def _check_tensor(name, x, ndim=4):
    torch = _torch()
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if x.dtype != torch.bfloat16 or not x.is_cuda or x.dim() != ndim or not x.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 4-D bfloat16 tensor on the GPU "
                         f"(got {x.dtype}, {x.device}, shape {tuple(x.shape)})")


def _stream(x):
    return ctypes.c_void_p(_torch().cuda.current_stream(x.device).cuda_stream)


def _scale(scale, head_dim):
    return 1.0 / math.sqrt(head_dim) if scale is None else float(scale)


def prefill(q, k, v, scale: float | None = None, out=None):
    """Causal full-sequence forward: q [B, Hq, S, 128], k/v [B, Hkv, S, 128]."""
    for n, x in (("q", q), ("k", k), ("v", v)):
        _check_tensor(n, x)
    B, Hq, S, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != S or k.shape[3] != D:
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    out = _torch().empty_like(q) if out is None else out
    _check_tensor("out", out)
    check(lib().kb_attn_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, S, Hq,
                                k.shape[1], D, _scale(scale, D), _stream(q)))
    return out


def partitioned(q, k_cache, v_cache, kv_len: int, scale: float | None = None, out=None):
    """q [B, Hq, q_len, 128] at positions kv_len - q_len .. kv_len - 1 against
    caches [B, Hkv, capacity, 128] holding kv_len keys."""
    for n, x in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _check_tensor(n, x)
    B, Hq, q_len, D = q.shape
    if k_cache.shape != v_cache.shape or k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError("cache shape mismatch")
    out = _torch().empty_like(q) if out is None else out
    _check_tensor("out", out)
    check(lib().kb_attn_partitioned(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(), B,
                                    q_len, int(kv_len), k_cache.shape[2], Hq, k_cache.shape[1], D,
                                    _scale(scale, D), _stream(q)))
    return out


def decode(q, k_cache, v_cache, kv_len: int | None = None, scale: float | None = None, out=None,
           workspace=None):
    """q [B, Hq, 1, 128] at position kv_len - 1 against caches [B, Hkv, capacity, 128]."""
    torch = _torch()
    for n, x in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _check_tensor(n, x)
    B, Hq, one, D = q.shape
    if one != 1:
        raise ValueError("decode takes one query token per sequence")
    if k_cache.shape != v_cache.shape or k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError("cache shape mismatch")
    kv_len = k_cache.shape[2] if kv_len is None else int(kv_len)
    need = decode_workspace_bytes(B, kv_len, Hq, D) if kv_len >= 1 else 0
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    out = torch.empty_like(q) if out is None else out
    _check_tensor("out", out)
    check(lib().kb_attn_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(), B, kv_len,
                               k_cache.shape[2], Hq, k_cache.shape[1], D, _scale(scale, D), ws_ptr, ws_bytes,
                               _stream(q)))
    return out


def unified_prefill(q, k, v, H_Q: int, H_KV: int, scale: float | None = None):
    """The README's call shape: causal forward, output shaped like q."""
    if q.shape[1] != H_Q or k.shape[1] != H_KV:
        raise ValueError("head counts do not match the tensors")
    return prefill(q, k, v, scale)


def unified_decode(q_last, k, v, H_Q: int, H_KV: int, scale: float | None = None):
    """The README's call shape: one query token over the whole KV context."""
    if q_last.shape[1] != H_Q or k.shape[1] != H_KV:
        raise ValueError("head counts do not match the tensors")
    return decode(q_last, k, v, k.shape[2], scale)


__all__ = ["prefill", "partitioned", "decode", "unified_prefill", "unified_decode", "contract",
           "decode_workspace_bytes", "lib", "check", "KBAttnError", "LIB_PATH"]
