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
  decode_static(q, k_cache, v_cache, kv_len) the same without a workspace (library-held scratch)
  decode_multi(q, k_cache, v_cache, kv_len) the last 1..8 tokens (a short partitioned chunk, split-KV)
  unified_prefill / unified_decode          the README's call shapes
  prefill_varlen / partitioned_varlen / decode_varlen
                                            ragged batches, packed [heads, rows, 128]
  decode_paged                              decode over a paged KV cache
  prefill_lse / partitioned_lse / decode_lse
                                            the same, also returning each row's log-sum-exp
  backward(q, k, v, out, dout, lse)         deterministic dq, dk, dv of the causal prefill
  prefill_varlen_lse / backward_varlen      the same for ragged (packed) batches
  attention(q, k, v)                        differentiable prefill (autograd glue)
All forward entry points give bitwise-identical rows (and log-sum-exps) for
the same inputs and context.
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
        L.kb_attn_decode_static.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, f32, vp]
        L.kb_attn_decode_static.restype = ctypes.c_int
        L.kb_attn_decode_workspace_bytes.argtypes = [i64, i64, i32, i32]
        L.kb_attn_decode_workspace_bytes.restype = ctypes.c_size_t
        p64 = ctypes.POINTER(i64)
        L.kb_attn_prefill_varlen.argtypes = [vp, vp, vp, vp, p64, i64, i32, i32, i32, f32, vp]
        L.kb_attn_prefill_varlen.restype = ctypes.c_int
        L.kb_attn_partitioned_varlen.argtypes = [vp, vp, vp, vp, p64, p64, p64, i64, i32, i32, i32, f32, vp]
        L.kb_attn_partitioned_varlen.restype = ctypes.c_int
        L.kb_attn_decode_varlen.argtypes = [vp, vp, vp, vp, p64, p64, i64, i32, i32, i32, f32, vp, ctypes.c_size_t,
                                            vp]
        L.kb_attn_decode_varlen.restype = ctypes.c_int
        L.kb_attn_decode_paged.argtypes = [vp, vp, vp, vp, vp, i64, p64, i64, i64, i32, i32, i32, i32, f32, vp,
                                           ctypes.c_size_t, vp]
        L.kb_attn_decode_paged.restype = ctypes.c_int
        L.kb_attn_decode_varlen_workspace_bytes.argtypes = [p64, i64, i32, i32]
        L.kb_attn_decode_varlen_workspace_bytes.restype = ctypes.c_size_t
        L.kb_attn_prefill_lse.argtypes = [vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, f32, vp]
        L.kb_attn_prefill_lse.restype = ctypes.c_int
        L.kb_attn_partitioned_lse.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, i32, f32, vp]
        L.kb_attn_partitioned_lse.restype = ctypes.c_int
        L.kb_attn_decode_lse.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, f32, vp,
                                         ctypes.c_size_t, vp]
        L.kb_attn_decode_lse.restype = ctypes.c_int
        L.kb_attn_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, f32, vp,
                                       ctypes.c_size_t, vp]
        L.kb_attn_backward.restype = ctypes.c_int
        L.kb_attn_backward_workspace_bytes.argtypes = [i64, i64, i32, i32]
        L.kb_attn_backward_workspace_bytes.restype = ctypes.c_size_t
        L.kb_attn_prefill_varlen_lse.argtypes = [vp, vp, vp, vp, vp, p64, i64, i32, i32, i32, f32, vp]
        L.kb_attn_prefill_varlen_lse.restype = ctypes.c_int
        L.kb_attn_backward_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, p64, i64, i32, i32, i32, f32, vp,
                                              ctypes.c_size_t, vp]
        L.kb_attn_backward_varlen.restype = ctypes.c_int
        L.kb_attn_backward_varlen_workspace_bytes.argtypes = [p64, i64, i32, i32]
        L.kb_attn_backward_varlen_workspace_bytes.restype = ctypes.c_size_t
        L.kb_attn_decode_multi.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, i32, f32, vp,
                                           ctypes.c_size_t, vp]
        L.kb_attn_decode_multi.restype = ctypes.c_int
        L.kb_attn_decode_multi_workspace_bytes.argtypes = [i64, i64, i64, i32, i32]
        L.kb_attn_decode_multi_workspace_bytes.restype = ctypes.c_size_t
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


def _host_i64(values):
    """A ctypes int64 array holding `values` (host memory, kept alive by the caller)."""
    vals = [int(x) for x in values]
    return (ctypes.c_int64 * max(1, len(vals)))(*vals)


def decode_varlen_workspace_bytes(kv_lens, n_q_heads: int = 32, head_dim: int = HEAD_DIM) -> int:
    arr = _host_i64(kv_lens)
    return int(lib().kb_attn_decode_varlen_workspace_bytes(arr, len(kv_lens), n_q_heads, head_dim))


def _torch():
    import torch
    return torch


def _check_tensor(name, x, ndim=4):
    torch = _torch()
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if x.dtype != torch.bfloat16 or not x.is_cuda or x.dim() != ndim or not x.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-D bfloat16 tensor on the GPU "
                         f"(got {x.dtype}, {x.device}, shape {tuple(x.shape)})")


def _check_like(name, x, like, ndim=4):
    """x is a contiguous bf16 GPU tensor with exactly the shape and device of
    `like`: the library takes only a pointer for an output, so a smaller
    buffer would be written past its end."""
    _check_tensor(name, x, ndim)
    if tuple(x.shape) != tuple(like.shape) or x.device != like.device:
        raise ValueError(f"{name} must have shape {tuple(like.shape)} on {like.device} "
                         f"(got {tuple(x.shape)} on {x.device})")


def _same_device(*named):
    """Every tensor on the device of the first (the library checks residency on
    the current device, the binding that they agree with each other)."""
    dev = named[0][1].device
    for n, x in named[1:]:
        if x.device != dev:
            raise ValueError(f"{n} is on {x.device}, {named[0][0]} on {dev}")


def _stream(x):
    return ctypes.c_void_p(_torch().cuda.current_stream(x.device).cuda_stream)


def _scale(scale, head_dim):
    return 1.0 / math.sqrt(head_dim) if scale is None else float(scale)


def prefill(q, k, v, scale: float | None = None, out=None):
    """Causal full-sequence forward: q [B, Hq, S, 128], k/v [B, Hkv, S, 128]."""
    for n, x in (("q", q), ("k", k), ("v", v)):
        _check_tensor(n, x)
    _same_device(("q", q), ("k", k), ("v", v))
    B, Hq, S, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != S or k.shape[3] != D:
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    out = _torch().empty_like(q) if out is None else out
    _check_like("out", out, q)
    check(lib().kb_attn_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, S, Hq,
                                k.shape[1], D, _scale(scale, D), _stream(q)))
    return out


def partitioned(q, k_cache, v_cache, kv_len: int, scale: float | None = None, out=None):
    """q [B, Hq, q_len, 128] at positions kv_len - q_len .. kv_len - 1 against
    caches [B, Hkv, capacity, 128] holding kv_len keys."""
    for n, x in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _check_tensor(n, x)
    _same_device(("q", q), ("k_cache", k_cache), ("v_cache", v_cache))
    B, Hq, q_len, D = q.shape
    if k_cache.shape != v_cache.shape or k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError("cache shape mismatch")
    out = _torch().empty_like(q) if out is None else out
    _check_like("out", out, q)
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
    _same_device(("q", q), ("k_cache", k_cache), ("v_cache", v_cache))
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
    _check_like("out", out, q)
    check(lib().kb_attn_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(), B, kv_len,
                               k_cache.shape[2], Hq, k_cache.shape[1], D, _scale(scale, D), ws_ptr, ws_bytes,
                               _stream(q)))
    return out


def decode_static(q, k_cache, v_cache, kv_len: int | None = None, scale: float | None = None, out=None):
    """decode() without a workspace: the chunk partials go to the library's
    own per-GPU scratch (8 MiB), so the call allocates nothing when out is
    given.  Calls that may overlap on one GPU race on that scratch."""
    for n, x in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _check_tensor(n, x)
    _same_device(("q", q), ("k_cache", k_cache), ("v_cache", v_cache))
    B, Hq, one, D = q.shape
    if one != 1:
        raise ValueError("decode takes one query token per sequence")
    if k_cache.shape != v_cache.shape or k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError("cache shape mismatch")
    kv_len = k_cache.shape[2] if kv_len is None else int(kv_len)
    out = _torch().empty_like(q) if out is None else out
    _check_like("out", out, q)
    check(lib().kb_attn_decode_static(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(), B,
                                      kv_len, k_cache.shape[2], Hq, k_cache.shape[1], D, _scale(scale, D),
                                      _stream(q)))
    return out


DECODE_STATIC_SCRATCH_BYTES = 8 << 20


def decode_multi_workspace_bytes(batch: int, n_rows: int, kv_len: int, n_q_heads: int = 32,
                                 head_dim: int = HEAD_DIM) -> int:
    return int(lib().kb_attn_decode_multi_workspace_bytes(batch, n_rows, kv_len, n_q_heads, head_dim))


def decode_multi(q, k_cache, v_cache, kv_len: int | None = None, scale: float | None = None, out=None,
                 workspace=None):
    """Decode of the last n_rows <= 8 tokens: q [B, Hq, n_rows, 128], row r
    at position kv_len - n_rows + r, against caches [B, Hkv, capacity, 128]."""
    torch = _torch()
    for n, x in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _check_tensor(n, x)
    _same_device(("q", q), ("k_cache", k_cache), ("v_cache", v_cache))
    B, Hq, n_rows, D = q.shape
    if k_cache.shape != v_cache.shape or k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError("cache shape mismatch")
    kv_len = k_cache.shape[2] if kv_len is None else int(kv_len)
    need = decode_multi_workspace_bytes(B, n_rows, kv_len, Hq, D)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    out = torch.empty_like(q) if out is None else out
    _check_like("out", out, q)
    check(lib().kb_attn_decode_multi(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(), B, n_rows,
                                     kv_len, k_cache.shape[2], Hq, k_cache.shape[1], D, _scale(scale, D), ws_ptr,
                                     ws_bytes, _stream(q)))
    return out


def _check_packed(name, x):
    _check_tensor(name, x, ndim=3)
    if x.shape[2] != HEAD_DIM:
        raise ValueError(f"{name} must be [heads, rows, {HEAD_DIM}]")


def prefill_varlen(q, k, v, cu_seqlens, scale: float | None = None, out=None):
    """Ragged causal prefill.  q [Hq, T, 128], k/v [Hkv, T, 128] packed
    head-major; sequence i owns rows cu_seqlens[i] .. cu_seqlens[i+1] - 1
    (host list of batch + 1 offsets, T = cu_seqlens[-1])."""
    for n, x in (("q", q), ("k", k), ("v", v)):
        _check_packed(n, x)
    _same_device(("q", q), ("k", k), ("v", v))
    if k.shape != v.shape or k.shape[1] != q.shape[1]:
        raise ValueError("k/v must be [Hkv, T, 128] with the rows of q")
    cu = _host_i64(cu_seqlens)
    if int(cu_seqlens[-1]) != q.shape[1]:
        raise ValueError("cu_seqlens[-1] must equal the packed row count")
    out = _torch().empty_like(q) if out is None else out
    _check_like("out", out, q, ndim=3)
    check(lib().kb_attn_prefill_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), cu,
                                       len(cu_seqlens) - 1, q.shape[0], k.shape[0], HEAD_DIM,
                                       _scale(scale, HEAD_DIM), _stream(q)))
    return out


def partitioned_varlen(q, k_cache, v_cache, cu_q, cu_cache, kv_lens, scale: float | None = None, out=None):
    """Ragged partitioned forward.  q [Hq, cu_q[-1], 128]; caches [Hkv,
    cu_cache[-1], 128]; sequence i has cu_q[i+1] - cu_q[i] query rows ending at
    position kv_lens[i] - 1, against the first kv_lens[i] rows of its cache
    range cu_cache[i] .. cu_cache[i+1] - 1 (host lists)."""
    for n, x in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _check_packed(n, x)
    _same_device(("q", q), ("k_cache", k_cache), ("v_cache", v_cache))
    if k_cache.shape != v_cache.shape:
        raise ValueError("cache shape mismatch")
    if int(cu_q[-1]) != q.shape[1] or int(cu_cache[-1]) != k_cache.shape[1]:
        raise ValueError("offsets do not match the packed row counts")
    batch = len(cu_q) - 1
    if len(cu_cache) != batch + 1 or len(kv_lens) != batch:
        raise ValueError("cu_q, cu_cache and kv_lens describe different batch sizes")
    a_q, a_c, a_l = _host_i64(cu_q), _host_i64(cu_cache), _host_i64(kv_lens)
    out = _torch().empty_like(q) if out is None else out
    _check_like("out", out, q, ndim=3)
    check(lib().kb_attn_partitioned_varlen(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(),
                                           a_q, a_c, a_l, batch, q.shape[0], k_cache.shape[0], HEAD_DIM,
                                           _scale(scale, HEAD_DIM), _stream(q)))
    return out


def decode_varlen(q, k_cache, v_cache, cu_cache, kv_lens, scale: float | None = None, out=None, workspace=None):
    """Ragged one-token decode.  q [Hq, batch, 128] (row i is sequence i's
    token at position kv_lens[i] - 1); caches [Hkv, cu_cache[-1], 128]."""
    torch = _torch()
    for n, x in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _check_packed(n, x)
    _same_device(("q", q), ("k_cache", k_cache), ("v_cache", v_cache))
    batch = q.shape[1]
    if len(cu_cache) != batch + 1 or len(kv_lens) != batch or int(cu_cache[-1]) != k_cache.shape[1]:
        raise ValueError("cu_cache / kv_lens do not match q and the caches")
    need = decode_varlen_workspace_bytes(kv_lens, q.shape[0])
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    a_c, a_l = _host_i64(cu_cache), _host_i64(kv_lens)
    out = torch.empty_like(q) if out is None else out
    _check_like("out", out, q, ndim=3)
    check(lib().kb_attn_decode_varlen(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(), a_c,
                                      a_l, batch, q.shape[0], k_cache.shape[0], HEAD_DIM, _scale(scale, HEAD_DIM),
                                      ws_ptr, ws_bytes, _stream(q)))
    return out


def decode_paged(q, k_pages, v_pages, block_table, kv_lens, scale: float | None = None, out=None, workspace=None):
    """One-token decode over a paged cache.  q [B, Hq, 128]; pools [n_pages,
    Hkv, page_size, 128]; block_table int32 [B, max_pages] on the GPU; kv_lens
    a host list.  Key j of sequence i is row j % page_size of page
    block_table[i, j // page_size]."""
    torch = _torch()
    _check_tensor("q", q, ndim=3)
    _check_tensor("k_pages", k_pages)
    _check_tensor("v_pages", v_pages)
    if k_pages.shape != v_pages.shape or k_pages.shape[3] != HEAD_DIM or q.shape[2] != HEAD_DIM:
        raise ValueError("page pools must be [n_pages, Hkv, page_size, 128] and q [B, Hq, 128]")
    if (not isinstance(block_table, torch.Tensor) or block_table.dtype != torch.int32 or not block_table.is_cuda
            or block_table.dim() != 2 or not block_table.is_contiguous() or block_table.shape[0] != q.shape[0]):
        raise ValueError("block_table must be a contiguous int32 [B, max_pages] tensor on the GPU")
    _same_device(("q", q), ("k_pages", k_pages), ("v_pages", v_pages), ("block_table", block_table))
    B, Hq = q.shape[0], q.shape[1]
    if len(kv_lens) != B:
        raise ValueError("kv_lens must have one entry per sequence")
    need = decode_varlen_workspace_bytes(kv_lens, Hq)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    a_l = _host_i64(kv_lens)
    out = torch.empty_like(q) if out is None else out
    _check_like("out", out, q, ndim=3)
    check(lib().kb_attn_decode_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), out.data_ptr(),
                                     block_table.data_ptr(), block_table.shape[1], a_l, B, k_pages.shape[0],
                                     k_pages.shape[2], Hq, k_pages.shape[1], HEAD_DIM, _scale(scale, HEAD_DIM), ws_ptr,
                                     ws_bytes, _stream(q)))
    return out


def _lse_out(lse, shape, like):
    torch = _torch()
    if lse is None:
        return torch.empty(shape, dtype=torch.float32, device=like.device)
    if (not isinstance(lse, torch.Tensor) or lse.dtype != torch.float32 or not lse.is_cuda
            or tuple(lse.shape) != tuple(shape) or not lse.is_contiguous()):
        raise ValueError(f"lse must be a contiguous float32 GPU tensor of shape {tuple(shape)}")
    return lse


def _check_lse_in(lse, shape, layout):
    torch = _torch()
    if (not isinstance(lse, torch.Tensor) or lse.dtype != torch.float32 or not lse.is_cuda
            or tuple(lse.shape) != tuple(shape) or not lse.is_contiguous()):
        raise ValueError(f"lse must be the contiguous float32 {layout} GPU tensor of the forward")


def prefill_lse(q, k, v, scale: float | None = None, out=None, lse=None):
    """prefill() that also returns the fp32 log-sum-exp of every row, [B, Hq, S]."""
    for n, x in (("q", q), ("k", k), ("v", v)):
        _check_tensor(n, x)
    _same_device(("q", q), ("k", k), ("v", v))
    B, Hq, S, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != S or k.shape[3] != D:
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    out = _torch().empty_like(q) if out is None else out
    _check_like("out", out, q)
    lse = _lse_out(lse, (B, Hq, S), q)
    check(lib().kb_attn_prefill_lse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, S,
                                    Hq, k.shape[1], D, _scale(scale, D), _stream(q)))
    return out, lse


def partitioned_lse(q, k_cache, v_cache, kv_len: int, scale: float | None = None, out=None, lse=None):
    """partitioned() that also returns the fp32 log-sum-exp of every row, [B, Hq, q_len]."""
    for n, x in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _check_tensor(n, x)
    _same_device(("q", q), ("k_cache", k_cache), ("v_cache", v_cache))
    B, Hq, q_len, D = q.shape
    if k_cache.shape != v_cache.shape or k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError("cache shape mismatch")
    out = _torch().empty_like(q) if out is None else out
    _check_like("out", out, q)
    lse = _lse_out(lse, (B, Hq, q_len), q)
    check(lib().kb_attn_partitioned_lse(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(),
                                        lse.data_ptr(), B, q_len, int(kv_len), k_cache.shape[2], Hq,
                                        k_cache.shape[1], D, _scale(scale, D), _stream(q)))
    return out, lse


def decode_lse(q, k_cache, v_cache, kv_len: int | None = None, scale: float | None = None, out=None, lse=None,
               workspace=None):
    """decode() that also returns the fp32 log-sum-exp of every row, [B, Hq, 1]."""
    torch = _torch()
    for n, x in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _check_tensor(n, x)
    _same_device(("q", q), ("k_cache", k_cache), ("v_cache", v_cache))
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
    _check_like("out", out, q)
    lse = _lse_out(lse, (B, Hq, 1), q)
    check(lib().kb_attn_decode_lse(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(),
                                   lse.data_ptr(), B, kv_len, k_cache.shape[2], Hq, k_cache.shape[1], D,
                                   _scale(scale, D), ws_ptr, ws_bytes, _stream(q)))
    return out, lse


def backward_workspace_bytes(batch: int, seq_len: int, n_q_heads: int = 32, head_dim: int = HEAD_DIM) -> int:
    return int(lib().kb_attn_backward_workspace_bytes(batch, seq_len, n_q_heads, head_dim))


def backward(q, k, v, out, dout, lse, scale: float | None = None, dq=None, dk=None, dv=None, workspace=None):
    """Gradients (dq, dk, dv) of the causal full-sequence forward for the
    upstream gradient dout, from the forward's out and lse (prefill_lse)."""
    torch = _torch()
    for n, x in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        _check_tensor(n, x)
    _same_device(("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout))
    B, Hq, S, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != S or k.shape[3] != D:
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    if out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("out and dout must be shaped like q")
    _check_lse_in(lse, (B, Hq, S), "[B, Hq, S]")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for n, x, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_like(n, x, like)
    need = backward_workspace_bytes(B, S, Hq, D)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    check(lib().kb_attn_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                                 lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, S, Hq, k.shape[1], D,
                                 _scale(scale, D), workspace.data_ptr(), ws_bytes, _stream(q)))
    return dq, dk, dv


def prefill_varlen_lse(q, k, v, cu_seqlens, scale: float | None = None, out=None, lse=None):
    """prefill_varlen() that also returns the fp32 log-sum-exp of every row, [Hq, T]."""
    for n, x in (("q", q), ("k", k), ("v", v)):
        _check_packed(n, x)
    _same_device(("q", q), ("k", k), ("v", v))
    if k.shape != v.shape or k.shape[1] != q.shape[1]:
        raise ValueError("k/v must be [Hkv, T, 128] with the rows of q")
    if int(cu_seqlens[-1]) != q.shape[1]:
        raise ValueError("cu_seqlens[-1] must equal the packed row count")
    cu = _host_i64(cu_seqlens)
    out = _torch().empty_like(q) if out is None else out
    _check_like("out", out, q, ndim=3)
    lse = _lse_out(lse, (q.shape[0], q.shape[1]), q)
    check(lib().kb_attn_prefill_varlen_lse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                           cu, len(cu_seqlens) - 1, q.shape[0], k.shape[0], HEAD_DIM,
                                           _scale(scale, HEAD_DIM), _stream(q)))
    return out, lse


def backward_varlen_workspace_bytes(cu_seqlens, n_q_heads: int = 32, head_dim: int = HEAD_DIM) -> int:
    cu = _host_i64(cu_seqlens)
    return int(lib().kb_attn_backward_varlen_workspace_bytes(cu, len(cu_seqlens) - 1, n_q_heads, head_dim))


def backward_varlen(q, k, v, out, dout, lse, cu_seqlens, scale: float | None = None, dq=None, dk=None, dv=None,
                    workspace=None):
    """Gradients of the ragged causal prefill: packed q, out, dout [Hq, T,
    128], k, v [Hkv, T, 128], lse [Hq, T] from prefill_varlen_lse; sequence i
    is rows cu_seqlens[i] .. cu_seqlens[i+1] - 1 (host list)."""
    torch = _torch()
    for n, x in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        _check_packed(n, x)
    _same_device(("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout))
    T = q.shape[1]
    if k.shape != v.shape or k.shape[1] != T or out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("packed shapes do not match")
    if int(cu_seqlens[-1]) != T:
        raise ValueError("cu_seqlens[-1] must equal the packed row count")
    _check_lse_in(lse, (q.shape[0], T), "[Hq, T]")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for n, x, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_like(n, x, like, ndim=3)
    need = backward_varlen_workspace_bytes(cu_seqlens, q.shape[0])
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    cu = _host_i64(cu_seqlens)
    check(lib().kb_attn_backward_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                                        lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), cu,
                                        len(cu_seqlens) - 1, q.shape[0], k.shape[0], HEAD_DIM,
                                        _scale(scale, HEAD_DIM), ws_ptr, ws_bytes, _stream(q)))
    return dq, dk, dv


def attention(q, k, v, scale: float | None = None):
    """Differentiable causal attention: forward through prefill_lse, backward
    through backward (torch autograd glue only)."""
    torch = _torch()

    class _Attention(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q_, k_, v_):
            o, lse = prefill_lse(q_, k_, v_, scale)
            ctx.save_for_backward(q_, k_, v_, o, lse)
            return o

        @staticmethod
        def backward(ctx, do):
            q_, k_, v_, o, lse = ctx.saved_tensors
            return backward(q_, k_, v_, o, do.contiguous(), lse, scale)

    return _Attention.apply(q, k, v)


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


__all__ = ["prefill", "partitioned", "decode", "decode_static", "unified_prefill", "unified_decode", "contract",
           "decode_workspace_bytes", "prefill_varlen", "partitioned_varlen", "decode_varlen",
           "decode_varlen_workspace_bytes", "decode_paged", "prefill_lse", "partitioned_lse", "decode_lse",
           "decode_multi", "decode_multi_workspace_bytes", "backward", "backward_workspace_bytes", "prefill_varlen_lse", "backward_varlen",
           "backward_varlen_workspace_bytes", "attention", "lib", "check", "KBAttnError", "LIB_PATH"]
