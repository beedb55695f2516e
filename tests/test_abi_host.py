"""The C-ABI library on the host: it loads, exports every declared symbol and
rejects malformed calls before touching the GPU (CPU only, no compute)."""
import ctypes
import os
import re

import pytest

import bitwise_aligned_causal_amd as kb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kb_attn.h")

OK, INVALID, UNSUPPORTED, LENGTH, ALIGN, DEVICE, WORKSPACE, ALIAS, HIP, SCRATCH = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9
SCALE = 128 ** -0.5

# fake, aligned, non-overlapping "device" addresses: every call below must
# return before dereferencing or querying them
Q, K, V, O, W = (ctypes.c_void_p(0x10_0000_0000 + i * 0x1_0000_0000) for i in range(5))


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*|void)\s+(kb_attn_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"kb_attn_prefill", "kb_attn_partitioned", "kb_attn_decode", "kb_attn_decode_workspace_bytes",
            "kb_attn_strerror", "kb_attn_contract"} <= set(names)
    lib = kb.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_contract_matches_header():
    text = open(HEADER).read()
    tile = int(re.search(r"#define KB_ATTN_KV_TILE (\d+)", text).group(1))
    chunk = int(re.search(r"#define KB_ATTN_KV_CHUNK (\d+)", text).group(1))
    c = kb.contract()
    assert (c["kv_tile"], c["kv_chunk"]) == (tile, chunk) == (64, 1024)
    kb.lib().kb_attn_contract(None, None, None)  # NULL outputs are allowed


def test_strerror():
    for code in (OK, INVALID, UNSUPPORTED, LENGTH, ALIGN, DEVICE, WORKSPACE, ALIAS, HIP, 12345):
        assert kb.lib().kb_attn_strerror(code)


@pytest.mark.parametrize("batch,kv_len,expect", [
    (1, 1, 0), (1, 1024, 0), (16, 8192, 16 * 32 * 8 * 130 * 4), (4, 1025, 4 * 32 * 2 * 130 * 4),
    (0, 100, 0), (1, 0, 0),
])
def test_workspace_bytes(batch, kv_len, expect):
    assert kb.decode_workspace_bytes(batch, kv_len) == expect


def prefill(**kw):
    a = dict(q=Q, k=K, v=V, o=O, batch=1, seq=16, hq=32, hkv=8, d=128, scale=SCALE)
    a.update(kw)
    return kb.lib().kb_attn_prefill(a["q"], a["k"], a["v"], a["o"], a["batch"], a["seq"], a["hq"], a["hkv"],
                                    a["d"], a["scale"], None)


def partitioned(**kw):
    a = dict(q=Q, k=K, v=V, o=O, batch=1, q_len=8, kv_len=16, cap=16, hq=32, hkv=8, d=128, scale=SCALE)
    a.update(kw)
    return kb.lib().kb_attn_partitioned(a["q"], a["k"], a["v"], a["o"], a["batch"], a["q_len"], a["kv_len"],
                                        a["cap"], a["hq"], a["hkv"], a["d"], a["scale"], None)


def decode(**kw):
    a = dict(q=Q, k=K, v=V, o=O, batch=1, kv_len=2048, cap=4096, hq=32, hkv=8, d=128, scale=SCALE, ws=W,
             ws_bytes=1 << 20)
    a.update(kw)
    return kb.lib().kb_attn_decode(a["q"], a["k"], a["v"], a["o"], a["batch"], a["kv_len"], a["cap"], a["hq"],
                                   a["hkv"], a["d"], a["scale"], a["ws"], a["ws_bytes"], None)


def decode_static(**kw):
    a = dict(q=Q, k=K, v=V, o=O, batch=1, kv_len=2048, cap=4096, hq=32, hkv=8, d=128, scale=SCALE)
    a.update(kw)
    return kb.lib().kb_attn_decode_static(a["q"], a["k"], a["v"], a["o"], a["batch"], a["kv_len"], a["cap"],
                                          a["hq"], a["hkv"], a["d"], a["scale"], None)


@pytest.mark.parametrize("call", [prefill, partitioned, decode, decode_static])
@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID), (dict(o=None), INVALID),
    (dict(batch=0), INVALID), (dict(scale=0.0), INVALID), (dict(scale=-1.0), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(d=64), UNSUPPORTED), (dict(hq=16), UNSUPPORTED), (dict(hq=32, hkv=4), UNSUPPORTED),
    (dict(hkv=0), INVALID),
    (dict(q=ctypes.c_void_p(Q.value + 2)), ALIGN), (dict(o=ctypes.c_void_p(O.value + 8)), ALIGN),
    (dict(o=Q), ALIAS), (dict(o=K), ALIAS), (dict(o=V), ALIAS),
])
def test_rejected_before_launch(call, kw, expect):
    assert call(**kw) == expect


@pytest.mark.parametrize("kw", [dict(q_len=0), dict(q_len=17), dict(kv_len=17), dict(cap=1 << 31, kv_len=1 << 31)])
def test_partitioned_lengths(kw):
    assert partitioned(**kw) == LENGTH


@pytest.mark.parametrize("kw", [dict(kv_len=0), dict(kv_len=4097), dict(cap=(1 << 30) + 1)])
def test_decode_lengths(kw):
    assert decode(**kw) == LENGTH


def test_prefill_length():
    assert prefill(seq=0) == INVALID
    assert prefill(seq=(1 << 30) + 1) == LENGTH


def test_decode_workspace_checks():
    need = kb.decode_workspace_bytes(1, 2048)
    assert decode(ws=None) == WORKSPACE
    assert decode(ws_bytes=need - 1) == WORKSPACE
    assert decode(ws=ctypes.c_void_p(W.value + 4)) == ALIGN
    assert decode(ws=O, ws_bytes=need) == ALIAS
    assert decode(ws=ctypes.c_void_p(K.value + 64)) == ALIAS


def test_python_binding_refuses_cpu_tensors():
    import torch

    q = torch.zeros(1, 32, 4, 128, dtype=torch.bfloat16)
    k = torch.zeros(1, 8, 4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        kb.prefill(q, k, k)
    with pytest.raises(ValueError):
        kb.decode(q[:, :, :1].contiguous(), k, k)


# ---- log-sum-exp entry points and the backward --------------------------------
L = ctypes.c_void_p(0x10_0000_0000 + 5 * 0x1_0000_0000)


def prefill_lse(**kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, batch=1, seq=16, hq=32, hkv=8, d=128, scale=SCALE)
    a.update(kw)
    return kb.lib().kb_attn_prefill_lse(a["q"], a["k"], a["v"], a["o"], a["lse"], a["batch"], a["seq"], a["hq"],
                                        a["hkv"], a["d"], a["scale"], None)


def partitioned_lse(**kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, batch=1, q_len=8, kv_len=16, cap=16, hq=32, hkv=8, d=128, scale=SCALE)
    a.update(kw)
    return kb.lib().kb_attn_partitioned_lse(a["q"], a["k"], a["v"], a["o"], a["lse"], a["batch"], a["q_len"],
                                            a["kv_len"], a["cap"], a["hq"], a["hkv"], a["d"], a["scale"], None)


def decode_lse(**kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, batch=1, kv_len=2048, cap=4096, hq=32, hkv=8, d=128, scale=SCALE, ws=W,
             ws_bytes=1 << 20)
    a.update(kw)
    return kb.lib().kb_attn_decode_lse(a["q"], a["k"], a["v"], a["o"], a["lse"], a["batch"], a["kv_len"], a["cap"],
                                       a["hq"], a["hkv"], a["d"], a["scale"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("call", [prefill_lse, partitioned_lse, decode_lse])
@pytest.mark.parametrize("kw,expect", [
    (dict(lse=None), INVALID), (dict(q=None), INVALID), (dict(d=64), UNSUPPORTED),
    (dict(lse=ctypes.c_void_p(L.value + 2)), ALIGN),
    (dict(lse=Q), ALIAS), (dict(lse=ctypes.c_void_p(O.value + 4)), ALIAS), (dict(lse=K), ALIAS),
])
def test_lse_rejected_before_launch(call, kw, expect):
    assert call(**kw) == expect


def test_decode_lse_must_not_overlap_workspace():
    assert decode_lse(lse=ctypes.c_void_p(W.value + 64)) == ALIAS


DQ, DK, DV, DO = (ctypes.c_void_p(0x20_0000_0000 + i * 0x1_0000_0000) for i in range(4))


def backward(**kw):
    a = dict(q=Q, k=K, v=V, o=O, do=DO, lse=L, dq=DQ, dk=DK, dv=DV, batch=2, seq=300, hq=32, hkv=8, d=128,
             scale=SCALE, ws=W, ws_bytes=1 << 20)
    a.update(kw)
    return kb.lib().kb_attn_backward(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                                     a["batch"], a["seq"], a["hq"], a["hkv"], a["d"], a["scale"], a["ws"],
                                     a["ws_bytes"], None)


def test_backward_workspace_bytes():
    # D and lse2 per row, rows padded to a multiple of 64
    assert kb.backward_workspace_bytes(2, 300) == 2 * 2 * 32 * 320 * 4
    assert kb.backward_workspace_bytes(1, 64) == 2 * 32 * 64 * 4
    assert kb.backward_workspace_bytes(0, 64) == 0
    assert kb.backward_workspace_bytes(1, 0) == 0
    assert kb.lib().kb_attn_backward_workspace_bytes(1, 64, 32, 64) == 0


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), INVALID), (dict(do=None), INVALID), (dict(lse=None), INVALID), (dict(dq=None), INVALID),
    (dict(dk=None), INVALID), (dict(dv=None), INVALID), (dict(o=None), INVALID),
    (dict(batch=0), INVALID), (dict(seq=0), INVALID), (dict(scale=0.0), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(d=64), UNSUPPORTED), (dict(hq=16), UNSUPPORTED), (dict(seq=(1 << 30) + 1), LENGTH),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=2 * 2 * 32 * 320 * 4 - 1), WORKSPACE),
    (dict(dq=ctypes.c_void_p(DQ.value + 8)), ALIGN), (dict(lse=ctypes.c_void_p(L.value + 2)), ALIGN),
    (dict(ws=ctypes.c_void_p(W.value + 4)), ALIGN),
    (dict(dq=Q), ALIAS), (dict(dk=V), ALIAS), (dict(dv=DK), ALIAS), (dict(dq=DO), ALIAS),
    (dict(dk=ctypes.c_void_p(L.value + 16)), ALIAS), (dict(ws=ctypes.c_void_p(DV.value + 4096)), ALIAS),
    (dict(dv=O), ALIAS),
])
def test_backward_rejected_before_launch(kw, expect):
    assert backward(**kw) == expect


def backward_varlen(cu=(0, 100, 164, 300), **kw):
    a = dict(q=Q, k=K, v=V, o=O, do=DO, lse=L, dq=DQ, dk=DK, dv=DV, hq=32, hkv=8, d=128, scale=SCALE, ws=W,
             ws_bytes=1 << 20)
    a.update(kw)
    arr = (ctypes.c_int64 * len(cu))(*cu)
    return kb.lib().kb_attn_backward_varlen(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"],
                                            a["dv"], arr, len(cu) - 1, a["hq"], a["hkv"], a["d"], a["scale"], a["ws"],
                                            a["ws_bytes"], None)


def test_backward_varlen_workspace_bytes():
    # each sequence padded to a multiple of 64 rows: 128 + 64 + 192 = 384
    assert kb.backward_varlen_workspace_bytes([0, 100, 164, 300]) == 2 * 32 * 384 * 4
    assert kb.backward_varlen_workspace_bytes([0, 0, 0]) == 0
    assert kb.backward_varlen_workspace_bytes([0, 5, 3]) == 0  # decreasing offsets


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), INVALID), (dict(lse=None), INVALID), (dict(dv=None), INVALID), (dict(scale=0.0), INVALID),
    (dict(d=64), UNSUPPORTED), (dict(hq=16), UNSUPPORTED),
    (dict(cu=(0, 10, 5)), LENGTH), (dict(cu=(-1, 10)), LENGTH), (dict(cu=(0, (1 << 30) + 1)), LENGTH),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=2 * 32 * 384 * 4 - 1), WORKSPACE),
    (dict(dq=ctypes.c_void_p(DQ.value + 8)), ALIGN), (dict(lse=ctypes.c_void_p(L.value + 1)), ALIGN),
    (dict(dq=Q), ALIAS), (dict(dv=DK), ALIAS), (dict(ws=ctypes.c_void_p(DO.value + 64)), ALIAS),
])
def test_backward_varlen_rejected_before_launch(kw, expect):
    assert backward_varlen(**kw) == expect


def test_prefill_varlen_lse_rejected_before_launch():
    cu = (ctypes.c_int64 * 3)(0, 10, 30)
    f = kb.lib().kb_attn_prefill_varlen_lse
    assert f(Q, K, V, O, None, cu, 2, 32, 8, 128, SCALE, None) == INVALID
    assert f(Q, K, V, O, ctypes.c_void_p(L.value + 2), cu, 2, 32, 8, 128, SCALE, None) == ALIGN
    assert f(Q, K, V, O, ctypes.c_void_p(O.value + 64), cu, 2, 32, 8, 128, SCALE, None) == ALIAS


def decode_multi(**kw):
    a = dict(q=Q, k=K, v=V, o=O, batch=1, rows=4, kv_len=2048, cap=4096, hq=32, hkv=8, d=128, scale=SCALE, ws=W,
             ws_bytes=1 << 20)
    a.update(kw)
    return kb.lib().kb_attn_decode_multi(a["q"], a["k"], a["v"], a["o"], a["batch"], a["rows"], a["kv_len"], a["cap"],
                                         a["hq"], a["hkv"], a["d"], a["scale"], a["ws"], a["ws_bytes"], None)


def test_decode_multi_workspace_bytes():
    assert kb.decode_multi_workspace_bytes(2, 3, 2048) == 2 * 32 * 3 * 2 * 130 * 4
    assert kb.decode_multi_workspace_bytes(2, 3, 1024) == 0
    assert kb.decode_multi_workspace_bytes(1, 1, 5000) == kb.decode_workspace_bytes(1, 5000)
    assert kb.decode_multi_workspace_bytes(1, 9, 5000) == 0
    assert kb.decode_multi_workspace_bytes(1, 4, 3) == 0


@pytest.mark.parametrize("kw,expect", [
    (dict(rows=0), UNSUPPORTED), (dict(rows=9), UNSUPPORTED), (dict(kv_len=3), LENGTH),
    (dict(kv_len=4097), LENGTH), (dict(q=None), INVALID), (dict(d=64), UNSUPPORTED),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=32 * 4 * 2 * 130 * 4 - 1), WORKSPACE),
    (dict(o=Q), ALIAS), (dict(o=ctypes.c_void_p(O.value + 8)), ALIGN),
])
def test_decode_multi_rejected_before_launch(kw, expect):
    assert decode_multi(**kw) == expect


@pytest.mark.parametrize("kw", [dict(kv_len=0), dict(kv_len=4097), dict(cap=(1 << 30) + 1)])
def test_decode_static_lengths(kw):
    assert decode_static(**kw) == LENGTH


def test_decode_static_scratch_limit():
    # 8 MiB holds 16131 partial rows of 130 floats: batch 1 with 32 heads fits
    # 504 chunks.  At the limit the size check passes and the (fake) pointers
    # fail the device check; one key more needs a 505th chunk and is refused
    # for its size, before any device query.
    limit = 504 * 1024
    assert kb.decode_workspace_bytes(1, limit) <= kb.DECODE_STATIC_SCRATCH_BYTES
    assert kb.decode_workspace_bytes(1, limit + 1) > kb.DECODE_STATIC_SCRATCH_BYTES
    assert decode_static(kv_len=limit, cap=limit) == DEVICE
    assert decode_static(kv_len=limit + 1, cap=limit + 1) == SCRATCH
    assert decode_static(batch=16, kv_len=31 * 1024, cap=31 * 1024) == DEVICE
    assert decode_static(batch=16, kv_len=31 * 1024 + 1, cap=32 * 1024) == SCRATCH
    assert b"scratch" in kb.lib().kb_attn_strerror(SCRATCH)
    # the header's size and the binding's agree
    text = open(HEADER).read()
    assert re.search(r"#define KB_ATTN_DECODE_STATIC_SCRATCH_BYTES \(8u << 20\)", text)
    assert kb.DECODE_STATIC_SCRATCH_BYTES == 8 << 20
