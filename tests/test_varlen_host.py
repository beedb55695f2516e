"""Ragged entry points on the host: malformed calls are rejected before any
device query or launch (CPU only, fake device addresses)."""
import ctypes

import pytest

import bitwise_aligned_causal_amd as kb
from test_abi_host import ALIAS, ALIGN, INVALID, LENGTH, O, OK, Q, SCALE, UNSUPPORTED, V, W, WORKSPACE, K


def arr(values):
    return (ctypes.c_int64 * max(1, len(values)))(*values)


def prefill_v(offs=(0, 5, 70, 200), **kw):
    a = dict(q=Q, k=K, v=V, o=O, hq=32, hkv=8, d=128, scale=SCALE, batch=len(offs) - 1, cu=arr(list(offs)))
    a.update(kw)
    return kb.lib().kb_attn_prefill_varlen(a["q"], a["k"], a["v"], a["o"], a["cu"], a["batch"], a["hq"], a["hkv"],
                                           a["d"], a["scale"], None)


def part_v(cu_q=(0, 3, 10), cu_c=(0, 64, 200), lens=(20, 130), **kw):
    a = dict(q=Q, k=K, v=V, o=O, hq=32, hkv=8, d=128, scale=SCALE, batch=len(lens), cq=arr(list(cu_q)),
             cc=arr(list(cu_c)), kl=arr(list(lens)))
    a.update(kw)
    return kb.lib().kb_attn_partitioned_varlen(a["q"], a["k"], a["v"], a["o"], a["cq"], a["cc"], a["kl"],
                                               a["batch"], a["hq"], a["hkv"], a["d"], a["scale"], None)


def decode_v(cu_c=(0, 64, 3000), lens=(20, 2100), ws=W, ws_bytes=1 << 24, **kw):
    # kw may replace any argument, including the host arrays (cc, kl) by None
    a = dict(q=Q, k=K, v=V, o=O, hq=32, hkv=8, d=128, scale=SCALE, batch=len(lens), cc=arr(list(cu_c)),
             kl=arr(list(lens)))
    a.update(kw)
    return kb.lib().kb_attn_decode_varlen(a["q"], a["k"], a["v"], a["o"], a["cc"], a["kl"], a["batch"], a["hq"],
                                          a["hkv"], a["d"], a["scale"], ws, ws_bytes, None)


@pytest.mark.parametrize("call", [prefill_v, part_v, decode_v])
@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), INVALID), (dict(o=None), INVALID), (dict(batch=0), INVALID), (dict(scale=0.0), INVALID),
    (dict(d=64), UNSUPPORTED), (dict(hq=16), UNSUPPORTED),
    (dict(q=ctypes.c_void_p(Q.value + 2)), ALIGN), (dict(o=Q), ALIAS), (dict(o=K), ALIAS),
])
def test_rejected_before_launch(call, kw, expect):
    assert call(**kw) == expect


def test_null_host_arrays():
    assert prefill_v(cu=None) == INVALID
    assert part_v(cq=None) == INVALID
    assert part_v(cc=None) == INVALID
    assert part_v(kl=None) == INVALID
    assert decode_v(cc=None) == INVALID
    assert decode_v(kl=None) == INVALID


@pytest.mark.parametrize("cu", [(0, 5, 4), (-1, 5, 9), (0, 10, 9, 20)])
def test_prefill_offsets_must_not_decrease(cu):
    assert prefill_v(offs=cu) == LENGTH


@pytest.mark.parametrize("cu_q,cu_c,lens", [
    ((0, 3, 10), (0, 64, 200), (2, 130)),     # q_len 3 > kv_len 2
    ((0, 3, 10), (0, 64, 200), (65, 130)),    # kv_len 65 > capacity 64
    ((0, 3, 10), (0, 64, 200), (20, -1)),     # negative kv_len
    ((0, 3, 2), (0, 64, 200), (20, 130)),     # decreasing query offsets
    ((0, 3, 10), (0, 64, 60), (20, 130)),     # decreasing cache offsets
])
def test_partitioned_lengths(cu_q, cu_c, lens):
    assert part_v(cu_q=cu_q, cu_c=cu_c, lens=lens) == LENGTH


@pytest.mark.parametrize("cu_c,lens", [((0, 64, 3000), (0, 2100)), ((0, 64, 3000), (65, 2100))])
def test_decode_lengths(cu_c, lens):
    assert decode_v(cu_c=cu_c, lens=lens) == LENGTH


def test_decode_workspace():
    lens = [100, 1025, 5000]
    need = kb.decode_varlen_workspace_bytes(lens)
    assert need == 32 * (2 + 5) * 130 * 4
    assert kb.decode_varlen_workspace_bytes([1, 1024]) == 0
    assert kb.decode_varlen_workspace_bytes([0, 5]) == 0  # invalid length
    cu_c = (0, 100, 1200, 6200)
    assert decode_v(cu_c=cu_c, lens=lens, ws=None) == WORKSPACE
    assert decode_v(cu_c=cu_c, lens=lens, ws_bytes=need - 1) == WORKSPACE
    assert decode_v(cu_c=cu_c, lens=lens, ws=ctypes.c_void_p(W.value + 4), ws_bytes=need) == ALIGN
    assert decode_v(cu_c=cu_c, lens=lens, ws=O, ws_bytes=need) == ALIAS


def test_binding_checks_offsets_against_tensors():
    import torch

    q = torch.zeros(32, 10, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        kb.prefill_varlen(q, q[:8], q[:8], [0, 5, 10])  # CPU tensors are refused


def paged(lens=(100, 3000), page_size=64, max_pages=64, n_pages=200, table=None, ws=W, ws_bytes=1 << 24, **kw):
    a = dict(q=Q, k=K, v=V, o=O, hq=32, hkv=8, d=128, scale=SCALE, batch=len(lens), kl=arr(list(lens)),
             table=ctypes.c_void_p(0x20_0000_0000) if table is None else table)
    a.update(kw)
    return kb.lib().kb_attn_decode_paged(a["q"], a["k"], a["v"], a["o"], a["table"], max_pages, a["kl"], a["batch"],
                                         n_pages, page_size, a["hq"], a["hkv"], a["d"], a["scale"], ws, ws_bytes, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), INVALID), (dict(table=ctypes.c_void_p(0)), INVALID), (dict(kl=None), INVALID),
    (dict(batch=0), INVALID), (dict(max_pages=0), INVALID), (dict(n_pages=0), INVALID),
    (dict(page_size=32), UNSUPPORTED), (dict(page_size=100), UNSUPPORTED), (dict(d=64), UNSUPPORTED),
    (dict(lens=(0, 10)), LENGTH), (dict(lens=(64 * 64 + 1, 10)), LENGTH),
    (dict(table=ctypes.c_void_p(0x20_0000_0002)), ALIGN), (dict(q=ctypes.c_void_p(Q.value + 4)), ALIGN),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=100), WORKSPACE),
    (dict(o=Q), ALIAS), (dict(o=ctypes.c_void_p(0x20_0000_0000)), ALIAS),
])
def test_paged_rejected_before_launch(kw, expect):
    base = dict(lens=(100, 3000), page_size=64, max_pages=64, n_pages=200)
    for key in list(kw):
        if key in base:
            base[key] = kw.pop(key)
    assert paged(**base, **kw) == expect
