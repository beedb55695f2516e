"""kb_attn_decode_static (no workspace argument, library-held per-GPU
scratch) against kb_attn_decode with a caller workspace: bit for bit, on
consecutive calls that reuse the scratch (a large call, then a smaller one),
at the scratch's size limit, and a refused oversize call."""
import ctypes

import numpy as np
import pytest

import kb_gen
from gpu_util import bits, dev, note

pytestmark = pytest.mark.gpu


def _inputs(seed, batch, cap, n_kv_heads=8):
    q, k, v = kb_gen.attention_inputs(seed, batch, cap, 4 * n_kv_heads, n_kv_heads, 128)
    return dev(q), dev(k), dev(v)


def _both(kb, qd, kd, vd, kv_len):
    qt = qd[:, :, kv_len - 1:kv_len].contiguous()
    ref = kb.decode(qt, kd, vd, kv_len=kv_len)
    got = kb.decode_static(qt, kd, vd, kv_len=kv_len)
    return bits(got), bits(ref)


def test_static_decode_matches_workspace_decode_on_consecutive_calls():
    import bitwise_aligned_causal_amd as kb

    # a large call (B=16, 8 chunks: 2.1 MB of partials), then smaller ones
    # that reuse the front of the same scratch, then a one-chunk call
    cases = [(16, 8192, 8192, 71), (2, 3000, 4096, 72), (3, 1025, 1500, 73), (1, 700, 700, 74),
             (16, 8192, 8192, 75)]
    for batch, kv_len, cap, seed in cases:
        note(f"decode_static B={batch} kv_len={kv_len} cap={cap} seed={seed}")
        qd, kd, vd = _inputs(seed, batch, cap)
        got, ref = _both(kb, qd, kd, vd, kv_len)
        assert np.array_equal(got, ref), f"B={batch} kv_len={kv_len}: {int((got != ref).sum())} bits differ"


def test_static_decode_at_the_scratch_limit():
    import torch

    import bitwise_aligned_causal_amd as kb

    # batch 1 with 32 query heads: 504 chunks of partials fill 8 MiB up to its
    # last 3 KiB (K and V of 516096 keys, 1 GiB each)
    kv_len = 504 * 1024
    assert kb.decode_workspace_bytes(1, kv_len) <= kb.DECODE_STATIC_SCRATCH_BYTES
    note(f"decode_static at the scratch limit: B=1 kv_len={kv_len}")
    g = torch.Generator(device="cuda:0").manual_seed(7)
    kd = torch.randn((1, 8, kv_len, 128), generator=g, device="cuda:0").to(torch.bfloat16)
    vd = torch.randn((1, 8, kv_len, 128), generator=g, device="cuda:0").to(torch.bfloat16)
    qd = torch.randn((1, 32, 1, 128), generator=g, device="cuda:0").to(torch.bfloat16)
    ref = bits(kb.decode(qd, kd, vd, kv_len=kv_len))
    got = bits(kb.decode_static(qd, kd, vd, kv_len=kv_len))
    assert np.array_equal(got, ref)
    # one key more needs a 505th chunk: refused before any launch
    kd2 = torch.zeros((1, 8, kv_len + 1, 128), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(kb.KBAttnError) as e:
        kb.decode_static(qd, kd2, kd2, kv_len=kv_len + 1)
    assert e.value.code == -9
    # and a smaller call afterwards still agrees
    small = bits(kb.decode_static(qd, kd, vd, kv_len=5000))
    assert np.array_equal(small, bits(kb.decode(qd, kd, vd, kv_len=5000)))
