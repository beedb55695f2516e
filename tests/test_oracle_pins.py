"""Pins of the oracle against what the mathematics fixes (CPU only).

The pages print no numeric values for their worked example (KernelBraid
README, "Usage": it only asserts bitwise equality of the last prefill row and
the decode output), so the oracle is pinned by independent formulations and
closed forms:
  - brute force in pure Python, matrix form with an explicit -inf mask and no
    max subtraction, on tiny shapes;
  - torch's scaled_dot_product_attention on the CPU in float64 (library
    reduction), with is_causal for full prefill and an explicit bottom-right
    mask for partitioned calls;
  - softmax rows sum to one; causality; GQA equals MHA with repeated KV heads;
    constant V; row 0 equals V_0; Q = 0 gives the running mean of V;
    two-key closed forms (tests/golden/closed_forms.json);
  - decode of the last token and partitioned chunks equal the matching
    prefill rows (the equalities the README's "Method" and "Usage" state).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import kb_gen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32(x):
    return kb_gen.bf16_bits_to_f32(x).astype(np.float64)


def inputs(seed, B, Hq, Hkv, q_len, kv_len, D, cap=None):
    cap = kv_len if cap is None else cap
    q = kb_gen.normal_bf16(seed, 1, (B, Hq, q_len, D))
    k = kb_gen.normal_bf16(seed, 2, (B, Hkv, cap, D))
    v = kb_gen.normal_bf16(seed, 3, (B, Hkv, cap, D))
    return q, k, v


def brute_force(q, k, v, kv_len, scale):
    """Matrix form in pure Python floats: explicit mask, no max subtraction."""
    B, Hq, q_len, D = q.shape
    Hkv = k.shape[1]
    Q, K, V = f32(q), f32(k), f32(v)
    out = np.zeros((B, Hq, q_len, D))
    for b in range(B):
        for h in range(Hq):
            g = h * Hkv // Hq
            for r in range(q_len):
                limit = kv_len - q_len + r
                scores = []
                for j in range(kv_len):
                    if j > limit:
                        scores.append(-math.inf)
                    else:
                        scores.append(scale * math.fsum(Q[b, h, r, d] * K[b, g, j, d] for d in range(D)))
                ex = [math.exp(s) if s != -math.inf else 0.0 for s in scores]
                z = math.fsum(ex)
                for d in range(D):
                    out[b, h, r, d] = math.fsum(ex[j] * V[b, g, j, d] for j in range(kv_len)) / z
    return out


TINY = [
    # B, Hq, Hkv, q_len, kv_len, D
    (1, 1, 1, 1, 1, 1),
    (1, 2, 1, 3, 3, 2),
    (2, 4, 2, 5, 5, 8),
    (1, 8, 2, 9, 9, 8),
    (2, 4, 1, 4, 9, 8),
    (1, 2, 2, 1, 7, 2),
    (1, 4, 4, 17, 17, 2),
    (1, 4, 1, 3, 65, 8),
    (1, 2, 1, 6, 6, 128),
    (1, 8, 2, 2, 17, 128),
]


@pytest.mark.parametrize("shape", TINY)
def test_brute_force(shape):
    B, Hq, Hkv, q_len, kv_len, D = shape
    q, k, v = inputs(101 + sum(shape), B, Hq, Hkv, q_len, kv_len, D)
    scale = 1.0 / math.sqrt(D)
    ref = brute_force(q, k, v, kv_len, scale)
    got = oracle.attention(q, k, v, kv_len=kv_len, scale=scale)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    got32 = oracle.attention(q, k, v, kv_len=kv_len, scale=scale, precision="f32")
    np.testing.assert_allclose(got32, ref, rtol=0, atol=2e-5 * max(1.0, np.abs(ref).max()))


def sdpa_reference(q, k, v, kv_len, scale):
    B, Hq, q_len, D = q.shape
    Q = torch.from_numpy(f32(q))
    K = torch.from_numpy(f32(k[:, :, :kv_len]))
    V = torch.from_numpy(f32(v[:, :, :kv_len]))
    if q_len == kv_len:
        o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=scale,
                                                             enable_gqa=True)
    else:
        pos = torch.arange(q_len)[:, None] + (kv_len - q_len)
        mask = torch.arange(kv_len)[None, :] <= pos
        o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=scale,
                                                             enable_gqa=True)
    return o.numpy()


@pytest.mark.parametrize("shape", [
    (1, 32, 8, 200, 200, 128),
    (2, 32, 8, 64, 300, 128),
    (1, 32, 8, 1, 257, 128),
    (2, 8, 2, 130, 130, 64),
])
def test_library_sdpa(shape):
    B, Hq, Hkv, q_len, kv_len, D = shape
    q, k, v = inputs(7 + q_len, B, Hq, Hkv, q_len, kv_len, D, cap=kv_len + 5)
    scale = 1.0 / math.sqrt(D)
    ref = sdpa_reference(q, k, v, kv_len, scale)
    got = oracle.attention(q, k, v, kv_len=kv_len, scale=scale)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("prec,eps", [("f64", 2.0 ** -53), ("f32", 2.0 ** -24)])
def test_rows_sum_to_one(prec, eps):
    q, k, v = inputs(3, 1, 8, 2, 300, 300, 128)
    for row in (0, 1, 63, 64, 150, 299, 300 + 17, 8 * 300 - 1):
        w = oracle.weights(q, k, v, row, precision=prec)
        pos = row % 300
        assert w.shape == (pos + 1,)
        assert np.all(w >= 0)
        assert abs(1.0 - math.fsum(w)) <= 4 * (pos + 1) * eps


def test_causality_bitwise():
    q, k, v = inputs(5, 2, 8, 2, 96, 96, 128)
    base = oracle.attention(q, k, v)
    for p in (0, 31, 64, 95):
        k2, v2 = k.copy(), v.copy()
        k2[:, :, p + 1:] = kb_gen.normal_bf16(99, 2, k2[:, :, p + 1:].shape)
        v2[:, :, p + 1:] = kb_gen.normal_bf16(99, 3, v2[:, :, p + 1:].shape)
        got = oracle.attention(q, k2, v2)
        assert np.array_equal(got[:, :, :p + 1], base[:, :, :p + 1])
        if p < 95:
            assert not np.array_equal(got[:, :, p + 1:], base[:, :, p + 1:])


def test_gqa_equals_mha_bitwise():
    q, k, v = inputs(9, 2, 32, 8, 70, 70, 128)
    gqa = oracle.attention(q, k, v)
    k_rep = np.ascontiguousarray(np.repeat(k, 4, axis=1))
    v_rep = np.ascontiguousarray(np.repeat(v, 4, axis=1))
    mha = oracle.attention(q, k_rep, v_rep)
    assert np.array_equal(gqa, mha)


@pytest.mark.parametrize("const", [1.5, -0.375, 3.0])
def test_constant_v(const):
    q, k, v = inputs(11, 1, 8, 2, 130, 130, 128)
    v[:] = kb_gen.f32_to_bf16_bits(np.full(v.shape, const, dtype=np.float32))
    # numerator and denominator are sums of pos+1 terms: relative error <= (2*(pos+1) + 1) u
    n = np.arange(1, 131, dtype=np.float64)[None, None, :, None]
    for prec, u in (("f64", 2.0 ** -53), ("f32", 2.0 ** -24)):
        got = oracle.attention(q, k, v, precision=prec)
        assert np.all(np.abs(got - const) <= (2 * n + 1) * u * abs(const))


def test_row_zero_is_v0_exactly():
    q, k, v = inputs(13, 2, 32, 8, 40, 40, 128)
    got = oracle.attention(q, k, v)
    v0 = f32(v[:, :, 0])  # [B, Hkv, D]
    for h in range(32):
        assert np.array_equal(got[:, h, 0], v0[:, h // 4])
    got32 = oracle.attention(q, k, v, precision="f32")
    assert np.array_equal(got32[:, :, 0], got[:, :, 0])


def test_zero_q_gives_running_mean():
    q, k, v = inputs(17, 1, 4, 1, 50, 50, 16)
    q[:] = 0
    got = oracle.attention(q, k, v)
    V = f32(v)[0, 0]
    for r in range(50):
        mean = np.array([math.fsum(V[: r + 1, d]) / (r + 1) for d in range(16)])
        np.testing.assert_allclose(got[0, :, r], np.broadcast_to(mean, (4, 16)), rtol=1e-13, atol=1e-13)


def test_decode_equals_last_prefill_row_bitwise():
    # README "Usage": decode of q[:, :, -1:] over the same k, v equals the last prefill row
    q, k, v = inputs(17, 1, 32, 8, 256, 256, 128)
    pre = oracle.attention(q, k, v)
    dec = oracle.attention(np.ascontiguousarray(q[:, :, -1:]), k, v)
    assert np.array_equal(dec[:, :, 0], pre[:, :, -1])
    # decode at an earlier context over a larger cache (kv_len < capacity)
    for c in (1, 64, 65, 200):
        dec = oracle.attention(np.ascontiguousarray(q[:, :, c - 1:c]), k, v, kv_len=c)
        assert np.array_equal(dec[:, :, 0], pre[:, :, c - 1])


def test_partitioned_equals_prefill_bitwise():
    q, k, v = inputs(19, 2, 8, 2, 300, 300, 128)
    pre = oracle.attention(q, k, v)
    start = 0
    for chunk in (1, 7, 100, 64, 128):
        stop = start + chunk
        part = oracle.attention(np.ascontiguousarray(q[:, :, start:stop]), k, v, kv_len=stop)
        assert np.array_equal(part, pre[:, :, start:stop])
        start = stop


def test_row_subset_matches_full():
    q, k, v = inputs(23, 2, 8, 2, 77, 77, 128)
    full = oracle.attention(q, k, v).reshape(-1, 128)
    rows = np.array([0, 5, 76, 77, 300, 2 * 8 * 77 - 1], dtype=np.int64)
    sub = oracle.attention(q, k, v, rows=rows, threads=3)
    assert np.array_equal(sub, full[rows])


def test_f32_and_f64_agree():
    q, k, v = inputs(29, 1, 8, 2, 512, 512, 128)
    a = oracle.attention(q, k, v)
    b = oracle.attention(q, k, v, precision="f32")
    # fp32 sums of <= 512 terms of magnitude <= ~1: a few hundred ulp at most
    assert np.abs(a - b).max() < 1e-4


def test_closed_forms_golden():
    with open(os.path.join(GOLDEN, "closed_forms.json")) as fh:
        cases = json.load(fh)["cases"]
    assert cases
    for case in cases:
        D = case["head_dim"]
        q = kb_gen.f32_to_bf16_bits(np.array(case["q"], dtype=np.float32)).reshape(1, 1, -1, D)
        k = kb_gen.f32_to_bf16_bits(np.array(case["k"], dtype=np.float32)).reshape(1, 1, -1, D)
        v = kb_gen.f32_to_bf16_bits(np.array(case["v"], dtype=np.float32)).reshape(1, 1, -1, D)
        # the golden values must be representable exactly in bf16
        assert np.array_equal(f32(q).ravel(), np.array(case["q"], dtype=np.float64).ravel())
        assert np.array_equal(f32(k).ravel(), np.array(case["k"], dtype=np.float64).ravel())
        assert np.array_equal(f32(v).ravel(), np.array(case["v"], dtype=np.float64).ravel())
        got = oracle.attention(q, k, v, kv_len=case["kv_len"], scale=case["scale"])
        expect = np.array(eval(case["expected"], {"math": math}), dtype=np.float64)  # noqa: S307
        np.testing.assert_allclose(got.reshape(expect.shape), expect, rtol=1e-14, atol=1e-14)


def test_rejects_malformed():
    q, k, v = inputs(31, 1, 4, 2, 8, 8, 16)
    with pytest.raises(ValueError):
        oracle.attention(q, k, v, kv_len=4)  # q_len > kv_len
    with pytest.raises(ValueError):
        oracle.attention(q, k, v, kv_len=9)  # kv_len > capacity
    q3, k3, v3 = inputs(31, 1, 3, 2, 8, 8, 16)
    with pytest.raises(ValueError):
        oracle.attention(q3, k3, v3)  # Hq not a multiple of Hkv
