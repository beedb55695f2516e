"""Pins of the oracle's log-sum-exp and backward (CPU only).

The pages cover the forward only (README "Background": training forward and
backward still run; "Features": this release covers forward attention), so
the gradient is pinned to the mathematics rather than to printed values:
  - torch autograd through scaled_dot_product_attention in float64 (library
    derivative of a library forward, with is_causal and enable_gqa);
  - central finite differences of torch's float64 forward on single
    coordinates (no derivative formula at all);
  - identities that hold for any input: sum_j dK_j = 0 (a softmax row does
    not move when every key is shifted by one vector), sum_j dV_j =
    sum_i dO_i summed over the heads of a group (each row of P sums to one),
    dQ = 0 when every key is the same vector, and a one-token sequence
    (dQ = dK = 0, dV_0 = sum of the group's dO_0);
  - log-sum-exp against torch.logsumexp of the masked float64 scores, and the
    closed form log(i + 1) + scale <q_i, k> when every key is the same.
"""
import math

import numpy as np
import pytest
import torch

import kb_gen
import oracle
from test_oracle_pins import f32, inputs


def grads_inputs(seed, B, Hq, Hkv, S, D):
    q, k, v = inputs(seed, B, Hq, Hkv, S, S, D)
    do = kb_gen.normal_bf16(seed, 4, (B, Hq, S, D))
    return q, k, v, do


def sdpa_autograd(q, k, v, do, scale):
    Q = torch.from_numpy(f32(q)).requires_grad_()
    K = torch.from_numpy(f32(k)).requires_grad_()
    V = torch.from_numpy(f32(v)).requires_grad_()
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=scale, enable_gqa=True)
    o.backward(torch.from_numpy(f32(do)))
    return Q.grad.numpy(), K.grad.numpy(), V.grad.numpy()


SHAPES = [
    # B, Hq, Hkv, S, D
    (1, 1, 1, 1, 4),
    (1, 2, 1, 3, 2),
    (2, 4, 2, 7, 8),
    (1, 8, 2, 17, 16),
    (1, 4, 1, 65, 8),
    (2, 32, 8, 40, 128),
]


@pytest.mark.parametrize("shape", SHAPES)
def test_backward_matches_autograd(shape):
    B, Hq, Hkv, S, D = shape
    q, k, v, do = grads_inputs(211 + sum(shape), B, Hq, Hkv, S, D)
    scale = 1.0 / math.sqrt(D)
    dq, dk, dv = sdpa_autograd(q, k, v, do, scale)
    got = oracle.backward(q, k, v, do, scale=scale)
    for name, ref in (("dq", dq), ("dk", dk), ("dv", dv)):
        tol = 1e-11 * max(1.0, np.abs(ref).max())
        np.testing.assert_allclose(got[name], ref, rtol=0, atol=tol, err_msg=name)


def test_backward_finite_differences():
    B, Hq, Hkv, S, D = 1, 4, 2, 9, 8
    q, k, v, do = grads_inputs(5, B, Hq, Hkv, S, D)
    scale = 0.3
    got = oracle.backward(q, k, v, do, scale=scale)
    base = {"q": f32(q), "k": f32(k), "v": f32(v)}
    DO = torch.from_numpy(f32(do))

    def loss(x):
        t = {n: torch.from_numpy(a) for n, a in x.items()}
        o = torch.nn.functional.scaled_dot_product_attention(t["q"], t["k"], t["v"], is_causal=True, scale=scale,
                                                             enable_gqa=True)
        return float((o * DO).sum())

    h = 1e-5
    coords = {"q": [(0, 0, 0, 3), (0, 3, 8, 7), (0, 2, 4, 0)],
              "k": [(0, 0, 0, 1), (0, 1, 5, 6), (0, 1, 8, 2)],
              "v": [(0, 0, 0, 0), (0, 1, 3, 5), (0, 0, 8, 7)]}
    for name, pts in coords.items():
        for idx in pts:
            plus = {n: a.copy() for n, a in base.items()}
            minus = {n: a.copy() for n, a in base.items()}
            plus[name][idx] += h
            minus[name][idx] -= h
            fd = (loss(plus) - loss(minus)) / (2 * h)
            assert abs(got["d" + name][idx] - fd) <= 1e-7, (name, idx, got["d" + name][idx], fd)


@pytest.mark.parametrize("shape", [(2, 8, 2, 50, 16), (1, 32, 8, 33, 128)])
def test_backward_identities(shape):
    B, Hq, Hkv, S, D = shape
    q, k, v, do = grads_inputs(17 + S, B, Hq, Hkv, S, D)
    got = oracle.backward(q, k, v, do)
    g = Hq // Hkv
    # shifting every key by one vector leaves each softmax row unchanged
    sk = got["dk"].sum(axis=2)
    assert np.abs(sk).max() <= 1e-12 * max(1.0, np.abs(got["dk"]).sum(axis=2).max())
    # each row of P sums to one: sum_j dV_j = sum over the group's rows of dO
    dos = f32(do).reshape(B, Hkv, g, S, D).sum(axis=(2, 3))
    np.testing.assert_allclose(got["dv"].sum(axis=2), dos, rtol=0, atol=1e-11)


def test_backward_identical_keys_and_single_token():
    q, k, v, do = grads_inputs(23, 1, 8, 2, 30, 16)
    k[:] = k[:, :, :1]
    got = oracle.backward(q, k, v, do)
    assert np.abs(got["dq"]).max() <= 1e-13
    q1, k1, v1, do1 = grads_inputs(29, 2, 8, 2, 1, 16)
    g1 = oracle.backward(q1, k1, v1, do1)
    assert np.abs(g1["dq"]).max() == 0 and np.abs(g1["dk"]).max() == 0
    np.testing.assert_allclose(g1["dv"][:, :, 0], f32(do1)[:, :, 0].reshape(2, 2, 4, 16).sum(axis=2),
                               rtol=0, atol=1e-14)


def test_backward_row_forms_agree():
    B, Hq, Hkv, S, D = 2, 8, 2, 70, 32
    q, k, v, do = grads_inputs(31, B, Hq, Hkv, S, D)
    full = oracle.backward(q, k, v, do, budgets=True)
    rows = np.array([0, 1, 69, 70, 3 * 70 + 35, B * Hq * S - 1], dtype=np.int64)
    dq, eq = oracle.backward_dq_rows(q, k, v, do, rows, budgets=True, threads=3)
    assert np.array_equal(dq, full["dq"].reshape(-1, D)[rows])
    assert np.array_equal(eq, full["eq"].reshape(-1, D)[rows])
    tail = oracle.backward(q, k, v, do, row_from=50, budgets=True)
    for name in ("dk", "dv", "ek", "ev"):
        np.testing.assert_allclose(tail[name][:, :, 50:], full[name][:, :, 50:], rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(tail["dq"][:, :, 50:], full["dq"][:, :, 50:])


def budgets_torch(q, k, v, do, scale):
    """The error budgets from their definitions, in float64 matrix form
    (torch, independent of the oracle's loops): with P the causal softmax,
    dS = P (dO V^T - D), D_i = <dO_i, (P V)_i>, A_i = sum_j P_ij <|dO_i|, |v_j|>,
      eq = scale (|dS| + P A) |K|,   ek = scale (|dS| + P A)^T |Q|,
      ev = P^T |dO|,
    with ek and ev summed over the query heads of each KV head."""
    B, Hq, S, D = q.shape
    g = Hq // k.shape[1]
    Q, K, V, dO = (torch.from_numpy(f32(x)).double() for x in (q, k, v, do))
    K, V = K.repeat_interleave(g, dim=1), V.repeat_interleave(g, dim=1)
    scores = scale * Q @ K.transpose(-1, -2)
    mask = torch.ones(S, S, dtype=torch.bool).triu(1)
    P = torch.softmax(scores.masked_fill(mask, float("-inf")), dim=-1)
    O = P @ V
    Drow = (dO * O).sum(-1, keepdim=True)
    dS = P * (dO @ V.transpose(-1, -2) - Drow)
    A = (P * (dO.abs() @ V.abs().transpose(-1, -2))).sum(-1, keepdim=True)
    W = dS.abs() + P * A
    eq = scale * W @ K.abs()
    ek = (scale * W.transpose(-1, -2) @ Q.abs()).reshape(B, Hq // g, g, S, D).sum(2)
    ev = (P.transpose(-1, -2) @ dO.abs()).reshape(B, Hq // g, g, S, D).sum(2)
    return eq.numpy(), ek.numpy(), ev.numpy()


@pytest.mark.parametrize("shape", [(1, 8, 2, 45, 32), (2, 4, 1, 9, 8), (1, 4, 4, 3, 4)])
def test_backward_budgets_equal_their_definition(shape):
    # pinned from both sides: a budget inflated by a dropped weight or an extra
    # factor, or one missing a term, differs from the matrix form
    B, Hq, Hkv, S, D = shape
    q, k, v, do = grads_inputs(37 + S, B, Hq, Hkv, S, D)
    scale = 1.0 / math.sqrt(D)
    g = oracle.backward(q, k, v, do, scale=scale, budgets=True)
    for name, ref in zip(("eq", "ek", "ev"), budgets_torch(q, k, v, do, scale)):
        np.testing.assert_allclose(g[name], ref, rtol=1e-11, atol=1e-13, err_msg=name)


def test_backward_budgets_cover_terms():
    # the budgets are sums of the absolute values of the terms whose sums are
    # the gradients, so they bound the gradients themselves
    q, k, v, do = grads_inputs(37, 1, 8, 2, 45, 32)
    g = oracle.backward(q, k, v, do, budgets=True)
    for grad, bud in (("dq", "eq"), ("dk", "ek"), ("dv", "ev")):
        assert np.all(g[bud] >= np.abs(g[grad]) * (1 - 1e-12)), grad


def test_value_budget_is_tight_for_nonnegative_upstream():
    # with dO >= 0 every term P_ij dO_id of dV is >= 0, so the sum of their
    # absolute values is dV itself: the budget may not exceed it
    q, k, v, do = grads_inputs(41, 2, 8, 2, 30, 16)
    do = kb_gen.f32_to_bf16_bits(np.abs(f32(do)))
    g = oracle.backward(q, k, v, do, budgets=True)
    np.testing.assert_allclose(g["ev"], g["dv"], rtol=1e-12, atol=0)
    assert np.all(g["eq"] >= np.abs(g["dq"]) * (1 - 1e-12))
    assert np.all(g["ek"] >= np.abs(g["dk"]) * (1 - 1e-12))


def masked_lse_torch(q, k, kv_len, scale):
    B, Hq, q_len, D = q.shape
    Hkv = k.shape[1]
    Q = torch.from_numpy(f32(q))
    K = torch.from_numpy(f32(k[:, :, :kv_len])).repeat_interleave(Hq // Hkv, dim=1)
    s = (Q @ K.transpose(-1, -2).contiguous()) * scale
    pos = torch.arange(q_len)[:, None] + (kv_len - q_len)
    s = s.masked_fill(torch.arange(kv_len)[None, :] > pos, -math.inf)
    return torch.logsumexp(s, dim=-1).numpy()


@pytest.mark.parametrize("shape", [(1, 4, 1, 1, 1, 8), (2, 8, 2, 20, 20, 16), (1, 32, 8, 5, 130, 128),
                                   (2, 32, 8, 100, 100, 128)])
def test_lse_matches_library(shape):
    B, Hq, Hkv, q_len, kv_len, D = shape
    q, k, v = inputs(41 + q_len, B, Hq, Hkv, q_len, kv_len, D, cap=kv_len + 3)
    scale = 1.0 / math.sqrt(D)
    ref = masked_lse_torch(q, k, kv_len, scale)
    got = oracle.lse(q, k, v, kv_len=kv_len, scale=scale)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    rows = np.array([0, B * Hq * q_len - 1], dtype=np.int64)
    np.testing.assert_array_equal(oracle.lse(q, k, v, kv_len=kv_len, scale=scale, rows=rows), got.reshape(-1)[rows])


def test_lse_closed_form_identical_keys():
    q, k, v = inputs(43, 1, 8, 2, 60, 60, 32)
    k[:] = k[:, :, 7:8]
    scale = 0.125
    got = oracle.lse(q, k, v, scale=scale)
    Q, K = f32(q)[0], f32(k)[0, :, 0]
    for h in range(8):
        dots = Q[h] @ K[h // 4]
        expect = np.log(np.arange(1, 61)) + scale * dots
        np.testing.assert_allclose(got[0, h], expect, rtol=0, atol=1e-12)
