"""GPU parity of the log-sum-exp outputs and of the backward (through the C-ABI).

Log-sum-exp: the library computes it from the contract's final fp32 state as
(Mc + log2 L) ln 2, where L sums bf16-rounded terms; each term carries a
relative rounding of at most 2^-9, so |lse - exact| <= 2^-9 + fp32 rounding.
The test allows 2^-8 + 2^-20 |lse|.

Gradients: the oracle returns, per element, the sum of the absolute values of
the terms (its error budget e, see oracle/oracle.c).  The HIP path rounds P
and dS to bf16 (2^-9 relative each), normalises P with a row sum of
bf16-rounded terms (2^-9), computes D_i from the bf16 forward output
(2^-9 of the output, plus the output's own error) and rounds the result to
bf16 (2^-9 relative); fp32 accumulation adds far less.  Every term's relative
error is below 2^-7, so |got - exact| <= 2^-7 e + 2^-8 |exact| element by
element.  Those roundings have random signs, so the typical error is far
smaller (measured: mean error 0.3-2% of the mean bound), and the test also
holds the mean error to a tenth of the mean bound.  (A bound relative to the
gradient's own size does not follow from the roundings: where the sums cancel,
as with outlier channels, the gradient is small beside its terms.)
"""
import math

import numpy as np
import pytest

import kb_gen
import oracle
from gpu_util import bits, dev, note, oracle_threads

pytestmark = pytest.mark.gpu

HQ, HKV, D = 32, 8, 128
SCALE = 1.0 / math.sqrt(D)


def kb():
    import bitwise_aligned_causal_amd as m

    return m


def f32(x):
    return kb_gen.bf16_bits_to_f32(x).astype(np.float64)


def make(seed, B, S):
    q = kb_gen.normal_bf16(seed, 1, (B, HQ, S, D))
    k = kb_gen.normal_bf16(seed, 2, (B, HKV, S, D))
    v = kb_gen.normal_bf16(seed, 3, (B, HKV, S, D))
    do = kb_gen.normal_bf16(seed, 4, (B, HQ, S, D))
    return q, k, v, do


def gpu_lse(t):
    import torch

    torch.cuda.synchronize()
    return t.cpu().numpy().astype(np.float64)


def check_lse(got, ref, what):
    err = np.abs(got - ref)
    tol = 2.0 ** -8 + 2.0 ** -20 * np.abs(ref)
    worst = np.unravel_index(int((err - tol).argmax()), err.shape)
    assert np.all(err <= tol), f"{what}: lse error {err[worst]:.3e} > {tol[worst]:.3e} at {worst}"


def check_grad(got_bits, ref, budget, what):
    got = kb_gen.bf16_bits_to_f32(got_bits).astype(np.float64).reshape(ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite gradient"
    err = np.abs(got - ref)
    bound = 2.0 ** -7 * budget + 2.0 ** -8 * np.abs(ref) + 1e-30
    ratio = err / bound
    worst = np.unravel_index(int(ratio.argmax()), ratio.shape)
    assert ratio.max() <= 1.0, (f"{what}: error {err[worst]:.3e} at {worst} exceeds {bound[worst]:.3e} "
                                f"(ref {ref[worst]:.3e}, budget {budget[worst]:.3e})")
    # typical errors are random-signed roundings, far below the worst case
    assert err.mean() <= 0.1 * bound.mean(), f"{what}: mean error {err.mean():.3e} vs bound {bound.mean():.3e}"
    return float(ratio.max())


def run_backward(q, k, v, do, seed_note=""):
    m = kb()
    Q, K, V, DO = dev(q), dev(k), dev(v), dev(do)
    note(f"prefill_lse + backward B={q.shape[0]} S={q.shape[2]} {seed_note}")
    o, lse = m.prefill_lse(Q, K, V)
    dq, dk, dv = m.backward(Q, K, V, o, DO, lse)
    return o, lse, dq, dk, dv


# 257, 513 and 800 end one key past, one key past two, and 32 keys into the
# fourth of the dK/dV kernel's 256-key blocks (waves with no valid key, a
# partial last 32-row tile)
@pytest.mark.parametrize("B,S", [(1, 1), (1, 17), (2, 64), (1, 100), (1, 257), (2, 300), (1, 513), (1, 800),
                                 (1, 1024)])
def test_backward_matches_oracle(B, S):
    q, k, v, do = make(1000 + S, B, S)
    _, lse, dq, dk, dv = run_backward(q, k, v, do)
    check_lse(gpu_lse(lse), oracle.lse(q, k, v, threads=oracle_threads()), f"lse S={S}")
    ref = oracle.backward(q, k, v, do, budgets=True, threads=oracle_threads())
    check_grad(bits(dq), ref["dq"], ref["eq"], f"dq B={B} S={S}")
    check_grad(bits(dk), ref["dk"], ref["ek"], f"dk B={B} S={S}")
    check_grad(bits(dv), ref["dv"], ref["ev"], f"dv B={B} S={S}")


def test_backward_outlier_inputs():
    # strong outlier channels in q and k (score spread of tens of log2 units)
    B, S = 1, 200
    q, k, v, do = make(77, B, S)
    qf, kf = kb_gen.bf16_bits_to_f32(q), kb_gen.bf16_bits_to_f32(k)
    qf[..., :4] *= 8.0
    kf[..., :4] *= 8.0
    q, k = kb_gen.f32_to_bf16_bits(qf), kb_gen.f32_to_bf16_bits(kf)
    _, lse, dq, dk, dv = run_backward(q, k, v, do, "outliers")
    check_lse(gpu_lse(lse), oracle.lse(q, k, v, threads=oracle_threads()), "lse outliers")
    ref = oracle.backward(q, k, v, do, budgets=True, threads=oracle_threads())
    check_grad(bits(dq), ref["dq"], ref["eq"], "dq outliers")
    check_grad(bits(dk), ref["dk"], ref["ek"], "dk outliers")
    check_grad(bits(dv), ref["dv"], ref["ev"], "dv outliers")


def test_backward_deterministic_and_batch_invariant():
    import torch

    m = kb()
    B, S = 3, 333
    q, k, v, do = make(5, B, S)
    o, lse, dq, dk, dv = run_backward(q, k, v, do)
    first = [bits(x) for x in (dq, dk, dv)]
    Q, K, V, DO = dev(q), dev(k), dev(v), dev(do)
    note("backward again, same inputs")
    again = [bits(x) for x in m.backward(Q, K, V, o, DO, lse)]
    for a, b in zip(first, again):
        assert np.array_equal(a, b)
    for i in range(B):
        note(f"backward of sequence {i} alone")
        sl = lambda x: np.ascontiguousarray(x[i:i + 1])
        qi, ki, vi, doi = dev(sl(q)), dev(sl(k)), dev(sl(v)), dev(sl(do))
        oi, lsei = m.prefill_lse(qi, ki, vi)
        assert np.array_equal(bits(oi), bits(o)[i:i + 1])
        assert torch.equal(lsei.cpu(), lse[i:i + 1].cpu())
        one = [bits(x) for x in m.backward(qi, ki, vi, oi, doi, lsei)]
        for name, a, b in zip(("dq", "dk", "dv"), one, first):
            assert np.array_equal(a, b[i:i + 1]), f"{name} of sequence {i} depends on the batch"


def test_lse_bitwise_across_entry_points():
    import torch

    m = kb()
    B, S = 2, 2500
    q, k, v, _ = make(11, B, S)
    Q, K, V = dev(q), dev(k), dev(v)
    note("prefill_lse vs prefill")
    o, lse = m.prefill_lse(Q, K, V)
    assert np.array_equal(bits(o), bits(m.prefill(Q, K, V)))
    lse_np = lse.cpu().numpy()
    # partitioned chunks that cross tile and chunk boundaries
    start = 0
    for n in (1, 63, 700, 1024, 712):
        stop = start + n
        note(f"partitioned_lse rows {start}..{stop}")
        qc = dev(np.ascontiguousarray(q[:, :, start:stop]))
        oc, lc = m.partitioned_lse(qc, K, V, stop)
        assert np.array_equal(bits(oc), bits(o)[:, :, start:stop])
        assert np.array_equal(lc.cpu().numpy().view(np.uint32), lse_np[:, :, start:stop].view(np.uint32))
        start = stop
    assert start == S
    # decode of the last token at several contexts (one chunk and several)
    for ctx in (1, 64, 1024, 1025, 2500):
        note(f"decode_lse at context {ctx}")
        qd = dev(np.ascontiguousarray(q[:, :, ctx - 1:ctx]))
        od, ld = m.decode_lse(qd, K, V, ctx)
        assert np.array_equal(bits(od)[:, :, 0], bits(o)[:, :, ctx - 1])
        assert np.array_equal(ld.cpu().numpy()[:, :, 0].view(np.uint32), lse_np[:, :, ctx - 1].view(np.uint32))
    torch.cuda.synchronize()


def test_autograd_glue_matches_explicit_calls():
    import torch

    m = kb()
    B, S = 1, 130
    q, k, v, do = make(13, B, S)
    Q, K, V, DO = (dev(x).requires_grad_(i < 3) for i, x in enumerate((q, k, v, do)))
    note("autograd attention")
    out = m.attention(Q, K, V)
    out.backward(DO)
    o, lse = m.prefill_lse(Q.detach(), K.detach(), V.detach())
    dq, dk, dv = m.backward(Q.detach(), K.detach(), V.detach(), o, DO, lse)
    assert np.array_equal(bits(out.detach()), bits(o))
    for g, e in ((Q.grad, dq), (K.grad, dk), (V.grad, dv)):
        assert np.array_equal(bits(g), bits(e))


def test_backward_full_size_sampled():
    """B=4, S=16384 (the training-shaped size the bench times): dq on sampled
    rows, dk / dv on the last 64 keys (which only the last rows see), and the
    softmax identities on every key."""
    B, S = 4, 16384
    q, k, v, do = make(21, B, S)
    _, lse, dq, dk, dv = run_backward(q, k, v, do, "full size")
    dq_b, dk_b, dv_b, lse_h = bits(dq), bits(dk), bits(dv), gpu_lse(lse)
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([
        rng.integers(0, B * HQ * S, size=48),
        np.array([0, S - 1, S, 2 * S + 1023, B * HQ * S - 1]),
    ])).astype(np.int64)
    ref, budget = oracle.backward_dq_rows(q, k, v, do, rows, budgets=True, threads=oracle_threads())
    check_grad(dq_b.reshape(-1, D)[rows], ref, budget, "dq sampled rows")
    lref = oracle.lse(q, k, v, rows=rows, threads=oracle_threads())
    check_lse(lse_h.reshape(-1)[rows], lref, "lse sampled rows")
    # keys S-64 .. S-1 of sequence 0, all KV heads
    q0, k0, v0, do0 = (np.ascontiguousarray(x[:1]) for x in (q, k, v, do))
    tail = oracle.backward(q0, k0, v0, do0, row_from=S - 64, budgets=True, threads=oracle_threads())
    check_grad(dk_b[:1, :, S - 64:], tail["dk"][:, :, S - 64:], tail["ek"][:, :, S - 64:], "dk last 64 keys")
    check_grad(dv_b[:1, :, S - 64:], tail["dv"][:, :, S - 64:], tail["ev"][:, :, S - 64:], "dv last 64 keys")
    # identities over all keys: sum_j dK_j = 0 and sum_j dV_j = sum of the group's dO
    dkf = kb_gen.bf16_bits_to_f32(dk_b).astype(np.float64)
    dvf = kb_gen.bf16_bits_to_f32(dv_b).astype(np.float64)
    sk, ak = dkf.sum(axis=2), np.abs(dkf).sum(axis=2)
    assert np.all(np.abs(sk) <= 2.0 ** -6 * ak), "sum_j dK_j is not ~0"
    sv = dvf.sum(axis=2)
    dos = kb_gen.bf16_bits_to_f32(do).astype(np.float64).reshape(B, HKV, 4, S, D).sum(axis=(2, 3))
    scale_v = np.abs(dvf).sum(axis=2)
    assert np.all(np.abs(sv - dos) <= 2.0 ** -6 * scale_v), "sum_j dV_j differs from the summed dO"


@pytest.mark.parametrize("hq,hkv,S,scale", [(4, 1, 129, 0.05), (8, 2, 70, None), (12, 3, 257, 0.2), (4, 1, 600, 0.1)])
def test_backward_other_heads_and_scale(hq, hkv, S, scale):
    m = kb()
    q = kb_gen.normal_bf16(300 + S, 1, (1, hq, S, D))
    k = kb_gen.normal_bf16(300 + S, 2, (1, hkv, S, D))
    v = kb_gen.normal_bf16(300 + S, 3, (1, hkv, S, D))
    do = kb_gen.normal_bf16(300 + S, 4, (1, hq, S, D))
    Q, K, V, DO = dev(q), dev(k), dev(v), dev(do)
    note(f"backward Hq={hq} Hkv={hkv} S={S} scale={scale}")
    o, lse = m.prefill_lse(Q, K, V, scale)
    dq, dk, dv = m.backward(Q, K, V, o, DO, lse, scale)
    sc = SCALE if scale is None else scale
    check_lse(gpu_lse(lse), oracle.lse(q, k, v, scale=sc, threads=oracle_threads()), f"lse Hq={hq}")
    ref = oracle.backward(q, k, v, do, scale=sc, budgets=True, threads=oracle_threads())
    check_grad(bits(dq), ref["dq"], ref["eq"], f"dq Hq={hq}")
    check_grad(bits(dk), ref["dk"], ref["ek"], f"dk Hq={hq}")
    check_grad(bits(dv), ref["dv"], ref["ev"], f"dv Hq={hq}")


def test_backward_from_partitioned_forward_is_bitwise_the_same():
    """o and lse assembled from partitioned chunks give the prefill-based
    gradients bit for bit (the forward contract makes both inputs identical)."""
    import torch

    m = kb()
    B, S = 2, 1500
    q, k, v, do = make(31, B, S)
    Q, K, V, DO = dev(q), dev(k), dev(v), dev(do)
    note("backward from prefill_lse vs from partitioned_lse chunks")
    o, lse = m.prefill_lse(Q, K, V)
    ref = [bits(x) for x in m.backward(Q, K, V, o, DO, lse)]
    outs, lses, start = [], [], 0
    for stop in (513, 1024, 1100, S):
        oc, lc = m.partitioned_lse(Q[:, :, start:stop].contiguous(), K, V, stop)
        outs.append(oc)
        lses.append(lc)
        start = stop
    o2 = torch.cat(outs, dim=2).contiguous()
    lse2 = torch.cat(lses, dim=2).contiguous()
    got = [bits(x) for x in m.backward(Q, K, V, o2, DO, lse2)]
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert np.array_equal(a, b), name


def test_backward_seeded_random_shapes():
    """Eight seeded random shapes (B 1-2, Hkv 1-2, S 1-900, scale 0.03-0.2):
    the gradients against the oracle's budgets, and a second call's bits equal
    the first's."""
    m = kb()
    rng = np.random.default_rng(2024)
    for case in range(8):
        B = int(rng.integers(1, 3))
        hkv = int(rng.integers(1, 3))
        hq = 4 * hkv
        S = int(rng.integers(1, 901))
        sc = float(rng.uniform(0.03, 0.2))
        seed = 500 + case
        q = kb_gen.normal_bf16(seed, 1, (B, hq, S, D))
        k = kb_gen.normal_bf16(seed, 2, (B, hkv, S, D))
        v = kb_gen.normal_bf16(seed, 3, (B, hkv, S, D))
        do = kb_gen.normal_bf16(seed, 4, (B, hq, S, D))
        Q, K, V, DO = dev(q), dev(k), dev(v), dev(do)
        what = f"case {case}: B={B} Hq={hq} Hkv={hkv} S={S} scale={sc:.4f}"
        note(f"backward {what}")
        o, lse = m.prefill_lse(Q, K, V, sc)
        dq, dk, dv = m.backward(Q, K, V, o, DO, lse, sc)
        first = [bits(x) for x in (dq, dk, dv)]
        ref = oracle.backward(q, k, v, do, scale=sc, budgets=True, threads=oracle_threads())
        check_grad(first[0], ref["dq"], ref["eq"], f"dq {what}")
        check_grad(first[1], ref["dk"], ref["ek"], f"dk {what}")
        check_grad(first[2], ref["dv"], ref["ev"], f"dv {what}")
        again = [bits(x) for x in m.backward(Q, K, V, o, DO, lse, sc)]
        for name, a, b in zip(("dq", "dk", "dv"), again, first):
            assert np.array_equal(a, b), f"{name} {what}: a rerun changed bits"
