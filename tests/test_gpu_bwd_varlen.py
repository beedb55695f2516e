"""GPU tests of the ragged log-sum-exp and backward (through the C-ABI).

A ragged call must give every sequence exactly the bits of the dense call on
that sequence alone (the kernels are the dense ones with a table lookup), so
the ragged results inherit the dense parity with the oracle; one sequence is
also checked against the oracle directly."""
import math

import numpy as np
import pytest

import kb_gen
import oracle
from gpu_util import bits, dev, note, oracle_threads
from test_gpu_bwd import check_grad, check_lse

pytestmark = pytest.mark.gpu

HQ, HKV, D = 32, 8, 128


def kb():
    import bitwise_aligned_causal_amd as m

    return m


def packed(seed, lens):
    """Per-sequence dense tensors and their packed head-major concatenation."""
    seqs = []
    for i, L in enumerate(lens):
        q = kb_gen.normal_bf16(seed + i, 1, (1, HQ, L, D))
        k = kb_gen.normal_bf16(seed + i, 2, (1, HKV, L, D))
        v = kb_gen.normal_bf16(seed + i, 3, (1, HKV, L, D))
        do = kb_gen.normal_bf16(seed + i, 4, (1, HQ, L, D))
        seqs.append((q, k, v, do))
    cat = [np.ascontiguousarray(np.concatenate([s[t][0] for s in seqs], axis=1)) for t in range(4)]
    cu = [0]
    for L in lens:
        cu.append(cu[-1] + L)
    return seqs, cat, cu


def run_case(lens, seed, check_oracle=False):
    m = kb()
    seqs, (qp, kp, vp, dop), cu = packed(seed, lens)
    Q, K, V, DO = dev(qp), dev(kp), dev(vp), dev(dop)
    note(f"ragged prefill_lse + backward, {len(lens)} sequences, T={cu[-1]}")
    o, lse = m.prefill_varlen_lse(Q, K, V, cu)
    dq, dk, dv = m.backward_varlen(Q, K, V, o, DO, lse, cu)
    ob, lb = bits(o), lse.cpu().numpy()
    dqb, dkb, dvb = bits(dq), bits(dk), bits(dv)
    assert np.array_equal(ob, bits(m.prefill_varlen(Q, K, V, cu)))
    for i, (q, k, v, do) in enumerate(seqs):
        L = lens[i]
        if L == 0:
            continue
        a, b = cu[i], cu[i + 1]
        qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
        od, ld = m.prefill_lse(qd, kd, vd)
        g = m.backward(qd, kd, vd, od, dod, ld)
        assert np.array_equal(lb[:, a:b].view(np.uint32), ld.cpu().numpy()[0].view(np.uint32)), f"lse seq {i}"
        assert np.array_equal(ob[:, a:b], bits(od)[0]), f"o seq {i}"
        for name, got, ref in (("dq", dqb, g[0]), ("dk", dkb, g[1]), ("dv", dvb, g[2])):
            assert np.array_equal(got[:, a:b], bits(ref)[0]), f"{name} of sequence {i} (length {L})"
        if check_oracle and L >= 64:
            ref = oracle.backward(q, k, v, do, budgets=True, threads=oracle_threads())
            check_lse(lb[:, a:b].astype(np.float64), oracle.lse(q, k, v, threads=oracle_threads())[0], "lse")
            check_grad(dqb[:, a:b], ref["dq"][0], ref["eq"][0], f"dq seq {i}")
            check_grad(dkb[:, a:b], ref["dk"][0], ref["ek"][0], f"dk seq {i}")
            check_grad(dvb[:, a:b], ref["dv"][0], ref["ev"][0], f"dv seq {i}")
            check_oracle = False


def test_ragged_backward_equals_dense_per_sequence():
    run_case([1, 63, 64, 65, 0, 130, 1000, 300, 2049], seed=500, check_oracle=True)


def test_ragged_backward_two_launches():
    # 70 non-empty sequences: more than one launch's table
    run_case([1 + (i * 37) % 150 for i in range(70)], seed=900)


def test_ragged_backward_other_heads():
    """Hq = 8, Hkv = 2: each sequence's ragged bits equal the dense call's."""
    m = kb()
    hq, hkv = 8, 2
    lens = [77, 1, 200, 64]
    seqs = []
    for i, L in enumerate(lens):
        seqs.append(tuple(kb_gen.normal_bf16(700 + i, t, (1, hq if t in (1, 4) else hkv, L, D)) for t in (1, 2, 3, 4)))
    cat = [np.ascontiguousarray(np.concatenate([s[t][0] for s in seqs], axis=1)) for t in range(4)]
    cu = [0]
    for L in lens:
        cu.append(cu[-1] + L)
    Q, K, V, DO = (dev(x) for x in cat)
    note("ragged backward Hq=8 Hkv=2")
    o, lse = m.prefill_varlen_lse(Q, K, V, cu, scale=0.1)
    dq, dk, dv = m.backward_varlen(Q, K, V, o, DO, lse, cu, scale=0.1)
    got = [bits(x) for x in (dq, dk, dv)]
    for i, (q, k, v, do) in enumerate(seqs):
        a, b = cu[i], cu[i + 1]
        qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
        od, ld = m.prefill_lse(qd, kd, vd, scale=0.1)
        ref = [bits(x) for x in m.backward(qd, kd, vd, od, dod, ld, scale=0.1)]
        for name, g, r in zip(("dq", "dk", "dv"), got, ref):
            assert np.array_equal(g[:, a:b], r[0]), f"{name} of sequence {i}"
