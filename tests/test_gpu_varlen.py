"""GPU parity of the ragged (variable-length) entry points.

A ragged call must give, for every sequence, exactly the bits of the dense
call on that sequence alone (the contract is per row), and so agree with the
oracle; its partitioned splits and decodes must reproduce the prefill rows bit
for bit.  All calls go through the C-ABI.
"""
import numpy as np
import pytest

import kb_gen
import oracle
from gpu_util import bits, compare, dev, note, oracle_threads

pytestmark = pytest.mark.gpu

HQ, HKV, D = 32, 8, 128


@pytest.fixture(scope="module")
def kb():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bitwise_aligned_causal_amd as kb

    kb.lib()
    return kb


def same_bits(a, b, what):
    assert a.shape == b.shape, f"{what}: shapes {a.shape} vs {b.shape}"
    n = int(np.count_nonzero(a != b))
    assert n == 0, f"{what}: {n} of {a.size} bf16 bit patterns differ"


def ragged_inputs(lengths, seed0, hkv=HKV, outliers=0):
    """Per-sequence inputs ([1, H, L, 128] each) and their packed head-major form."""
    seqs = [kb_gen.attention_inputs(seed0 + i, 1, max(L, 1), 4 * hkv, hkv, D, outliers=outliers) for i, L in
            enumerate(lengths)]
    seqs = [(q[:, :, :L], k[:, :, :L], v[:, :, :L]) for (q, k, v), L in zip(seqs, lengths)]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    pack = lambda xs: np.ascontiguousarray(np.concatenate([x[0] for x in xs], axis=1))
    return seqs, cu, pack([s[0] for s in seqs]), pack([s[1] for s in seqs]), pack([s[2] for s in seqs])


LENGTHS = [1, 63, 64, 65, 0, 130, 1000, 2049, 300, 1024, 1025]


def test_prefill_varlen_matches_dense_and_oracle(kb):
    note(f"prefill_varlen lengths {LENGTHS}")
    seqs, cu, qp, kp, vp = ragged_inputs(LENGTHS, 900)
    out = bits(kb.prefill_varlen(dev(qp), dev(kp), dev(vp), cu.tolist()))
    for i, ((q, k, v), L) in enumerate(zip(seqs, LENGTHS)):
        if L == 0:
            continue
        dense = bits(kb.prefill(dev(q), dev(k), dev(v)))[0]
        same_bits(out[:, cu[i]:cu[i + 1]], dense, f"sequence {i} (L={L}) ragged vs dense")
        if L <= 1100:
            compare(out[:, cu[i]:cu[i + 1]], oracle.attention(q, k, v, threads=oracle_threads())[0],
                    f"sequence {i} (L={L}) vs oracle")


def test_partitioned_varlen_prompt_answer_splits(kb):
    lengths = [L for L in LENGTHS if L > 1]
    note(f"partitioned_varlen lengths {lengths}")
    seqs, cu, qp, kp, vp = ragged_inputs(lengths, 950)
    full = bits(kb.prefill_varlen(dev(qp), dev(kp), dev(vp), cu.tolist()))
    rng = np.random.default_rng(3)
    split = [int(rng.integers(1, L)) for L in lengths]
    # prompt: rows 0..split-1 against kv_len = split; answer: rows split..L-1 against the whole sequence
    for part in ("prompt", "answer"):
        rows = [(0, s) if part == "prompt" else (s, L) for s, L in zip(split, lengths)]
        qchunk = np.concatenate([qp[:, cu[i] + a:cu[i] + b] for i, (a, b) in enumerate(rows)], axis=1)
        cu_q = np.concatenate([[0], np.cumsum([b - a for a, b in rows])]).tolist()
        kv_lens = [b for _, b in rows]
        got = bits(kb.partitioned_varlen(dev(np.ascontiguousarray(qchunk)), dev(kp), dev(vp), cu_q, cu.tolist(),
                                         kv_lens))
        for i, (a, b) in enumerate(rows):
            same_bits(got[:, cu_q[i]:cu_q[i + 1]], full[:, cu[i] + a:cu[i] + b],
                      f"{part} of sequence {i} (rows {a}..{b - 1})")


def test_decode_varlen_equals_prefill_rows(kb):
    lengths = [L for L in LENGTHS if L > 0]
    note(f"decode_varlen lengths {lengths}")
    seqs, cu, qp, kp, vp = ragged_inputs(lengths, 990)
    full = bits(kb.prefill_varlen(dev(qp), dev(kp), dev(vp), cu.tolist()))
    for ctx_of in (lambda L: L, lambda L: L // 2 + 1):
        ctx = [ctx_of(L) for L in lengths]
        qtok = np.stack([qp[:, cu[i] + c - 1] for i, c in enumerate(ctx)], axis=1)  # [Hq, batch, 128]
        got = bits(kb.decode_varlen(dev(np.ascontiguousarray(qtok)), dev(kp), dev(vp), cu.tolist(), ctx))
        for i, c in enumerate(ctx):
            same_bits(got[:, i], full[:, cu[i] + c - 1], f"decode of sequence {i} at context {c}")


def test_many_sequences_split_into_launches(kb):
    rng = np.random.default_rng(11)
    lengths = [int(x) for x in rng.integers(1, 400, size=70)] + [1500]
    note(f"prefill/decode_varlen with {len(lengths)} sequences")
    seqs, cu, qp, kp, vp = ragged_inputs(lengths, 1100, hkv=1)
    kd, vd = dev(kp), dev(vp)
    full = bits(kb.prefill_varlen(dev(qp), kd, vd, cu.tolist()))
    for i in (0, 31, 63, 64, 65, 69, 70):
        q, k, v = seqs[i]
        same_bits(full[:, cu[i]:cu[i + 1]], bits(kb.prefill(dev(q), dev(k), dev(v)))[0], f"sequence {i}")
    qtok = np.stack([qp[:, cu[i + 1] - 1] for i in range(len(lengths))], axis=1)
    got = bits(kb.decode_varlen(dev(np.ascontiguousarray(qtok)), kd, vd, cu.tolist(), lengths))
    same_bits(got, full[:, cu[1:] - 1], "decode of every sequence")


def test_decode_varlen_over_larger_cache_ranges(kb):
    # cache ranges longer than the valid keys, GQA with 2 KV heads
    lengths = [70, 1100, 5]
    caps = [128, 2048, 64]
    note(f"decode_varlen kv_lens {lengths} capacities {caps}")
    rng_seqs = [kb_gen.attention_inputs(1200 + i, 1, c, 8, 2, D) for i, c in enumerate(caps)]
    cu_c = np.concatenate([[0], np.cumsum(caps)]).tolist()
    kp = np.ascontiguousarray(np.concatenate([s[1][0] for s in rng_seqs], axis=1))
    vp = np.ascontiguousarray(np.concatenate([s[2][0] for s in rng_seqs], axis=1))
    qtok = np.ascontiguousarray(np.stack([s[0][0, :, L - 1] for s, L in zip(rng_seqs, lengths)], axis=1))
    got = bits(kb.decode_varlen(dev(qtok), dev(kp), dev(vp), cu_c, lengths))
    for i, ((q, k, v), L) in enumerate(zip(rng_seqs, lengths)):
        ref = bits(kb.decode(dev(np.ascontiguousarray(q[:, :, L - 1:L])), dev(k), dev(v), kv_len=L))
        same_bits(got[:, i], ref[0, :, 0], f"sequence {i} ragged decode vs dense decode")
        compare(got[:, i], oracle.attention(np.ascontiguousarray(q[:, :, L - 1:L]), k, v, kv_len=L,
                                            threads=oracle_threads())[0, :, 0],
                f"sequence {i} decode vs oracle")
