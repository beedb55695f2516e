"""GPU tests of the multi-row decode (the last 1..8 tokens of each sequence,
split over 1024-key chunks): every row equals the prefill row at its
position bit for bit ("Method": one contract for prefill, partitioned forward
and decode), over contexts that cross tile and chunk boundaries and over a
cache larger than the context."""
import numpy as np
import pytest

import kb_gen
import oracle
from gpu_util import bits, compare, dev, note, oracle_threads

pytestmark = pytest.mark.gpu


def kb():
    import bitwise_aligned_causal_amd as m

    return m


@pytest.fixture(scope="module")
def seq():
    B, S = 2, 4200
    q, k, v = (kb_gen.normal_bf16(41, t, (B, 32 if t == 1 else 8, S, 128)) for t in (1, 2, 3))
    Q, K, V = dev(q), dev(k), dev(v)
    note("prefill for the multi-row decode tests")
    pre = bits(kb().prefill(Q, K, V))
    return q, k, v, Q, K, V, pre


@pytest.mark.parametrize("n_rows", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("kv_len", [8, 63, 64, 65, 1024, 1025, 1027, 1030, 2049, 4100])
def test_decode_multi_equals_prefill(seq, n_rows, kv_len):
    q, k, v, Q, K, V, pre = seq
    m = kb()
    note(f"decode_multi n_rows={n_rows} kv_len={kv_len}")
    qm = dev(np.ascontiguousarray(q[:, :, kv_len - n_rows:kv_len]))
    got = bits(m.decode_multi(qm, K, V, kv_len))
    assert np.array_equal(got, pre[:, :, kv_len - n_rows:kv_len]), f"n_rows={n_rows} kv_len={kv_len}"


def test_decode_multi_against_oracle_and_exact_cache(seq):
    q, k, v, Q, K, V, pre = seq
    m = kb()
    kv_len, n_rows = 3001, 7
    kc = dev(np.ascontiguousarray(k[:, :, :kv_len]))
    vc = dev(np.ascontiguousarray(v[:, :, :kv_len]))
    qm = np.ascontiguousarray(q[:, :, kv_len - n_rows:kv_len])
    note("decode_multi over an exactly sized cache")
    got = bits(m.decode_multi(dev(qm), kc, vc))
    assert np.array_equal(got, pre[:, :, kv_len - n_rows:kv_len])
    ref = oracle.attention(qm, np.ascontiguousarray(k[:, :, :kv_len]), np.ascontiguousarray(v[:, :, :kv_len]),
                           threads=oracle_threads())
    compare(got, ref, "decode_multi vs oracle")
