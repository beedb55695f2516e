"""Seeded random shapes through all three entry points (GPU).

Each case draws batch, KV heads, sequence length, a random cut of the
sequence into partitioned chunks and a set of decode contexts; every output
is checked against the fp64 oracle within tolerance and the three entry
points are checked for identical bits.
"""
import os

import numpy as np
import pytest

import kb_gen
import oracle
from gpu_util import bits, compare, dev, note, oracle_threads, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kb():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bitwise_aligned_causal_amd as kb

    kb.lib()
    return kb


@pytest.mark.parametrize("case", range(12))
def test_random_shapes(kb, case):
    rng = np.random.default_rng(2024 + case)
    B = int(rng.integers(1, 4))
    hkv = int(rng.integers(1, 3))
    S = int(rng.integers(1, 1400))
    seed = 500 + case
    q, k, v = kb_gen.attention_inputs(seed, B, S, n_q_heads=4 * hkv, n_kv_heads=hkv)
    note(f"fuzz case {case}: B={B} Hkv={hkv} S={S} seed={seed}")
    qd, kd, vd = dev(q), dev(k), dev(v)
    pre = bits(kb.prefill(qd, kd, vd))
    compare(pre, oracle.attention(q, k, v, threads=oracle_threads()), f"fuzz {case} prefill")
    # a random cut into partitioned chunks
    cuts = sorted(set(rng.integers(1, S, size=min(4, max(S - 1, 0))).tolist())) if S > 1 else []
    start = 0
    for stop in cuts + [S]:
        part = bits(kb.partitioned(qd[:, :, start:stop].contiguous(), kd, vd, kv_len=stop))
        n = int(np.count_nonzero(part != pre[:, :, start:stop]))
        assert n == 0, f"fuzz {case}: partitioned rows {start}..{stop}: {n} bit patterns differ"
        start = stop
    # decode at random contexts, over the full cache and over an exact-size copy
    for c in sorted(set(rng.integers(1, S + 1, size=3).tolist()) | {S}):
        d1 = bits(kb.decode(qd[:, :, c - 1:c].contiguous(), kd, vd, kv_len=c))
        d2 = bits(kb.decode(qd[:, :, c - 1:c].contiguous(), kd[:, :, :c].contiguous(), vd[:, :, :c].contiguous()))
        for name, d in (("full cache", d1), ("exact cache", d2)):
            n = int(np.count_nonzero(d[:, :, 0] != pre[:, :, c - 1]))
            assert n == 0, f"fuzz {case}: decode context {c} ({name}): {n} bit patterns differ"


# long cases: several 1024-key chunks, so the chunk folds of the prefill and
# the decode's combine run at random lengths; KB_FUZZ_LONG_CASES widens the
# sweep (default 6)
N_LONG = int(os.environ.get("KB_FUZZ_LONG_CASES", "6"))


@pytest.mark.parametrize("case", range(N_LONG))
def test_random_long_shapes(kb, case):
    rng = np.random.default_rng(7100 + case)
    B = int(rng.integers(1, 3))
    hkv = int(rng.integers(1, 3))
    S = int(rng.integers(1400, 6000))
    seed = 900 + case
    q, k, v = kb_gen.attention_inputs(seed, B, S, n_q_heads=4 * hkv, n_kv_heads=hkv)
    note(f"long fuzz case {case}: B={B} Hkv={hkv} S={S} seed={seed}")
    qd, kd, vd = dev(q), dev(k), dev(v)
    pre = bits(kb.prefill(qd, kd, vd))
    rows = sample_rows(rng, B, 4 * hkv, S, extra=6)
    ref = oracle.attention(q, k, v, rows=rows, threads=oracle_threads())
    compare(pre.reshape(-1, q.shape[-1])[rows], ref, f"long fuzz {case} prefill sampled rows")
    cuts = sorted(set(rng.integers(1, S, size=5).tolist()))
    start = 0
    for stop in cuts + [S]:
        part = bits(kb.partitioned(qd[:, :, start:stop].contiguous(), kd, vd, kv_len=stop))
        n = int(np.count_nonzero(part != pre[:, :, start:stop]))
        assert n == 0, f"long fuzz {case}: partitioned rows {start}..{stop}: {n} bit patterns differ"
        start = stop
    for c in sorted(set(rng.integers(1, S + 1, size=4).tolist()) | {S}):
        d = bits(kb.decode(qd[:, :, c - 1:c].contiguous(), kd, vd, kv_len=c))
        n = int(np.count_nonzero(d[:, :, 0] != pre[:, :, c - 1]))
        assert n == 0, f"long fuzz {case}: decode context {c}: {n} bit patterns differ"
