"""GPU parity of the paged-KV decode: for the same keys, paged decode gives
the dense decode's bits (through the C-ABI), whatever the page order."""
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


def paged_cache(k, page_size, rng, extra_pages=5):
    """Pool [n_pages, Hkv, page_size, 128] holding k [B, Hkv, cap, 128] in
    shuffled pages, and the block table [B, cap / page_size]."""
    B, hkv, cap, d = k.shape
    mp = cap // page_size
    n_pages = B * mp + extra_pages
    phys = rng.permutation(n_pages)[: B * mp].reshape(B, mp)
    pool = np.zeros((n_pages, hkv, page_size, d), dtype=k.dtype)
    for b in range(B):
        for p in range(mp):
            pool[phys[b, p]] = k[b, :, p * page_size:(p + 1) * page_size]
    return pool, phys.astype(np.int32)


@pytest.mark.parametrize("page_size", [64, 128, 256])
def test_paged_decode_equals_dense(kb, page_size):
    import torch

    lengths = [1, 63, 64, 65, 1000, 1024, 1025, 3000, 4097]
    cap = 4608  # a multiple of every page size here
    B = len(lengths)
    note(f"decode_paged page_size {page_size} lengths {lengths}")
    q, k, v = kb_gen.attention_inputs(1300 + page_size, B, cap, HQ, HKV, D)
    rng = np.random.default_rng(page_size)
    kpool, table = paged_cache(k, page_size, rng)
    vpool, _ = paged_cache(v, page_size, np.random.default_rng(page_size))  # same permutation
    qtok = np.ascontiguousarray(np.stack([q[b, :, L - 1] for b, L in enumerate(lengths)]))  # [B, Hq, 128]
    tab = torch.from_numpy(table).cuda()
    got = bits(kb.decode_paged(dev(qtok), dev(kpool), dev(vpool), tab, lengths))
    kd, vd = dev(k), dev(v)
    for b, L in enumerate(lengths):
        ref = bits(kb.decode(dev(np.ascontiguousarray(q[b:b + 1, :, L - 1:L])), kd[b:b + 1], vd[b:b + 1],
                             kv_len=L))
        n = int(np.count_nonzero(got[b] != ref[0, :, 0]))
        assert n == 0, f"page size {page_size}, sequence {b} (L={L}): {n} bit patterns differ from dense decode"
    b = lengths.index(1025)
    compare(got[b], oracle.attention(np.ascontiguousarray(q[b:b + 1, :, 1024:1025]), k[b:b + 1], v[b:b + 1],
                                     kv_len=1025, threads=oracle_threads())[0, :, 0], "paged decode L=1025 vs oracle")


def test_unused_and_out_of_pool_table_entries(kb):
    import torch

    page_size, lengths, cap = 128, [300, 130], 512
    note("decode_paged table entries beyond the context and outside the pool")
    q, k, v = kb_gen.attention_inputs(1400, 2, cap, HQ, HKV, D)
    kpool, table = paged_cache(k, page_size, np.random.default_rng(0))
    vpool, _ = paged_cache(v, page_size, np.random.default_rng(0))
    qtok = np.ascontiguousarray(np.stack([q[b, :, L - 1] for b, L in enumerate(lengths)]))
    qd, kp, vp = dev(qtok), dev(kpool), dev(vpool)
    ref = bits(kb.decode_paged(qd, kp, vp, torch.from_numpy(table).cuda(), lengths))
    # entries past each context's last page are never read
    junk = table.copy()
    junk[0, 3:] = -7
    junk[1, 2:] = 1 << 30
    same = bits(kb.decode_paged(qd, kp, vp, torch.from_numpy(junk).cuda(), lengths))
    assert np.array_equal(same, ref)
    # an entry in use but outside the pool is clamped into it: the call stays
    # inside the pool and equals the call that names the pool's last page
    n_pages = kpool.shape[0]
    bad, last = table.copy(), table.copy()
    bad[0, 1], last[0, 1] = n_pages + 100, n_pages - 1
    got = bits(kb.decode_paged(qd, kp, vp, torch.from_numpy(bad).cuda(), lengths))
    want = bits(kb.decode_paged(qd, kp, vp, torch.from_numpy(last).cuda(), lengths))
    assert np.array_equal(got, want)
    assert np.isfinite(kb_gen.bf16_bits_to_f32(got)).all()
