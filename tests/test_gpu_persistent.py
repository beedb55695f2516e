"""GPU: the prefill's two launch forms give the same bits.

A prefill or partitioned launch of 2 to 16 position blocks per CU (when its
blocks split evenly into the persistent schedule's rounds) runs the
persistent kernel, one workgroup per CU walking a fixed list of blocks;
any other launch runs one workgroup per block.  Rows of launches of the
first kind are compared bit for bit with the same rows from launches of the
second (partitioned calls of 128 rows: at most 64 blocks), and sampled rows
with the oracle.  The block counts below are those of a 256-CU MI355X; on
another CU count the comparisons still hold, whichever form runs.
"""
import numpy as np
import pytest

import kb_gen
import oracle
from gpu_util import bits, compare, dev, note, oracle_threads, sample_rows

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
    n = int(np.count_nonzero(a != b))
    assert a.shape == b.shape and n == 0, f"{what}: {n} of {a.size} bf16 bit patterns differ"


def test_persistent_prefill_equals_one_block_launches(kb):
    # B=2 S=8192: 2 * 8 * 128 = 2048 blocks, 8 per CU
    B, S, seed = 2, 8192, 11
    q, k, v = kb_gen.attention_inputs(seed, B, S)
    qd, kd, vd = dev(q), dev(k), dev(v)
    note(f"persistent prefill B={B} S={S} seed={seed}")
    pre = bits(kb.prefill(qd, kd, vd))
    for r0 in (0, 64, 1000, 4096, 8064):
        note(f"partitioned rows {r0}..{r0 + 127} at kv_len {r0 + 128} (one workgroup per block)")
        part = kb.partitioned(qd[:, :, r0:r0 + 128].contiguous(), kd, vd, kv_len=r0 + 128)
        same_bits(bits(part), pre[:, :, r0:r0 + 128], f"prefill rows {r0}..{r0 + 127}")
    rows = sample_rows(np.random.default_rng(seed), B, HQ, S, extra=4)
    compare(pre.reshape(-1, D)[rows], oracle.attention(q, k, v, rows=rows, threads=oracle_threads()),
            f"persistent prefill B={B} S={S} sampled rows")


def test_persistent_partitioned_equals_one_block_launches(kb):
    # B=4, 2048 rows at positions 6144..8191: 4 * 8 * 32 = 1024 blocks, 4 per CU
    B, S, seed, q_len = 4, 8192, 12, 2048
    q, k, v = kb_gen.attention_inputs(seed, B, S)
    qd, kd, vd = dev(q), dev(k), dev(v)
    r0 = S - q_len
    note(f"persistent partitioned B={B} rows {r0}..{S - 1} kv_len {S}")
    part = bits(kb.partitioned(qd[:, :, r0:].contiguous(), kd, vd, kv_len=S))
    for a in (0, 128, 1920):
        note(f"partitioned rows {r0 + a}..{r0 + a + 127} (one workgroup per block)")
        small = kb.partitioned(qd[:, :, r0 + a:r0 + a + 128].contiguous(), kd, vd, kv_len=r0 + a + 128)
        same_bits(bits(small), part[:, :, a:a + 128], f"rows {r0 + a}..{r0 + a + 127}")
    rows = sample_rows(np.random.default_rng(seed), B, HQ, q_len, extra=4, fixed=(0, 1, 63, 64, 65, 1023, 1024))
    flat = (rows // q_len) * S + r0 + rows % q_len
    ref = oracle.attention(q, k, v, rows=flat, threads=oracle_threads())
    compare(part.reshape(-1, D)[rows], ref, f"persistent partitioned B={B} sampled rows")


def test_persistent_partitioned_rows_off_the_block_grid(kb):
    # B=8, 1000 rows at positions 15384..16383: the first 64-position block
    # (15360..15423) holds 24 positions before the first row, so its lanes
    # for them store nothing; 8 * 8 * 16 = 1024 blocks, 4 per CU
    B, S, seed, q_len = 8, 16384, 13, 1000
    q, k, v = kb_gen.attention_inputs(seed, B, S)
    qd, kd, vd = dev(q), dev(k), dev(v)
    r0 = S - q_len
    note(f"persistent partitioned B={B} rows {r0}..{S - 1} kv_len {S}")
    out = kb.partitioned(qd[:, :, r0:].contiguous(), kd, vd, kv_len=S)
    part = bits(out)
    for a, n in ((0, 40), (40, 128), (872, 128)):
        note(f"partitioned rows {r0 + a}..{r0 + a + n - 1} (one workgroup per block)")
        small = kb.partitioned(qd[:, :, r0 + a:r0 + a + n].contiguous(), kd, vd, kv_len=r0 + a + n)
        same_bits(bits(small), part[:, :, a:a + n], f"rows {r0 + a}..{r0 + a + n - 1}")
    rows = sample_rows(np.random.default_rng(seed), B, HQ, q_len, extra=2, fixed=(0, 1, 23, 24, 25, 39, 40, 999))
    flat = (rows // q_len) * S + r0 + rows % q_len
    ref = oracle.attention(q, k, v, rows=flat, threads=oracle_threads())
    compare(part.reshape(-1, D)[rows], ref, f"persistent partitioned B={B} q_len={q_len} sampled rows")


def test_persistent_prefill_two_blocks_per_cu(kb):
    # B=1 S=4096: 8 * 64 = 512 blocks, 2 per CU (one even round, one odd)
    B, S, seed = 1, 4096, 14
    q, k, v = kb_gen.attention_inputs(seed, B, S)
    qd, kd, vd = dev(q), dev(k), dev(v)
    note(f"persistent prefill B={B} S={S} seed={seed}")
    pre = bits(kb.prefill(qd, kd, vd))
    for r0 in (0, 1984, 3968):
        note(f"partitioned rows {r0}..{r0 + 127} at kv_len {r0 + 128} (one workgroup per block)")
        part = kb.partitioned(qd[:, :, r0:r0 + 128].contiguous(), kd, vd, kv_len=r0 + 128)
        same_bits(bits(part), pre[:, :, r0:r0 + 128], f"prefill rows {r0}..{r0 + 127}")
    rows = sample_rows(np.random.default_rng(seed), B, HQ, S, extra=8)
    compare(pre.reshape(-1, D)[rows], oracle.attention(q, k, v, rows=rows, threads=oracle_threads()),
            f"persistent prefill B={B} S={S} sampled rows")


def test_persistent_prefill_lse_equals_one_block_launches(kb):
    # the log-sum-exp output of the persistent path (B=2 S=8192, 8 blocks per
    # CU) against one-workgroup-per-block partitioned_lse calls, bit for bit
    B, S, seed = 2, 8192, 15
    q, k, v = kb_gen.attention_inputs(seed, B, S)
    qd, kd, vd = dev(q), dev(k), dev(v)
    note(f"persistent prefill_lse B={B} S={S} seed={seed}")
    o, lse = kb.prefill_lse(qd, kd, vd)
    o_bits, lse_bits = bits(o), lse.cpu().numpy().view(np.uint32)
    for r0 in (0, 2048, 8064):
        note(f"partitioned_lse rows {r0}..{r0 + 127} (one workgroup per block)")
        oc, lc = kb.partitioned_lse(qd[:, :, r0:r0 + 128].contiguous(), kd, vd, r0 + 128)
        same_bits(bits(oc), o_bits[:, :, r0:r0 + 128], f"o rows {r0}..{r0 + 127}")
        same_bits(lc.cpu().numpy().view(np.uint32), lse_bits[:, :, r0:r0 + 128], f"lse rows {r0}..{r0 + 127}")
