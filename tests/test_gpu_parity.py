"""GPU parity: the HIP path against the oracle, and the three entry points
against each other bit for bit, on the workloads of the KernelBraid README
("Features": prefill 1K-16K, decode contexts 128-8K, batch 1-16, 32/8 heads,
D = 128; "Usage": decode of the last token equals the last prefill row).

Every call goes through the C-ABI (the binding only marshals pointers).
Tolerance against the fp64 oracle: max-abs 2e-2 and mean-abs 2e-3 over the
compared elements; across entry points: zero differing bf16 bit patterns.
"""
import json
import os

import numpy as np
import pytest

import kb_gen
import oracle
from gpu_util import bits, compare, dev, note, oracle_threads, sample_rows

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
HQ, HKV, D = 32, 8, 128


@pytest.fixture(scope="module")
def kb():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bitwise_aligned_causal_amd as kb

    kb.lib()  # fails loudly when the HIP library is missing
    return kb


def assert_same_bits(a: np.ndarray, b: np.ndarray, what: str):
    assert a.shape == b.shape, f"{what}: shapes {a.shape} vs {b.shape}"
    n = int(np.count_nonzero(a != b))
    assert n == 0, f"{what}: {n} of {a.size} bf16 bit patterns differ"


def test_worked_example(kb):
    """README 'Usage': B=1, S=1024, seed 17; last prefill row == decode, as raw bits;
    plus decode at contexts 1..128 over the same K/V (capacity 1024)."""
    with open(os.path.join(GOLDEN, "worked_example.json")) as fh:
        case = json.load(fh)["case"]
    B, S, seed = case["batch"], case["seq_len"], case["seed"]
    q, k, v = kb_gen.attention_inputs(seed, B, S, case["n_q_heads"], case["n_kv_heads"], case["head_dim"])
    note(f"worked example B={B} S={S} seed={seed}: prefill + decode")
    qd, kd, vd = dev(q), dev(k), dev(v)
    pre = kb.unified_prefill(qd, kd, vd, HQ, HKV)
    dec = kb.unified_decode(qd[:, :, -1:].contiguous(), kd, vd, HQ, HKV)
    pre_bits = bits(pre)
    assert pre.shape == qd.shape and dec.shape == (B, HQ, 1, D)
    assert_same_bits(bits(dec)[:, :, 0], pre_bits[:, :, -1], "decode vs last prefill row")
    compare(pre_bits, oracle.attention(q, k, v, threads=oracle_threads()), "prefill S=1024 vs oracle")
    for c in range(1, 129):
        d = kb.decode(qd[:, :, c - 1:c].contiguous(), kd, vd, kv_len=c)
        assert_same_bits(bits(d)[:, :, 0], pre_bits[:, :, c - 1], f"decode context {c}")


def test_prefill_b4_s4096_and_decode_1024(kb):
    B, S, seed = 4, 4096, 2
    q, k, v = kb_gen.attention_inputs(seed, B, S)
    note(f"prefill B={B} S={S} seed={seed}")
    qd, kd, vd = dev(q), dev(k), dev(v)
    pre_bits = bits(kb.prefill(qd, kd, vd))
    note("decode kv_len=1024 over the S=4096 cache")
    dec = kb.decode(qd[:, :, 1023:1024].contiguous(), kd, vd, kv_len=1024)
    assert_same_bits(bits(dec)[:, :, 0], pre_bits[:, :, 1023], "decode(1024) vs prefill row 1023")
    rows = sample_rows(np.random.default_rng(seed), B, HQ, S, extra=14)
    ref = oracle.attention(q, k, v, rows=rows, threads=oracle_threads())
    compare(pre_bits.reshape(-1, D)[rows], ref, f"prefill B={B} S={S} sampled rows")


def test_prefill_b8_s8192_partitioned_chunks(kb):
    B, S, seed = 8, 8192, 3
    q, k, v = kb_gen.attention_inputs(seed, B, S)
    note(f"prefill B={B} S={S} seed={seed}")
    qd, kd, vd = dev(q), dev(k), dev(v)
    pre_bits = bits(kb.prefill(qd, kd, vd))
    for c in range(8):
        note(f"partitioned chunk {c}: q_len=1024 kv_len={1024 * (c + 1)} capacity={S}")
        part = kb.partitioned(qd[:, :, 1024 * c:1024 * (c + 1)].contiguous(), kd, vd, kv_len=1024 * (c + 1))
        assert_same_bits(bits(part), pre_bits[:, :, 1024 * c:1024 * (c + 1)], f"partitioned chunk {c}")
    rows = sample_rows(np.random.default_rng(seed), B, HQ, S, extra=6)
    ref = oracle.attention(q, k, v, rows=rows, threads=oracle_threads())
    compare(pre_bits.reshape(-1, D)[rows], ref, f"prefill B={B} S={S} sampled rows")


@pytest.mark.parametrize("B", [1, 4, 8, 16])
@pytest.mark.parametrize("L", [128, 1024, 4096, 8192])
def test_decode_sweep(kb, B, L):
    seed = 1000 + 10 * B + L
    q_full, k, v = kb_gen.attention_inputs(seed, B, L)
    q = np.ascontiguousarray(q_full[:, :, -1:])
    note(f"decode sweep B={B} L={L} seed={seed}")
    qd, kd, vd = dev(q), dev(k), dev(v)
    dec_bits = bits(kb.decode(qd, kd, vd))
    ref = oracle.attention(q, k, v, threads=oracle_threads())
    compare(dec_bits, ref, f"decode B={B} L={L}")
    note(f"prefill of the same cache B={B} L={L}")
    pre = kb.prefill(dev(q_full), kd, vd)
    assert_same_bits(dec_bits[:, :, 0], bits(pre[:, :, -1]), f"decode vs prefill row {L - 1}")


def test_prefill_b16_s16384_outliers_and_decode_8192(kb):
    import torch

    B, S, seed = 16, 16384, 5
    q, k, v = kb_gen.attention_inputs(seed, B, S, outliers=4)
    note(f"prefill B={B} S={S} seed={seed} with 4 outlier channels x8")
    qd, kd, vd = dev(q), dev(k), dev(v)
    pre = kb.prefill(qd, kd, vd)
    note("decode kv_len=8192 over the S=16384 cache")
    dec = kb.decode(qd[:, :, 8191:8192].contiguous(), kd, vd, kv_len=8192)
    assert_same_bits(bits(dec)[:, :, 0], bits(pre[:, :, 8191]), "decode(8192) vs prefill row 8191")
    # the bench's partitioned calls (1024 rows against the cache; 2048 blocks,
    # the persistent kernel on a 256-CU device) for three of its 16 chunks
    for c in (0, 7, 15):
        note(f"partitioned chunk {c}: q_len=1024 kv_len={1024 * (c + 1)} capacity={S}")
        part = kb.partitioned(qd[:, :, 1024 * c:1024 * (c + 1)].contiguous(), kd, vd, kv_len=1024 * (c + 1))
        assert_same_bits(bits(part), bits(pre[:, :, 1024 * c:1024 * (c + 1)]), f"partitioned chunk {c}")
        del part
    rng = np.random.default_rng(seed)
    rows = sample_rows(rng, B, HQ, S, extra=4, fixed=(0, 1, 63, 64, 65, 1023, 1024, 1025, 8191))
    flat = pre.view(-1, D)
    got = bits(flat[torch.from_numpy(rows).to(flat.device)])
    del pre, flat, qd
    ref = oracle.attention(q, k, v, rows=rows, threads=oracle_threads())
    compare(got, ref, f"prefill B={B} S={S} outliers sampled rows")


@pytest.mark.parametrize("S", [1, 2, 31, 32, 33, 63, 64, 65, 100, 127, 129, 1023, 1025, 2049])
def test_ragged_prefill_against_oracle(kb, S):
    q, k, v = kb_gen.attention_inputs(40 + S, 1, S)
    note(f"ragged prefill S={S}")
    got = bits(kb.prefill(dev(q), dev(k), dev(v)))
    compare(got, oracle.attention(q, k, v, threads=oracle_threads()), f"prefill S={S}")


def test_partitioned_odd_chunks(kb):
    B, S = 2, 2100
    q, k, v = kb_gen.attention_inputs(77, B, S)
    qd, kd, vd = dev(q), dev(k), dev(v)
    note(f"prefill B={B} S={S}")
    pre_bits = bits(kb.prefill(qd, kd, vd))
    start = 0
    for size in (1, 7, 100, 1000, 31, 33, 64, 1, 863):
        stop = start + size
        note(f"partitioned rows {start}..{stop}")
        part = kb.partitioned(qd[:, :, start:stop].contiguous(), kd, vd, kv_len=stop)
        assert_same_bits(bits(part), pre_bits[:, :, start:stop], f"partitioned rows {start}..{stop}")
        start = stop
    assert start == S


def test_decode_contexts_not_multiple_of_tile_or_chunk(kb):
    B, S = 2, 4097
    q, k, v = kb_gen.attention_inputs(81, B, S)
    qd, kd, vd = dev(q), dev(k), dev(v)
    note(f"prefill B={B} S={S}")
    pre_bits = bits(kb.prefill(qd, kd, vd))
    for c in (1, 2, 63, 64, 65, 1023, 1024, 1025, 2048, 2049, 3000, 4096, 4097):
        note(f"decode context {c} over capacity {S}")
        dec = kb.decode(qd[:, :, c - 1:c].contiguous(), kd, vd, kv_len=c)
        assert_same_bits(bits(dec)[:, :, 0], pre_bits[:, :, c - 1], f"decode context {c}")
        note(f"decode context {c} over an exactly sized cache")
        dec2 = kb.decode(qd[:, :, c - 1:c].contiguous(), kd[:, :, :c].contiguous(), vd[:, :, :c].contiguous())
        assert_same_bits(bits(dec2)[:, :, 0], pre_bits[:, :, c - 1], f"decode context {c}, exact cache")


def test_causality_on_gpu(kb):
    q, k, v = kb_gen.attention_inputs(91, 1, 700)
    qd = dev(q)
    base = bits(kb.prefill(qd, dev(k), dev(v)))
    for p in (0, 63, 64, 500):
        k2, v2 = k.copy(), v.copy()
        k2[:, :, p + 1:] = kb_gen.normal_bf16(92, 2, k2[:, :, p + 1:].shape)
        v2[:, :, p + 1:] = kb_gen.normal_bf16(92, 3, v2[:, :, p + 1:].shape)
        note(f"causality: perturbed keys > {p}")
        got = bits(kb.prefill(qd, dev(k2), dev(v2)))
        assert_same_bits(got[:, :, :p + 1], base[:, :, :p + 1], f"rows <= {p} after perturbing keys > {p}")


def test_row_zero_is_v0_bitwise(kb):
    q, k, v = kb_gen.attention_inputs(93, 3, 130)
    note("row 0 == V0")
    got = bits(kb.prefill(dev(q), dev(k), dev(v)))
    assert_same_bits(got[:, :, 0], np.repeat(v[:, :, 0], 4, axis=1), "row 0 vs V[:, h // 4, 0]")


def test_batch_independence_and_determinism(kb):
    q, k, v = kb_gen.attention_inputs(95, 4, 1500)
    qd, kd, vd = dev(q), dev(k), dev(v)
    note("batch 4 prefill twice")
    full = bits(kb.prefill(qd, kd, vd))
    again = bits(kb.prefill(qd, kd, vd))
    assert_same_bits(again, full, "two identical runs")
    for b in range(4):
        note(f"batch element {b} alone")
        one = bits(kb.prefill(qd[b:b + 1].contiguous(), kd[b:b + 1].contiguous(), vd[b:b + 1].contiguous()))
        assert_same_bits(one, full[b:b + 1], f"batch element {b} alone vs in batch 4")
        dec = bits(kb.decode(qd[b:b + 1, :, 1499:1500].contiguous(), kd[b:b + 1].contiguous(),
                             vd[b:b + 1].contiguous()))
        assert_same_bits(dec[:, :, 0], full[b:b + 1, :, 1499], f"decode of batch element {b}")


@pytest.mark.parametrize("hkv", [1, 2, 3])
def test_small_gqa_shapes(kb, hkv):
    hq = 4 * hkv
    q, k, v = kb_gen.attention_inputs(97 + hkv, 2, 300, n_q_heads=hq, n_kv_heads=hkv)
    qd, kd, vd = dev(q), dev(k), dev(v)
    note(f"GQA Hq={hq} Hkv={hkv}")
    pre = bits(kb.prefill(qd, kd, vd))
    compare(pre, oracle.attention(q, k, v, threads=oracle_threads()), f"Hq={hq} Hkv={hkv}")
    dec = bits(kb.decode(qd[:, :, 299:300].contiguous(), kd, vd))
    assert_same_bits(dec[:, :, 0], pre[:, :, 299], "decode vs last row")


def test_constant_v(kb):
    q, k, v = kb_gen.attention_inputs(99, 1, 600)
    v[:] = kb_gen.f32_to_bf16_bits(np.full(v.shape, 1.5, dtype=np.float32))
    note("constant V")
    got = kb_gen.bf16_bits_to_f32(bits(kb.prefill(dev(q), dev(k), dev(v))))
    # the weights sum to one up to fp32 rounding; the output lands within one bf16 ulp of 1.5
    assert np.abs(got - 1.5).max() <= 2.0 ** -7


@pytest.mark.parametrize("scale", [1.0, 1e-3])
def test_extreme_scales(kb, scale):
    """A sharp softmax (scale 1: score spreads of hundreds of log2 units, so
    reference-max moves, exponentials that underflow to zero and chunk folds
    with a zero weight) and a nearly flat one (scale 1e-3: row sums close to
    the context length): the three entry points agree bit for bit and the
    prefill meets the oracle's tolerance on sampled rows."""
    B, S, seed = 2, 2100, 4242
    q, k, v = kb_gen.attention_inputs(seed, B, S)
    qd, kd, vd = dev(q), dev(k), dev(v)
    note(f"prefill B={B} S={S} scale={scale}")
    pre = bits(kb.prefill(qd, kd, vd, scale=scale))
    note(f"partitioned rows 1024.. and decode of the last row, scale={scale}")
    part = bits(kb.partitioned(qd[:, :, 1024:].contiguous(), kd, vd, kv_len=S, scale=scale))
    assert_same_bits(part, pre[:, :, 1024:], f"partitioned vs prefill, scale={scale}")
    dec = bits(kb.decode(qd[:, :, -1:].contiguous(), kd, vd, scale=scale))
    assert_same_bits(dec[:, :, 0], pre[:, :, -1], f"decode vs last prefill row, scale={scale}")
    rows = sample_rows(np.random.default_rng(seed), B, HQ, S, extra=10)
    ref = oracle.attention(q, k, v, scale=scale, rows=rows, threads=oracle_threads())
    compare(pre.reshape(-1, D)[rows], ref, f"prefill scale={scale} sampled rows")


def test_stale_workspace_does_not_matter(kb):
    import torch

    q, k, v = kb_gen.attention_inputs(101, 2, 3000)
    qd, kd, vd = dev(q), dev(k), dev(v)
    q_last = qd[:, :, -1:].contiguous()
    need = kb.decode_workspace_bytes(2, 3000)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda:0")
    note("decode with a NaN-filled workspace")
    a = bits(kb.decode(q_last, kd, vd, workspace=ws))
    ws.fill_(1e30)
    b = bits(kb.decode(q_last, kd, vd, workspace=ws))
    assert_same_bits(a, b, "decode with different stale workspaces")


def test_error_paths_on_gpu(kb):
    import ctypes

    import torch

    q = torch.zeros(1, 32, 64, 128, dtype=torch.bfloat16, device="cuda:0")
    k = torch.zeros(1, 8, 64, 128, dtype=torch.bfloat16, device="cuda:0")
    v = torch.zeros_like(k)
    o = torch.empty_like(q)
    host = torch.zeros(1, 32, 64, 128, dtype=torch.bfloat16).pin_memory()
    L = kb.lib()
    s = 128 ** -0.5
    note("error paths")
    assert L.kb_attn_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), host.data_ptr(), 1, 64, 32, 8, 128, s,
                             None) == -5
    assert L.kb_attn_prefill(q.data_ptr() + 2, k.data_ptr(), v.data_ptr(), o.data_ptr(), 1, 64, 32, 8, 128, s,
                             None) == -4
    plain = (ctypes.c_uint16 * 64)()
    assert L.kb_attn_prefill(ctypes.addressof(plain), k.data_ptr(), v.data_ptr(), o.data_ptr(), 1, 64, 32, 8, 128,
                             s, None) in (-4, -5)
    assert L.kb_attn_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), 1, 64, 32, 8, 128, s,
                             None) == 0
    torch.cuda.synchronize()
