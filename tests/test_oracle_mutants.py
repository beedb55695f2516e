"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case copies oracle/oracle.c, applies one plausible mistake (a dropped
term, a wrong sign or index, a transposed operand, an off-by-one mask, a wrong
stride), builds it with gcc in a temporary folder and runs a compact battery
of the same pins used in test_oracle_pins.py.  The unmodified copy must pass
the battery and every mutant must fail it.
"""
import math
import os
import subprocess

import numpy as np
import pytest

import kb_gen
import oracle
from test_oracle_pins import brute_force, f32, inputs

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "gqa_modulo_mapping": [("h / (p->n_q_heads / p->n_kv_heads)", "h % p->n_kv_heads")],
    "top_left_causal": [("const int64_t pos = p->kv_len - p->q_len + r;", "const int64_t pos = r;")],
    "dropped_scale": [("s[j] = p->scale * dot;", "s[j] = dot;")],
    "reversed_k_channels": [("widen(kbase[j * D + d])", "widen(kbase[j * D + (D - 1 - d)])")],
    "v_read_from_k": [("widen(vbase[j * D + d])", "widen(kbase[j * D + d])")],
    "dropped_normalisation": [("for (int64_t d = 0; d < D; ++d) out[d] /= l;", "")],
    "exp_sign": [("s[j] = kbo_exp(s[j] - m);", "s[j] = kbo_exp(m - s[j]);")],
    "sees_one_future_key": [("j <= pos;", "j <= pos + (pos + 1 < p->kv_len);")],
    "drops_diagonal_key": [("j <= pos;", "j < pos + (pos == 0);")],
    "dropped_first_channel": [("for (int64_t d = 0; d < D; ++d) dot +=", "for (int64_t d = 1; d < D; ++d) dot +=")],
    "kv_stride_uses_length": [("(b * p->n_kv_heads + g) * p->kv_capacity * D",
                               "(b * p->n_kv_heads + g) * p->kv_len * D")],
    "weights_not_normalised": [("w[j] = (double)(s[j] / l);", "w[j] = (double)s[j];")],
}


def build_variant(tmp_path, name, edits):
    text = open(SRC).read()
    for old, new in edits:
        assert old in text, f"mutation anchor not found: {old!r}"
        text = text.replace(old, new)
    src = tmp_path / f"{name}.c"
    lib = tmp_path / f"lib{name}.so"
    src.write_text(text)
    subprocess.run(["gcc", "-std=c11", "-O1", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
                    "-DKBO_REAL=double", "-DKBO_SUFFIX=_f64", str(src), "-o", str(lib), "-lm"], check=True)
    return oracle.bind(str(lib), "f64")


def battery(entry) -> bool:
    """True when the build passes every pin in the compact battery."""
    ok = True
    # brute force, including GQA, a partitioned split and a cache larger than kv_len
    for (B, Hq, Hkv, q_len, kv_len, D, cap) in [(2, 4, 2, 5, 5, 8, 5), (2, 4, 2, 3, 9, 8, 12),
                                                (1, 8, 2, 6, 6, 16, 6)]:
        q, k, v = inputs(1000 + q_len, B, Hq, Hkv, q_len, kv_len, D, cap=cap)
        ref = brute_force(q, k, v, kv_len, 1 / math.sqrt(D))
        got = oracle.attention(q, k, v, kv_len=kv_len, entry=entry)
        ok &= bool(np.allclose(got, ref, rtol=1e-12, atol=1e-12))
    # rows sum to one
    q, k, v = inputs(5, 1, 4, 2, 20, 20, 8)
    for row in (0, 7, 19, 45):
        w = oracle.weights(q, k, v, row, entry=entry)
        ok &= abs(1 - math.fsum(w)) < 1e-12
    # causality
    base = oracle.attention(q, k, v, entry=entry)
    k2 = k.copy()
    k2[:, :, 11:] = kb_gen.normal_bf16(77, 2, k2[:, :, 11:].shape)
    ok &= bool(np.array_equal(oracle.attention(q, k2, v, entry=entry)[:, :, :11], base[:, :, :11]))
    # GQA == MHA with repeated heads
    mha = oracle.attention(q, np.ascontiguousarray(np.repeat(k, 2, axis=1)),
                           np.ascontiguousarray(np.repeat(v, 2, axis=1)), entry=entry)
    ok &= bool(np.array_equal(base, mha))
    # constant V and row 0
    vc = kb_gen.f32_to_bf16_bits(np.full(v.shape, 1.5, dtype=np.float32))
    ok &= bool(np.allclose(oracle.attention(q, k, vc, entry=entry), 1.5, rtol=1e-13, atol=0))
    ok &= bool(np.array_equal(base[:, :, 0], np.repeat(f32(v[:, :, 0]), 2, axis=1)))
    return ok


def test_unmodified_copy_passes(tmp_path):
    entry = build_variant(tmp_path, "clean", [])
    assert battery(entry)
    assert bwd_battery(entry)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    assert not battery(build_variant(tmp_path, name, MUTANTS[name])), f"pins missed mutant {name}"


# Mistakes planted in the log-sum-exp and the backward; caught by the
# backward pins of test_oracle_bwd_pins.py.
BWD_MUTANTS = {
    "lse_drops_max": [("if (lse) *lse = m + kbo_log(l);", "if (lse) *lse = kbo_log(l);")],
    "ds_drops_d_term": [("ds[j] = (real)w[j] * (dp - Di);", "ds[j] = (real)w[j] * dp;")],
    "ds_sign": [("ds[j] = (real)w[j] * (dp - Di);", "ds[j] = (real)w[j] * (Di - dp);")],
    "dp_reads_k": [("const uint16_t* vrows = p->v + (b * p->n_kv_heads + g) * S * D;",
                    "const uint16_t* vrows = p->k + (b * p->n_kv_heads + g) * S * D;")],
    "dv_uses_q": [("if (dvb) dvb[j * D + d] += (double)((real)w[j] * dod);",
                   "if (dvb) dvb[j * D + d] += (double)((real)w[j] * qd);")],
    "dk_unscaled": [("if (dkb) dkb[j * D + d] += (double)(p->scale * ds[j] * qd);",
                     "if (dkb) dkb[j * D + d] += (double)(ds[j] * qd);")],
    "dq_reversed_channels": [("acc += ds[j] * widen(krows[j * D + d]);",
                              "acc += ds[j] * widen(krows[j * D + (D - 1 - d)]);")],
    "d_uses_v0": [("for (int64_t d = 0; d < D; ++d) Di += widen(dorow[d]) * o[d];",
                   "for (int64_t d = 0; d < D; ++d) Di += widen(dorow[d]) * widen(vrows[d]);")],
    "dk_to_wrong_group": [("b = x / Hkv;\n            g = x % Hkv;\n            h_first = g * hpg;",
                           "b = x / Hkv;\n            g = x % Hkv;\n            h_first = ((g + 1) % Hkv) * hpg;")],
    # mistakes in the error budgets that leave every gradient bit unchanged
    "ev_drops_weight": [("if (evb) evb[j * D + d] += w[j] * fabs((double)dod);",
                         "if (evb) evb[j * D + d] += fabs((double)dod);")],
    "ek_times_length": [("if (ekb) ekb[j * D + d] += (double)p->scale * (fabs((double)ds[j]) + w[j] * Ai)",
                         "if (ekb) ekb[j * D + d] += (double)S * p->scale * (fabs((double)ds[j]) + w[j] * Ai)")],
    "eq_drops_pa_term": [("if (eqr) bud += (fabs((double)ds[j]) + w[j] * Ai)",
                          "if (eqr) bud += (fabs((double)ds[j]))")],
}


def bwd_battery(entry) -> bool:
    """True when the build passes the backward and log-sum-exp pins."""
    import test_oracle_bwd_pins as bp

    ok = True
    for shape in [(2, 4, 2, 7, 8), (1, 8, 2, 17, 16)]:
        B, Hq, Hkv, S, D = shape
        q, k, v, do = bp.grads_inputs(211 + sum(shape), B, Hq, Hkv, S, D)
        scale = 1.0 / math.sqrt(D)
        ref = bp.sdpa_autograd(q, k, v, do, scale)
        got = oracle.backward(q, k, v, do, scale=scale, entry=entry)
        for name, r in zip(("dq", "dk", "dv"), ref):
            ok &= bool(np.allclose(got[name], r, rtol=0, atol=1e-11 * max(1.0, np.abs(r).max())))
        lref = bp.masked_lse_torch(q, k, S, scale)
        ok &= bool(np.allclose(oracle.lse(q, k, v, scale=scale, entry=entry), lref, rtol=0, atol=1e-12))
        bud = oracle.backward(q, k, v, do, scale=scale, budgets=True, entry=entry)
        for name, r in zip(("eq", "ek", "ev"), bp.budgets_torch(q, k, v, do, scale)):
            ok &= bool(np.allclose(bud[name], r, rtol=1e-11, atol=1e-13))
    return ok


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_bwd_mutant_is_caught(tmp_path, name):
    assert not bwd_battery(build_variant(tmp_path, name, BWD_MUTANTS[name])), f"pins missed mutant {name}"
