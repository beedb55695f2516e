"""Helpers for the GPU tests: move generator output to the device, read bits
back, compare with the oracle."""
import os
import sys

import numpy as np

import kb_gen

MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def note(msg: str) -> None:
    """Name the case on stderr before a GPU step."""
    sys.stderr.write(f"[gpu-case] {msg}\n")
    sys.stderr.flush()


def dev(x: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to("cuda:0").view(torch.bfloat16)


def bits(t) -> np.ndarray:
    import torch

    torch.cuda.synchronize()
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def compare(got_bits: np.ndarray, ref: np.ndarray, what: str):
    """Tolerance check of bf16 GPU output against the fp64 oracle."""
    got = kb_gen.bf16_bits_to_f32(got_bits).astype(np.float64).reshape(ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    worst = np.unravel_index(int(err.argmax()), err.shape)
    msg = f"{what}: max_abs {err.max():.3e} at {worst}, mean_abs {err.mean():.3e}"
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, msg
    return float(err.max()), float(err.mean())


def sample_rows(rng: np.random.Generator, batch: int, n_heads: int, q_len: int, extra: int,
                fixed=(0, 1, 63, 64, 65, 1023, 1024, 1025)) -> np.ndarray:
    """Flat row ids: per (b, h) the fixed positions that exist, q_len/2, q_len-1 and `extra` random rows."""
    out = []
    base = sorted({r for r in fixed if r < q_len} | {q_len // 2, q_len - 1})
    for bh in range(batch * n_heads):
        rows = set(base) | set(rng.integers(0, q_len, size=extra).tolist())
        out.extend(bh * q_len + r for r in sorted(rows))
    return np.array(out, dtype=np.int64)


def oracle_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))
