"""Host-side behaviour of the binding and the bench (CPU only)."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import bitwise_aligned_causal_amd as kb

    monkeypatch.setattr(kb, "_lib", None)
    monkeypatch.setattr(kb, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        kb.lib()


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_bench_flop_count_matches_oracle_rows():
    sys.path.insert(0, ROOT)
    import bench
    import oracle

    # prefill_flops sums 4*D*(pos+1) over positions for every (b, h)
    for first, n in ((0, 1), (0, 100), (1024, 1024), (5, 37)):
        per_bh = oracle.row_flops(np.arange(first, first + n))
        assert bench.prefill_flops(3, first, n) == 3 * bench.HQ * per_bh
    s = 16384
    assert bench.prefill_flops(16, 0, s) == 2 * 16 * 32 * 128 * s * (s + 1)


def test_kernel_source_hash_is_stable():
    sys.path.insert(0, ROOT)
    import bench

    assert bench.kernel_source_hash() == bench.kernel_source_hash()
    assert len(bench.kernel_source_hash()) == 16


def test_build_flags_that_the_kernels_rely_on():
    """The contract places every fused multiply-add explicitly (no contraction),
    packed fp32 arithmetic stays off, the code targets gfx950 only, and MFMA
    operands stay in ordinary vector registers."""
    from bitwise_aligned_causal_amd import _build

    flags = _build.HIPCC_FLAGS
    assert "-ffp-contract=off" in flags
    i = flags.index("-packed-fp32-ops")
    assert flags[i - 3:i] == ["-Xclang", "-target-feature", "-Xclang"]
    assert [f for f in flags if f.startswith("--offload-arch")] == ["--offload-arch=gfx950"]
    assert "-mllvm=-amdgpu-mfma-vgpr-form" in flags


def test_kernel_hash_covers_the_build_flags(monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    from bitwise_aligned_causal_amd import _build

    before = bench.kernel_source_hash()
    monkeypatch.setattr(_build, "HIPCC_FLAGS", _build.HIPCC_FLAGS + ["-DKB_EXTRA"])
    assert bench.kernel_source_hash() != before
