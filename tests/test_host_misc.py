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


def test_bench_flop_counts():
    sys.path.insert(0, ROOT)
    import bench

    # prefill_flops sums 4*D*(pos+1) over positions for every (b, h)
    for first, n in ((0, 1), (0, 100), (1024, 1024), (5, 37)):
        per_bh = bench.row_flops(np.arange(first, first + n))
        assert per_bh == sum(4 * 128 * (p + 1) for p in range(first, first + n))
        assert bench.prefill_flops(3, first, n) == 3 * bench.HQ * per_bh
    s = 16384
    assert bench.prefill_flops(16, 0, s) == 2 * 16 * 32 * 128 * s * (s + 1)


def test_kernel_source_hash_is_stable():
    sys.path.insert(0, ROOT)
    import bench

    assert bench.kernel_source_hash() == bench.kernel_source_hash()
    assert len(bench.kernel_source_hash()) == 16


def test_git_record_without_helper_processes(monkeypatch):
    """Profiled bench runs take the commit from the build record, never from git."""
    sys.path.insert(0, ROOT)
    import bench

    def refuse(*a, **k):
        raise AssertionError("subprocess started")

    monkeypatch.setattr(subprocess, "run", refuse)
    rec = bench.git_head(spawn=False)
    assert rec["from"] in ("build record", "unavailable")


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


class _FakeLib:
    """Stands in for libkb_attn.so: workspace queries answer 64 bytes, any
    other call is recorded (a compute call must never be reached)."""

    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def fn(*args):
            if name.endswith("_workspace_bytes"):
                return 64
            self.calls.append(name)
            return 0
        return fn


@pytest.fixture
def cpu_binding(monkeypatch):
    """The binding with its GPU-residency check relaxed to CPU tensors and a
    fake library, so that the shape checks run without a GPU."""
    import torch

    import bitwise_aligned_causal_amd as kb

    def check_tensor(name, x, ndim=4):
        if x.dtype != torch.bfloat16 or x.dim() != ndim or not x.is_contiguous():
            raise ValueError(f"{name}: bad tensor")

    fake = _FakeLib()
    monkeypatch.setattr(kb, "_check_tensor", check_tensor)
    monkeypatch.setattr(kb, "lib", lambda: fake)
    return kb, fake


def _bf(*shape):
    import torch
    return torch.zeros(shape, dtype=torch.bfloat16)


def test_binding_rejects_wrong_output_shape_before_any_launch(cpu_binding):
    kb, fake = cpu_binding
    q, k, v = _bf(1, 4, 64, 128), _bf(1, 1, 64, 128), _bf(1, 1, 64, 128)
    q1 = _bf(1, 4, 1, 128)
    small, wrong_heads = _bf(1, 4, 32, 128), _bf(1, 8, 64, 128)
    calls = [
        lambda: kb.prefill(q, k, v, out=small),
        lambda: kb.prefill(q, k, v, out=wrong_heads),
        lambda: kb.prefill_lse(q, k, v, out=small),
        lambda: kb.partitioned(q, k, v, kv_len=64, out=small),
        lambda: kb.partitioned_lse(q, k, v, kv_len=64, out=small),
        lambda: kb.decode(q1, k, v, kv_len=64, out=_bf(1, 4, 2, 128)),
        lambda: kb.decode_lse(q1, k, v, kv_len=64, out=_bf(2, 4, 1, 128)),
        lambda: kb.decode_multi(_bf(1, 4, 2, 128), k, v, kv_len=64, out=_bf(1, 4, 1, 128)),
        lambda: kb.prefill_varlen(_bf(4, 64, 128), _bf(1, 64, 128), _bf(1, 64, 128), [0, 64],
                                  out=_bf(4, 63, 128)),
        lambda: kb.prefill_varlen_lse(_bf(4, 64, 128), _bf(1, 64, 128), _bf(1, 64, 128), [0, 64],
                                      out=_bf(4, 63, 128)),
        lambda: kb.partitioned_varlen(_bf(4, 8, 128), _bf(1, 64, 128), _bf(1, 64, 128), [0, 8], [0, 64], [64],
                                      out=_bf(4, 7, 128)),
        lambda: kb.decode_varlen(_bf(4, 1, 128), _bf(1, 64, 128), _bf(1, 64, 128), [0, 64], [64],
                                 out=_bf(2, 1, 128)),
    ]
    for i, call in enumerate(calls):
        with pytest.raises(ValueError):
            call()
        assert fake.calls == [], f"case {i} reached the library"


def test_binding_rejects_wrong_gradient_shapes_before_any_launch(cpu_binding, monkeypatch):
    import torch

    kb, fake = cpu_binding
    q, k, v = _bf(1, 4, 64, 128), _bf(1, 1, 64, 128), _bf(1, 1, 64, 128)
    o, do = _bf(1, 4, 64, 128), _bf(1, 4, 64, 128)
    lse = torch.zeros((1, 4, 64), dtype=torch.float32)
    # lse is an input that must live on the GPU; its own check is covered elsewhere
    monkeypatch.setattr(kb, "_check_lse_in", lambda *a: None)
    bad_grads = {"dq": _bf(1, 4, 32, 128), "dk": _bf(1, 2, 64, 128), "dv": _bf(1, 1, 63, 128)}
    for name, bad in bad_grads.items():
        with pytest.raises(ValueError, match=name):
            kb.backward(q, k, v, o, do, lse, **{name: bad})
        assert fake.calls == []
    packed = {"dq": _bf(4, 63, 128), "dk": _bf(1, 64, 127), "dv": _bf(2, 64, 128)}
    qp, kp, vp = _bf(4, 64, 128), _bf(1, 64, 128), _bf(1, 64, 128)
    for name, bad in packed.items():
        with pytest.raises(ValueError):
            kb.backward_varlen(qp, kp, vp, _bf(4, 64, 128), _bf(4, 64, 128), torch.zeros((4, 64)), [0, 64],
                               **{name: bad})
        assert fake.calls == []


def test_binding_accepts_matching_output(cpu_binding, monkeypatch):
    kb, fake = cpu_binding
    monkeypatch.setattr(kb, "_stream", lambda x: None)
    q, k, v = _bf(1, 4, 64, 128), _bf(1, 1, 64, 128), _bf(1, 1, 64, 128)
    out = _bf(1, 4, 64, 128)
    assert kb.prefill(q, k, v, out=out) is out
    assert fake.calls == ["kb_attn_prefill"]


def test_data_study_summary_reads_clock_per_case(tmp_path):
    """bench_profile's clock-by-input summary: per case (launches in
    bench.DATA_STUDY_CASES order, the first of each dropped), the median
    duration and GRBM_COUNT / (8 XCDs x duration)."""
    sys.path.insert(0, ROOT)
    import bench
    import bench_profile

    reps = 3
    src = tmp_path / "data" / "run_counter_collection.csv"
    src.parent.mkdir()
    lines = ["Dispatch_Id,Kernel_Name,Grid_Size,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp"]
    d = 0
    for i, _ in enumerate(bench.DATA_STUDY_CASES):
        ghz = 1.5 + 0.25 * i
        for r in range(reps):
            d += 1
            ns = 20_000_000 + 1_000_000 * i + (5_000_000 if r == 0 else 0)  # the first launch is slower
            lines.append(f"{d},prefill_kernel<false>(kb::PrefillArgs),1,GRBM_COUNT,{8 * ghz * ns},0,{ns}")
            lines.append(f"{d},prefill_kernel<false>(kb::PrefillArgs),1,GRBM_GUI_ACTIVE,{8 * ghz * ns},0,{ns}")
        d += 1
        lines.append(f"{d},decode_kernel(kb::DecodeArgs),1,GRBM_COUNT,1,0,1")
    src.write_text("\n".join(lines) + "\n")
    bench_profile.data_study_summary(str(tmp_path / "data"), str(tmp_path / "out"), "h", reps=reps)
    text = (tmp_path / "out" / "prefill_kernel_b16_s16384_clock_by_data.txt").read_text()
    for i, name in enumerate(bench.DATA_STUDY_CASES):
        line = next(l for l in text.splitlines() if l.strip().startswith(name + " "))
        assert f"{20 + i:.3f} ms" in line and f"{1.5 + 0.25 * i:.3f} GHz" in line, line
