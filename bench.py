"""Benchmark of the bitwise-aligned causal GQA attention hot path on one MI355X.

One step is one pass of the whole path over one batch of synthetic input
(B=16, S=16384, Hq=32, Hkv=8, D=128, bf16, Q/K ~ N(0,1) with 4 seeded outlier
channels x8, V ~ N(0,1), scale 1/sqrt(128)):
  1. full causal prefill of the 16384 rows              (prefill_kernel<false>)
  2. partitioned forward of the same rows in 16 chunks of 1024 against the
     cached K/V (2048 blocks per call, 8 per CU)     (prefill_persistent_kernel<true>)
  3. one-token decode at context 8192 (split-KV chunks + in-order combine)
Inputs are resident in HBM before the timed region.  Outside the step the
line also reports a decode sweep, a ragged batch, a paged-cache decode, a
multi-row decode and the backward of the prefill (each with its own bitwise
checks).  After timing, the
partitioned output and the decode output are compared bit for bit with the
prefill output.

Prints ONE JSON line (rank 0).  `value` is the step's algorithmic FLOPs
(causal work only: 4*D*(pos+1) per row) over the measured step time.  The
roofline object is for the dominant kernel (the full prefill launch), timed
with HIP events on the stream it runs on.  The CPU baseline times the oracle
on a bounded sample of the same rows.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

B, S, HQ, HKV, D = 16, 16384, 32, 8, 128
SEED = 5
PART = 1024
DEC_LEN = 8192
PEAK_BF16 = 2.5e15
PEAK_HBM = 8.0e12
METRIC = "prefill TFLOP/s + decode KV GB/s (frac of peak), bitwise prefill≡decode"
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "prefill_kernel_b16_s16384_traffic.json")


def prefill_flops(batch: int, n_rows_first_pos: int, n_rows: int) -> int:
    """4*D*(pos+1) summed over positions first..first+n_rows-1, per (b, h)."""
    p0, p1 = n_rows_first_pos, n_rows_first_pos + n_rows
    s = (p1 * (p1 + 1) - p0 * (p0 + 1)) // 2
    return 4 * D * s * batch * HQ


def row_flops(positions) -> int:
    """Algorithmic FLOPs of query rows at the given positions: QK^T and PV,
    2*D each per visible key, 4*D*(pos+1) per row."""
    positions = np.asarray(positions, dtype=np.int64)
    return int((4 * D * (positions + 1)).sum())


def backward_flops(batch: int, n_q_heads: int, seq_len: int, head_dim: int = D) -> int:
    """Algorithmic FLOPs of the causal backward: five products of 2*D FLOPs
    per visible (query, key) pair (S recomputed, dP, dV, dQ, dK)."""
    pairs = seq_len * (seq_len + 1) // 2
    return int(10 * head_dim * pairs * batch * n_q_heads)


def source_hash(names) -> str:
    """Hash of kernel sources with comments and whitespace removed, and of the
    compiler flags they are built with, so that a counter summary stays valid
    across edits that change no code and lapses when the code or the flags
    change."""
    from bitwise_aligned_causal_amd import _build

    h = hashlib.sha256()
    h.update(" ".join(_build.HIPCC_FLAGS).encode())
    for name in names:
        with open(os.path.join(ROOT, "bitwise_aligned_causal_amd", "csrc", name)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def device_env(torch, dev) -> dict:
    """The GPU and software the line was measured on."""
    p = torch.cuda.get_device_properties(dev)
    env = {"gpu": torch.cuda.get_device_name(dev), "arch": getattr(p, "gcnArchName", None),
           "compute_units": p.multi_processor_count, "hip": torch.version.hip, "torch": torch.__version__}
    clock = getattr(p, "clock_rate", None)
    if clock:
        env["clock_mhz"] = round(clock / 1000)
    return env


def gpu_clocks() -> dict | None:
    """Clock levels as rocm-smi reports them (text fields, as printed), or None."""
    import subprocess

    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=60)
        data = json.loads(r.stdout[r.stdout.index("{"):])
    except (OSError, ValueError, subprocess.SubprocessError):
        return None
    card = next(iter(data.values()), {}) if isinstance(data, dict) else {}
    return {k.strip(" :"): v for k, v in card.items() if "clk" in k.lower() or "clock" in k.lower()} or None


def git_head(spawn: bool = True) -> dict:
    """The commit the tree comes from: git itself in a checkout, else the record
    the library build leaves beside libkb_attn.so (a copied tree has no .git)."""
    import subprocess

    try:
        if not spawn or not os.path.isdir(os.path.join(ROOT, ".git")):
            raise FileNotFoundError(".git")
        head = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True,
                              timeout=30)
        if head.returncode == 0:
            dirty = subprocess.run(["git", "-C", ROOT, "status", "--porcelain", "--untracked-files=no"],
                                   capture_output=True, text=True, timeout=30)
            return {"commit": head.stdout.strip(), "dirty": bool(dirty.stdout.strip()), "from": "git"}
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open(os.path.join(ROOT, "bitwise_aligned_causal_amd", "_build_info.json")) as fh:
            rec = json.load(fh)
        return {"commit": rec.get("git_head"), "dirty": rec.get("dirty"), "from": "build record"}
    except (OSError, ValueError):
        return {"commit": None, "dirty": None, "from": "unavailable"}


def worst_error(got, ref, shape) -> dict:
    """max-abs and mean-abs of got - ref and where the max sits: (b, h, row,
    d) for a full [B, H, rows, D] output, or (flat row, d) for listed rows."""
    err = np.abs(got - ref)
    i = int(np.argmax(err))
    idx = [int(x) for x in np.unravel_index(i, err.shape)]
    where = dict(zip(shape, idx))
    return {"max_abs": float(err.flat[i]), "mean_abs": float(err.mean()), "at": where,
            "got": float(got.flat[i]), "ref": float(ref.flat[i])}


def kernel_source_hash() -> str:
    """Source hash of the forward kernels."""
    return source_hash(("kb_attn.hip", "kb_contract.h"))


def backward_source_hash() -> str:
    """Source hash of the backward kernels."""
    return source_hash(("kb_bwd.hip", "kb_contract.h"))


def load_traffic(launch_flops: float):
    """HBM bytes per prefill launch from the committed rocprofv3 counter
    summary, or None when it is missing or was taken on other kernel source."""
    try:
        with open(PROFILE_TRAFFIC) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(q, k, v, target_s: float):
    """Oracle (fp64, all host threads) on a bounded sample of prefill rows."""
    import oracle

    threads = len(os.sched_getaffinity(0))
    rng = np.random.default_rng(1234)

    def sample(n):
        b = rng.integers(0, B, n)
        h = rng.integers(0, HQ, n)
        r = rng.integers(0, S, n)
        return (b * HQ + h) * S + r, r

    # batches of random rows until about target_s seconds of oracle work have
    # run, each batch sized from the rate measured so far
    all_rows, refs = [], []
    flops, dt, n = 0, 0.0, 4 * threads
    while dt < target_s:
        rows, pos = sample(n)
        t0 = time.perf_counter()
        refs.append(oracle.attention(q, k, v, rows=rows, threads=threads))
        dt += time.perf_counter() - t0
        flops += row_flops(pos)
        all_rows.append(rows)
        rate = flops / max(dt, 1e-6)
        left = target_s - dt
        n = int(min(200000, max(threads, 0.5 * left * rate / (4 * D * (S / 2)) + threads)))
    rows = np.concatenate(all_rows)
    ref = np.concatenate(refs)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows.size} random prefill rows of the same B=16 S=16384 input (fp64 oracle), "
                      f"{flops:.3e} FLOPs in {dt:.2f} s",
            "rows": int(rows.size), "seconds": round(dt, 3), "rows_per_s": round(rows.size / dt, 1)}, rows, ref


def prefill_workloads(kb, torch, dev, stream, reps: int = 5):
    """The pages' prefill set (B=1, S = 1K, 4K, 8K and 16K, N(0,1), seed 17;
    S=1024 is the worked example's case) and the two other prefill workloads
    (B=4 S=4096, seed 2; B=8 S=8192, seed 3, also as its 8 partitioned calls
    of 1024 rows against the cache), each timed with HIP events on the launch
    stream in two ways: calls back to back (the mean per call over enough
    calls to fill about 150 ms between one pair of events: the rate a stream
    of calls sees, with the chip at its working clock; `ms` and the rates
    below it) and each call alone (median of `reps` after one untimed call,
    a synchronisation between calls: `ms_alone`, which also pays the clock's
    climb back after the idle gap).  Returns the rows for the JSON line and
    the host copies the CPU leg checks."""
    import kb_gen

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, window_ms: float = 150.0, max_calls: int = 1000):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        alone = float(np.median(ts))
        n = int(min(max_calls, max(3, window_ms / max(alone, 1e-3))))
        fn()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n, alone, n

    def to_dev(x):
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)

    rows, keep = [], {}
    cases = [("pages B=1", 17, 1, 1024), ("pages B=1", 17, 1, 4096), ("pages B=1", 17, 1, 8192),
             ("pages B=1", 17, 1, 16384), ("B=4 S=4096", 2, 4, 4096), ("B=8 S=8192", 3, 8, 8192)]
    for name, seed, bs, sl in cases:
        q, k, v = kb_gen.attention_inputs(seed, bs, sl)
        qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
        out = torch.empty_like(qd)
        ms, ms_alone, calls = timed(lambda: kb.prefill(qd, kd, vd, out=out))
        fl = 2 * bs * HQ * D * sl * (sl + 1)
        rec = {"workload": name, "batch": bs, "seq_len": sl, "seed": seed, "ms": round(ms, 4),
               "tflops": round(fl / ms / 1e9, 2), "frac_of_peak": round(fl / (ms * 1e-3) / PEAK_BF16, 4),
               "back_to_back_calls": calls, "ms_alone": round(ms_alone, 4),
               "frac_of_peak_alone": round(fl / (ms_alone * 1e-3) / PEAK_BF16, 4),
               "workgroups": bs * HKV * ((sl + 63) // 64)}
        if bs == 8:
            chunks = [qd[:, :, c * PART:(c + 1) * PART].contiguous() for c in range(sl // PART)]
            outs = [torch.empty_like(c) for c in chunks]

            def parts():
                for c in range(sl // PART):
                    kb.partitioned(chunks[c], kd, vd, kv_len=(c + 1) * PART, out=outs[c])
            pms, pms_alone, pcalls = timed(parts)
            mism = sum(int((outs[c].view(torch.int16) != out.view(torch.int16)[:, :, c * PART:(c + 1) * PART])
                           .sum()) for c in range(sl // PART))
            rec["partitioned"] = {"calls": sl // PART, "rows_per_call": PART, "ms": round(pms, 4),
                                  "tflops": round(fl / pms / 1e9, 2),
                                  "frac_of_peak": round(fl / (pms * 1e-3) / PEAK_BF16, 4),
                                  "back_to_back_sequences": pcalls, "ms_alone": round(pms_alone, 4),
                                  "frac_of_peak_alone": round(fl / (pms_alone * 1e-3) / PEAK_BF16, 4),
                                  "bitwise_mismatch_vs_prefill": mism}
            del chunks, outs
        if (bs, sl) in ((1, 1024), (4, 4096)):
            keep[(bs, sl)] = (q, k, v, out.view(torch.int16).cpu().numpy())
        rows.append(rec)
        del qd, kd, vd, out
    return rows, keep


def cpu_leg(q, k, v, out_pre, keep, sweep_cells, target_s: float, dev, torch):
    """The oracle as it stands, on the host cores of this run: (1) the worked
    example's case B=1 S=1024 in full on all threads and on one thread, (2)
    B=4 S=4096 in full, (3) every decode-sweep cell, (4) randomly sampled rows
    of the bench's B=16 S=16384 input for about target_s seconds.  Each is also
    the parity check of the GPU output it covers."""
    import kb_gen
    import oracle

    threads = len(os.sched_getaffinity(0))
    full = {}
    for (bs, sl), (qq, kk, vv, bits) in sorted(keep.items()):
        t0 = time.perf_counter()
        ref = oracle.attention(qq, kk, vv, threads=threads)
        dt = time.perf_counter() - t0
        got = kb_gen.bf16_bits_to_f32(bits.view(np.uint16)).astype(np.float64)
        nrows = bs * HQ * sl
        rec = {"seconds": round(dt, 3), "threads": threads, "rows": nrows, "rows_per_s": round(nrows / dt, 1),
               "tflops": round(2 * bs * HQ * D * sl * (sl + 1) / dt / 1e12, 5),
               "check": worst_error(got, ref, ("b", "h", "row", "d"))}
        if (bs, sl) == (1, 1024):
            t0 = time.perf_counter()
            oracle.attention(qq, kk, vv, threads=1)
            rec["single_thread_seconds"] = round(time.perf_counter() - t0, 3)
        full[f"B={bs} S={sl}"] = rec
    # decode sweep cells: one query row per head at position kv_len - 1
    t_dec, n_dec, worst = 0.0, 0, None
    for bs, ctx, got_bits in sweep_cells:
        qs = np.ascontiguousarray(q[:bs, :, ctx - 1:ctx])
        t0 = time.perf_counter()
        ref = oracle.attention(qs, np.ascontiguousarray(k[:bs]), np.ascontiguousarray(v[:bs]), kv_len=ctx,
                               threads=threads)
        t_dec += time.perf_counter() - t0
        n_dec += bs * HQ
        w = worst_error(kb_gen.bf16_bits_to_f32(got_bits.view(np.uint16)).astype(np.float64), ref,
                        ("b", "h", "row", "d"))
        w["cell"] = {"batch": bs, "kv_len": ctx}
        if worst is None or w["max_abs"] > worst["max_abs"]:
            worst = w
    full["decode sweep (16 cells)"] = {"seconds": round(t_dec, 3), "threads": threads, "rows": n_dec,
                                       "rows_per_s": round(n_dec / max(t_dec, 1e-9), 1), "check": worst}
    base, rows, ref = cpu_baseline(q, k, v, target_s)
    flat = out_pre.view(-1, D)
    got = flat[torch.from_numpy(rows).to(dev)].float().cpu().numpy().astype(np.float64)
    check = worst_error(got, ref, ("flat_row", "d"))
    fr = check["at"]["flat_row"]
    check["at"] = {"b": int(rows[fr] // (HQ * S)), "h": int(rows[fr] // S % HQ), "row": int(rows[fr] % S),
                   "d": check["at"]["d"]}
    check.update({"rows": int(rows.size), "tol_max_abs": 2e-2, "tol_mean_abs": 2e-3})
    base["full_oracle"] = full
    return base, check


def backward_section(kb, torch, dev, qd, kd, vd, out_pre, reps: int, check: bool):
    """The backward of the full causal prefill on the bench input (B=16,
    S=16384) with a seeded N(0, 1) upstream gradient: prefill_lse, then the
    backward timed with HIP events on its stream.  FLOPs are the five
    products' algorithmic count (10*D per visible pair; the dQ kernel's
    recomputation of S and dP is not counted).  With check: the lse forward's
    output must equal the plain prefill's bit for bit, and a second backward
    must reproduce the gradients bit for bit."""
    import kb_gen

    stream = torch.cuda.current_stream(dev)
    do = torch.from_numpy(kb_gen.normal_bf16(SEED, 4, (B, HQ, S, D)).view(np.int16)).to(dev).view(torch.bfloat16)
    o, lse = kb.prefill_lse(qd, kd, vd)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    ws = torch.empty(kb.backward_workspace_bytes(B, S, HQ, D), dtype=torch.uint8, device=dev)
    kb.backward(qd, kd, vd, o, do, lse, dq=dq, dk=dk, dv=dv, workspace=ws)
    torch.cuda.synchronize()
    times = []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(reps):
        e0.record(stream)
        kb.backward(qd, kd, vd, o, do, lse, dq=dq, dk=dk, dv=dv, workspace=ws)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = float(np.median(times))
    flops = backward_flops(B, HQ, S, D)
    res = {"batch": B, "seq_len": S, "ms": round(ms, 3), "tflops": round(flops / ms / 1e9, 2),
           "frac_of_peak": round(flops / (ms * 1e-3) / PEAK_BF16, 4), "flops": flops,
           "flops_count": "5 products x 2*D per visible (query, key) pair"}
    if check:
        first = [x.view(torch.int16).clone() for x in (dq, dk, dv)]
        kb.backward(qd, kd, vd, o, do, lse, dq=dq, dk=dk, dv=dv, workspace=ws)
        torch.cuda.synchronize()
        res["bitwise_mismatch"] = {
            "lse_forward_vs_prefill": int((o.view(torch.int16) != out_pre.view(torch.int16)).sum()),
            "rerun": sum(int((a != b.view(torch.int16)).sum()) for a, b in zip(first, (dq, dk, dv)))}
        del first
    del do, o, lse, dq, dk, dv, ws
    return res


DATA_STUDY_CASES = ("bench inputs", "V = 0", "Q = 0", "Q = K = V = 0")


def data_study(kb, torch, qd, kd, vd, reps: int) -> list:
    """The prefill on the bench shape, `reps` launches on each case of
    DATA_STUDY_CASES in that order; median launch time of each (HIP events)."""
    z = torch.zeros_like
    cases = {"bench inputs": (qd, kd, vd), "V = 0": (qd, kd, z(vd)), "Q = 0": (z(qd), kd, vd),
             "Q = K = V = 0": (z(qd), z(kd), z(vd))}
    out = torch.empty_like(qd)
    stream = torch.cuda.current_stream()
    res = []
    for name in DATA_STUDY_CASES:
        qx, kx, vx = cases[name]
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            kb.prefill(qx, kx, vx, out=out)
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        res.append({"case": name, "ms_median": float(np.median(ts)), "launches": reps})
    return res


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the decode sweep and the ragged batch (profiling runs: one kernel configuration each)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (calibrates HBM byte counters)")
    ap.add_argument("--backward-only", type=int, default=0, metavar="N",
                    help="only run prefill_lse once and the backward N times (profiling runs of the backward)")
    ap.add_argument("--data-study", type=int, default=0, metavar="N",
                    help="only run the prefill N times on each of four inputs of the bench shape (the bench's, "
                         "V = 0, Q = 0, Q = K = V = 0): same instructions and traffic, different operand switching")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this operator is built and measured per GPU "
              "(no sharding, no collectives); use --gpus 1", file=sys.stderr)
        return 2

    import torch

    import bitwise_aligned_causal_amd as kb
    import kb_gen

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": 1 << 30, "copies": 3}))
        return 0
    kb.lib()
    q, k, v = kb_gen.attention_inputs(SEED, B, S, HQ, HKV, D, outliers=4)

    def to_dev(x):
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)

    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    if args.backward_only:
        bwd = backward_section(kb, torch, dev, qd, kd, vd, None, reps=args.backward_only, check=False)
        print(json.dumps({"backward": bwd}))
        return 0
    if args.data_study:
        print(json.dumps({"data_study": data_study(kb, torch, qd, kd, vd, args.data_study)}))
        return 0
    q_chunks = [qd[:, :, c * PART:(c + 1) * PART].contiguous() for c in range(S // PART)]
    q_dec = qd[:, :, DEC_LEN - 1:DEC_LEN].contiguous()
    out_pre = torch.empty_like(qd)
    out_part = [torch.empty_like(c) for c in q_chunks]
    out_dec = torch.empty_like(q_dec)
    ws = torch.empty(kb.decode_workspace_bytes(B, DEC_LEN, HQ, D), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    f_pre = prefill_flops(B, 0, S)
    f_part = sum(prefill_flops(B, c * PART, PART) for c in range(S // PART))
    f_dec = 4 * D * DEC_LEN * B * HQ
    dec_bytes = 4096 * B * DEC_LEN + 16384 * B

    names = ("pre", "part", "dec")
    ev = [{n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for n in names}
          for _ in range(args.steps)]

    def step(e):
        if e:
            e["pre"][0].record(stream)
        kb.prefill(qd, kd, vd, out=out_pre)
        if e:
            e["pre"][1].record(stream)
            e["part"][0].record(stream)
        for c in range(S // PART):
            kb.partitioned(q_chunks[c], kd, vd, kv_len=(c + 1) * PART, out=out_part[c])
        if e:
            e["part"][1].record(stream)
            e["dec"][0].record(stream)
        kb.decode(q_dec, kd, vd, kv_len=DEC_LEN, out=out_dec, workspace=ws)
        if e:
            e["dec"][1].record(stream)

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    # timed region: exactly K steps between two synchronisations
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    times = {n: [e[n][0].elapsed_time(e[n][1]) for e in ev] for n in names}

    # bitwise identity across entry points
    pre_bits = out_pre.view(torch.int16)
    mism = sum(int((out_part[c].view(torch.int16) != pre_bits[:, :, c * PART:(c + 1) * PART]).sum())
               for c in range(S // PART))
    mism_dec = int((out_dec.view(torch.int16)[:, :, 0] != pre_bits[:, :, DEC_LEN - 1]).sum())

    # cold decode: evict the 256 MB last-level cache by reading 512 MiB between
    # reps (a read leaves no dirty lines whose write-back would be charged to
    # the decode)
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    cold = []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(20):
        flush.sum()
        e0.record(stream)
        kb.decode(q_dec, kd, vd, kv_len=DEC_LEN, out=out_dec, workspace=ws)
        e1.record(stream)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))

    sweep, varlen, paged, decode_multi, pre_sweep = None, None, None, None, None
    sweep_cells, keep = [], {}
    if not args.no_extras:
        # decode sweep: batch 1/4/8/16 x context 128/1K/4K/8K over the resident
        # cache (capacity 16384, first kv_len keys), cold, one query token per head
        sweep, sweep_cells = [], []
        for bs in (1, 4, 8, 16):
            for ctx in (128, 1024, 4096, 8192):
                qs = qd[:bs, :, ctx - 1:ctx].contiguous()
                os_ = torch.empty_like(qs)
                wss = torch.empty(max(1, kb.decode_workspace_bytes(bs, ctx, HQ, D)), dtype=torch.uint8, device=dev)
                kv_b, vv_b = kd[:bs], vd[:bs]
                reps = []
                for i in range(11):
                    flush.sum()
                    e0.record(stream)
                    kb.decode(qs, kv_b, vv_b, kv_len=ctx, out=os_, workspace=wss)
                    e1.record(stream)
                    torch.cuda.synchronize()
                    reps.append(e0.elapsed_time(e1))
                us = float(np.median(reps[1:])) * 1e3
                nbytes = 4096 * bs * ctx + 16384 * bs
                sweep.append({"batch": bs, "kv_len": ctx, "us_cold": round(us, 2), "gbs": round(nbytes / us / 1e3, 1),
                              "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / PEAK_HBM, 4)})
                sweep_cells.append((bs, ctx, os_.view(torch.int16).cpu().numpy()))

        # ragged batch: 16 sequences of mixed lengths, sequence i = the first L_i
        # rows of batch i, packed head-major; its rows must equal the dense
        # prefill's rows bit for bit (row r of batch i sees the same keys 0..r)
        lens = [16384, 12000, 9000, 7000, 5000, 4096, 3000, 2500, 2049, 1500, 1025, 900, 600, 300, 130, 64]
        cu = [0]
        for L in lens:
            cu.append(cu[-1] + L)
        qv = torch.cat([qd[i, :, :L] for i, L in enumerate(lens)], dim=1).contiguous()
        kv_ = torch.cat([kd[i, :, :L] for i, L in enumerate(lens)], dim=1).contiguous()
        vv_ = torch.cat([vd[i, :, :L] for i, L in enumerate(lens)], dim=1).contiguous()
        ov = torch.empty_like(qv)
        qtok = torch.stack([qv[:, cu[i + 1] - 1] for i in range(len(lens))], dim=1).contiguous()
        otok = torch.empty_like(qtok)
        wsv = torch.empty(max(1, kb.decode_varlen_workspace_bytes(lens)), dtype=torch.uint8, device=dev)
        kb.prefill_varlen(qv, kv_, vv_, cu, out=ov)
        torch.cuda.synchronize()
        vt = []
        for _ in range(5):
            e0.record(stream)
            kb.prefill_varlen(qv, kv_, vv_, cu, out=ov)
            e1.record(stream)
            torch.cuda.synchronize()
            vt.append(e0.elapsed_time(e1))
        vd_t = []
        for _ in range(11):
            flush.sum()
            e0.record(stream)
            kb.decode_varlen(qtok, kv_, vv_, cu, lens, out=otok, workspace=wsv)
            e1.record(stream)
            torch.cuda.synchronize()
            vd_t.append(e0.elapsed_time(e1))
        ov_bits = ov.view(torch.int16)
        v_mism = sum(int((ov_bits[:, cu[i]:cu[i + 1]] != pre_bits[i, :, :L]).sum()) for i, L in enumerate(lens))
        v_mism_dec = sum(int((otok.view(torch.int16)[:, i] != ov_bits[:, cu[i + 1] - 1]).sum())
                         for i in range(len(lens)))
        v_flops = sum(2 * HQ * D * L * (L + 1) for L in lens)
        v_ms = float(np.median(vt))
        v_dec_us = float(np.median(vd_t[1:])) * 1e3
        v_bytes = sum(4096 * L + 16384 for L in lens)
        varlen = {"sequences": len(lens), "lengths": lens, "prefill_ms": round(v_ms, 3),
                  "prefill_tflops": round(v_flops / v_ms / 1e9, 2),
                  "prefill_frac_of_peak": round(v_flops / (v_ms * 1e-3) / PEAK_BF16, 4),
                  "decode_us_cold": round(v_dec_us, 2), "decode_gbs": round(v_bytes / v_dec_us / 1e3, 1),
                  "bitwise_mismatch": {"prefill_vs_dense_prefill": v_mism, "decode_vs_prefill": v_mism_dec}}
        del qv, kv_, vv_, ov

        # paged decode: the same B=16, context-8192 decode over 64-key pages in
        # shuffled pool order; must give the dense decode's bits
        ps = 64
        npg = DEC_LEN // ps

        def to_pool(x):
            logical = x[:, :, :DEC_LEN].reshape(B, HKV, npg, ps, D).permute(0, 2, 1, 3, 4).reshape(B * npg, HKV, ps, D)
            pool = torch.empty_like(logical)
            pool[perm] = logical
            return pool

        perm = torch.randperm(B * npg, generator=torch.Generator().manual_seed(7)).to(dev)
        kpool, vpool = to_pool(kd), to_pool(vd)
        table = perm.view(B, npg).to(torch.int32).contiguous()
        qpg = q_dec.view(B, HQ, D)
        opg = torch.empty_like(qpg)
        wsp = torch.empty(max(1, kb.decode_varlen_workspace_bytes([DEC_LEN] * B)), dtype=torch.uint8, device=dev)
        pt = []
        for _ in range(11):
            flush.sum()
            e0.record(stream)
            kb.decode_paged(qpg, kpool, vpool, table, [DEC_LEN] * B, out=opg, workspace=wsp)
            e1.record(stream)
            torch.cuda.synchronize()
            pt.append(e0.elapsed_time(e1))
        p_us = float(np.median(pt[1:])) * 1e3
        paged = {"batch": B, "kv_len": DEC_LEN, "page_size": ps, "us_cold": round(p_us, 2),
                 "gbs": round(dec_bytes / p_us / 1e3, 1),
                 "frac_of_hbm_peak": round(dec_bytes / (p_us * 1e-6) / PEAK_HBM, 4),
                 "bitwise_mismatch_vs_dense_decode": int((opg.view(torch.int16)
                                                          != out_dec.view(B, HQ, D).view(torch.int16)).sum())}
        del kpool, vpool

        # multi-row decode: the last 4 tokens of every sequence at context 8192
        # (B=16) in one call, against the same rows of the prefill output
        nr = 4
        qm = qd[:, :, DEC_LEN - nr:DEC_LEN].contiguous()
        om = torch.empty_like(qm)
        wsm = torch.empty(max(1, kb.decode_multi_workspace_bytes(B, nr, DEC_LEN, HQ, D)), dtype=torch.uint8,
                          device=dev)
        mt = []
        for _ in range(11):
            flush.sum()
            e0.record(stream)
            kb.decode_multi(qm, kd, vd, kv_len=DEC_LEN, out=om, workspace=wsm)
            e1.record(stream)
            torch.cuda.synchronize()
            mt.append(e0.elapsed_time(e1))
        m_us = float(np.median(mt[1:])) * 1e3
        m_bytes = 4096 * B * DEC_LEN + 16384 * B * nr
        decode_multi = {"batch": B, "kv_len": DEC_LEN, "rows": nr, "us_cold": round(m_us, 2),
                        "gbs": round(m_bytes / m_us / 1e3, 1),
                        "frac_of_hbm_peak": round(m_bytes / (m_us * 1e-6) / PEAK_HBM, 4),
                        "bitwise_mismatch_vs_prefill": int((om.view(torch.int16)
                                                            != pre_bits[:, :, DEC_LEN - nr:DEC_LEN]).sum())}
        del qm, om, wsm
    del flush
    backward = None if args.no_extras else backward_section(kb, torch, dev, qd, kd, vd, out_pre, reps=3, check=True)
    if not args.no_extras:
        pre_sweep, keep = prefill_workloads(kb, torch, dev, stream)
    # clock levels while the GPU is busy with prefill launches (about 1.2 s
    # of queued work), then idle
    clocks_busy = None
    if not args.no_extras:
        for _ in range(40):
            kb.prefill(qd, kd, vd, out=out_pre)
        clocks_busy = gpu_clocks()
        torch.cuda.synchronize()

    pre_ms = float(np.mean(times["pre"]))
    part_ms = float(np.mean(times["part"]))
    dec_ms = float(np.mean(times["dec"]))
    cold_ms = float(np.median(cold))
    achieved = f_pre / (pre_ms * 1e-3)
    traffic = load_traffic(f_pre)
    result = {
        "metric": METRIC,
        "value": round((f_pre + f_part + f_dec) / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal GQA attention forward: prefill B=16 S=16384 + partitioned 16x1024 "
                               "+ decode at context 8192",
                   "batch": B, "seq_len": S, "n_q_heads": HQ, "n_kv_heads": HKV, "head_dim": D,
                   "partition_rows": PART, "decode_context": DEC_LEN, "outlier_channels": 4, "seed": SEED},
        "roofline": {"bound": "mfma", "achieved": round(achieved / 1e12, 2), "peak": PEAK_BF16 / 1e12,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16, 4),
                     "traffic": traffic, "kernel": "prefill_kernel<false>", "launch_ms": round(pre_ms, 3),
                     "flops_per_launch": f_pre,
                     "timing": "HIP events on the launch stream around each of the timed steps' prefill launches, "
                               "mean"},
        "prefill": {"ms": round(pre_ms, 3), "tflops": round(f_pre / pre_ms / 1e9, 2),
                    "frac_of_peak": round(f_pre / (pre_ms * 1e-3) / PEAK_BF16, 4)},
        "partitioned": {"calls": S // PART, "ms": round(part_ms, 3), "tflops": round(f_part / part_ms / 1e9, 2),
                        "frac_of_peak": round(f_part / (part_ms * 1e-3) / PEAK_BF16, 4)},
        "decode": {"kv_len": DEC_LEN, "bytes": dec_bytes, "ms_in_step": round(dec_ms, 4),
                   "gbs_in_step": round(dec_bytes / dec_ms / 1e6, 1),
                   "ms_cold": round(cold_ms, 4), "gbs_cold": round(dec_bytes / cold_ms / 1e6, 1),
                   "frac_of_peak_cold": round(dec_bytes / (cold_ms * 1e-3) / PEAK_HBM, 4)},
        "decode_sweep": sweep,
        "prefill_sweep": pre_sweep,
        "varlen": varlen,
        "paged_decode": paged,
        "decode_multi": decode_multi,
        "backward": backward,
        "bitwise_mismatch": {"partitioned_vs_prefill": mism, "decode_vs_prefill": mism_dec},
        "contract": kb.contract(),
        "kernel_source_hash": kernel_source_hash(),
        "inputs_sha256": {name: hashlib.sha256(np.ascontiguousarray(x).data).hexdigest()[:16]
                          for name, x in (("q", q), ("k", k), ("v", v))},
        "env": {**device_env(torch, dev), "clocks_idle": None if args.no_extras else gpu_clocks(),
                "clocks_busy": clocks_busy},
        # profiled runs (--no-extras) start no helper programs: the profiler's
        # preloaded library would follow them
        "git": git_head(spawn=not args.no_extras),
    }
    if not args.no_cpu_baseline:
        base, check = cpu_leg(q, k, v, out_pre, keep, sweep_cells, args.cpu_seconds, dev, torch)
        result["cpu_baseline"] = base
        result["oracle_check"] = check
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
