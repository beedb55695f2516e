"""Turn rocprofv3 output of bench.py into the short summaries kept in profiles/.

The GPU runs (each command runs committed files only):
  rocprofv3 --kernel-trace --stats -d <stats> -o run --output-format csv -- python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline --no-extras
  rocprofv3 --pmc FETCH_SIZE -d <fetch> -o run --output-format csv -- python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline --no-extras
  rocprofv3 --pmc WRITE_SIZE -d <write> -o run --output-format csv -- python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline --no-extras
  rocprofv3 --pmc FETCH_SIZE -d <copy_fetch> -o run --output-format csv -- python3 bench.py --copy-probe
  rocprofv3 --pmc WRITE_SIZE -d <copy_write> -o run --output-format csv -- python3 bench.py --copy-probe
  rocprofv3 --pmc <8 SQ counters> -d <sqN> -o run --output-format csv -- python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline --no-extras
      (three passes, SQ_PASSES below; the third reads the GPU's active cycles, so that
      cycles / dispatch time gives the clock the kernel ran at)
  and for the backward kernels, the same --kernel-trace --stats, FETCH_SIZE and
  WRITE_SIZE runs of `python3 bench.py --backward-only 3`; and, for the
  prefill's clock against its input data,
  rocprofv3 --pmc GRBM_GUI_ACTIVE GRBM_COUNT -d <data> -o run --output-format csv -- python3 bench.py --data-study 7
Then, on any host:
  python bench_profile.py --stats <stats> --fetch <fetch> --write <write> \
      --copy-fetch <copy_fetch> --copy-write <copy_write> [--sq <sq1> <sq2>] \
      [--bwd-stats <s> --bwd-fetch <f> --bwd-write <w>] --out profiles

FETCH_SIZE / WRITE_SIZE are in KiB per dispatch.  Each is scaled by the
factor that makes the plain 1 GiB copy read and write exactly 1 GiB.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import statistics

import bench

COPY_BYTES = 1 << 30
SQ_PASSES = (
    "SQ_WAVE_CYCLES SQ_BUSY_CU_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS "
    "SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_LDS",
    "SQ_WAIT_INST_LDS SQ_WAIT_ANY SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_ANY SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_SALU "
    "SQ_LDS_ADDR_CONFLICT SQ_INSTS_VALU_MFMA_MOPS_BF16",
    "GRBM_GUI_ACTIVE GRBM_COUNT",
)
STATS_ARGS = "--steps 5 --warmup 2 --no-cpu-baseline --no-extras"
STATS_WARMUP_STEPS = 2
KERNELS = {
    "prefill_kernel<false>": ("prefill_kernel_b16_s16384", "full causal prefill B=16 S=16384 (one launch per step)"),
    "prefill_persistent_kernel<true>": ("prefill_kernel_partitioned_b16_16x1024",
                                        "partitioned forward, 16 launches of 1024 rows against the S=16384 cache "
                                        "(2048 blocks per launch, 8 per CU: the persistent kernel)"),
    "decode_kernel": ("decode_kernel_b16_l8192", "decode split-KV at context 8192, B=16 (8 chunks)"),
    "combine_kernel": ("combine_kernel_b16_l8192", "decode combine of 8 chunks, B=16"),
}


# the backward of the bench's prefill (B=16, S=16384), profiled with
# `bench.py --backward-only 3` (one prefill_lse launch, four backward calls)
BWD_KERNELS = {
    "bwd_dkdv_kernel": ("bwd_dkdv_kernel_b16_s16384", "backward dK, dV of the causal prefill B=16 S=16384"),
    "bwd_dq_kernel": ("bwd_dq_kernel_b16_s16384", "backward dQ of the causal prefill B=16 S=16384"),
    "bwd_prep_kernel": ("bwd_prep_kernel_b16_s16384", "backward D_i = <dO_i, O_i> and lse2 per row, B=16 S=16384"),
}
BWD_ARGS = "--backward-only 3"


def bwd_flops() -> dict:
    """Products each backward kernel executes, 2*D FLOPs per visible pair each:
    dK/dV kernel S, dP, dV, dK (4 of the algorithm's 5); dQ kernel dQ plus its
    recomputation of S and dP (3, of which 1 is new)."""
    pairs = bench.S * (bench.S + 1) // 2 * bench.B * bench.HQ
    return {"bwd_dkdv_kernel": 4 * 2 * bench.D * pairs, "bwd_dq_kernel": 3 * 2 * bench.D * pairs}


def find_csv(d: str, suffix: str) -> str:
    hits = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[0]


def short(name: str, kernels=None):
    for k in (kernels or KERNELS):
        if k in name:
            return k
    return None


def per_dispatch(d: str):
    out = {}
    for r in csv.DictReader(open(find_csv(d, "counter_collection.csv"))):
        out.setdefault(r["Kernel_Name"], []).append(
            (int(r["Dispatch_Id"]), int(r["Grid_Size"]), float(r["Counter_Value"]),
             int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    return out


def trace_durations(d: str, kernels) -> dict:
    """{kernel: [duration ns in dispatch order]} from a --kernel-trace run."""
    rows = []
    for r in csv.DictReader(open(find_csv(d, "kernel_trace.csv"))):
        k = short(r["Kernel_Name"], kernels)
        if k:
            rows.append((int(r["Dispatch_Id"]), k, int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    out = {}
    for _, k, dur in sorted(rows):
        out.setdefault(k, []).append(dur)
    return out


def steady_average(durs, warmup_steps: int, steps: int):
    """Mean duration over the timed steps' dispatches: the first warmup_steps
    steps' dispatches (untimed warm-up, first touches of the inputs) dropped."""
    per_step = max(1, len(durs) // (warmup_steps + steps))
    kept = durs[warmup_steps * per_step:] or durs
    return statistics.mean(kept), len(kept)


def copy_factor(d: str) -> float:
    vals = [v for name, rows in per_dispatch(d).items() if "copyBuffer" in name for (_, _, v, _) in rows]
    return COPY_BYTES / 1024.0 / statistics.mean(vals)


def prefill_wave_tiles() -> int:
    """64-key tiles visited per wave, summed over the full-prefill launch:
    a workgroup covers 4 heads x 64 positions with 8 waves, and position
    block pb visits pb + 1 tiles."""
    blocks = bench.S // 64
    return bench.B * (bench.HQ // 4) * (blocks * (blocks + 1) // 2) * 8


def sq_summary(dirs, out: str, src_hash: str, kernel: str = "prefill_kernel<false>", kernels=None,
               fname: str = "prefill_kernel_b16_s16384", title: str = f"full causal prefill B={bench.B} S={bench.S}",
               run_args: str = "--steps 1 --warmup 0 --no-cpu-baseline --no-extras",
               unit: tuple[str, int] | None = None) -> None:
    """SQ / GRBM counters of one kernel, mean over its dispatches in each pass,
    per dispatch, per MFMA instruction and (if given) per work unit."""
    kernels = kernels or KERNELS
    vals, durs = {}, []
    for d in dirs:
        for name, rows in per_counter(d, kernel, kernels).items():
            vals[name] = statistics.mean(rows)
    if unit is None and kernel == "prefill_kernel<false>":
        unit = ("wave per 64-key tile", prefill_wave_tiles())
    lines = [f"# {kernel} SQ and GRBM counters, {title}",
             f"kernel hash (code without comments, and compiler flags): {src_hash}", "",
             "commands (one pass each, counters split to stay within the SQ block limit):"]
    lines += [f"  rocprofv3 --pmc {p} -d <dir> -o run --output-format csv -- python3 bench.py {run_args}"
              for p in SQ_PASSES]
    head = f"  {'counter':<32} {'per dispatch':>12}   {'per MFMA':>9}"
    if unit:
        head += f"   per {unit[0]}"
    lines += ["", "mean per dispatch (SQ_WAVE_CYCLES, SQ_BUSY_CU_CYCLES, SQ_WAIT_* and SQ_ACTIVE_* are in 4-cycle "
                  "units; per MFMA = divided by SQ_INSTS_MFMA):", head]
    mfma = vals.get("SQ_INSTS_MFMA")
    for k, v in sorted(vals.items()):
        row = f"  {k:<32} {v:>12.4g}   {v / mfma if mfma else float('nan'):>9.3f}"
        if unit:
            row += f"   {v / unit[1]:>9.2f}"
        lines.append(row)
    if "SQ_VALU_MFMA_BUSY_CYCLES" in vals and "SQ_BUSY_CU_CYCLES" in vals:
        # MFMA busy cycles are summed over SIMDs, CU busy cycles over CUs (4 SIMDs each)
        util = vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (4.0 * vals["SQ_BUSY_CU_CYCLES"])
        lines += ["", f"MFMA utilisation: SQ_VALU_MFMA_BUSY_CYCLES / (4 x SQ_BUSY_CU_CYCLES) = {util:.3f} of the "
                      "SIMD cycles while the CUs are busy (at the clock the chip runs under this load)"]
    if "SQ_WAIT_ANY" in vals and "SQ_WAVE_CYCLES" in vals:
        lines += [f"waits: SQ_WAIT_ANY / SQ_WAVE_CYCLES = {vals['SQ_WAIT_ANY'] / vals['SQ_WAVE_CYCLES']:.3f} of the "
                  "wave cycles; SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES = "
                  f"{vals.get('SQ_WAIT_INST_LDS', float('nan')) / vals['SQ_WAVE_CYCLES']:.3f}"]
    if "SQ_INSTS_VALU" in vals and mfma:
        lines += [f"VALU instructions (MFMA included) per MFMA: {vals['SQ_INSTS_VALU'] / mfma:.2f}; "
                  f"transcendental per MFMA: {vals.get('SQ_INSTS_VALU_TRANS_F32', float('nan')) / mfma:.2f}"]
    if "GRBM_COUNT" in vals and "GRBM_GUI_ACTIVE" in vals:
        dur = [d for name, rows in per_dispatch(dirs[-1]).items() if short(name, kernels) == kernel
               for (_, _, _, d) in rows]
        if dur:
            sec = statistics.mean(dur) * 1e-9
            # the GRBM counters are summed over the 8 XCDs (each counts its own clock)
            lines += ["", f"clock under this load: GRBM_COUNT / (8 XCDs x dispatch time {sec * 1e3:.2f} ms) = "
                          f"{vals['GRBM_COUNT'] / (8 * sec) / 1e6:.0f} MHz; GRBM_GUI_ACTIVE / GRBM_COUNT = "
                          f"{vals['GRBM_GUI_ACTIVE'] / vals['GRBM_COUNT']:.3f}"]
    with open(os.path.join(out, f"{fname}_sq_counters.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")


def per_counter(d: str, kernel: str, kernels):
    """{counter: [value per dispatch of `kernel`]} of one pass."""
    out = {}
    for r in csv.DictReader(open(find_csv(d, "counter_collection.csv"))):
        if short(r["Kernel_Name"], kernels) == kernel:
            out.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return out


def write_summaries(kernels, stats, fetch, write, f_fetch, f_write, src_hash, out, stats_args, pmc_args, flops,
                    trace=None, warmup_steps=0, steps=0):
    for k, (fname, what) in kernels.items():
        st = stats.get(k)
        fr = [v for n, rows in fetch.items() if short(n, kernels) == k for v in rows]
        wr = [v for n, rows in write.items() if short(n, kernels) == k for v in rows]
        if not st or not fr or not wr:
            continue
        fetch_kib = statistics.mean(v for _, _, v, _ in fr)
        write_kib = statistics.mean(v for _, _, v, _ in wr)
        hbm = (fetch_kib * f_fetch + write_kib * f_write) * 1024.0
        avg_all_us = float(st["AverageNs"]) / 1e3
        avg_us, n_kept = avg_all_us, int(st["Calls"])
        if trace and trace.get(k) and warmup_steps:
            avg_ns, n_kept = steady_average(trace[k], warmup_steps, steps)
            avg_us = avg_ns / 1e3
        lines = [
            f"# {k}: {what}",
            f"kernel hash (code without comments, and compiler flags): {src_hash}",
            "",
            "commands:",
            f"  rocprofv3 --kernel-trace --stats -d <stats> -o run --output-format csv -- python3 bench.py {stats_args}",
            f"  rocprofv3 --pmc FETCH_SIZE -d <fetch> -o run --output-format csv -- python3 bench.py {pmc_args}",
            f"  rocprofv3 --pmc WRITE_SIZE -d <write> -o run --output-format csv -- python3 bench.py {pmc_args}",
            "  rocprofv3 --pmc FETCH_SIZE|WRITE_SIZE ... -- python3 bench.py --copy-probe   (1 GiB copy)",
            "  python bench_profile.py --stats <stats> --fetch <fetch> --write <write> "
            "--copy-fetch <copy_fetch> --copy-write <copy_write> "
            "[--bwd-stats <s> --bwd-fetch <f> --bwd-write <w>] --out profiles",
            "",
            "kernel-trace --stats:",
            f"  calls {st['Calls']}, average {avg_all_us:.1f} us, "
            f"min {float(st['MinNs']) / 1e3:.1f} us, max {float(st['MaxNs']) / 1e3:.1f} us, "
            f"{float(st['Percentage']):.2f} % of GPU time",
            f"  average over the {n_kept} dispatches of the timed steps (warm-up steps' dispatches dropped): "
            f"{avg_us:.1f} us",
            "",
            "counters (per dispatch, mean over the profiled dispatches):",
            f"  dispatches {len(fr)}, FETCH_SIZE {fetch_kib:.1f} KiB, WRITE_SIZE {write_kib:.1f} KiB",
            f"  copy calibration: 1 GiB copy reads {COPY_BYTES / 1024 / f_fetch:.0f} KiB, "
            f"writes {COPY_BYTES / 1024 / f_write:.0f} KiB -> factors fetch x{f_fetch:.3f}, write x{f_write:.3f}",
            f"  HBM bytes per dispatch (scaled): {hbm:.4e}",
        ]
        if k in flops:
            lines += ["", f"FLOPs per dispatch (algorithmic for the forward kernels, mean over the calls; "
                          f"products executed for the backward ones): {flops[k]:.4e} -> "
                          f"{flops[k] / (avg_us * 1e-6) / 1e12:.1f} TFLOP/s at the average duration "
                          f"({flops[k] / (avg_us * 1e-6) / bench.PEAK_BF16:.3f} of the 2.5 PFLOP/s bf16 peak)"]
        with open(os.path.join(out, fname + ".txt"), "w") as fh:
            fh.write("\n".join(lines) + "\n")
        rec = {"kernel": k, "workload": what, "kernel_source_hash": src_hash, "fetch_kib": fetch_kib,
               "write_kib": write_kib, "fetch_factor": f_fetch, "write_factor": f_write,
               "hbm_bytes_per_launch": hbm, "avg_duration_us": avg_us, "calls_in_stats_run": int(st["Calls"])}
        with open(os.path.join(out, fname + "_traffic.json"), "w") as fh:
            json.dump(rec, fh, indent=1)
        print(f"{k}: avg {avg_us:.1f} us, HBM {hbm:.3e} B/launch")


def data_study_summary(d: str, out: str, src_hash: str, reps: int = 7) -> None:
    """Per-case duration and clock of the prefill launches of bench.py
    --data-study (cases in bench.DATA_STUDY_CASES order, `reps` each)."""
    rows = {}
    for r in csv.DictReader(open(find_csv(d, "counter_collection.csv"))):
        if short(r["Kernel_Name"]) != "prefill_kernel<false>":
            continue
        x = rows.setdefault(int(r["Dispatch_Id"]), {})
        x[r["Counter_Name"]] = float(r["Counter_Value"])
        x["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    disp = [rows[k] for k in sorted(rows)]
    assert len(disp) == reps * len(bench.DATA_STUDY_CASES), len(disp)
    lines = ["# prefill_kernel<false>: clock and duration by input data, B=16 S=16384 (same instructions and traffic)",
             f"kernel hash (code without comments, and compiler flags): {src_hash}", "",
             "command:",
             f"  rocprofv3 --pmc GRBM_GUI_ACTIVE GRBM_COUNT -d <data> -o run --output-format csv -- python3 bench.py "
             f"--data-study {reps}",
             "  python bench_profile.py ... --data-study <data> --out profiles", "",
             "per case, median over its launches but the first (clock = GRBM_COUNT / (8 XCDs x duration)):"]
    for i, name in enumerate(bench.DATA_STUDY_CASES):
        sel = disp[i * reps + 1:(i + 1) * reps]
        ms = statistics.median(x["ns"] for x in sel) * 1e-6
        ghz = statistics.median(x["GRBM_COUNT"] / 8 / x["ns"] for x in sel)
        lines.append(f"  {name:16s} {ms:8.3f} ms  {ghz:5.3f} GHz  time x clock {ms * ghz:6.1f} million cycles  "
                     f"({bench.prefill_flops(bench.B, 0, bench.S) / (ms * 1e-3) / 2.5e15:.3f} of the 2.5 PFLOP/s peak)")
    os.makedirs(out, exist_ok=True)
    with open(os.path.join(out, "prefill_kernel_b16_s16384_clock_by_data.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines[-len(bench.DATA_STUDY_CASES):]))


def main():
    ap = argparse.ArgumentParser()
    for a in ("stats", "fetch", "write", "copy_fetch", "copy_write", "out"):
        ap.add_argument("--" + a.replace("_", "-"), required=True)
    ap.add_argument("--sq", nargs="*", default=[], help="directories of the SQ counter passes")
    ap.add_argument("--bwd-sq", nargs="*", default=[],
                    help="directories of the SQ counter passes over bench.py --backward-only 3")
    for a in ("bwd_stats", "bwd_fetch", "bwd_write"):
        ap.add_argument("--" + a.replace("_", "-"), default=None,
                        help="rocprofv3 output of bench.py --backward-only 3 (stats, FETCH_SIZE, WRITE_SIZE)")
    ap.add_argument("--data-study", default=None,
                    help="rocprofv3 GRBM counter run of bench.py --data-study N (the prefill's clock by input data)")
    args = ap.parse_args()
    if args.data_study:
        data_study_summary(args.data_study, args.out, bench.kernel_source_hash())
    f_fetch, f_write = copy_factor(args.copy_fetch), copy_factor(args.copy_write)
    stats = {}
    for r in csv.DictReader(open(find_csv(args.stats, "kernel_stats.csv"))):
        k = short(r["Name"])
        if k:
            stats[k] = r
    src_hash = bench.kernel_source_hash()
    os.makedirs(args.out, exist_ok=True)
    write_summaries(KERNELS, stats, per_dispatch(args.fetch), per_dispatch(args.write), f_fetch, f_write, src_hash,
                    args.out, STATS_ARGS, "--steps 1 --warmup 0 --no-cpu-baseline --no-extras",
                    {"prefill_kernel<false>": bench.prefill_flops(bench.B, 0, bench.S),
                     "prefill_persistent_kernel<true>":
                         bench.prefill_flops(bench.B, 0, bench.S) // (bench.S // bench.PART)},
                    trace_durations(args.stats, KERNELS), STATS_WARMUP_STEPS, 5)
    if args.bwd_stats:
        bstats = {}
        for r in csv.DictReader(open(find_csv(args.bwd_stats, "kernel_stats.csv"))):
            k = short(r["Name"], BWD_KERNELS)
            if k:
                bstats[k] = r
        write_summaries(BWD_KERNELS, bstats, per_dispatch(args.bwd_fetch), per_dispatch(args.bwd_write), f_fetch,
                        f_write, bench.backward_source_hash(), args.out, BWD_ARGS, BWD_ARGS, bwd_flops())
    if args.sq:
        sq_summary(args.sq, args.out, src_hash)
    for k in ("bwd_dkdv_kernel", "bwd_dq_kernel") if args.bwd_sq else ():
        fname, what = BWD_KERNELS[k]
        sq_summary(args.bwd_sq, args.out, bench.backward_source_hash(), k, BWD_KERNELS, fname, what, BWD_ARGS)


if __name__ == "__main__":
    main()
