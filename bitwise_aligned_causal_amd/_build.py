"""Compile the HIP library libkb_attn.so in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libkb_attn.so")
# the forward (the bitwise contract's kernels) and the backward
SOURCES = ["kb_attn.hip", "kb_bwd.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # the contract places every fused multiply-add explicitly
    "-ffp-contract=off",
    # keep the compiler from emitting packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA operands and results in ordinary vector registers: without it the
    # decode kernels put 48 registers in the accumulation file and spend ~180
    # copy instructions moving them back and forth
    "-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Always recompiles libkb_attn.so; returns its path."""
    srcs = [os.path.join(CSRC, name) for name in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), *srcs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, LIB)
    write_build_info()
    return LIB


def write_build_info() -> None:
    """Record beside the library the commit it was built from, for runs on a
    copy of the tree that has no .git (the benchmark reports it)."""
    import datetime
    import json

    def git(*args):
        try:
            r = subprocess.run(["git", "-C", ROOT, *args], capture_output=True, text=True, timeout=30)
            return r.stdout.strip() if r.returncode == 0 else None
        except (OSError, subprocess.SubprocessError):
            return None

    head = git("rev-parse", "HEAD")
    dirty = git("status", "--porcelain", "--untracked-files=no")
    rec = {"git_head": head, "dirty": None if dirty is None else bool(dirty),
           "built_utc": datetime.datetime.now(datetime.timezone.utc).isoformat(timespec="seconds")}
    with open(os.path.join(PKG, "_build_info.json"), "w") as fh:
        json.dump(rec, fh)


if __name__ == "__main__":
    print(build(verbose=True))
