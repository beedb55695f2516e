"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

A copy of the tree gets sanitizer builds of the host-side C and C++: the
oracle (both precisions), the input generator, and the host part of
libkb_attn.so (argument validation, the ragged and paged table readers,
workspace sizing; the GPU code is built as usual).  The CPU tests that drive
that code run against the copy in a child process with the sanitizer runtime
preloaded; any report ends the run with an error.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-shared-libsan", "-fno-omit-frame-pointer",
       "-g"]
SUITES = ["tests/test_abi_host.py", "tests/test_varlen_host.py", "tests/test_gen.py", "tests/test_oracle_pins.py",
          "tests/test_oracle_bwd_pins.py"]


def asan_runtime():
    hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return hits[0] if hits else None


def copy_tree(dst):
    for d in ("bitwise_aligned_causal_amd", "oracle", "kb_gen", "include", "tests"):
        shutil.copytree(os.path.join(ROOT, d), os.path.join(dst, d),
                        ignore=shutil.ignore_patterns("*.so", "__pycache__", "*.tmp"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), dst)


def build_sanitized(tree):
    sys.path.insert(0, ROOT)
    from bitwise_aligned_causal_amd import _build

    host = [f for flag in SAN for f in ("-Xarch_host", flag)]
    pkg = os.path.join(tree, "bitwise_aligned_causal_amd")
    srcs = [os.path.join(pkg, "csrc", n) for n in _build.SOURCES]
    subprocess.run([_build.hipcc(), *_build.HIPCC_FLAGS, *host, "-I", os.path.join(tree, "include"), *srcs,
                    "-o", os.path.join(pkg, "libkb_attn.so")], check=True, capture_output=True)
    for prec, real in (("f64", "double"), ("f32", "float")):
        subprocess.run([CLANG, "-std=c11", "-O1", "-ffp-contract=off", "-fPIC", "-shared", "-pthread", *SAN,
                        f"-DKBO_REAL={real}", f"-DKBO_SUFFIX=_{prec}", os.path.join(tree, "oracle", "oracle.c"),
                        "-o", os.path.join(tree, "oracle", f"liboracle_{prec}.so"), "-lm"], check=True)
    subprocess.run([CLANG, "-std=c11", "-O1", "-ffp-contract=off", "-fPIC", "-shared", "-pthread", *SAN,
                    os.path.join(tree, "kb_gen", "gen.c"), "-o", os.path.join(tree, "kb_gen", "libkb_gen.so"),
                    "-lm"], check=True)


@pytest.mark.skipif(asan_runtime() is None or not os.path.exists(CLANG), reason="no clang sanitizer runtime")
def test_host_code_under_asan_and_ubsan(tmp_path):
    tree = str(tmp_path / "tree")
    copy_tree(tree)
    build_sanitized(tree)
    rc, out, reports = run_suites(tree, SUITES)
    assert not reports, "\n".join(reports)[-6000:]
    assert rc == 0 and "passed" in out, out[-4000:]


def run_suites(tree, suites):
    """Run the suites in the copy with the sanitizer runtime preloaded; the
    reports go to files (pytest's capture would swallow a report written to a
    dying process's stderr).  Returns (exit code, output, report texts)."""
    logs = os.path.join(tree, "sanitizer-logs")
    os.makedirs(logs, exist_ok=True)
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": asan_runtime(),
        # leaks and one-definition reports come from the interpreter and the
        # libraries it loads (never built with the sanitizer), not this code
        "ASAN_OPTIONS": f"detect_leaks=0:detect_odr_violation=0:halt_on_error=1:log_path={logs}/asan",
        "UBSAN_OPTIONS": f"halt_on_error=1:print_stacktrace=1:log_path={logs}/ubsan",
        "PYTHONDONTWRITEBYTECODE": "1",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        *suites], cwd=tree, env=env, capture_output=True, text=True, timeout=1500)
    reports = [open(os.path.join(logs, f)).read() for f in sorted(os.listdir(logs))]
    return r.returncode, r.stdout + r.stderr, reports


@pytest.mark.skipif(asan_runtime() is None or not os.path.exists(CLANG), reason="no clang sanitizer runtime")
def test_harness_reports_a_planted_overflow(tmp_path):
    # one past the end of a heap array, planted in the oracle copy: the run
    # must fail with a report (the harness is not silently inactive)
    tree = str(tmp_path / "tree")
    copy_tree(tree)
    src = os.path.join(tree, "oracle", "oracle.c")
    text = open(src).read()
    anchor = "real* s = (real*)malloc(sizeof(real) * (size_t)kv_len);"
    assert anchor in text
    open(src, "w").write(text.replace(anchor, anchor + "\n    if (s) s[kv_len] = 0;", 1))
    build_sanitized(tree)
    rc, out, reports = run_suites(tree, ["tests/test_oracle_pins.py"])
    assert rc != 0
    assert any("heap-buffer-overflow" in r for r in reports), (out[-2000:], reports)
