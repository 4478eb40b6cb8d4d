"""Host sanitizers on the CPU (no GPU is touched).

1. The C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
   (gcc), running every oracle pin test: an out-of-bounds access, a use after
   free or an undefined operation anywhere in the oracle's codecs, quantiser or
   GEMM aborts the child process.
2. The HIP library's host code built with AddressSanitizer (clang, host pass
   only: the GPU code objects are built as usual), running the C-ABI tests,
   which drive every entry point's argument validation with bad sizes,
   pointers and overlaps before anything reaches the GPU."""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_PINS = ["tests/test_oracle_codecs.py", "tests/test_oracle_quantize.py",
               "tests/test_oracle_gemm.py", "tests/test_oracle_swiglu.py",
               "tests/test_oracle_combine.py"]


def _gcc_runtime(name):
    try:
        p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                           check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _child(tests, env_extra):
    env = dict(os.environ, OMP_NUM_THREADS="2", **env_extra)
    # -s: no output capture in the child, so a sanitizer report reaches this log
    # (the runtime aborts the process, which would lose a captured report).
    res = subprocess.run([sys.executable, "-m", "pytest", *tests, "-x", "-q", "-s", "-m", "not gpu",
                          "-p", "no:cacheprovider"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    return res.returncode, res.stdout + res.stderr


def test_oracle_pins_under_asan_and_ubsan():
    asan = _gcc_runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    from oracle import oracle as orc
    with tempfile.TemporaryDirectory(prefix="oracle_asan_") as tmp:
        out = os.path.join(tmp, "liboracle_fp4_asan.so")
        cmd = ["gcc", "-O1", "-g", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=undefined", "-Wall", "-shared", "-fPIC",
               os.path.join(ROOT, "oracle", "fp4_oracle.c"), "-o", out, "-lm"]
        subprocess.run(cmd, check=True)
        assert orc.LIB_PATH != out
        rc, log = _child(ORACLE_PINS, {"FP4_ORACLE_LIB": out, "LD_PRELOAD": asan,
                                       "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                                       "UBSAN_OPTIONS": "print_stacktrace=1"})
    assert "AddressSanitizer" not in log and "runtime error" not in log, log[-4000:]
    assert rc == 0, log[-4000:]


def _clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_library_host_validation_under_asan():
    rt = _clang_asan_runtime()
    if rt is None:
        pytest.skip("the ROCm clang AddressSanitizer runtime is not installed")
    from block_scaled_fp4_05_amd import build as hipbuild
    with tempfile.TemporaryDirectory(prefix="moe_fp4_asan_") as tmp:
        out = os.path.join(tmp, "libmoe_fp4_asan.so")
        # Host pass only: each -fsanitize goes to the host compilation.
        hipbuild.build(out=out, extra_flags=["-g", "-Xarch_host", "-fsanitize=address",
                                             "-Xarch_host", "-fno-omit-frame-pointer"])
        rc, log = _child(["tests/test_abi.py"], {"MOE_FP4_LIB": out, "LD_PRELOAD": rt,
                                                 "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1"})
    assert "AddressSanitizer" not in log, log[-4000:]
    assert rc == 0, log[-4000:]
