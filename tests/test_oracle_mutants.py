"""The oracle's pins catch plausible mistakes (CPU only).

Each case compiles a copy of oracle/fp4_oracle.c with one deliberate mistake of
the kind that could slip into a hand-written reference (a tie sent the wrong
way, a threshold off by one step, a wrong exponent bias, swapped nibbles, a
transposed or dropped operand, a wrong index, a reciprocal in place of a
division, a forgotten factor) and runs the oracle's own tests against that
build, through FP4_ORACLE_LIB, in a child process.  Every mutant must make them
fail; an unmutated copy built the same way must pass.  Nothing here touches a
GPU or the HIP library."""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from oracle import oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "fp4_oracle.c")
PIN_TESTS = ["tests/test_oracle_codecs.py", "tests/test_oracle_quantize.py",
             "tests/test_oracle_gemm.py", "tests/test_oracle_swiglu.py",
             "tests/test_oracle_combine.py"]

# name -> (text in fp4_oracle.c, replacement, which occurrence (0-based)), or a
# list of such edits applied in order
MUTANTS = {
    "e2m1 subnormal step 1 instead of 0.5": ("0.5 * m : ldexp", "1.0 * m : ldexp", 0),
    "e2m1 tie at 0.25 rounds up": ("if (a <= 0.25f) c = 0;", "if (a < 0.25f) c = 0;", 0),
    "e2m1 tie at 3.5 rounds down": ("else if (a < 3.5f) c = 5;", "else if (a <= 3.5f) c = 5;", 0),
    "e2m1 sign from y < 0 (loses -0)": ("int sign = signbit(y) ? 8 : 0;", "int sign = (y < 0.0f) ? 8 : 0;", 0),
    "e2m1 saturates at 4": ("else c = 7;", "else c = 6;", 0),
    "e4m3 exponent bias 6": ("ldexp(8.0 + m, e - 10)", "ldexp(8.0 + m, e - 9)", 0),
    "e4m3 subnormal spacing 2^-8": ("ldexp((double)m, -9)", "ldexp((double)m, -8)", 0),
    "e4m3 encode ties away from zero": ("rn = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "rn = fl + 1.0;", 0),
    "e4m3 encode truncates": ("if (frac > 0.5) rn = fl + 1.0;", "if (frac > 2.0) rn = fl + 1.0;", 0),
    # The encoder clamps both before and after rounding; dropping one alone
    # changes nothing, so this mutant drops both.
    "e4m3 encode no saturation": [("if (a >= 448.0) {", "if (a > 1e300) {", 0),
                                  ("if (v > 448.0) v = 448.0;", "", 0)],
    "bf16 ties away from zero": ("rn = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "rn = fl + 1.0;", 1),
    "tensor scale amax / 2048": ("g = (amax > 0.0f) ? amax / 2688.0f : 1.0f;", "g = (amax > 0.0f) ? amax / 2048.0f : 1.0f;", 0),
    "all-zero tensor scale 0": ("g = (amax > 0.0f) ? amax / 2688.0f : 1.0f;", "g = (amax > 0.0f) ? amax / 2688.0f : 0.0f;", 0),
    "block scale without the 6": ("float rr = amax_b / six_g;", "float rr = amax_b / g;", 0),
    "reciprocal multiply for x / s": ("float y = (s == 0.0f) ? 0.0f : xb[i] / s;", "float y = (s == 0.0f) ? 0.0f : xb[i] * (1.0f / s);", 0),
    "block amax over 15 elements": ("for (int i = 0; i < 16; ++i) {\n        float a = fabsf(xb[i]);", "for (int i = 1; i < 16; ++i) {\n        float a = fabsf(xb[i]);", 0),
    "nibbles swapped in the pack": ("(codes[2 * i] | (codes[2 * i + 1] << 4))", "(codes[2 * i + 1] | (codes[2 * i] << 4))", 0),
    "gemm weight nibbles swapped": ("int cw = (wq[kk / 2] >> (4 * (kk % 2))) & 15;\n          p +=", "int cw = (wq[kk / 2] >> (4 * (1 - kk % 2))) & 15;\n          p +=", 0),
    "gemm activation scale used for weights": ("acc += k512[as[b]] * k512[ws[b]] * p;", "acc += k512[as[b]] * k512[as[b]] * p;", 0),
    "gemm scale of the wrong block": ("acc += k512[as[b]] * k512[ws[b]] * p;", "acc += k512[as[b]] * k512[ws[b ^ 1]] * p;", 0),
    "gemm weight tensor scale dropped": ("double alpha = (double)a_scale * (double)w_scale[e];", "double alpha = (double)a_scale;", 0),
    "gemm every expert reads expert 0": ("const uint8_t* wq = w_q + ((int64_t)e * n + j) * kb;\n      const uint8_t* ws = w_sf + ((int64_t)e * n + j) * nb;\n      int64_t acc", "const uint8_t* wq = w_q + ((int64_t)j) * kb;\n      const uint8_t* ws = w_sf + ((int64_t)e * n + j) * nb;\n      int64_t acc", 0),
    "gemm row index ignored": ("int64_t src = a_row_index ? a_row_index[r] : r;", "int64_t src = r;", 0),
    "gemm exponent 2^-18": ("ldexp((double)acc, -20)", "ldexp((double)acc, -18)", 0),
    "gemm row on an expert boundary goes to the earlier expert": ("if (off[e] <= r && r < off[e + 1]) return e;", "if (off[e] <= r && r <= off[e + 1]) return e;", 0),
    "f64 cross-check drops the weight tensor scale": ("R_out[t * n + j] = sum * (double)a_scale * (double)w_scale[e];", "R_out[t * n + j] = sum * (double)a_scale;", 0),
}


def _mutate(text: str, old: str, new: str, which: int) -> str:
    pos = -1
    for _ in range(which + 1):
        pos = text.find(old, pos + 1)
        assert pos >= 0, f"mutation site not found: {old!r} (occurrence {which})"
    return text[:pos] + new + text[pos + len(old):]


def _run_pins(lib: str) -> int:
    env = dict(os.environ, FP4_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    res = subprocess.run([sys.executable, "-m", "pytest", *PIN_TESTS, "-x", "-q",
                          "-p", "no:cacheprovider"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return res.returncode


def _build_and_run(tmp: str, name: str, text: str) -> tuple[str, int]:
    src = os.path.join(tmp, f"m{abs(hash(name))}.c")
    with open(src, "w") as f:
        f.write(text)
    lib = orc.build(force=True, src=src, out=src[:-2] + ".so")
    return name, _run_pins(lib)


def test_unmutated_copy_passes_the_pins():
    with open(SRC) as f:
        text = f.read()
    with tempfile.TemporaryDirectory(prefix="oracle_control_") as tmp:
        _, rc = _build_and_run(tmp, "control", text)
    assert rc == 0, "the pin tests fail on an unmutated copy of the oracle"


def test_every_mutant_fails_a_pin():
    with open(SRC) as f:
        text = f.read()
    jobs = {}
    for name, m in MUTANTS.items():
        t = text
        for edit in (m if isinstance(m, list) else [m]):
            t = _mutate(t, *edit)
        jobs[name] = t
    with tempfile.TemporaryDirectory(prefix="oracle_mutants_") as tmp:
        with ThreadPoolExecutor(max_workers=4) as pool:
            results = list(pool.map(lambda kv: _build_and_run(tmp, *kv), jobs.items()))
    # 1 = some test failed; anything else (a crash, a collection error) is not
    # the pins doing their job.
    survivors = [name for name, rc in results if rc == 0]
    odd = [(name, rc) for name, rc in results if rc not in (0, 1)]
    assert not survivors, f"mutants the pins do not catch: {survivors}"
    assert not odd, f"mutants that broke the test run instead of failing a test: {odd}"


# Mistakes in the oracle's numpy half (oracle/oracle.py): name -> (text, replacement).
PY_MUTANTS = {
    "silu with exp(+x)": ("return x / (1.0 + np.exp(-x))", "return x / (1.0 + np.exp(x))"),
    "swiglu gate and up swapped": ("return silu(R[:, :inter]) * R[:, inter:]",
                                   "return silu(R[:, inter:]) * R[:, :inter]"),
    "swiglu re-quantised with a dynamic scale": (
        "q, sf, _ = quantize(h.astype(np.float32), g=float(np.float32(g)))",
        "q, sf, _ = quantize(h.astype(np.float32))"),
    "combine ignores the routing weights": ("np.add.at(out, out_token, row_weight[:, None] * R)",
                                            "np.add.at(out, out_token, R)"),
    "combine ignores the initial rows": ("else np.array(init, dtype=np.float64, copy=True))",
                                         "else np.zeros((num_tokens, R.shape[1])))"),
    "bf16 widened with a 15-bit shift": ("astype(np.uint32) << 16", "astype(np.uint32) << 15"),
    "row error reads as zero": ("    err = np.where(norm > 0, diff / safe, np.where(diff > 0, np.inf, 0.0))\n    return err, norm\n\n\ndef combine",
                                "    err = np.zeros_like(norm)\n    return err, norm\n\n\ndef combine"),
    "static and dynamic scale swapped in the wrapper": ("1 if g is None else 0,", "0 if g is None else 1,"),
}


def _run_py_mutant(tmp: str, name: str, old: str, new: str) -> tuple[str, int]:
    import shutil
    root = os.path.join(tmp, f"r{abs(hash(name))}")
    for d in ("tests", "workloads", "oracle"):
        shutil.copytree(os.path.join(ROOT, d), os.path.join(root, d),
                        ignore=shutil.ignore_patterns("__pycache__", "*.so", "*.tmp*"))
    path = os.path.join(root, "oracle", "oracle.py")
    with open(path) as f:
        text = f.read()
    with open(path, "w") as f:
        f.write(_mutate(text, old, new, 0))
    env = dict(os.environ, FP4_ORACLE_LIB=orc.build(), OMP_NUM_THREADS="2")
    res = subprocess.run([sys.executable, "-m", "pytest", *PIN_TESTS, "-x", "-q",
                          "-p", "no:cacheprovider"],
                         cwd=root, env=env, capture_output=True, text=True, timeout=600)
    return name, res.returncode


def test_every_python_mutant_fails_a_pin():
    with tempfile.TemporaryDirectory(prefix="oracle_py_mutants_") as tmp:
        with ThreadPoolExecutor(max_workers=4) as pool:
            results = list(pool.map(lambda kv: _run_py_mutant(tmp, kv[0], *kv[1]),
                                    PY_MUTANTS.items()))
    survivors = [name for name, rc in results if rc == 0]
    odd = [(name, rc) for name, rc in results if rc not in (0, 1)]
    assert not survivors, f"mutants the pins do not catch: {survivors}"
    assert not odd, f"mutants that broke the test run instead of failing a test: {odd}"


def test_unmutated_python_copy_passes_the_pins():
    anchor = "def silu(x: np.ndarray) -> np.ndarray:"
    with tempfile.TemporaryDirectory(prefix="oracle_py_control_") as tmp:
        _, rc = _run_py_mutant(tmp, "control", anchor, anchor)
    assert rc == 0, "the pin tests fail on an unmutated copy of the oracle package"
