"""The quantiser kernel's shared-divisor quotient (CPU only, no GPU).

The kernel replaces the 16 IEEE divisions of a block, x / s, by one reciprocal
and Markstein's FMA correction (csrc/quantize.hip, k_quantize).  The codes must
stay those of the true division, bit for bit; tests/quotient_check.c models the
sequence in C with fmaf and compares codes (and the quotient bits where they
decide a code) on random and adversarial pairs.  The GPU side of the same claim
is test_gpu_quantize.py (bit-exact against the oracle, which divides)."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_shared_divisor_quotient_gives_the_division_codes():
    with tempfile.TemporaryDirectory(prefix="quotient_") as tmp:
        exe = os.path.join(tmp, "quotient_check")
        subprocess.run(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-o", exe,
                        os.path.join(HERE, "quotient_check.c"), "-lm"], check=True)
        res = subprocess.run([exe, "20000000"], capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "0 code mismatches, 0 bit mismatches" in res.stdout, res.stdout
