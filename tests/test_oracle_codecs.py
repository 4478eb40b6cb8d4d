"""Pins of the oracle's E2M1, E4M3 and BF16 codecs against things other than itself:
the OCP format tables (golden files), torch's float8_e4m3fn conversion, and the
exhaustive-search brute force."""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import read_golden
from oracle import bruteforce as bf
from oracle import oracle as orc


def f32(x):
    return struct.unpack("<f", struct.pack("<f", x))[0]


def next_f32(x, direction):
    return float(np.nextafter(np.float32(x), np.float32(direction)))


# ------------------------------------------------------------------- E2M1 --

def test_e2m1_decode_matches_ocp_table():
    for code_s, val_s in read_golden("e2m1_ocp_mx.txt"):
        code, want = int(code_s, 16), float(val_s)
        got = orc.e2m1_decode(code)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (code, got, want)


def test_e2m1_roundtrip_all_codes():
    for code in range(16):
        assert orc.e2m1_encode(orc.e2m1_decode(code)) == code


def _e2m1_sweep():
    vals = [0.0, -0.0, 1e-45, -1e-45, 1e-38, 7.0, -7.0, 1e30, -1e30, 6.0, 6.4, 5.6]
    for t in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0):
        for s in (1.0, -1.0):
            x = s * t
            vals.append(x)
            a, b = x, x
            for _ in range(3):
                a = next_f32(a, math.inf)
                b = next_f32(b, -math.inf)
                vals += [a, b]
    rng = np.random.default_rng(7)
    vals += [float(v) for v in rng.uniform(-8, 8, 4000).astype(np.float32)]
    return vals


def test_e2m1_encode_matches_bruteforce():
    for y in _e2m1_sweep():
        sign = 8 if math.copysign(1.0, y) < 0 else 0
        want = sign | bf.e2m1_nearest(abs(Fraction(y)))
        assert orc.e2m1_encode(y) == want, y


# ------------------------------------------------------------------- E4M3 --

def _torch_e4m3_decode(codes):
    t = torch.tensor(codes, dtype=torch.uint8).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy()


def test_e4m3_decode_matches_torch_all_codes():
    ref = _torch_e4m3_decode(list(range(256)))
    for c in range(256):
        got = orc.e4m3_decode(c)
        if math.isnan(ref[c]):
            assert math.isnan(got), c
        else:
            assert got == float(ref[c]) and math.copysign(1, got) == math.copysign(1, ref[c]), c


def test_e4m3_decode_matches_ocp_specials():
    for code_s, val_s in read_golden("e4m3_ocp_ofp8.txt"):
        code = int(code_s, 16)
        got = orc.e4m3_decode(code)
        if val_s == "nan":
            assert math.isnan(got)
        else:
            want = float(val_s)
            assert got == want and math.copysign(1, got) == math.copysign(1, want), code


def test_e4m3_roundtrip_finite_codes():
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue
        assert orc.e4m3_encode(orc.e4m3_decode(c)) == c, hex(c)


def _e4m3_sweep():
    vals = set()
    pos = [float(v) for v in _torch_e4m3_decode(list(range(0x7F)))]
    for i in range(len(pos) - 1):
        mid = f32((pos[i] + pos[i + 1]) / 2)  # exact: 5 significant bits
        vals.update([mid, next_f32(mid, math.inf), next_f32(mid, -math.inf), pos[i]])
    vals.update([448.0, 449.0, 463.9, 464.0, 465.0, 500.0, 1e6, 3.4e38, 0.0,
                 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -11, 1e-45, 2.0 ** -9, 2.0 ** -6])
    rng = np.random.default_rng(11)
    vals.update(float(v) for v in (2.0 ** rng.uniform(-14, 10, 20000)).astype(np.float32))
    out = sorted(vals)
    return out + [-v for v in out]


def test_e4m3_encode_matches_torch_rne_after_clamp():
    vals = np.array(_e4m3_sweep(), dtype=np.float32)
    clamped = torch.from_numpy(np.clip(vals, -448.0, 448.0))
    ref = clamped.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = orc.e4m3_encode_array(vals)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(vals[i]), hex(got[i]), hex(ref[i])) for i in bad[:10]]


def test_e4m3_encode_matches_bruteforce_nonneg():
    vals = [v for v in _e4m3_sweep() if v >= 0][::7]
    for v in vals:
        assert orc.e4m3_encode(v) == bf.e4m3_nearest(Fraction(v)), v


def test_e4m3_ties_go_to_even():
    # 2^-10 lies halfway between 0 (code 0x00) and 2^-9 (0x01): even -> 0x00.
    assert orc.e4m3_encode(2.0 ** -10) == 0x00
    # 3*2^-10 lies halfway between 0x01 (odd) and 0x02 (even).
    assert orc.e4m3_encode(3 * 2.0 ** -10) == 0x02
    # 1.0625 lies halfway between 1.0 (0x38, even) and 1.125 (0x39).
    assert orc.e4m3_encode(1.0625) == 0x38
    # 464 is halfway between 448 and the NaN slot: saturate to 448.
    assert orc.e4m3_encode(464.0) == 0x7E
    assert orc.e4m3_encode(-1e9) == 0xFE


# ------------------------------------------------------------------- BF16 --

def test_bf16_rounding_golden():
    for m, e, bits, *_ in read_golden("bf16_rounding.txt"):
        x = Fraction(int(m)) * Fraction(2) ** int(e)
        assert orc.bf16_bits(float(x)) == int(bits, 16), (m, e)
        assert float(x) == x  # each case is exact in double


def test_bf16_rounding_matches_bruteforce():
    rng = np.random.default_rng(5)
    vals = list(rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, 3000))
    for v in vals:
        want = float(bf.bf16(Fraction(v)))
        got = float(orc.bf16_bits_to_float(np.array([orc.bf16_bits(v)], dtype=np.uint16))[0])
        assert got == want, v
