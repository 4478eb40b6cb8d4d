"""Exact rational brute force of the quantiser and the grouped GEMM.

TEST INFRASTRUCTURE ONLY (pins the C oracle on tiny inputs; never imported by
the library).  Written separately from ``fp4_oracle.c``: every rounding here is
"pick the nearest representable value by exhaustive search, ties to the even
code", and every FP32 operation is the exact rational result rounded to the
nearest float32 by search over its binade.  Slow by design: tiny shapes only.

Formats: E2M1 per the OCP Microscaling (MX) v1.0 specification, E4M3 per the
OCP 8-bit Floating Point (OFP8) v1.0 specification.  Block of 16 elements with
one FP8 scale, two 4-bit values per byte: "Peering into the CUTLASS
SharedStorage", section "Input Knowledge", item 3.
"""
from __future__ import annotations

import math
from fractions import Fraction

# Non-negative E2M1 values in code order 0..7 (sign is bit 3).
E2M1_MAGS = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2),
             Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def e4m3_value(code: int) -> Fraction | None:
    """Exact value of an E4M3 code (None for NaN)."""
    s, e, m = (code >> 7) & 1, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return None
    if e == 0:
        v = Fraction(m, 8) * Fraction(1, 2 ** 6)
    else:
        v = (1 + Fraction(m, 8)) * (Fraction(2) ** (e - 7))
    return -v if s else v


E4M3_NONNEG = [(c, e4m3_value(c)) for c in range(0x7F)]  # 0x00..0x7E, all finite


def _round_half_even(q: Fraction) -> int:
    return round(q)  # Fraction.__round__ rounds half to even


def _binade_exp(a: Fraction) -> int:
    """e with 2^e <= a < 2^(e+1), for a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_to_format(x: Fraction, mant_bits: int, min_exp: int) -> Fraction:
    """Nearest value with `mant_bits` fraction bits, exponent >= min_exp (subnormals
    below), ties to even; no overflow handling (callers stay in range)."""
    if x == 0:
        return Fraction(0)
    a = abs(x)
    e = max(_binade_exp(a), min_exp)
    spacing = Fraction(2) ** (e - mant_bits)
    v = _round_half_even(a / spacing) * spacing
    return v if x > 0 else -v


def fl32(x: Fraction) -> Fraction:
    return round_to_format(x, 23, -126)


def bf16(x: Fraction) -> Fraction:
    return round_to_format(x, 7, -126)


def e2m1_nearest(mag: Fraction) -> int:
    """Code 0..7 of the E2M1 magnitude nearest to mag >= 0; ties to the even code."""
    best = None
    for c, v in enumerate(E2M1_MAGS):
        d = abs(mag - v)
        key = (d, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def e4m3_nearest(r: Fraction) -> int:
    """Code of the finite non-negative E4M3 value nearest to r >= 0; ties to even code."""
    best = None
    for c, v in E4M3_NONNEG:
        d = abs(r - v)
        key = (d, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def quantize(x_rows: list[list[float]], g: float | None = None):
    """Quantise a matrix given as rows of float32-representable Python floats.

    Returns (q bytes per row, sf codes per row, g as a Python float).
    """
    k = len(x_rows[0]) if x_rows else 0
    assert k % 16 == 0
    if g is None:
        amax = max((abs(Fraction(v)) for row in x_rows for v in row), default=Fraction(0))
        G = fl32(amax / 2688) if amax > 0 else Fraction(1)
    else:
        G = Fraction(g)
    six_g = fl32(6 * G)
    q_out, sf_out = [], []
    for row in x_rows:
        qrow, sfrow = [], []
        for b in range(k // 16):
            blk = row[16 * b:16 * b + 16]
            amax_b = max(abs(Fraction(v)) for v in blk)
            r = fl32(amax_b / six_g)
            sf = e4m3_nearest(r)
            s = fl32(e4m3_value(sf) * G)
            codes = []
            for v in blk:
                if s == 0:
                    codes.append(0)
                    continue
                y = fl32(Fraction(v) / s)
                sign = 8 if math.copysign(1.0, v) < 0 else 0
                codes.append(sign | e2m1_nearest(abs(y)))
            sfrow.append(sf)
            for i in range(8):
                qrow.append(codes[2 * i] | (codes[2 * i + 1] << 4))
        q_out.append(qrow)
        sf_out.append(sfrow)
    return q_out, sf_out, float(G)


def _elem(qrow, sfrow, kk: int) -> Fraction:
    code = (qrow[kk // 2] >> (4 * (kk % 2))) & 15
    mag = E2M1_MAGS[code & 7]
    v = -mag if code & 8 else mag
    return v * e4m3_value(sfrow[kk // 16])


def grouped_gemm(a_q, a_sf, a_scale, w_q, w_sf, w_scale, offsets, a_row_index=None):
    """Exact R (list of rows of Fractions) and bf16(R) (Fractions), all m_total rows."""
    E = len(offsets) - 1
    n = len(w_q[0])
    k = 2 * len(w_q[0][0])
    R, B = [], []
    for e in range(E):
        for r in range(offsets[e], offsets[e + 1]):
            src = a_row_index[r] if a_row_index is not None else r
            arow = [_elem(a_q[src], a_sf[src], kk) for kk in range(k)]
            rr, bb = [], []
            for j in range(n):
                s = sum((arow[kk] * _elem(w_q[e][j], w_sf[e][j], kk) for kk in range(k)),
                        Fraction(0))
                val = Fraction(a_scale) * Fraction(w_scale[e]) * s
                rr.append(val)
                bb.append(bf16(val))
            R.append(rr)
            B.append(bb)
    return R, B
