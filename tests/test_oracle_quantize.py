"""Pins of the oracle quantiser: the rational brute force on tiny tensors, and
invariants that hold for the definition whatever the data."""
import math

import numpy as np
import pytest

from oracle import bruteforce as bf
from oracle import oracle as orc
from workloads import gen


def _tiny_inputs():
    rng = np.random.default_rng(3)
    cases = {}
    cases["normal"] = rng.standard_normal((3, 32)).astype(np.float32)
    x = rng.standard_normal((2, 48)).astype(np.float32)
    x[0, 16:32] = 0.0                                   # an all-zero block
    x[1, 0:16] *= np.float32(1e-3)                      # a block with a subnormal E4M3 scale
    x[1, 5] = -0.0
    cases["zeros_and_small"] = x
    # values placed on the E2M1 midpoints of the block scale: block amax 6 -> r = 1/448*...
    y = np.array([[6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, -0.25, -0.75, -1.25, -1.75, -2.5,
                   -3.5, -5, 0.1]], dtype=np.float32)
    cases["midpoints"] = y
    cases["wide_range"] = (rng.standard_normal((2, 32)) * 10.0 ** rng.integers(-6, 6, (2, 32))
                           ).astype(np.float32)
    cases["bf16_values"] = gen.bf16_round(rng.standard_normal((2, 64)).astype(np.float32))
    return cases


@pytest.mark.parametrize("name", list(_tiny_inputs().keys()))
@pytest.mark.parametrize("static_g", [None, 0.01, 3.0e-4])
def test_quantize_matches_bruteforce(name, static_g):
    x = _tiny_inputs()[name]
    q, sf, g = orc.quantize(x, g=static_g)
    bq, bsf, bg = bf.quantize([[float(v) for v in row] for row in x], g=static_g)
    assert np.float32(bg) == g
    assert np.array_equal(sf, np.array(bsf, dtype=np.uint8)), (sf, bsf)
    assert np.array_equal(q, np.array(bq, dtype=np.uint8))


def _dequant(q, sf, g):
    rows, kb = q.shape
    lo, hi = q & 15, q >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(rows, kb * 2)
    vals = np.vectorize(orc.e2m1_decode)(codes)
    scales = np.vectorize(orc.e4m3_decode)(sf)
    return vals * np.repeat(scales, 16, axis=1) * float(g)


def test_all_zero_tensor():
    x = np.zeros((4, 64), dtype=np.float32)
    q, sf, g = orc.quantize(x)
    assert g == np.float32(1.0) and not q.any() and not sf.any()


def test_block_holding_tensor_amax_gets_max_scale():
    x = np.random.default_rng(1).standard_normal((16, 256)).astype(np.float32)
    q, sf, g = orc.quantize(x)
    r, c = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert sf[r, c // 16] == 0x7E        # amax_b / (6 g) = 448 exactly
    codes = np.where(np.arange(16) % 2 == 0, q[r, c // 16 * 8 + np.arange(16) // 2] & 15,
                     q[r, c // 16 * 8 + np.arange(16) // 2] >> 4)
    assert (codes[c % 16] & 7) == 7      # the amax element maps to +-6


def test_normal_scale_blocks_use_the_top_code():
    x = np.random.default_rng(2).standard_normal((32, 512)).astype(np.float32)
    q, sf, g = orc.quantize(x)
    lo, hi = q & 7, (q >> 4) & 7
    mags = np.stack([lo, hi], -1).reshape(32, 512)
    normal = (sf & 0x78) != 0            # exponent field non-zero
    top = mags.reshape(32, 32, 16).max(axis=2)
    assert normal.any() and np.all(top[normal] == 7)


def test_row_permutation_equivariance():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((24, 128)).astype(np.float32)
    perm = rng.permutation(24)
    q, sf, g = orc.quantize(x)
    qp, sfp, gp = orc.quantize(x[perm])
    assert g == gp and np.array_equal(q[perm], qp) and np.array_equal(sf[perm], sfp)


@pytest.mark.parametrize("p", [-3, 1, 5])
def test_power_of_two_scaling_moves_only_the_tensor_scale(p):
    x = np.random.default_rng(6).standard_normal((8, 128)).astype(np.float32)
    q, sf, g = orc.quantize(x)
    q2, sf2, g2 = orc.quantize(x * np.float32(2.0 ** p))
    assert np.array_equal(q, q2) and np.array_equal(sf, sf2)
    assert g2 == g * np.float32(2.0 ** p)


def test_dequantisation_error_is_within_half_a_grid_step():
    x = np.random.default_rng(8).standard_normal((16, 256)).astype(np.float32)
    q, sf, g = orc.quantize(x)
    xh = _dequant(q, sf, g)
    s = np.repeat(np.vectorize(orc.e4m3_decode)(sf), 16, axis=1) * float(g)
    # Largest half-gap of the E2M1 grid is 1 (between 4 and 6); saturation adds at
    # most 0.4 (|y| <= 6.4 when the block scale is a normal E4M3 value).
    assert np.all(np.abs(x - xh) <= 1.0 * s * (1 + 1e-6))
    rel = np.linalg.norm(x - xh) / np.linalg.norm(x)
    assert rel < 0.15


def test_static_scale_is_used_as_given():
    x = np.random.default_rng(9).standard_normal((4, 64)).astype(np.float32)
    q, sf, g = orc.quantize(x, g=0.5)
    assert g == np.float32(0.5)
    bq, bsf, _ = bf.quantize([[float(v) for v in row] for row in x], g=0.5)
    assert np.array_equal(q, np.array(bq, dtype=np.uint8)) and np.array_equal(sf, np.array(bsf, dtype=np.uint8))


def test_rejects_k_not_multiple_of_16():
    with pytest.raises(ValueError):
        orc.quantize(np.zeros((2, 24), dtype=np.float32))


def _threshold_block_rows():
    """Rows of 16 whose block scale is an E4M3 value with an odd mantissa (so 1/s is
    not exact) and whose other elements sit on an E2M1 rounding threshold times s,
    or one or two float32 ulps away.  With g = 1 the block amax 6*v gives s = v."""
    rows = []
    thresholds = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    for v in (1.125 * 2 ** -2, 1.375 * 2 ** -5, 1.625, 1.875 * 2 ** 3, 1.25 * 2 ** -1, 1.75 * 2 ** 2,
              1.375 * 2 ** 6, 1.625 * 2 ** -4):
        for t in thresholds:
            base = np.float32(t * v)  # exact: at most 7 significant bits
            row = [np.float32(6 * v)]
            x = base
            for _ in range(7):
                row.append(x)
                x = np.nextafter(x, np.float32(np.inf))
            x = np.nextafter(base, np.float32(-np.inf))
            for _ in range(7):
                row.append(x)
                x = np.nextafter(x, np.float32(-np.inf))
            row.append(-base)
            rows.append(row)
    return np.array(rows, dtype=np.float32)


def test_division_is_ieee_division_near_thresholds():
    x = _threshold_block_rows()
    q, sf, g = orc.quantize(x, g=1.0)
    bq, bsf, _ = bf.quantize([[float(v) for v in row] for row in x], g=1.0)
    assert np.array_equal(sf, np.array(bsf, dtype=np.uint8))
    assert np.array_equal(q, np.array(bq, dtype=np.uint8))
    # The inputs have teeth: multiplying by a rounded reciprocal instead of dividing
    # changes at least one code.
    s = np.array([np.float32(orc.e4m3_decode(int(c))) for c in sf[:, 0]], dtype=np.float32)
    y_div = x / s[:, None]
    y_rcp = x * (np.float32(1.0) / s)[:, None]
    assert not np.array_equal(orc.e2m1_encode_array(y_div), orc.e2m1_encode_array(y_rcp))
