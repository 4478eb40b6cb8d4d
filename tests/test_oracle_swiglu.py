"""Pins of the oracle's gate+up activation step (oracle.silu, oracle.swiglu,
oracle.swiglu_quantize): closed forms of the sigmoid, torch's SiLU as a library
routine, a hand-computed case that fixes which half of the GEMM result is the
gate, and hand-encoded NVFP4 bytes for the quantised output (E2M1 codes from the
OCP MX table: 0, 0.5, 1, 1.5, 2, 3, 4, 6 are codes 0..7, bit 3 the sign)."""
import math

import numpy as np
import pytest
import torch

from oracle import oracle as orc


def test_silu_closed_forms():
    # sigmoid(ln 3) = 3/4 and sigmoid(ln 2) = 2/3, so silu(x) = x * sigmoid(x) is known there.
    x = np.array([0.0, math.log(3.0), -math.log(3.0), math.log(2.0), -math.log(2.0)])
    want = np.array([0.0, 0.75 * math.log(3.0), -0.25 * math.log(3.0),
                     (2.0 / 3.0) * math.log(2.0), -(1.0 / 3.0) * math.log(2.0)])
    assert np.allclose(orc.silu(x), want, rtol=1e-15, atol=0.0)


def test_silu_odd_part_is_half_identity():
    # sigmoid(x) + sigmoid(-x) = 1, so silu(x) - silu(-x) = x.
    x = np.random.default_rng(1).uniform(-30.0, 30.0, 1000)
    assert np.allclose(orc.silu(x) - orc.silu(-x), x, rtol=1e-13, atol=1e-13)


def test_silu_limits():
    got = orc.silu(np.array([1000.0, -1000.0, 64.0]))
    assert got[0] == 1000.0
    assert got[1] == 0.0 and np.signbit(got[1])  # exp overflows: the limit -0, not NaN
    assert got[2] == 64.0


def test_silu_matches_torch():
    x = np.random.default_rng(2).standard_normal(4096) * 8.0
    want = torch.nn.functional.silu(torch.from_numpy(x)).numpy()
    assert np.allclose(orc.silu(x), want, rtol=1e-15, atol=1e-300)


def test_swiglu_gate_is_first_half():
    # Two output columns: gate = (ln 3, 0), up = (4, 5).
    R = np.array([[math.log(3.0), 0.0, 4.0, 5.0]])
    h = orc.swiglu(R)
    assert h.shape == (1, 2)
    assert h[0, 0] == pytest.approx(3.0 * math.log(3.0), rel=1e-15)  # silu(ln 3) * 4
    assert h[0, 1] == 0.0                                            # silu(0) * 5
    # Swapping the halves would give silu(4) * ln 3, which is different.
    assert abs(h[0, 0] - orc.silu(np.array([4.0]))[0] * math.log(3.0)) > 0.1


def test_swiglu_rejects_odd_width():
    with pytest.raises(ValueError):
        orc.swiglu(np.ones((2, 3)))


def _gate_up(up_rows):
    # A large gate makes silu(gate) = gate exactly (64 * (1 - 1.6e-28) rounds to 64),
    # so h = 64 * up: every row below is chosen to land on E2M1 values times a scale.
    up = np.array(up_rows, dtype=np.float64) / 64.0
    return np.concatenate([np.full_like(up, 64.0), up], axis=1)


def test_swiglu_quantize_hand_encoded():
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    row0 = grid + [-v for v in grid]          # amax 6: block scale 1.0 (E4M3 0x38)
    row1 = [v / 2 for v in row0]              # amax 3: block scale 0.5 (E4M3 0x30)
    R = _gate_up([row0, row1])
    h, q, sf = orc.swiglu_quantize(R, 1.0)
    assert np.array_equal(h[0], np.array(row0))
    # Codes 0..15 in element order, two per byte, element 2i in the low nibble.
    want_q = np.array([0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE], dtype=np.uint8)
    assert np.array_equal(q[0], want_q) and np.array_equal(q[1], want_q)
    assert sf[0, 0] == 0x38 and sf[1, 0] == 0x30


def test_swiglu_quantize_saturates_under_a_small_static_scale():
    # g = 1e-4: the block scale wants 6 / 6e-4 = 10^4 and saturates to 448 (E4M3 0x7E);
    # 6 / (448 * 1e-4) then exceeds 6 and the element saturates to code 7 (and 15).
    R = _gate_up([[6.0, -6.0] + [0.0] * 14])
    _, q, sf = orc.swiglu_quantize(R, 1e-4)
    assert sf[0, 0] == 0x7E
    assert q[0, 0] == 0xF7 and not np.any(q[0, 1:])


def test_swiglu_quantize_zero_block():
    # All-zero up projection: block amax 0, scale code 0, every element code 0.
    R = _gate_up([[0.0] * 16])
    _, q, sf = orc.swiglu_quantize(R, 1.0)
    assert sf[0, 0] == 0 and not np.any(q)
