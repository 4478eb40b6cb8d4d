"""Pins of the oracle's MoE finalize step (oracle.combine): a hand-computed case,
a plain Python loop on random inputs, the top-1 / unit-weight case (a row
scatter), accumulation onto an initial value and argument checks."""
import numpy as np
import pytest

from oracle import oracle as orc


def test_hand_computed_case():
    # Rows 0 and 2 belong to token 1, row 1 to token 0; token 2 receives nothing.
    R = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]])
    tok = np.array([1, 0, 1])
    w = np.array([0.5, 2.0, 0.25], np.float32)
    out = orc.combine(R, tok, w, 3)
    # token 0: 2 * [3, 4]; token 1: 0.5 * [1, 2] + 0.25 * [5, 6]; token 2: zeros.
    assert np.array_equal(out, np.array([[6.0, 8.0], [1.75, 2.5], [0.0, 0.0]]))


def test_matches_a_plain_loop():
    rng = np.random.default_rng(5)
    m, n, T = 40, 7, 9
    R = rng.standard_normal((m, n))
    tok = rng.integers(0, T, m)
    w = rng.uniform(0.0, 1.0, m).astype(np.float32)
    init = rng.standard_normal((T, n))
    want = init.copy()
    for r in range(m):
        for j in range(n):
            want[tok[r], j] += float(w[r]) * R[r, j]
    init_copy = init.copy()
    got = orc.combine(R, tok, w, T, init=init)
    assert np.allclose(got, want, rtol=1e-14, atol=1e-14)
    assert np.array_equal(init, init_copy)  # the caller's init is not modified


def test_top1_unit_weights_scatter_rows():
    rng = np.random.default_rng(6)
    R = rng.standard_normal((5, 3))
    tok = np.array([4, 0, 2, 6, 1])
    out = orc.combine(R, tok, np.ones(5, np.float32), 7)
    assert np.array_equal(out[tok], R)
    assert not np.any(out[[3, 5]])


def test_weights_enter_as_float32_values():
    # The weight is the FP32 value the GPU reads (0.1f, not 0.1).
    R = np.ones((1, 1))
    out = orc.combine(R, np.array([0]), np.array([0.1], np.float32), 1)
    assert out[0, 0] == float(np.float32(0.1))


def test_rejects_tokens_out_of_range():
    with pytest.raises(ValueError):
        orc.combine(np.ones((2, 2)), np.array([0, 3]), np.ones(2, np.float32), 3)
    with pytest.raises(ValueError):
        orc.combine(np.ones((2, 2)), np.array([-1, 0]), np.ones(2, np.float32), 3)


def test_token_row_error_conventions():
    ref = np.array([[3.0, 4.0], [0.0, 0.0], [0.0, 0.0]])
    got = np.array([[3.0, 4.5], [0.0, 0.0], [0.0, 1e-30]])
    err, norm = orc.token_row_error(got, ref)
    assert err[0] == pytest.approx(0.1) and norm[0] == 5.0
    assert err[1] == 0.0 and np.isinf(err[2])
