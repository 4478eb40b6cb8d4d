"""Pins of the oracle grouped GEMM: the exact int64 path against the FP64 path,
the rational brute force, numpy's matmul on dequantised matrices (decoded with
the golden E2M1 table and torch's float8_e4m3fn), closed forms and invariants."""
import math

import numpy as np
import pytest
import torch

from conftest import read_golden
from oracle import bruteforce as bf
from oracle import oracle as orc
from workloads import gen


def _problem(E, rows_per_expert, n, k, seed, a_rows=None):
    rng = np.random.default_rng(seed)
    counts = np.array(rows_per_expert, dtype=np.int64)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    m = int(offsets[-1])
    a_rows = m if a_rows is None else a_rows
    a_q = gen.random_fp4_bytes((a_rows, k // 2), seed)
    a_sf = gen.random_e4m3_codes((a_rows, k // 16), seed + 1, 0x20, 0x48)
    w_q = gen.random_fp4_bytes((E, n, k // 2), seed + 2)
    w_sf = gen.random_e4m3_codes((E, n, k // 16), seed + 3, 0x20, 0x48)
    w_scale = rng.uniform(0.5, 2.0, E).astype(np.float32)
    a_scale = np.float32(rng.uniform(0.5, 2.0))
    return a_q, a_sf, a_scale, w_q, w_sf, w_scale, offsets


def _golden_e2m1():
    return np.array([float(v) for _, v in read_golden("e2m1_ocp_mx.txt")])


def _dequant_indep(q, sf):
    """Dequantise with the golden E2M1 table and torch's E4M3 decode (no oracle code)."""
    table = _golden_e2m1()
    lo, hi = q & 15, q >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(*q.shape[:-1], q.shape[-1] * 2)
    scales = torch.from_numpy(np.ascontiguousarray(sf)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return table[codes] * np.repeat(scales, 16, axis=-1)


@pytest.mark.parametrize("E,rows,n,k", [(1, [5], 3, 16), (3, [1, 0, 5], 3, 48), (3, [0, 1, 1], 1, 32),
                                        (1, [1], 1, 16)])
def test_exact_matches_bruteforce(E, rows, n, k):
    a_q, a_sf, a_scale, w_q, w_sf, w_scale, off = _problem(E, rows, n, k, 21)
    R, out = orc.grouped_gemm(a_q, a_sf, a_scale, w_q, w_sf, w_scale, off)
    bR, bB = bf.grouped_gemm(a_q.tolist(), a_sf.tolist(), float(a_scale), w_q.tolist(),
                             w_sf.tolist(), [float(s) for s in w_scale], off.tolist())
    assert R.shape == (int(off[-1]), n)
    for r in range(R.shape[0]):
        for j in range(n):
            assert math.isclose(R[r, j], float(bR[r][j]), rel_tol=1e-15, abs_tol=0)
            assert orc.bf16_bits_to_float(out[r:r + 1, j:j + 1])[0, 0] == float(bB[r][j])


def test_exact_matches_f64_path():
    a_q, a_sf, a_scale, w_q, w_sf, w_scale, off = _problem(4, [7, 0, 3, 9], 40, 256, 22)
    R, _ = orc.grouped_gemm(a_q, a_sf, a_scale, w_q, w_sf, w_scale, off)
    R64 = orc.grouped_gemm_f64(a_q, a_sf, a_scale, w_q, w_sf, w_scale, off)
    scale = np.abs(R).max()
    assert np.max(np.abs(R - R64)) <= 1e-12 * scale


def test_dense_single_expert_matches_numpy_matmul():
    m, n, k = 24, 40, 192
    a_q, a_sf, a_scale, w_q, w_sf, w_scale, off = _problem(1, [m], n, k, 23)
    R, _ = orc.grouped_gemm(a_q, a_sf, a_scale, w_q, w_sf, w_scale, off)
    A = _dequant_indep(a_q, a_sf)            # [m][k]
    W = _dequant_indep(w_q[0], w_sf[0])      # [n][k]
    ref = np.matmul(A, W.T) * float(a_scale) * float(w_scale[0])
    assert np.max(np.abs(R - ref)) <= 1e-12 * np.abs(ref).max()


def test_grouped_matches_numpy_per_expert_with_row_index():
    E, rows, n, k = 3, [4, 0, 6], 24, 64
    a_q, a_sf, a_scale, w_q, w_sf, w_scale, off = _problem(E, rows, n, k, 24, a_rows=7)
    idx = np.array([6, 0, 3, 3, 1, 2, 5, 4, 0, 6], dtype=np.int32)
    R, _ = orc.grouped_gemm(a_q, a_sf, a_scale, w_q, w_sf, w_scale, off, a_row_index=idx)
    A = _dequant_indep(a_q, a_sf)
    for e in range(E):
        W = _dequant_indep(w_q[e], w_sf[e])
        for r in range(off[e], off[e + 1]):
            ref = A[idx[r]] @ W.T * float(a_scale) * float(w_scale[e])
            assert np.max(np.abs(R[r] - ref)) <= 1e-12 * max(np.abs(ref).max(), 1e-300)


def test_single_nonzero_element_closed_form():
    n, k = 2, 32
    a_q = np.zeros((1, k // 2), np.uint8)
    a_sf = np.zeros((1, k // 16), np.uint8)
    w_q = np.zeros((1, n, k // 2), np.uint8)
    w_sf = np.zeros((1, n, k // 16), np.uint8)
    a_q[0, 9] = 0x70           # element 19 = +6
    a_sf[0, 1] = 0x39          # block 1 scale 1.125
    w_q[0, 1, 9] = 0xD0        # weight row 1, element 19 = -3
    w_sf[0, 1, 1] = 0x01       # 2^-9
    off = np.array([0, 1], np.int32)
    R, out = orc.grouped_gemm(a_q, a_sf, 2.0, w_q, w_sf, np.array([0.25], np.float32), off)
    assert R[0, 0] == 0.0
    assert R[0, 1] == 6 * 1.125 * -3 * 2.0 ** -9 * 2.0 * 0.25


def test_zero_activations_give_zero():
    a_q, a_sf, a_scale, w_q, w_sf, w_scale, off = _problem(2, [3, 2], 8, 64, 25)
    R, out = orc.grouped_gemm(np.zeros_like(a_q), a_sf, a_scale, w_q, w_sf, w_scale, off)
    assert not R.any() and not (out & 0x7FFF).any()


def test_doubling_a_scale_doubles_exactly():
    a_q, a_sf, a_scale, w_q, w_sf, w_scale, off = _problem(2, [3, 4], 16, 128, 26)
    R1, _ = orc.grouped_gemm(a_q, a_sf, a_scale, w_q, w_sf, w_scale, off)
    R2, _ = orc.grouped_gemm(a_q, a_sf, a_scale * np.float32(2), w_q, w_sf, w_scale, off)
    assert np.array_equal(R2, 2 * R1)


def test_block_scale_exponent_step_adds_that_blocks_term():
    a_q, a_sf, a_scale, w_q, w_sf, w_scale, off = _problem(1, [2], 4, 64, 27)
    R1, _ = orc.grouped_gemm(a_q, a_sf, a_scale, w_q, w_sf, w_scale, off)
    w_sf2 = w_sf.copy()
    j, b = 2, 1
    w_sf2[0, j, b] += 0x08        # exponent + 1: this block's scale doubles
    R2, _ = orc.grouped_gemm(a_q, a_sf, a_scale, w_q, w_sf2, w_scale, off)
    A = _dequant_indep(a_q, a_sf)
    W = _dequant_indep(w_q[0], w_sf[0])
    term = A[:, 16 * b:16 * b + 16] @ W[j, 16 * b:16 * b + 16] * float(a_scale) * float(w_scale[0])
    other = [c for c in range(4) if c != j]
    assert np.array_equal(R2[:, other], R1[:, other])
    assert np.allclose(R2[:, j] - R1[:, j], term, rtol=1e-12, atol=1e-12 * np.abs(R1).max())


def test_expert_permutation_permutes_rows():
    E, rows = 4, [2, 3, 1, 2]
    a_q, a_sf, a_scale, w_q, w_sf, w_scale, off = _problem(E, rows, 8, 64, 28)
    R, _ = orc.grouped_gemm(a_q, a_sf, a_scale, w_q, w_sf, w_scale, off)
    perm = [2, 0, 3, 1]
    # expert perm[i] becomes expert i; its rows move with it
    row_lists = [list(range(off[e], off[e + 1])) for e in range(E)]
    new_rows = [r for e in perm for r in row_lists[e]]
    off2 = np.zeros(E + 1, np.int32)
    off2[1:] = np.cumsum([rows[e] for e in perm])
    R2, _ = orc.grouped_gemm(a_q[new_rows], a_sf[new_rows], a_scale, w_q[perm], w_sf[perm],
                             w_scale[perm], off2)
    assert np.array_equal(R2, R[new_rows])


def test_selected_rows_equal_full_rows():
    a_q, a_sf, a_scale, w_q, w_sf, w_scale, off = _problem(3, [5, 2, 6], 12, 96, 29)
    R, out = orc.grouped_gemm(a_q, a_sf, a_scale, w_q, w_sf, w_scale, off)
    sel = np.array([12, 0, 6, 5], np.int64)
    Rs, outs = orc.grouped_gemm(a_q, a_sf, a_scale, w_q, w_sf, w_scale, off, rows_sel=sel)
    assert np.array_equal(Rs, R[sel]) and np.array_equal(outs, out[sel])


def test_row_error_metric():
    R = np.array([[3.0, 4.0], [0.0, 0.0]])
    ref = orc.bf16_bits_array(R)
    got = ref.copy()
    err, norm = orc.row_error(got, ref, R)
    assert np.array_equal(err, [0.0, 0.0]) and np.array_equal(norm, [5.0, 0.0])
    got[1, 0] = 0x3F80
    err, _ = orc.row_error(got, ref, R)
    assert err[1] == np.inf
