"""GPU parity of moe_grouped_gemm_fp4 and moe_fp4_combine at the largest sizes the
library accepts.

The header's limits: at most 8192 experts; m_total below 2^29 - 1024; n * k/2 and a_rows * k/2 below
2^31 - 4096 (every byte offset into one expert's weights and into the
activations is a 32-bit buffer offset); ldo at most 2^23; each combine buffer
below 2^31 - 4096 bytes.  Each case sits at its limit, the oracle computing
sampled rows and columns (the bar of the other GEMM tests: per-row relative L2
error <= 2e-3 on the sampled columns; the combine's FP32 sums against FP64)."""
import numpy as np
import pytest
import torch

from gpu_util import TOL, bf16_bits_of, dev, require_gpu, say
from oracle import oracle as orc
from workloads import gen

pytestmark = pytest.mark.gpu

LIMIT = 2 ** 31 - 4096


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _gemm(a_q, a_sf, a_scale, w_q, w_sf, w_scale, offsets, m, row_index=None, ldo=None,
          tile=None, packed=False):
    """Device inputs in, BF16 bits [m][n] out; columns n .. ldo-1 must keep the canary."""
    import os
    from block_scaled_fp4_05_amd import moe_fp4
    n = w_q.shape[1]
    ldo = n if ldo is None else ldo
    out = torch.full((m, ldo), -777.0, dtype=torch.bfloat16, device="cuda")
    old = os.environ.get("MOE_FP4_TILE")
    if tile:
        os.environ["MOE_FP4_TILE"] = tile
    try:
        moe_fp4.grouped_gemm(a_q, a_sf, a_scale, w_q, w_sf, w_scale, offsets,
                             a_row_index=row_index, out=out, m_total=m, packed=packed)
        torch.cuda.synchronize()
    finally:
        if tile:
            if old is None:
                del os.environ["MOE_FP4_TILE"]
            else:
                os.environ["MOE_FP4_TILE"] = old
    return out


def _check(got_bits, R, ref, label):
    err, norm = orc.row_error(got_bits, ref, R)
    worst = int(np.argmax(err))
    assert np.all(err <= TOL), f"{label}: row {worst} err {err[worst]:.3g} (norm {norm[worst]:.3g})"


@pytest.mark.parametrize("tile", [None, "16x32", "128x128"])
def test_most_experts(tile):
    """8192 experts (the limit), most of them empty, the rest ragged; every row checked."""
    E, n, k = 8192, 64, 256
    rng = np.random.default_rng(8192)
    cnt = np.zeros(E, np.int64)
    live = rng.choice(E, size=700, replace=False)
    cnt[live] = rng.integers(1, 40, size=700)
    cnt[E - 1] = 17                       # the last expert is never empty
    off = np.zeros(E + 1, np.int32)
    off[1:] = np.cumsum(cnt)
    m = int(off[-1])
    a_q = gen.random_fp4_bytes((m, k // 2), 1)
    a_sf = gen.random_e4m3_codes((m, k // 16), 2, 0x20, 0x50)
    w_q = gen.random_fp4_bytes((E, n, k // 2), 3)
    w_sf = gen.random_e4m3_codes((E, n, k // 16), 4, 0x20, 0x50)
    w_scale = rng.uniform(0.25, 4.0, E).astype(np.float32)
    a_scale = np.float32(0.75)
    say(f"limits: {E} experts, m_total={m}, tile={tile}")
    out = _gemm(dev(a_q), dev(a_sf), dev(np.array([a_scale])), dev(w_q), dev(w_sf), dev(w_scale),
                dev(off), m, tile=tile)
    R, ref = orc.grouped_gemm(a_q, a_sf, a_scale, w_q, w_sf, w_scale, off)
    _check(bf16_bits_of(out), R, ref, f"{E} experts, tile {tile}")


def test_largest_ldo():
    """ldo = 2^23 (the limit): rows 16 MB apart, padding columns untouched."""
    E, n, k, ldo = 3, 64, 256, 2 ** 23
    off = np.array([0, 5, 5, 21], np.int32)
    m = int(off[-1])
    a_q = gen.random_fp4_bytes((m, k // 2), 11)
    a_sf = gen.random_e4m3_codes((m, k // 16), 12, 0x20, 0x50)
    w_q = gen.random_fp4_bytes((E, n, k // 2), 13)
    w_sf = gen.random_e4m3_codes((E, n, k // 16), 14, 0x20, 0x50)
    w_scale = np.array([0.5, 1.0, 2.0], np.float32)
    a_scale = np.float32(1.5)
    say(f"limits: ldo={ldo}")
    out = _gemm(dev(a_q), dev(a_sf), dev(np.array([a_scale])), dev(w_q), dev(w_sf), dev(w_scale),
                dev(off), m, ldo=ldo)
    canary = bf16_bits_of(torch.tensor([-777.0], dtype=torch.bfloat16))[0]
    pad = out[:, n:]
    assert bool((pad == pad[0, 0]).all()) and bf16_bits_of(pad[:1, :1])[0, 0] == canary
    R, ref = orc.grouped_gemm(a_q, a_sf, a_scale, w_q, w_sf, w_scale, off)
    _check(bf16_bits_of(out[:, :n]), R, ref, "ldo 2^23")


@pytest.mark.parametrize("tile,ldo", [
    (None, 2 ** 23), ("256x256!", 2 ** 23), ("128x128", 2 ** 23),
    ("256x256!", (2 ** 31 - 4096) // 512 - 8), ("128x128", 2 ** 23 - 24),
    (None, (2 ** 31 - 4096) // 512 - 8)])
def test_workgroup_tiles_at_the_largest_ldo(tile, ldo):
    """A 300-row expert (two 256-row M-tiles), an empty one and a 17-row one, n = 272
    (a partial last 256-column N-tile), with output rows ldo apart: at ldo = 2^23 the
    workgroup tiles' 128 or 256 rows would span 2^31 bytes or more, so the library
    falls back to per-wave items; just below that bound the workgroup tile itself
    runs.  Every row is checked, the padding columns and the rows past m_total keep
    their canary."""
    _workgroup_tile_case(tile, ldo, 256, np.array([0, 300, 300, 317], np.int32))


@pytest.mark.parametrize("ldo", [2 ** 23, 2 ** 23 - 24])
def test_mid_tile_at_the_largest_ldo(ldo):
    """48-row workgroup items at the largest accepted ldo: 48 rows of 2^23 BF16 values
    stay below 2^31 bytes, so the 48 x 512 kernel itself runs (K = 512, its smallest);
    a 100-row expert (items of 48, 48 and 4 rows), an empty one and a 17-row one, n = 272
    (a partial 512-column item), every row checked, canaries kept."""
    _workgroup_tile_case("48x512", ldo, 512, np.array([0, 100, 100, 117], np.int32))


def _workgroup_tile_case(tile, ldo, k, off):
    E, n = 3, 272
    m = int(off[-1])
    extra = 8
    a_q = gen.random_fp4_bytes((m, k // 2), 61)
    a_sf = gen.random_e4m3_codes((m, k // 16), 62, 0x20, 0x50)
    w_q = gen.random_fp4_bytes((E, n, k // 2), 63)
    w_sf = gen.random_e4m3_codes((E, n, k // 16), 64, 0x20, 0x50)
    w_scale = np.array([0.5, 1.0, 2.0], np.float32)
    a_scale = np.float32(1.5)
    say(f"limits: workgroup tiles, tile={tile}, ldo={ldo}, {(m + extra) * ldo * 2 / 2**30:.1f} GiB output")
    import os
    from block_scaled_fp4_05_amd import moe_fp4
    out = torch.full((m + extra, ldo), -777.0, dtype=torch.bfloat16, device="cuda")
    old = os.environ.get("MOE_FP4_TILE")
    if tile:
        os.environ["MOE_FP4_TILE"] = tile
    try:
        moe_fp4.grouped_gemm(dev(a_q), dev(a_sf), dev(np.array([a_scale])), dev(w_q), dev(w_sf),
                             dev(w_scale), dev(off), out=out, m_total=m)
        torch.cuda.synchronize()
    finally:
        if tile:
            if old is None:
                del os.environ["MOE_FP4_TILE"]
            else:
                os.environ["MOE_FP4_TILE"] = old
    canary = int(bf16_bits_of(torch.tensor([-777.0], dtype=torch.bfloat16))[0])
    cbits = torch.tensor(canary, dtype=torch.int16, device="cuda") if canary < 2 ** 15 else \
        torch.tensor(canary - 2 ** 16, dtype=torch.int16, device="cuda")
    assert bool((out[:, n:].view(torch.int16) == cbits).all()), "a padding column was written"
    assert bool((out[m:, :n].view(torch.int16) == cbits).all()), "a row past m_total was written"
    R, ref = orc.grouped_gemm(a_q, a_sf, a_scale, w_q, w_sf, w_scale, off)
    _check(bf16_bits_of(out[:m, :n]), R, ref, f"tile {tile}, ldo {ldo}")
    del out
    torch.cuda.empty_cache()


def test_byte_offsets_at_the_32_bit_limit():
    """One expert whose weights fill n * k/2 just below 2^31 - 4096 bytes, behind an
    empty expert of the same size (so its base is 2 GB into w_q), and activations of
    the same size, gathered from rows at both ends through the row index."""
    k = 65536
    n = (LIMIT - 1) // (k // 2) // 16 * 16          # 65520 rows of 32 KB
    a_rows = n
    assert n * (k // 2) < LIMIT and (n + 16) * (k // 2) >= LIMIT
    E = 2
    rng = np.random.default_rng(31)
    m = 48
    picks = np.concatenate([np.arange(a_rows - 24, a_rows), np.arange(0, 12),
                            rng.choice(a_rows, 12, replace=False)]).astype(np.int32)
    off = np.array([0, 0, m], np.int32)
    cols = np.unique(np.concatenate([np.arange(0, 16), np.arange(n - 32, n),
                                     rng.choice(n, 16, replace=False)]))
    say(f"limits: n={n} k={k} a_rows={a_rows}: generating {2 * n * k // 2 / 2**30:.1f} GiB of codes")
    w1_q = gen.random_fp4_bytes((n, k // 2), 32)
    w1_sf = gen.random_e4m3_codes((n, k // 16), 33, 0x30, 0x40)
    w_q = torch.empty((E, n, k // 2), dtype=torch.uint8, device="cuda")
    w_sf = torch.empty((E, n, k // 16), dtype=torch.uint8, device="cuda")
    w_q[1].copy_(torch.from_numpy(w1_q))
    w_sf[1].copy_(torch.from_numpy(w1_sf))
    w_q[0].zero_()
    w_sf[0].zero_()
    a_q_h = gen.random_fp4_bytes((a_rows, k // 2), 34)
    a_sf_h = gen.random_e4m3_codes((a_rows, k // 16), 35, 0x30, 0x40)
    a_q, a_sf = dev(a_q_h), dev(a_sf_h)
    w_scale = np.array([1.0, 0.5], np.float32)
    a_scale = np.float32(2.0)
    # Oracle on the gathered rows and the sampled columns only (expert 1 alone).
    R, ref = orc.grouped_gemm(a_q_h[picks], a_sf_h[picks], a_scale, w1_q[cols][None],
                              w1_sf[cols][None], w_scale[1:], np.array([0, m], np.int32))
    del a_q_h, a_sf_h
    args = (a_q, a_sf, dev(np.array([a_scale])), w_q, w_sf, dev(w_scale), dev(off), m)
    for tile in [None, "16x64", "64x64", "128x128", "256x256!", "48x512"]:
        say(f"limits: byte offsets, tile={tile}")
        out = _gemm(*args, row_index=dev(picks), tile=tile)
        _check(bf16_bits_of(out)[:, cols], R, ref, f"32-bit byte offsets, tile {tile}")
    say("limits: byte offsets, packed weights")
    from block_scaled_fp4_05_amd import moe_fp4
    packed = moe_fp4.pack_weights(w_q)
    out = _gemm(a_q, a_sf, args[2], packed, w_sf, args[5], args[6], m, row_index=dev(picks),
                packed=True)
    _check(bf16_bits_of(out)[:, cols], R, ref, "32-bit byte offsets, packed")
    say("limits: byte offsets, packed weights, 48x512 workgroup items")
    out = _gemm(a_q, a_sf, args[2], packed, w_sf, args[5], args[6], m, row_index=dev(picks),
                tile="48x512", packed=True)
    _check(bf16_bits_of(out)[:, cols], R, ref, "32-bit byte offsets, packed, 48x512")


def test_combine_buffers_at_the_32_bit_limit():
    """moe_fp4_combine with its routed-row buffer and its FP32 output each just below
    2^31 - 4096 bytes: tokens near both ends, and a skipped slot, checked in FP64."""
    from block_scaled_fp4_05_amd import moe_fp4
    n = 16384
    m = (LIMIT - 1) // (2 * n)            # 65535 BF16 rows of 32 KB
    T = (LIMIT - 1) // (4 * n)            # 32767 FP32 token rows of 64 KB
    assert m * n * 2 < LIMIT and (m + 1) * n * 2 >= LIMIT
    assert T * n * 4 < LIMIT and (T + 1) * n * 4 >= LIMIT
    say(f"limits: combine rows {m}x{n} bf16, out {T}x{n} fp32")
    gen_t = torch.Generator(device="cuda").manual_seed(4242)
    rows = torch.randn((m, n), generator=gen_t, device="cuda").to(torch.bfloat16)
    topk = 2
    tr = torch.arange(T * topk, dtype=torch.int32, device="cuda").reshape(T, topk)
    tr[T - 1, 1] = -1                     # a skipped slot
    tr[T - 2, 0] = m - 1                  # the last routed row
    tw = torch.rand((T, topk), generator=gen_t, device="cuda")
    out = moe_fp4.combine(rows, tr, tw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    picks = np.unique(np.concatenate([[0, 1, T - 2, T - 1], rng.choice(T, 12, replace=False)]))
    tr_h, tw_h = tr.cpu().numpy(), tw.cpu().numpy().astype(np.float64)
    for t in picks:
        ref = np.zeros(n)
        mag = np.zeros(n)
        for s in range(topk):
            r = int(tr_h[t, s])
            if 0 <= r < m:
                v = rows[r].float().cpu().numpy().astype(np.float64)
                ref += tw_h[t, s] * v
                mag += abs(tw_h[t, s] * v)
        got = out[int(t)].cpu().numpy().astype(np.float64)
        # FP32 sums of two exactly representable products: within 2 ulps of the terms.
        assert np.all(np.abs(got - ref) <= 2.0 ** -22 * mag + 1e-30), f"token {t}"


def test_most_routed_rows():
    """m_total = 2^29 - 1025, the largest the header accepts (the row index's byte
    offsets then approach 2^31): two experts, 4 distinct token rows gathered by the
    row index, 16 output columns; sampled rows near both ends checked."""
    E, n, k, a_rows = 2, 16, 256, 4
    m = 2 ** 29 - 1025
    split = 1000
    off = np.array([0, split, m], np.int32)
    a_q = gen.random_fp4_bytes((a_rows, k // 2), 61)
    a_sf = gen.random_e4m3_codes((a_rows, k // 16), 62, 0x30, 0x40)
    w_q = gen.random_fp4_bytes((E, n, k // 2), 63)
    w_sf = gen.random_e4m3_codes((E, n, k // 16), 64, 0x30, 0x40)
    w_scale = np.array([0.5, 2.0], np.float32)
    a_scale = np.float32(1.0)
    say(f"limits: m_total={m} (row index {4 * m / 2**30:.2f} GiB, output {2 * m * n / 2**30:.1f} GiB)")
    idx = (torch.arange(m, dtype=torch.int64, device="cuda") * 7 % a_rows).to(torch.int32)
    out = _gemm(dev(a_q), dev(a_sf), dev(np.array([a_scale])), dev(w_q), dev(w_sf), dev(w_scale),
                dev(off), m, row_index=idx)
    rng = np.random.default_rng(7)
    sel = np.unique(np.concatenate([[0, split - 1, split, m - 2, m - 1],
                                    rng.integers(0, m, 24)])).astype(np.int64)
    idx_sel = idx[torch.from_numpy(sel).to("cuda")].cpu().numpy()
    sel_off = np.array([0, int(np.sum(sel < split)), len(sel)], np.int32)
    R, ref = orc.grouped_gemm(a_q, a_sf, a_scale, w_q, w_sf, w_scale, sel_off, a_row_index=idx_sel)
    _check(bf16_bits_of(out[torch.from_numpy(sel).to("cuda")]), R, ref, "m_total at its limit")
    del out, idx
