"""Host-side checks of the C-ABI library: it loads, exports every declared symbol,
and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

from conftest import ROOT, read_golden

HEADER = os.path.join(ROOT, "include", "moe_fp4.h")


def _lib():
    from block_scaled_fp4_05_amd import moe_fp4
    return moe_fp4


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    m = _lib()
    names = _declared()
    assert set(names) == set(m.EXPORTED), names
    L = m.lib()
    for nm in names:
        assert hasattr(L, nm), nm


def test_status_strings_cover_every_code():
    m = _lib()
    seen = set()
    for code in range(7):
        s = m.status_string(code)
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == 7
    assert m.status_string(99) == "unknown status"


def test_stage_bytes_matches_the_per_stage_transaction_formula():
    m = _lib()
    for bm, bn, bk, want in read_golden("stage_bytes.txt"):
        assert m.stage_bytes(int(bm), int(bn), int(bk)) == int(want)
    assert m.stage_bytes(0, 16, 16) == -1 and m.stage_bytes(16, 16, 8) == -1


def test_workspace_size_is_zero():
    """The work list lives in LDS: no entry point needs a workspace, for any sizes."""
    m = _lib()
    for args in [(256, 4096, 512, 6144), (1, 8192, 8192, 8192), (8192, 0, 16, 256), (0, -1, 0, 0)]:
        assert m.workspace_size(*args) == 0


def _log_of_empty_call(monkeypatch, capfd, tile, ldo, E=1, n=1024, k=8192):
    """Tile line MOE_FP4_LOG prints for a GEMM call with m_total = 0 (validated,
    logged, nothing launched: fake aligned pointers never reach the GPU)."""
    m = _lib()
    monkeypatch.setenv("MOE_FP4_LOG", "1")
    if tile:
        monkeypatch.setenv("MOE_FP4_TILE", tile)
    else:
        monkeypatch.delenv("MOE_FP4_TILE", raising=False)
    fake = ctypes.c_void_p(1 << 20)
    st = m.gemm_raw(fake, fake, fake, 1, None, fake, fake, fake, fake, E, 0, n, k, fake, ldo, None)
    assert st == 0
    return capfd.readouterr().err


def test_log_prints_the_chosen_tile_and_the_output_range_fallback(monkeypatch, capfd):
    """MOE_FP4_LOG names the tile; a 256-row workgroup tile whose output rows would
    span 2^31 - 4096 bytes or more gives way to 64-row per-wave items."""
    err = _log_of_empty_call(monkeypatch, capfd, "256x256!", 4096)
    assert "256x256 workgroup tile for every expert" in err, err
    # 256 rows of ldo BF16 values: 2^31 - 4096 - 4096 bytes, and exactly 2^31 - 4096.
    err = _log_of_empty_call(monkeypatch, capfd, "256x256!", (2 ** 31 - 4096) // 512 - 8)
    assert "256x256 workgroup tile for every expert" in err, err
    err = _log_of_empty_call(monkeypatch, capfd, "256x256!", (2 ** 31 - 4096) // 512)
    assert "per-wave items" in err and "tile 64x64" in err, err
    err = _log_of_empty_call(monkeypatch, capfd, "128x128", 2 ** 23 - 24)
    assert "128x128 workgroup tile" in err, err
    err = _log_of_empty_call(monkeypatch, capfd, "128x128", 2 ** 23 - 16)
    assert "per-wave items" in err and "tile 64x64" in err, err
    err = _log_of_empty_call(monkeypatch, capfd, "128x128", 2 ** 23)
    assert "per-wave items" in err and "tile 64x64" in err, err
    # Unset or "0": silent.
    monkeypatch.setenv("MOE_FP4_LOG", "0")
    fake = ctypes.c_void_p(1 << 20)
    assert _lib().gemm_raw(fake, fake, fake, 1, None, fake, fake, fake, fake, 2, 0, 64, 256, fake,
                           64, None) == 0
    assert capfd.readouterr().err == ""


def test_log_keeps_the_48_row_items_at_the_largest_ldo(monkeypatch, capfd):
    """48 rows of 2^23 BF16 values stay below 2^31 - 4096 bytes, so the 48 x 512 items
    run at every accepted ldo (test_gpu_limits checks their output there); with K not a
    multiple of 512 the request falls back to the default choice."""
    err = _log_of_empty_call(monkeypatch, capfd, "48x512", 2 ** 23, E=3, n=272, k=512)
    assert "48x512 workgroup items for every expert" in err, err
    err = _log_of_empty_call(monkeypatch, capfd, "48x512", 2 ** 23, E=3, n=272, k=256)
    assert "48x512" not in err, err


def test_plan_picks_tiles_by_rows_per_expert(monkeypatch):
    m = _lib()
    monkeypatch.delenv("MOE_FP4_TILE", raising=False)
    assert m.plan(256, 4096, 512, 6144)["tile_m"] == 16
    assert m.plan(256, 8192, 6144, 256)["tile_m"] == 32
    assert m.plan(1, 8192, 8192, 8192)["tile_m"] == 256   # compute-bound: large workgroup tile
    assert m.plan(256, 32768, 512, 6144)["tile_m"] == 256  # large experts in 256-row items
    assert m.plan(256, 16384, 512, 6144)["tile_m"] == 64
    monkeypatch.setenv("MOE_FP4_TILE", "64x32")
    p = m.plan(256, 4096, 512, 6144)
    assert (p["tile_m"], p["tile_n"]) == (64, 32)
    monkeypatch.setenv("MOE_FP4_TILE", "128x128")
    p = m.plan(256, 4096, 512, 6144)
    assert (p["tile_m"], p["tile_n"], p["k_step"]) == (128, 128, 64)
    monkeypatch.setenv("MOE_FP4_TILE", "256x256")
    p = m.plan(256, 4096, 512, 6144)
    assert (p["tile_m"], p["tile_n"], p["k_step"], p["lds_bytes"]) == (256, 256, 64, 2064 + 131072 + 16)
    # The large tile needs 128 KB of stages beside the work list: too many experts
    # to fit it keep the default choice.
    assert m.plan(8192, 512 * 8192, 512, 6144)["tile_m"] == 128
    monkeypatch.setenv("MOE_FP4_TILE", "48x64")  # unsupported -> ignored
    assert m.plan(256, 4096, 512, 6144)["tile_m"] == 16
    monkeypatch.setenv("MOE_FP4_TILE", "48x512")
    p = m.plan(256, 4096, 512, 6144)
    assert (p["tile_m"], p["tile_n"], p["k_step"], p["waves_per_group"]) == (48, 512, 256, 8)
    assert p["lds_bytes"] == 2064 + 2 * 48 * 528 + 8 * (2 * 4096 + 1024) + 16
    assert m.plan(256, 4096, 512, 6400)["tile_m"] == 16  # K not a multiple of 512 -> default
    for split in ("256x256m", "256x256mp"):
        monkeypatch.setenv("MOE_FP4_TILE", split)
        assert m.plan(256, 4096, 512, 6144)["tile_m"] == 256
    monkeypatch.setenv("MOE_FP4_TILE", "48x512p")
    assert m.plan(256, 4096, 512, 6144)["k_step"] == 256


@pytest.mark.parametrize("args,status", [
    ((0, 4096, 512, 6144), 2), ((256, -1, 512, 6144), 2), ((256, 16, 0, 6144), 2),
    ((256, 16, 24, 6144), 4), ((256, 16, 512, 6000), 4), ((256, 16, 512, 128), 4),
])
def test_plan_rejects(args, status):
    m = _lib()
    with pytest.raises(m.MoeFp4Error) as ei:
        m.plan(*args)
    assert ei.value.status == status


# Negative calls with pointer-sized integers that are never dereferenced: every
# case fails validation on the host.  Skipped where a GPU is present so that a
# validation bug could never turn into a launch on fake pointers.
needs_no_gpu = pytest.mark.skipif(
    __import__("torch").cuda.is_available(), reason="fake-pointer negative tests run on CPU only")

P16 = 0x10000  # 16-byte aligned fake address


def _q(**kw):
    a = dict(x=P16, dt=0, rows=4, k=64, ld=64, q=2 * P16, sf=3 * P16, ts=4 * P16, mode=1,
             stream=None)
    a.update(kw)
    return _lib().quantize_raw(a["x"], a["dt"], a["rows"], a["k"], a["ld"], a["q"], a["sf"],
                               a["ts"], a["mode"], a["stream"])


@needs_no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(dt=7), 6), (dict(mode=2), 6), (dict(ts=None), 1), (dict(x=None), 1), (dict(q=None), 1),
    (dict(sf=None), 1), (dict(rows=-1), 2), (dict(k=0), 2), (dict(k=24), 2), (dict(ld=32), 2),
    (dict(x=P16 + 8), 3), (dict(ld=68), 3), (dict(q=P16 + 4), 3), (dict(ts=P16 + 2), 3),
    (dict(dt=1, ld=66), 3), (dict(dt=1, ld=60), 2), (dict(dt=1, ld=65, k=48), 3),
    # overlapping buffers (x spans 4 rows x 128 bytes, q 128 bytes, sf 16 bytes)
    (dict(q=P16 + 504), 6), (dict(sf=P16 + 511), 6), (dict(ts=P16 + 508), 6),
    (dict(sf=2 * P16 + 120), 6), (dict(ts=2 * P16 + 124), 6), (dict(ts=3 * P16 + 12), 6),
    (dict(sf=P16, mode=0), 6),
    # an input extent beyond int64
    (dict(rows=1 << 20, ld=1 << 50), 2),
])
def test_quantize_rejects(kw, status):
    assert _q(**kw) == status


def _g(**kw):
    a = dict(a_q=P16, a_sf=P16, a_scale=P16, a_rows=64, idx=None, w_q=P16, w_sf=P16, w_scale=P16,
             off=P16, E=4, m=64, n=64, k=256, out=P16, ldo=64, stream=None)
    a.update(kw)
    return _lib().gemm_raw(a["a_q"], a["a_sf"], a["a_scale"], a["a_rows"], a["idx"], a["w_q"],
                           a["w_sf"], a["w_scale"], a["off"], a["E"], a["m"], a["n"], a["k"],
                           a["out"], a["ldo"], a["stream"])


@needs_no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(a_q=None), 1), (dict(a_sf=None), 1), (dict(a_scale=None), 1), (dict(w_q=None), 1),
    (dict(w_sf=None), 1), (dict(w_scale=None), 1), (dict(off=None), 1), (dict(out=None), 1),
    (dict(E=0), 2), (dict(m=-1), 2), (dict(n=0), 2), (dict(k=0), 2), (dict(ldo=32), 2),
    (dict(a_rows=63), 2), (dict(a_rows=0, idx=P16), 2), (dict(a_rows=-1), 2),
    (dict(n=24, ldo=24), 4), (dict(k=128), 4), (dict(k=320), 4), (dict(E=20000), 4), (dict(E=8193), 4),
    (dict(a_q=P16 + 8), 3), (dict(w_sf=P16 + 4), 3), (dict(out=P16 + 8), 3), (dict(ldo=68), 3),
    (dict(off=P16 + 2), 3), (dict(idx=P16 + 2), 3), (dict(a_scale=P16 + 1), 3),
    # sizes whose products would not fit in 64 bits are refused, not overflowed
    (dict(k=1 << 60), 4), (dict(a_rows=1 << 62), 4), (dict(a_rows=1 << 62, idx=P16), 4),
])
def test_gemm_rejects(kw, status):
    assert _g(**kw) == status


@needs_no_gpu
def test_gemm_empty_problem_is_a_noop():
    assert _g(m=0, a_rows=0) == 0


def _gp(**kw):
    a = dict(a_q=P16, a_sf=P16, a_scale=P16, a_rows=64, idx=None, w_q=P16, w_sf=P16, w_scale=P16,
             off=P16, E=4, m=64, n=64, k=512, out=P16, ldo=64, stream=None)
    a.update(kw)
    return _lib().gemm_packed_raw(a["a_q"], a["a_sf"], a["a_scale"], a["a_rows"], a["idx"], a["w_q"],
                                  a["w_sf"], a["w_scale"], a["off"], a["E"], a["m"], a["n"], a["k"],
                                  a["out"], a["ldo"], a["stream"])


@needs_no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(w_q=None), 1), (dict(out=None), 1), (dict(E=0), 2), (dict(n=0), 2), (dict(ldo=32), 2),
    (dict(n=24, ldo=24), 4), (dict(k=320), 4), (dict(w_q=P16 + 8), 3),
])
def test_packed_gemm_rejects(kw, status):
    assert _gp(**kw) == status


@needs_no_gpu
@pytest.mark.parametrize("tile", ["16x32", "16x64x256", "32x32x512"])
def test_packed_gemm_rejects_tiles_the_layout_cannot_feed(tile, monkeypatch):
    # k = 512: the packed granule is 512 elements and items are 64 columns wide.
    monkeypatch.setenv("MOE_FP4_TILE", tile)
    assert _gp() == 4


def _rp(fn, **kw):
    a = dict(src=P16, dst=P16 * 64, E=2, n=64, k=512, stream=None)
    a.update(kw)
    return getattr(_lib().lib(), fn)(a["src"], a["dst"], a["E"], a["n"], a["k"], a["stream"])


@needs_no_gpu
@pytest.mark.parametrize("fn", ["moe_fp4_pack_weights", "moe_fp4_unpack_weights"])
@pytest.mark.parametrize("kw,status", [
    (dict(src=None), 1), (dict(dst=None), 1), (dict(E=0), 2), (dict(n=0), 2), (dict(k=0), 2),
    (dict(n=24), 4), (dict(k=320), 4), (dict(src=P16 + 8), 3), (dict(dst=P16 * 64 + 4), 3),
    (dict(dst=P16 + 16), 6),
])
def test_repack_rejects(fn, kw, status):
    assert _rp(fn, **kw) == status


@pytest.mark.parametrize("n,k", [(16, 256), (48, 256), (64, 512), (80, 768), (144, 1024),
                                 (112, 2048), (64, 6144)])
def test_packed_layout_definition_is_a_group_preserving_permutation(n, k):
    import pack_layout
    kb = k // 2
    src = pack_layout.source_offsets(n, k)
    assert src.size * 16 == n * kb
    assert np.array_equal(np.sort(src), np.arange(0, n * kb, 16))
    # Every 64-row group keeps its byte range: packed offset and source share the group.
    dst = np.arange(src.size) * 16
    assert np.array_equal(dst // (64 * kb), src // (64 * kb))
    # One packed 1 KB run is one load instruction: 16 rows x 4 lane groups, same K piece.
    G = 512 if k % 512 == 0 else 256
    first = src[:64]
    assert np.array_equal(first[:16] // kb, np.arange(16))
    assert np.array_equal(first[16:32] - first[:16], np.full(16, G // 8))


def _gf(**kw):
    a = dict(a_q=P16, a_sf=P16, a_scale=P16, a_rows=64, idx=None, w_q=P16, w_sf=P16, w_scale=P16,
             pk=0, off=P16, E=4, m=64, n=64, k=512, tok=P16, wt=P16, out=P16, ldo=64, T=32,
             stream=None)
    a.update(kw)
    return _lib().finalize_raw(a["a_q"], a["a_sf"], a["a_scale"], a["a_rows"], a["idx"], a["w_q"],
                               a["w_sf"], a["w_scale"], a["pk"], a["off"], a["E"], a["m"], a["n"],
                               a["k"], a["tok"], a["wt"], a["out"], a["ldo"], a["T"], a["stream"])


@needs_no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(tok=None), 1), (dict(wt=None), 1), (dict(out=None), 1), (dict(w_q=None), 1),
    (dict(pk=2), 6), (dict(T=0), 2), (dict(ldo=32), 2), (dict(E=0), 2), (dict(n=24, ldo=24), 4),
    (dict(k=320), 4), (dict(out=P16 + 2), 3), (dict(tok=P16 + 2), 3), (dict(wt=P16 + 1), 3),
    (dict(T=1 << 24, ldo=64), 4), (dict(ldo=1 << 61), 4), (dict(a_rows=1 << 62), 4),
])
def test_finalize_rejects(kw, status):
    assert _gf(**kw) == status


@needs_no_gpu
def test_finalize_empty_problem_is_a_noop():
    assert _gf(m=0, a_rows=0) == 0


@needs_no_gpu
@pytest.mark.parametrize("tile,pk", [("16x32", 0), ("32x32x1024", 0), ("16x64x256", 1)])
def test_finalize_rejects_tiles_it_does_not_run(tile, pk, monkeypatch):
    # k = 1024: 32-column items and 1024-element stages are not run by the finalize
    # epilogue; packed weights (512-element granule) need 512-element stages.
    monkeypatch.setenv("MOE_FP4_TILE", tile)
    assert _gf(k=1024, pk=pk) == 4


H_Q, H_SF = 0x4000000, 0x8000000  # fake output addresses clear of the inputs at P16


def _gs(**kw):
    a = dict(a_q=P16, a_sf=P16, a_scale=P16, a_rows=64, idx=None, w_q=P16, w_sf=P16, w_scale=P16,
             pk=0, off=P16, E=4, m=64, n=128, k=512, hs=P16, hq=H_Q, hsf=H_SF, stream=None)
    a.update(kw)
    return _lib().swiglu_raw(a["a_q"], a["a_sf"], a["a_scale"], a["a_rows"], a["idx"], a["w_q"],
                             a["w_sf"], a["w_scale"], a["pk"], a["off"], a["E"], a["m"], a["n"],
                             a["k"], a["hs"], a["hq"], a["hsf"], a["stream"])


@needs_no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(hs=None), 1), (dict(hq=None), 1), (dict(hsf=None), 1), (dict(w_q=None), 1),
    (dict(off=None), 1), (dict(pk=2), 6), (dict(E=0), 2), (dict(m=-1), 2), (dict(a_rows=32), 2),
    (dict(n=48), 4), (dict(n=16), 4), (dict(pk=1, n=64), 4), (dict(pk=1, n=160), 4), (dict(k=320), 4),
    (dict(hq=H_Q + 4), 3), (dict(hsf=H_SF + 2), 3), (dict(hs=P16 + 2), 3), (dict(a_q=P16 + 8), 3),
    (dict(hq=P16), 6), (dict(hsf=P16 + 64), 6), (dict(hsf=H_Q + 512), 6),
])
def test_swiglu_rejects(kw, status):
    assert _gs(**kw) == status


@needs_no_gpu
def test_swiglu_empty_problem_is_a_noop():
    assert _gs(m=0, a_rows=0) == 0


@needs_no_gpu
@pytest.mark.parametrize("tile,pk", [("16x32", 0), ("32x32x1024", 0), ("16x64x256", 1)])
def test_swiglu_rejects_tiles_it_does_not_run(tile, pk, monkeypatch):
    # As for the finalize epilogue: 4 row blocks per item, stages of 256 or 512
    # elements, and packed weights need their granule as the stage.
    monkeypatch.setenv("MOE_FP4_TILE", tile)
    assert _gs(k=1024, pk=pk) == 4


def _cb(**kw):
    a = dict(rows=P16, ld_rows=64, m=64, tok=P16, wt=P16, topk=2, T=32, n=64, res=None, ld_res=0,
             out=P16, dt=0, ldo=64, stream=None)
    a.update(kw)
    return _lib().combine_raw(a["rows"], a["ld_rows"], a["m"], a["tok"], a["wt"], a["topk"], a["T"],
                              a["n"], a["res"], a["ld_res"], a["out"], a["dt"], a["ldo"], a["stream"])


@needs_no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(dt=2), 6), (dict(rows=None), 1), (dict(tok=None), 1), (dict(wt=None), 1),
    (dict(out=None), 1), (dict(topk=0), 2), (dict(T=-1), 2), (dict(n=0), 2), (dict(ldo=32), 2),
    (dict(ld_rows=32), 2), (dict(res=P16, ld_res=32), 2), (dict(m=-1), 2),
    (dict(rows=P16 + 8), 3), (dict(ld_rows=68), 3), (dict(out=P16 + 4), 3), (dict(ldo=68), 3),
    (dict(dt=1, ldo=66), 3), (dict(tok=P16 + 2), 3), (dict(res=P16 + 8, ld_res=64), 3),
    (dict(res=P16, ld_res=66), 3), (dict(n=24, ld_rows=32, ldo=32), 4),
    (dict(T=1 << 26, ldo=64), 4),
])
def test_combine_rejects(kw, status):
    assert _cb(**kw) == status


@needs_no_gpu
def test_combine_without_tokens_is_a_noop():
    assert _cb(T=0) == 0
