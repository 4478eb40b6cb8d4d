"""GPU parity of the MoE finalize step against the oracle: the exact per-row GEMM
result (oracle grouped_gemm) combined into token order in FP64 (oracle combine).

Fused epilogue (moe_grouped_gemm_fp4_finalize, FP32 sums): for every token row t,
||gpu[t] - ref[t]||_2 <= 2e-3 * ||ref[t]||_2, and a token with ref = 0 exactly 0 (or
exactly its initial value); its atomic adds run in no fixed order, so the comparison
is by tolerance only.  Two-pass (plain GEMM, then moe_fp4_combine): the per-term bar
of _check_two_pass; the combine alone is also checked on seeded BF16 rows, and for
bit-for-bit repeatability."""
import numpy as np
import pytest
import torch

import wl_data
from gpu_util import TOL, dev, require_gpu, say
from oracle import oracle as orc
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _routed_problem(T, E, topk, n, k, seed, scale_lo=0x20, scale_hi=0x50):
    """T tokens, each routed to topk distinct experts; routed rows sorted by (expert,
    token); activations are per token (gathered through the row index)."""
    rng = np.random.default_rng(seed)
    pairs = sorted((int(e), t) for t in range(T) for e in rng.choice(E, topk, replace=False))
    row_token = np.array([t for _, t in pairs], np.int32)
    counts = np.bincount([e for e, _ in pairs], minlength=E)
    off = np.zeros(E + 1, np.int32)
    off[1:] = np.cumsum(counts)
    return dict(
        a_q=gen.random_fp4_bytes((T, k // 2), seed + 1),
        a_sf=gen.random_e4m3_codes((T, k // 16), seed + 2, scale_lo, scale_hi),
        a_scale=np.float32(rng.uniform(0.25, 4.0)),
        w_q=gen.random_fp4_bytes((E, n, k // 2), seed + 3),
        w_sf=gen.random_e4m3_codes((E, n, k // 16), seed + 4, scale_lo, scale_hi),
        w_scale=rng.uniform(0.25, 4.0, E).astype(np.float32),
        offsets=off, m_total=int(off[-1]), row_token=row_token,
        row_weight=rng.uniform(0.0, 1.0, int(off[-1])).astype(np.float32), T=T)


def _gpu_finalize(P, packed=False, out_token=None, init=None, ldo=None):
    from block_scaled_fp4_05_amd import moe_fp4
    n = P["w_q"].shape[1]
    ldo = n if ldo is None else ldo
    canary = np.float32(-777.0)
    host = np.full((P["T"], ldo), canary, np.float32)
    host[:, :n] = 0.0 if init is None else init
    out = dev(host)
    w_q = dev(P["w_q"])
    if packed:
        w_q = moe_fp4.pack_weights(w_q)
    tok = P["row_token"] if out_token is None else out_token
    moe_fp4.grouped_gemm_finalize(
        dev(P["a_q"]), dev(P["a_sf"]), dev(np.array([P["a_scale"]], np.float32)), w_q,
        dev(P["w_sf"]), dev(P["w_scale"]), dev(P["offsets"]), dev(tok.astype(np.int32)),
        dev(P["row_weight"]), out, a_row_index=dev(P["row_token"]), m_total=P["m_total"],
        packed=packed)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(got[:, n:] == canary), "padding columns were written"
    return got[:, :n]


def _reference(P, out_token=None, init=None):
    R, _ = orc.grouped_gemm(P["a_q"], P["a_sf"], P["a_scale"], P["w_q"], P["w_sf"], P["w_scale"],
                            P["offsets"], a_row_index=P["row_token"])
    tok = P["row_token"] if out_token is None else out_token
    keep = (tok >= 0) & (tok < P["T"])
    return orc.combine(R[keep], tok[keep], P["row_weight"][keep], P["T"], init=init)


def _check_two_pass(got, P, label):
    """Bar for the two-pass finalize (plain GEMM with BF16 rows, then the combine):
    each routed row is rounded to BF16 before the sum and the sum is rounded again,
    so per token t the error is bounded by the rounding of every term plus that of
    the result: ||got[t] - ref[t]|| <= 2e-3 * (sum_s |w_s| ||R_s|| + ||ref[t]||)
    (2e-3 just above the BF16 unit round-off 2^-9).  Where a token's terms partly
    cancel, this is looser than 2e-3 of ||ref[t]||, which the fused FP32 path meets."""
    R, _ = orc.grouped_gemm(P["a_q"], P["a_sf"], P["a_scale"], P["w_q"], P["w_sf"], P["w_scale"],
                            P["offsets"], a_row_index=P["row_token"])
    ref = orc.combine(R, P["row_token"], P["row_weight"], P["T"])
    mag = orc.combine(np.linalg.norm(R, axis=1)[:, None], P["row_token"],
                      np.abs(P["row_weight"]), P["T"])[:, 0]
    diff = np.linalg.norm(np.asarray(got, np.float64) - ref, axis=1)
    bound = 2e-3 * (mag + np.linalg.norm(ref, axis=1))
    worst = int(np.argmax(diff / np.maximum(bound, 1e-300)))
    assert np.all(diff <= bound), f"{label}: token {worst} diff {diff[worst]:.3g} bound {bound[worst]:.3g}"


def _check(got, ref, label):
    err, _ = orc.token_row_error(got, ref)
    worst = int(np.argmax(err)) if err.size else 0
    assert np.all(err <= TOL), f"{label}: token {worst} err {err[worst]:.3g}"
    return float(err.max())


# (T, E, topk, n, k): rows per expert on average 8 / 24 / 32 / 66 / 150 (one, two
# and four row blocks, and experts the plain GEMM would give the workgroup tile),
# 256- and 512-element stages, LDS scale lines (k % 2048 == 0), and last 64-row
# groups of 16 and 48 rows.
CASES = [(32, 8, 2, 64, 256), (48, 6, 3, 80, 512), (64, 4, 2, 128, 2048), (100, 3, 2, 64, 768),
         (300, 2, 1, 112, 512), (40, 5, 4, 208, 6144)]


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_finalize_matches_oracle_combine(case, packed):
    T, E, topk, n, k = CASES[case]
    P = _routed_problem(T, E, topk, n, k, 500 + 10 * case)
    say(f"finalize T={T} E={E} top{topk} n={n} k={k} packed={packed}")
    got = _gpu_finalize(P, packed=packed, ldo=n + 4)
    _check(got, _reference(P), f"case {case}")


def test_finalize_accumulates_onto_initial_values():
    P = _routed_problem(24, 4, 2, 64, 512, 600)
    init = np.random.default_rng(601).standard_normal((24, 64)).astype(np.float32) * 50
    say("finalize onto a residual")
    got = _gpu_finalize(P, init=init)
    _check(got, _reference(P, init=init), "residual")


def test_finalize_drops_rows_of_out_of_range_tokens_and_empty_experts():
    P = _routed_problem(16, 32, 1, 64, 256, 610)  # top-1 over 32 experts: many are empty
    assert np.any(np.diff(P["offsets"]) == 0)
    tok = P["row_token"].copy()
    tok[::3] = P["T"] + 5
    tok[1::7] = -1
    say("finalize with dropped rows")
    got = _gpu_finalize(P, out_token=tok)
    ref = _reference(P, out_token=tok)
    _check(got, ref, "dropped")
    # Tokens that received no row stay exactly zero.
    untouched = np.setdiff1d(np.arange(P["T"]), tok[(tok >= 0) & (tok < P["T"])])
    assert not np.any(got[untouched])


def test_finalize_full_size_down_projection_shard():
    """The 32-rows-per-expert down-projection shard (256 experts, 1024 tokens top-8,
    K=256, N=6144), every token row, with seeded routing weights."""
    d = wl_data.workload("c4")
    rng = np.random.default_rng(620)
    P = dict(a_q=d["a_q"], a_sf=d["a_sf"], a_scale=d["a_scale"], w_q=d["w_q"], w_sf=d["w_sf"],
             w_scale=d["w_scale"], offsets=d["offsets"], m_total=d["m_total"],
             row_token=d["row_token"].astype(np.int32),
             row_weight=rng.uniform(0.0, 1.0, d["m_total"]).astype(np.float32),
             T=int(d["a_q"].shape[0]))
    say("finalize full-size down-projection shard, packed")
    got = _gpu_finalize(P, packed=True)
    worst = _check(got, _reference(P), "down shard")
    say(f"finalize down shard max token error {worst:.3g}")


# ------------------------------------------------------------- combine --

def _token_rows(row_token, T, topk):
    """Each token's routed rows in row order, padded with -1 to topk slots."""
    tr = np.full((T, topk), -1, np.int32)
    fill = np.zeros(T, np.int64)
    for r, t in enumerate(row_token):
        tr[t, fill[t]] = r
        fill[t] += 1
    return tr


def _random_bf16_rows(m, n, seed):
    """Seeded BF16 bit patterns: random sign and mantissa, exponents 2^-8 .. 2^7."""
    rng = np.random.default_rng(seed)
    sign = rng.integers(0, 2, (m, n)).astype(np.uint16) << 15
    exp = rng.integers(119, 135, (m, n)).astype(np.uint16) << 7
    man = rng.integers(0, 128, (m, n)).astype(np.uint16)
    return sign | exp | man


def _combine_reference(rows_f, token_rows, token_weights, T, residual=None):
    tok = np.repeat(np.arange(T), token_rows.shape[1])
    flat = token_rows.reshape(-1)
    keep = (flat >= 0) & (flat < rows_f.shape[0])
    return orc.combine(rows_f[flat[keep]], tok[keep], token_weights.reshape(-1)[keep], T,
                       init=residual)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_combine_matches_oracle_and_is_deterministic(out_dtype):
    from block_scaled_fp4_05_amd import moe_fp4
    m, n, T, topk = 200, 1040, 37, 6  # n spans two 512-column chunks and a ragged third
    rows_bits = _random_bf16_rows(m, n + 16, 630)
    rng = np.random.default_rng(631)
    tr = rng.integers(0, m, (T, topk)).astype(np.int32)
    tr[::4, -1] = -1           # empty slots
    tr[1::9, 0] = m + 3        # out of range: skipped
    tr[5] = -1                 # a token with no rows
    tw = rng.uniform(0.0, 1.0, (T, topk)).astype(np.float32)
    rows = dev(rows_bits.view(np.int16)).view(torch.bfloat16)[:, :n]
    say(f"combine {m}x{n} T={T} top{topk} -> {out_dtype}")
    out1 = moe_fp4.combine(rows, dev(tr), dev(tw), out_dtype=out_dtype)
    out2 = moe_fp4.combine(rows, dev(tr), dev(tw), out_dtype=out_dtype)
    torch.cuda.synchronize()
    a = out1.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32).cpu().numpy()
    b = out2.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32).cpu().numpy()
    assert np.array_equal(a, b), "combine is not deterministic"
    rows_f = orc.bf16_bits_to_float(rows_bits[:, :n]).astype(np.float64)
    ref = _combine_reference(rows_f, tr, tw, T)
    got = out1.float().cpu().numpy()
    err, _ = orc.token_row_error(got, ref)
    assert np.all(err <= (2e-3 if out_dtype == torch.bfloat16 else 1e-5)), err.max()
    assert not np.any(got[5])


def test_combine_adds_a_residual_in_place():
    from block_scaled_fp4_05_amd import moe_fp4
    m, n, T, topk = 64, 128, 16, 3
    rows_bits = _random_bf16_rows(m, n, 640)
    rng = np.random.default_rng(641)
    tr = rng.integers(0, m, (T, topk)).astype(np.int32)
    tw = rng.uniform(0.0, 1.0, (T, topk)).astype(np.float32)
    res = rng.standard_normal((T, n)).astype(np.float32) * 10
    buf = dev(res)
    rows = dev(rows_bits.view(np.int16)).view(torch.bfloat16)
    say("combine onto a residual, in place")
    moe_fp4.combine(rows, dev(tr), dev(tw), out=buf, residual=buf)
    torch.cuda.synchronize()
    ref = _combine_reference(orc.bf16_bits_to_float(rows_bits).astype(np.float64), tr, tw, T,
                             residual=res)
    err, _ = orc.token_row_error(buf.cpu().numpy(), ref)
    assert np.all(err <= 1e-5), err.max()


@pytest.mark.parametrize("packed", [False, True])
def test_gemm_then_combine_chain_matches_oracle(packed):
    """Plain grouped GEMM (BF16 rows) followed by the combine, against the oracle's
    exact rows combined in FP64."""
    from block_scaled_fp4_05_amd import moe_fp4
    T, E, topk, n, k = 60, 6, 3, 208, 512
    P = _routed_problem(T, E, topk, n, k, 650)
    w_q = dev(P["w_q"])
    if packed:
        w_q = moe_fp4.pack_weights(w_q)
    say(f"gemm + combine chain packed={packed}")
    rows = moe_fp4.grouped_gemm(dev(P["a_q"]), dev(P["a_sf"]), dev(np.array([P["a_scale"]], np.float32)),
                                w_q, dev(P["w_sf"]), dev(P["w_scale"]), dev(P["offsets"]),
                                a_row_index=dev(P["row_token"]), m_total=P["m_total"], packed=packed)
    tr = _token_rows(P["row_token"], T, topk)
    tw = np.zeros((T, topk), np.float32)
    for t in range(T):
        for s in range(topk):
            if tr[t, s] >= 0:
                tw[t, s] = P["row_weight"][tr[t, s]]
    got = moe_fp4.combine(rows, dev(tr), dev(tw), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    _check_two_pass(got.float().cpu().numpy(), P, "chain")


def test_gemm_then_combine_full_size_down_projection_shard():
    from block_scaled_fp4_05_amd import moe_fp4
    d = wl_data.workload("c4")
    rng = np.random.default_rng(660)
    T = int(d["a_q"].shape[0])
    P = dict(a_q=d["a_q"], a_sf=d["a_sf"], a_scale=d["a_scale"], w_q=d["w_q"], w_sf=d["w_sf"],
             w_scale=d["w_scale"], offsets=d["offsets"], m_total=d["m_total"],
             row_token=d["row_token"].astype(np.int32),
             row_weight=rng.uniform(0.0, 1.0, d["m_total"]).astype(np.float32), T=T)
    say("gemm + combine, full-size down-projection shard")
    rows = moe_fp4.grouped_gemm(dev(P["a_q"]), dev(P["a_sf"]), dev(np.array([P["a_scale"]], np.float32)),
                                moe_fp4.pack_weights(dev(P["w_q"])), dev(P["w_sf"]), dev(P["w_scale"]),
                                dev(P["offsets"]), a_row_index=dev(P["row_token"]),
                                m_total=P["m_total"], packed=True)
    tr = _token_rows(P["row_token"], T, 8)
    tw = np.where(tr >= 0, P["row_weight"][np.maximum(tr, 0)], 0).astype(np.float32)
    got = moe_fp4.combine(rows, dev(tr), dev(tw), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    _check_two_pass(got.float().cpu().numpy(), P, "down shard chain")
