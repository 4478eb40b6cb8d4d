"""A whole Mixture-of-Experts FFN from the library's entry points, against the
oracle's chain of the same steps:

  gate+up   moe_grouped_gemm_fp4_swiglu   (oracle: grouped_gemm, swiglu_quantize)
  down      moe_grouped_gemm_fp4 on the NVFP4 intermediate, routed rows in order
                                          (oracle: grouped_gemm on its own intermediate)
  finalize  moe_fp4_combine, BF16 tokens  (oracle: combine)

The gate+up inputs are built so that every FP32 sum is exact (block scales in
{0.5, 1, 2}, power-of-two tensor scales), so the kernel's intermediate must equal
the oracle's except where the FP32 SiLU lands within a few ulps of an encoding
boundary (at most 2 elements, as in the SwiGLU tests).  The down projection then
reads identical codes; each token's output is checked with the two-pass finalize
bar (per routed term: the down GEMM's BF16 rows, then the BF16 sum).  Tokens fed
by a routed row whose intermediate differs are excluded from that check and
counted."""
import numpy as np
import pytest
import torch

from gpu_util import dev, require_gpu, say
from oracle import oracle as orc
from workloads import configs, gen

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _layer(T, E, topk, hidden, inter, seed, routing=None):
    """Seeded layer inputs; routing = (row_token, offsets) replaces the random top-k."""
    rng = np.random.default_rng(seed)
    if routing is None:
        pairs = sorted((int(e), t) for t in range(T) for e in rng.choice(E, topk, replace=False))
        row_token = np.array([t for _, t in pairs], np.int32)
        counts = np.bincount([e for e, _ in pairs], minlength=E)
        off = np.zeros(E + 1, np.int32)
        off[1:] = np.cumsum(counts)
    else:
        row_token, off = routing
    exact = lambda c: (0x30 + 8 * (c % 3)).astype(np.uint8)  # E4M3 0.5, 1, 2
    # Gate+up pre-activations of standard deviation about 2 (see test_gpu_swiglu).
    s13 = 2.0 ** np.round(np.log2(2.0 / (18.0 * np.sqrt(hidden)) * rng.uniform(0.5, 2.0, E)))
    return dict(
        T=T, topk=topk, row_token=row_token, offsets=off, m_total=int(off[-1]),
        a_q=gen.random_fp4_bytes((T, hidden // 2), seed + 1),
        a_sf=exact(gen.random_e4m3_codes((T, hidden // 16), seed + 2)), a_scale=np.float32(1.0),
        w13_q=gen.random_fp4_bytes((E, 2 * inter, hidden // 2), seed + 3),
        w13_sf=exact(gen.random_e4m3_codes((E, 2 * inter, hidden // 16), seed + 4)),
        w13_scale=s13.astype(np.float32),
        w2_q=gen.random_fp4_bytes((E, hidden, inter // 2), seed + 5),
        w2_sf=gen.random_e4m3_codes((E, hidden, inter // 16), seed + 6, 0x30, 0x40),
        w2_scale=rng.uniform(0.01, 0.04, E).astype(np.float32),
        weight=rng.uniform(0.0, 1.0, int(off[-1])).astype(np.float32))


def _token_map(L):
    """token_rows [T][topk] (routed rows of each token, in row order) and their weights."""
    T, k = L["T"], L["topk"]
    rows = np.full((T, k), -1, np.int32)
    fill = np.zeros(T, np.int64)
    for r, t in enumerate(L["row_token"]):
        rows[t, fill[t]] = r
        fill[t] += 1
    return rows, np.where(rows >= 0, L["weight"][np.maximum(rows, 0)], 0.0).astype(np.float32)


def _gpu_layer(L, g2, packed):
    from block_scaled_fp4_05_amd import moe_fp4
    w13 = dev(L["w13_q"])
    w2 = dev(L["w2_q"])
    if packed:
        w13, w2 = moe_fp4.pack_weights(w13), moe_fp4.pack_weights(w2)
    off = dev(L["offsets"])
    g = dev(np.array([g2], np.float32))
    h_q, h_sf = moe_fp4.grouped_gemm_swiglu(
        dev(L["a_q"]), dev(L["a_sf"]), dev(np.array([L["a_scale"]], np.float32)), w13,
        dev(L["w13_sf"]), dev(L["w13_scale"]), off, g, a_row_index=dev(L["row_token"]),
        m_total=L["m_total"], packed=packed)
    rows = moe_fp4.grouped_gemm(h_q, h_sf, g, w2, dev(L["w2_sf"]), dev(L["w2_scale"]), off,
                                m_total=L["m_total"], packed=packed)
    tr, tw = _token_map(L)
    out = moe_fp4.combine(rows, dev(tr), dev(tw))
    torch.cuda.synchronize()
    return h_q.cpu().numpy(), h_sf.cpu().numpy(), out.float().cpu().numpy()


def _check(L, packed, label):
    T = L["T"]
    R1 = orc.grouped_gemm(L["a_q"], L["a_sf"], L["a_scale"], L["w13_q"], L["w13_sf"],
                          L["w13_scale"], L["offsets"], a_row_index=L["row_token"])[0]
    # The static scale a calibration pass would pick: amax of the FP32 activation / 2688.
    g2 = float(np.float32(np.max(np.abs(orc.swiglu(R1).astype(np.float32))) / np.float32(2688)))
    _, q_ref, sf_ref = orc.swiglu_quantize(R1, g2)
    R2, _ = orc.grouped_gemm(q_ref, sf_ref, np.float32(g2), L["w2_q"], L["w2_sf"], L["w2_scale"],
                             L["offsets"])
    say(f"moe layer {label} T={T} m_total={L['m_total']} packed={packed}")
    h_q, h_sf, got = _gpu_layer(L, g2, packed)
    # Intermediate: equal to the oracle's but for boundary cases of the FP32 SiLU.
    bad_rows = np.nonzero(np.any(h_q != q_ref, axis=1) | np.any(h_sf != sf_ref, axis=1))[0]
    n_bad = int(np.sum(h_q != q_ref)) + int(np.sum(h_sf != sf_ref))
    assert n_bad <= 2, f"{label}: {n_bad} intermediate bytes differ from the oracle's"
    # Output tokens: the two-pass finalize bar, per routed term.
    ref = orc.combine(R2, L["row_token"], L["weight"], T)
    mag = orc.combine(np.linalg.norm(R2, axis=1)[:, None], L["row_token"], L["weight"], T)[:, 0]
    keep = np.ones(T, bool)
    keep[L["row_token"][bad_rows]] = False
    diff = np.linalg.norm(got - ref, axis=1)
    bound = 2e-3 * (mag + np.linalg.norm(ref, axis=1))
    ok = (diff <= bound) | ~keep
    worst = int(np.argmax(np.where(keep, diff / np.maximum(bound, 1e-300), 0)))
    assert np.all(ok), f"{label}: token {worst} diff {diff[worst]:.3g} bound {bound[worst]:.3g}"
    assert np.count_nonzero(~keep) <= 2 * L["topk"]


@pytest.mark.parametrize("packed", [False, True])
def test_moe_layer_small(packed):
    # 96 tokens top-2 over 8 experts, hidden 512, intermediate 256.
    _check(_layer(96, 8, 2, 512, 256, 1200), packed, "small")


def test_moe_layer_empty_and_ragged_experts():
    # 24 tokens top-2 over 40 experts: many empty experts, the rest of 1 to 4 rows.
    _check(_layer(24, 40, 2, 256, 256, 1210), False, "ragged")


def test_moe_layer_decode_shard_full_size():
    """The decode layer shard at full size: 512 tokens top-8 over 256 experts (16 rows
    each), hidden 6144, intermediate 256 (gate+up N = 512, down K = 256), packed
    weights, the routing of the decode gate+up workload."""
    w = configs.WORKLOADS["c3"]
    L = _layer(w.tokens, w.experts, w.topk, w.k, w.n // 2, 1220, routing=configs.routing(w))
    _check(L, True, "decode shard")
