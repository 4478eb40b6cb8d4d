"""Seeded generators: Gaussian matrices, random packed codes, MoE routing tables.

Nothing here quantises, decodes or multiplies: these are the raw inputs that
both the oracle and the HIP library consume.  All randomness comes from numpy's
PCG64 (``numpy.random.default_rng``) so a seed fixes every value on any machine.
"""
from __future__ import annotations

import numpy as np


def rng(seed) -> np.random.Generator:
    return np.random.default_rng(seed)


def normal(shape, seed) -> np.ndarray:
    """Standard normal float32 values."""
    return rng(seed).standard_normal(shape, dtype=np.float32)


def expert_weight(e: int, n: int, k: int, seed: int) -> np.ndarray:
    """Float32 N(0,1) weight matrix [n][k] of expert e; each expert has its own
    stream (seed, e) so any subset of experts can be regenerated on its own."""
    return rng([seed, e]).standard_normal((n, k), dtype=np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 with torch's conversion (round to nearest
    even) and widen them back to float32, so the same values can feed a BF16 input
    on the GPU and a float32 input on the CPU."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def bf16_bits(x_bf16_valued: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bfloat16-representable."""
    u = np.ascontiguousarray(x_bf16_valued, dtype=np.float32).view(np.uint32)
    return (u >> 16).astype(np.uint16)


def random_fp4_bytes(shape, seed) -> np.ndarray:
    """Uniformly random packed bytes (every 4-bit code equally likely)."""
    return rng(seed).integers(0, 256, size=shape, dtype=np.uint8)


def random_e4m3_codes(shape, seed, lo: int = 0x00, hi: int = 0x7E) -> np.ndarray:
    """Random non-negative, non-NaN E4M3 codes in [lo, hi]."""
    if not (0 <= lo <= hi <= 0x7E):
        raise ValueError("code range must lie in [0x00, 0x7E]")
    return rng(seed).integers(lo, hi + 1, size=shape, dtype=np.uint8)


# ------------------------------------------------------------------ routing --

def route_uniform_topk(tokens: int, experts: int, topk: int, seed) -> np.ndarray:
    """Each token picks `topk` distinct experts uniformly at random -> int32 [tokens][topk]."""
    g = rng(seed)
    out = np.empty((tokens, topk), dtype=np.int32)
    for t in range(tokens):
        out[t] = g.choice(experts, size=topk, replace=False)
    return out


def route_balanced(tokens: int, experts: int, topk: int, seed) -> np.ndarray:
    """Token t goes to experts (topk*t + j) mod E, j < topk, relabelled by a seeded
    permutation: when tokens*topk is a multiple of E every expert gets exactly
    tokens*topk/E rows (the decode shapes with a fixed number of tokens per expert)."""
    perm = rng(seed).permutation(experts).astype(np.int32)
    t = np.arange(tokens, dtype=np.int64)[:, None]
    j = np.arange(topk, dtype=np.int64)[None, :]
    return perm[(topk * t + j) % experts]


def zipf_probs(experts: int, s: float, seed) -> np.ndarray:
    """Expert popularity p ~ rank^-s over ranks 1..E, ranks mapped to experts by a
    seeded permutation."""
    ranks = np.arange(1, experts + 1, dtype=np.float64)
    p_rank = ranks ** (-s)
    p_rank /= p_rank.sum()
    perm = rng([seed, 1]).permutation(experts)
    p = np.empty(experts, dtype=np.float64)
    p[perm] = p_rank
    return p


def route_zipf_topk(tokens: int, experts: int, topk: int, s: float, seed) -> np.ndarray:
    """Each token draws `topk` distinct experts from the Zipf popularity without
    replacement (Gumbel-top-k on log p)."""
    p = zipf_probs(experts, s, seed)
    gum = rng([seed, 2]).gumbel(size=(tokens, experts))
    keys = np.log(p)[None, :] + gum
    idx = np.argpartition(-keys, topk - 1, axis=1)[:, :topk]
    return idx.astype(np.int32)


def route_zipf_iid(rows: int, experts: int, s: float, seed) -> np.ndarray:
    """`rows` routed rows, each drawn i.i.d. from the Zipf popularity -> int32 [rows][1]."""
    p = zipf_probs(experts, s, seed)
    return rng([seed, 3]).choice(experts, size=(rows, 1), p=p).astype(np.int32)


def group_by_expert(assign: np.ndarray, experts: int):
    """Sort the (token, expert) pairs of a routing table by (expert, token).

    Returns (row_token int32[m_total], offsets int32[E+1]): row r of the grouped
    problem is token row_token[r], and expert e owns rows [offsets[e], offsets[e+1]).
    """
    tokens, topk = assign.shape
    tok = np.repeat(np.arange(tokens, dtype=np.int64), topk)
    exp = assign.reshape(-1).astype(np.int64)
    order = np.lexsort((tok, exp))
    row_token = tok[order].astype(np.int32)
    counts = np.bincount(exp, minlength=experts)
    offsets = np.zeros(experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return row_token, offsets
