"""Host-side inputs and oracle results for the named workloads, built once per
test session.  Activations and weights come from the seeded generators and are
quantised by the ORACLE; nothing here reads a GPU result."""
from __future__ import annotations

import numpy as np

from oracle import oracle as orc
from workloads import configs

_cache: dict = {}


def workload(name: str) -> dict:
    if name in _cache:
        return _cache[name]
    w = configs.WORKLOADS[name]
    row_token, offsets = configs.routing(w)
    x = configs.activations(w)                      # BF16-valued float32 [tokens][K]
    a_q, a_sf, a_scale = orc.quantize(x)            # one row per token, dynamic scale
    E, n, k = w.experts, w.n, w.k
    w_q = np.empty((E, n, k // 2), np.uint8)
    w_sf = np.empty((E, n, k // 16), np.uint8)
    w_scale = np.empty(E, np.float32)
    for e in range(E):
        q, sf, g = orc.quantize(configs.expert_weight(w, e))
        w_q[e], w_sf[e], w_scale[e] = q, sf, g
    d = dict(w=w, row_token=row_token, offsets=offsets, x=x, a_q=a_q, a_sf=a_sf,
             a_scale=a_scale, w_q=w_q, w_sf=w_sf, w_scale=w_scale, m_total=int(offsets[-1]))
    _cache[name] = d
    return d


def sample_rows(offsets: np.ndarray, count: int, seed: int) -> np.ndarray:
    """A spread of output rows: the first and last row of the problem, rows at expert
    boundaries, and random rows."""
    m = int(offsets[-1])
    rng = np.random.default_rng(seed)
    nz = np.nonzero(np.diff(offsets))[0]
    picks = {0, m - 1}
    for e in rng.choice(nz, size=min(len(nz), count // 3), replace=False):
        picks.add(int(offsets[e]))
        picks.add(int(offsets[e + 1]) - 1)
    while len(picks) < count:
        picks.add(int(rng.integers(0, m)))
    return np.array(sorted(picks), dtype=np.int64)


def large_tile_rows(offsets: np.ndarray, seed: int, per_tile: int = 2, min_rows: int = 96) -> np.ndarray:
    """Rows that cover the 256 x 256 workgroup tile of every expert with at least
    `min_rows` rows: `per_tile` rows in each 256-row M-tile, cycling through the 8
    32-row MFMA block positions of the tile's two 128-row wave halves (position
    i = row % 256 // 32), at a random row within the block, plus each such
    expert's first and last row."""
    rng = np.random.default_rng(seed)
    picks = set()
    pos = 0
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi - lo < min_rows:
            continue
        picks.update((lo, hi - 1))
        for t0 in range(lo, hi, 256):
            for _ in range(per_tile):
                block = pos % 8
                pos += 1
                r = t0 + 32 * block + int(rng.integers(0, 32))
                if r < hi:
                    picks.add(r)
    return np.array(sorted(picks), dtype=np.int64)
