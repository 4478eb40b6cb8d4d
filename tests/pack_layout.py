"""The packed weight-code layout of include/moe_fp4.h, written out in NumPy
from the header's definition (test helper; shares nothing with the kernels).

For one expert with n rows and k elements (kb = k/2 bytes) per row:
  G = 512 if k % 512 == 0 else 256, GB = G/2; rows in groups of 64 (the last
  group holds 16*rg rows); group q starts at byte 64*q*kb; inside it, block
  (granule t, row block j) starts at (t*rg + j) * 8G; inside a block the
  16-byte piece ((2s + h)*4 + g)*16 + r holds row 64q + 16j + r, row-major
  bytes t*GB + (GB/4)*g + 32s + 16h .. +15.
"""
import numpy as np


def source_offsets(n, k):
    """For every 16-byte piece of one packed expert, in packed order, the byte
    offset of the row-major piece it holds."""
    kb = k // 2
    G = 512 if k % 512 == 0 else 256
    GB = G // 2
    S = G // 256
    out = []
    for q in range((n + 63) // 64):
        rg = min(4, n // 16 - 4 * q)
        for t in range(k // G):
            for j in range(rg):
                for s in range(S):
                    for h in range(2):
                        for g in range(4):
                            r = np.arange(16)
                            row = 64 * q + 16 * j + r
                            out.append(row * kb + t * GB + (GB // 4) * g + 32 * s + 16 * h)
    return np.concatenate(out).astype(np.int64)


def pack(w_q):
    """Row-major [E][n][k/2] uint8 -> packed (same shape), per the definition."""
    E, n, kb = w_q.shape
    src = source_offsets(n, 2 * kb)
    flat = w_q.reshape(E, n * kb)
    gather = (src[:, None] + np.arange(16)[None, :]).reshape(-1)
    return flat[:, gather].reshape(E, n, kb)
