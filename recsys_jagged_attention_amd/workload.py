"""Work accounting for jagged attention (host side, counts only).

Useful FLOPs count every (query, key) pair that enters the output once, at
4*D FLOPs per pair per head (2*D for the score dot product, 2*D for the
weighted sum of values); softmax/GELU/normalisation FLOPs and every padded or
masked element are excluded.  Compulsory bytes read each input once and write
the output once.
"""
from __future__ import annotations

import numpy as np

BLOCK = 64


def attended_pairs(lq, lk, window: int = 0, variant: str = "self") -> int:
    """Pairs per head for samples with query lengths lq and key lengths lk
    (sliding: query i of a sample sees min(i + 1, window) keys)."""
    lq = np.asarray(lq, dtype=np.int64)
    lk = np.asarray(lk, dtype=np.int64)
    if variant == "sliding":
        w = int(window)
        n = np.minimum(lq, w)
        return int(np.sum(n * (n + 1) // 2 + (lq - n) * w))
    if window == 0:
        return int(np.sum(lq * lk))
    nb = window // BLOCK
    total = 0
    for L, K in zip(lq.tolist(), lk.tolist()):
        if L == 0 or K == 0:
            continue
        for blk in range((L + BLOCK - 1) // BLOCK):
            rows = min(L, BLOCK * (blk + 1)) - BLOCK * blk
            k0 = BLOCK * max(0, blk - nb + 1)
            k1 = min(K, BLOCK * (blk + 1))
            total += rows * max(0, k1 - k0)
    return total


def useful_flops(lq, lk, H: int, D: int, window: int = 0, variant: str = "self") -> int:
    return 4 * D * H * attended_pairs(lq, lk, window, variant)


def compulsory_bytes(total_q: int, total_kv: int, H: int, D: int, in_bytes: float,
                     out_bytes: int, mx_scales: bool = False) -> int:
    """Q read + K,V read + O written, each once (MX: plus one scale byte per 32 elements)."""
    elems_q = total_q * H * D
    elems_kv = total_kv * H * D
    b = (elems_q + 2 * elems_kv) * in_bytes + elems_q * out_bytes
    if mx_scales:
        b += (elems_q + 2 * elems_kv) // 32
    return int(b)


def padded_dense_flops(lq, lk, H: int, D: int, window: int = 0) -> int:
    """FLOPs of the same attention on a batch padded to the longest sample
    (every sample Lq_max query rows; each row Lk_max keys, or the window's
    keys when there is a window): what a padded dense kernel would spend."""
    lq = np.asarray(lq, dtype=np.int64)
    lk = np.asarray(lk, dtype=np.int64)
    if lq.size == 0:
        return 0
    keys = int(lk.max())
    if window > 0:
        keys = min(keys, int(window))
    return int(4 * D * H * lq.size * int(lq.max()) * keys)
