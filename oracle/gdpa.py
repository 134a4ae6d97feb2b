"""Jagged generalized dot-product attention, forward, in float64 (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring for the page names).

What is computed -- the plain definition, sample by sample and head by head:

  Jagged inputs: values [sum(L), H, D] + int32 offsets [B+1]; no padding to the
  maximum length ([GEM-T] "なぜLLM向けのインフラをそのまま使えないのか": padding wastes
  up to half the compute; [GEM-R] "効率向上はモデルとシステムの協調設計から生まれた").

  Three shapes share one definition ([GEM-T] same section: self-attention over
  long histories with a short window, cross-attention with long queries and short
  K/V, PMA with short queries and long K/V; [GEM-T] "Generalized Dot-Product
  Attention（GDPA）": one kernel for all three).

  For sample b and head h, with Q (Lq x D), K, V (Lk x D):
    S = Q K^T / sqrt(D)
    softmax:   O = softmax_rows(S restricted to the allowed keys) V
    gelu_tanh: Q, K are RMS-normalised per token and head first (the QK-norm of
               [GEM-T] GDPA section, which bounds the activation input), then
               O = gelu_tanh(S) V / Lk   (no max, no row sum)
  Block window ([GEM-T] "BlockAttention"; [GEM-S] "深いソフトウェア・ハードウェア
  協調設計によるスケーラブルなアーキテクチャ": 64-token blocks, window a whole number
  of blocks): query in block i sees every key of blocks i-W/64+1 .. i, blocks
  counted from the sample's first token, the last block possibly partial.
  Sliding window ([GEM-T] "BlockAttention": the token-level sliding window that
  block attention grew out of, cost O(L x window)): query i sees keys j with
  i - W < j <= i, positions counted from the sample's first token.

Readings where the pages are silent (each listed in the design notes):
  * no causal mask inside a block or in full attention; window 0 = no window;
  * the sliding window looks back: W keys ending at the query itself;
  * scale 1/sqrt(D) for every variant, no bias or positional term;
  * RMSNorm has unit weight and eps inside the square root (default 1e-6);
  * Lk == 0 gives O == 0; Lq == 0 gives no rows.
"""
from __future__ import annotations

import math

import numpy as np

BLOCK = 64
DEFAULT_EPS = 1e-6


def gelu_tanh(x):
    """0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))  -- the tanh form of GELU."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def rms_normalise(x, eps: float = DEFAULT_EPS):
    """Unit-weight RMSNorm over the last axis: x / sqrt(mean(x^2) + eps)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def block_window_allowed(lq: int, lk: int, window: int) -> np.ndarray:
    """Boolean [lq, lk]: may query i attend key j?

    window == 0: every key.  window > 0 (a multiple of 64): key block j//64 must
    lie in [i//64 - window/64 + 1, i//64]."""
    if window == 0:
        return np.ones((lq, lk), dtype=bool)
    if window % BLOCK:
        raise ValueError("window must be a multiple of 64")
    nb = window // BLOCK
    qi = (np.arange(lq) // BLOCK)[:, None]
    kj = (np.arange(lk) // BLOCK)[None, :]
    return (kj <= qi) & (kj >= qi - nb + 1)


def sliding_window_allowed(lq: int, lk: int, window: int) -> np.ndarray:
    """Boolean [lq, lk] for the token sliding window (window >= 1): key j is
    allowed for query i when i - window < j <= i."""
    if window < 1:
        raise ValueError("a sliding window needs window >= 1")
    qi = np.arange(lq)[:, None]
    kj = np.arange(lk)[None, :]
    return (kj <= qi) & (kj > qi - window)


def allowed_keys(lq: int, lk: int, window: int, variant: str = "self") -> np.ndarray:
    """The softmax mask of any variant: sliding window or block window / all keys."""
    if variant == "sliding":
        return sliding_window_allowed(lq, lk, window)
    return block_window_allowed(lq, lk, window)


def attention_dense(Q, K, V, act: str, window: int = 0, eps: float = DEFAULT_EPS, variant: str = "self"):
    """One (sample, head): Q [Lq,D], K, V [Lk,D] -> O [Lq,D] in float64."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    lq, d = Q.shape
    lk = K.shape[0]
    if lq == 0:
        return np.zeros((0, d))
    if lk == 0:
        return np.zeros((lq, d))
    if act == "softmax":
        S = (Q @ K.T) / math.sqrt(d)
        allowed = allowed_keys(lq, lk, window, variant)
        S = np.where(allowed, S, -np.inf)
        m = S.max(axis=1, keepdims=True)
        P = np.exp(S - m)            # exp(-inf) = 0 for disallowed keys
        P /= P.sum(axis=1, keepdims=True)
        return P @ V
    if act == "gelu_tanh":
        if window:
            raise ValueError("windowed GELU attention is not defined")
        S = (rms_normalise(Q, eps) @ rms_normalise(K, eps).T) / math.sqrt(d)
        return (gelu_tanh(S) @ V) / lk
    raise ValueError(f"unknown activation {act!r}")


def attention_lse(Q, K, window: int = 0, variant: str = "self"):
    """One (sample, head) of softmax attention: the natural log-sum-exp over the
    allowed keys of the scaled scores, log sum_j exp(q_i . k_j / sqrt(D)), per
    query row [Lq]; -inf for a row that sees no key (Lk == 0).  With it the
    softmax weights are exp(s_ij - lse_i) -- what the backward needs from the
    forward besides the output."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    lq, d = Q.shape
    lk = K.shape[0]
    if lk == 0:
        return np.full(lq, -np.inf)
    S = (Q @ K.T) / math.sqrt(d)
    S = np.where(allowed_keys(lq, lk, window, variant), S, -np.inf)
    m = S.max(axis=1)
    return m + np.log(np.exp(S - m[:, None]).sum(axis=1))


def gdpa_lse(q, k, q_offsets, kv_offsets, variant: str = "self", window: int = 0) -> np.ndarray:
    """Softmax attention's log-sum-exp per query row and head: float64 [Nq, H]
    (attention_lse of every sample and head)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    qo, ko = _check(q, k, k, q_offsets, kv_offsets, variant, "softmax", window)
    out = np.zeros(q.shape[:2], dtype=np.float64)
    for b in range(len(qo) - 1):
        for h in range(q.shape[1]):
            out[qo[b]:qo[b + 1], h] = attention_lse(q[qo[b]:qo[b + 1], h, :], k[ko[b]:ko[b + 1], h, :],
                                                    window, variant)
    return out


def _check(q, k, v, q_offsets, kv_offsets, variant, act, window):
    qo = np.asarray(q_offsets, dtype=np.int64)
    ko = np.asarray(kv_offsets, dtype=np.int64)
    if qo.ndim != 1 or ko.shape != qo.shape or qo[0] != 0 or ko[0] != 0:
        raise ValueError("offsets must be [B+1] and start at 0")
    if np.any(np.diff(qo) < 0) or np.any(np.diff(ko) < 0):
        raise ValueError("offsets must be non-decreasing")
    if qo[-1] != q.shape[0] or ko[-1] != k.shape[0] or k.shape != v.shape:
        raise ValueError("offsets do not match the value tensors")
    if variant not in ("self", "cross", "pma", "sliding"):
        raise ValueError(variant)
    if variant in ("self", "sliding") and not np.array_equal(qo, ko):
        raise ValueError("self-attention needs identical query and key offsets")
    if window and (variant not in ("self", "sliding") or act != "softmax"):
        raise ValueError("a window applies to softmax self-attention only")
    if variant == "sliding" and (window < 1 or act != "softmax"):
        raise ValueError("sliding-window attention needs window >= 1 and softmax")
    return qo, ko


def gdpa_forward(q, k, v, q_offsets, kv_offsets, variant: str = "self", act: str = "softmax",
                 window: int = 0, eps: float = DEFAULT_EPS) -> np.ndarray:
    """q [Nq,H,D], k/v [Nk,H,D] (any float dtype) -> out float64 [Nq,H,D]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    qo, ko = _check(q, k, v, q_offsets, kv_offsets, variant, act, window)
    out = np.zeros(q.shape, dtype=np.float64)
    for b in range(len(qo) - 1):
        for h in range(q.shape[1]):
            out[qo[b]:qo[b + 1], h, :] = attention_dense(
                q[qo[b]:qo[b + 1], h, :], k[ko[b]:ko[b + 1], h, :], v[ko[b]:ko[b + 1], h, :],
                act, window, eps, variant)
    return out


def gdpa_rows(q, k, v, q_offsets, kv_offsets, rows, variant: str = "self", act: str = "softmax",
              window: int = 0, eps: float = DEFAULT_EPS) -> np.ndarray:
    """Selected output rows only: rows = iterable of (token index t, head h).
    Returns float64 [len(rows), D]; row r is out[t, h, :] of gdpa_forward."""
    q = np.asarray(q)
    qo, ko = _check(q, k, v, q_offsets, kv_offsets, variant, act, window)
    res = []
    for t, h in rows:
        b = int(np.searchsorted(qo, t, side="right") - 1)
        i = t - qo[b]                                   # position inside the sample
        Qs = np.asarray(q[qo[b]:qo[b + 1], h, :], dtype=np.float64)
        Ks = np.asarray(k[ko[b]:ko[b + 1], h, :], dtype=np.float64)
        Vs = np.asarray(v[ko[b]:ko[b + 1], h, :], dtype=np.float64)
        lk = Ks.shape[0]
        if lk == 0:
            res.append(np.zeros(q.shape[2]))
            continue
        if act == "gelu_tanh":
            Qs, Ks = rms_normalise(Qs[i:i + 1], eps), rms_normalise(Ks, eps)
            s = (Qs @ Ks.T)[0] / math.sqrt(q.shape[2])
            res.append(gelu_tanh(s) @ Vs / lk)
            continue
        allowed = allowed_keys(Qs.shape[0], lk, window, variant)[i]
        s = (Ks @ Qs[i]) / math.sqrt(q.shape[2])
        s = np.where(allowed, s, -np.inf)
        p = np.exp(s - s.max())
        res.append((p / p.sum()) @ Vs)
    return np.array(res, dtype=np.float64).reshape(len(res), q.shape[2])


def attended_pairs(q_offsets, kv_offsets, act: str = "softmax", window: int = 0, variant: str = "self") -> int:
    """Number of (query, key) pairs that enter the output, per head:
    sum over samples of the allowed-mask population (dense count)."""
    qo = np.asarray(q_offsets, dtype=np.int64)
    ko = np.asarray(kv_offsets, dtype=np.int64)
    total = 0
    for b in range(len(qo) - 1):
        lq, lk = int(qo[b + 1] - qo[b]), int(ko[b + 1] - ko[b])
        if lq and lk:
            total += int(allowed_keys(lq, lk, window, variant).sum())
    return total
