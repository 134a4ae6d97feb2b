"""Backward of jagged softmax attention in float64 (oracle; test infrastructure only).

The gradient of the plain definition (see gdpa.py) with respect to Q, K and V,
for every softmax variant (full, block window, sliding window, cross, PMA).
The pages describe training (the whole GEM write-up is about training
efficiency) but not the backward pass; this is the derivative of the forward
as defined, by the chain rule, for one (sample, head):

  S = Q K^T / sqrt(D) on the allowed keys, P = softmax_rows(S), O = P V
  dV = P^T dO
  dP = dO V^T
  dS = P * (dP - rowsum(P * dP))        (softmax Jacobian, row by row)
  dQ = dS K / sqrt(D),  dK = dS^T Q / sqrt(D)

rowsum(P * dP) equals rowsum(dO * O).  Rows with no keys (Lk = 0) have O = 0
and zero gradients.
"""
from __future__ import annotations

import math

import numpy as np

from .gdpa import allowed_keys, _check


def attention_dense_bwd(Q, K, V, dO, window: int = 0, variant: str = "self"):
    """One (sample, head): Q, dO [Lq,D], K, V [Lk,D] -> (dQ, dK, dV) float64."""
    Q, K, V, dO = (np.asarray(a, dtype=np.float64) for a in (Q, K, V, dO))
    lq, d = Q.shape
    lk = K.shape[0]
    if lq == 0 or lk == 0:
        return np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    S = (Q @ K.T) / math.sqrt(d)
    S = np.where(allowed_keys(lq, lk, window, variant), S, -np.inf)
    P = np.exp(S - S.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    dV = P.T @ dO
    dP = dO @ V.T
    dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
    dQ = dS @ K / math.sqrt(d)
    dK = dS.T @ Q / math.sqrt(d)
    return dQ, dK, dV


def gdpa_backward(q, k, v, dout, q_offsets, kv_offsets, variant: str = "self", act: str = "softmax",
                  window: int = 0):
    """q, dout [Nq,H,D], k, v [Nk,H,D] -> (dq [Nq,H,D], dk, dv [Nk,H,D]) float64."""
    if act != "softmax":
        raise ValueError("the backward oracle covers softmax attention")
    q, k, v, dout = (np.asarray(a, dtype=np.float64) for a in (q, k, v, dout))
    qo, ko = _check(q, k, v, q_offsets, kv_offsets, variant, act, window)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(len(qo) - 1):
        qs, ks = slice(qo[b], qo[b + 1]), slice(ko[b], ko[b + 1])
        for h in range(q.shape[1]):
            gq, gk, gv = attention_dense_bwd(q[qs, h], k[ks, h], v[ks, h], dout[qs, h], window, variant)
            dq[qs, h], dk[ks, h], dv[ks, h] = gq, gk, gv
    return dq, dk, dv
