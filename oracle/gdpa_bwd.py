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

For the GELU scores (tanh form, with QK-RMSNorm; no window), with
Qn = rms(Q), Kn = rms(K), rms(x) = x r, r = (mean(x^2) + eps)^(-1/2):

  S = Qn Kn^T / sqrt(D),  G = gelu_tanh(S),  O = G V / Lk
  dV = G^T dO / Lk
  dS = gelu_tanh'(S) * (dO V^T) / Lk
  dQn = dS Kn / sqrt(D),  dKn = dS^T Qn / sqrt(D)
  dx = r dxn - x r^3 (dxn . x) / D        (RMSNorm, per row)

with gelu_tanh'(x) = 0.5 (1 + tanh u) + 0.5 x (1 - tanh^2 u) u',
u = sqrt(2/pi) (x + 0.044715 x^3), u' = sqrt(2/pi) (1 + 3 * 0.044715 x^2).
"""
from __future__ import annotations

import math

import numpy as np

from .gdpa import DEFAULT_EPS, allowed_keys, gelu_tanh, _check


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


def gelu_tanh_grad(x):
    """Derivative of 0.5 x (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3)."""
    x = np.asarray(x, dtype=np.float64)
    c = math.sqrt(2.0 / math.pi)
    t = np.tanh(c * (x + 0.044715 * x ** 3))
    return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * c * (1.0 + 3.0 * 0.044715 * x * x)


def rms_normalise_bwd(x, dy, eps: float = DEFAULT_EPS):
    """Gradient through y = x / sqrt(mean(x^2) + eps), row by row (last axis)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return r * dy - x * r ** 3 * np.sum(dy * x, axis=-1, keepdims=True) / d


def attention_dense_gelu_bwd(Q, K, V, dO, eps: float = DEFAULT_EPS):
    """One (sample, head), GELU scores with QK-RMSNorm -> (dQ, dK, dV) float64."""
    Q, K, V, dO = (np.asarray(a, dtype=np.float64) for a in (Q, K, V, dO))
    lq, d = Q.shape
    lk = K.shape[0]
    if lq == 0 or lk == 0:
        return np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    rq = 1.0 / np.sqrt(np.mean(Q * Q, axis=1, keepdims=True) + eps)
    rk = 1.0 / np.sqrt(np.mean(K * K, axis=1, keepdims=True) + eps)
    Qn, Kn = Q * rq, K * rk
    S = Qn @ Kn.T / math.sqrt(d)
    G = gelu_tanh(S)
    dV = G.T @ dO / lk
    dS = gelu_tanh_grad(S) * (dO @ V.T) / lk
    dQn = dS @ Kn / math.sqrt(d)
    dKn = dS.T @ Qn / math.sqrt(d)
    return rms_normalise_bwd(Q, dQn, eps), rms_normalise_bwd(K, dKn, eps), dV


def gdpa_backward(q, k, v, dout, q_offsets, kv_offsets, variant: str = "self", act: str = "softmax",
                  window: int = 0, eps: float = DEFAULT_EPS):
    """q, dout [Nq,H,D], k, v [Nk,H,D] -> (dq [Nq,H,D], dk, dv [Nk,H,D]) float64.
    act: "softmax" or "gelu_tanh" (no window)."""
    if act not in ("softmax", "gelu_tanh"):
        raise ValueError(f"unknown activation {act!r}")
    q, k, v, dout = (np.asarray(a, dtype=np.float64) for a in (q, k, v, dout))
    qo, ko = _check(q, k, v, q_offsets, kv_offsets, variant, act, window)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(len(qo) - 1):
        qs, ks = slice(qo[b], qo[b + 1]), slice(ko[b], ko[b + 1])
        for h in range(q.shape[1]):
            if act == "softmax":
                gq, gk, gv = attention_dense_bwd(q[qs, h], k[ks, h], v[ks, h], dout[qs, h], window, variant)
            else:
                gq, gk, gv = attention_dense_gelu_bwd(q[qs, h], k[ks, h], v[ks, h], dout[qs, h], eps)
            dq[qs, h], dk[ks, h], dv[ks, h] = gq, gk, gv
    return dq, dk, dv
