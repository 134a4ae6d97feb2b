"""Pins for the oracle's log-sum-exp of softmax attention (oracle.gdpa_lse,
attention_lse): what the backward takes from the forward besides its output.

Each test checks it against something fixed outside it: scipy's logsumexp
(an independent library routine) on the masked scores, closed forms, and the
pinned forward (the weights exp(s - lse) reproduce its output)."""
import math

import numpy as np
import pytest
from scipy.special import logsumexp

from oracle import gdpa_forward, gdpa_lse, attention_lse, block_window_allowed, sliding_window_allowed
from recsys_jagged_attention_amd.inputs import random_jagged


@pytest.mark.parametrize("variant,window", [("self", 0), ("self", 64), ("self", 128), ("sliding", 1),
                                            ("sliding", 37), ("cross", 0), ("pma", 0)])
def test_lse_against_scipy_logsumexp(variant, window):
    lq = [1, 70, 0, 130, 5] if variant != "pma" else [32, 32, 32, 32, 32]
    lk = [1, 70, 0, 130, 5] if variant in ("self", "sliding") else [3, 0, 90, 200, 64]
    qo, ko, q, k, v = random_jagged(31 + window, lq, lk, 2, 16)
    got = gdpa_lse(q, k, qo, ko, variant, window)
    for b in range(len(lq)):
        for h in range(2):
            Q = q[qo[b]:qo[b + 1], h].astype(np.float64)
            K = k[ko[b]:ko[b + 1], h].astype(np.float64)
            if len(Q) == 0:
                continue
            if len(K) == 0:
                assert np.all(got[qo[b]:qo[b + 1], h] == -np.inf)
                continue
            S = Q @ K.T / math.sqrt(Q.shape[1])
            if variant == "sliding":
                allowed = sliding_window_allowed(len(Q), len(K), window)
            else:
                allowed = block_window_allowed(len(Q), len(K), window)
            for i in range(len(Q)):
                ref = logsumexp(S[i][allowed[i]])
                assert abs(got[qo[b] + i, h] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_lse_closed_forms():
    rng = np.random.default_rng(3)
    Q = rng.standard_normal((4, 8))
    k = rng.standard_normal((1, 8))
    # one key: lse = q . k / sqrt(D)
    np.testing.assert_allclose(attention_lse(Q, k), (Q @ k.T)[:, 0] / math.sqrt(8), rtol=0, atol=1e-14)
    # n equal keys: lse = q . k / sqrt(D) + log n
    K = np.repeat(k, 7, axis=0)
    np.testing.assert_allclose(attention_lse(Q, K), (Q @ k.T)[:, 0] / math.sqrt(8) + math.log(7),
                               rtol=0, atol=1e-13)
    # sliding window of one token: each row sees only its own key
    X = rng.standard_normal((6, 8))
    np.testing.assert_allclose(attention_lse(X, X, 1, "sliding"), (X * X).sum(1) / math.sqrt(8),
                               rtol=0, atol=1e-13)


def test_lse_weights_reproduce_the_forward():
    """exp(s_ij - lse_i) over the allowed keys are the softmax weights: P V with
    them equals the pinned forward's output, and they sum to one."""
    lq = [50, 130, 1]
    qo, ko, q, k, v = random_jagged(9, lq, lq, 2, 16)
    lse = gdpa_lse(q, k, qo, ko, "self", 64)
    out = gdpa_forward(q, k, v, qo, ko, "self", "softmax", 64)
    for b in range(len(lq)):
        for h in range(2):
            Q, K, V = (x[qo[b]:qo[b + 1], h].astype(np.float64) for x in (q, k, v))
            S = Q @ K.T / math.sqrt(16)
            P = np.where(block_window_allowed(len(Q), len(K), 64), np.exp(S - lse[qo[b]:qo[b + 1], h][:, None]), 0.0)
            np.testing.assert_allclose(P.sum(1), 1.0, rtol=0, atol=1e-12)
            np.testing.assert_allclose(P @ V, out[qo[b]:qo[b + 1], h], rtol=0, atol=1e-12)
