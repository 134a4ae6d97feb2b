"""Pins for the oracle's GELU path: QK-RMSNorm + gelu_tanh + 1/Lk."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import gdpa_forward, gdpa_rows, gelu_tanh, rms_normalise
from recsys_jagged_attention_amd.inputs import random_jagged, rng_for


def test_gelu_tanh_matches_library():
    x = np.linspace(-12, 12, 4801)
    ref = F.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    np.testing.assert_allclose(gelu_tanh(x), ref, rtol=0, atol=1e-15)


def test_gelu_tanh_closed_forms():
    assert gelu_tanh(0.0) == 0.0
    x = np.linspace(-6, 6, 101)
    # gelu(x) - gelu(-x) = x for the tanh form (tanh is odd)
    np.testing.assert_allclose(gelu_tanh(x) - gelu_tanh(-x), x, atol=1e-14)
    # identity 1 + tanh(u) = 2 sigmoid(2u)
    u = math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3)
    np.testing.assert_allclose(gelu_tanh(x), x / (1 + np.exp(-2 * u)), atol=1e-14)
    assert abs(gelu_tanh(30.0) - 30.0) < 1e-12 and abs(gelu_tanh(-30.0)) < 1e-12


def test_rms_normalise_matches_library_and_closed_form():
    rng = rng_for(3)
    x = rng.standard_normal((50, 128))
    for eps in (1e-6, 0.5):
        ref = F.rms_norm(torch.from_numpy(x), (128,), eps=eps).numpy()
        np.testing.assert_allclose(rms_normalise(x, eps), ref, atol=1e-14)
        m = np.mean(x * x, axis=1)
        np.testing.assert_allclose(np.sum(rms_normalise(x, eps) ** 2, axis=1), 128 * m / (m + eps), rtol=1e-13)


def test_collinear_rows_closed_form():
    """q_i = a_i u, k_j = s_j b_j u (a, b > 0, s = +-1), eps = 0: the normalised
    rows are +-sqrt(D) u/|u|, so every score is s_j * sqrt(D) and
    O_i = (1/Lk) sum_j gelu(s_j sqrt(D)) v_j."""
    D, lq, lk = 16, 5, 7
    rng = rng_for(4)
    u = rng.standard_normal(D)
    a = rng.uniform(0.5, 3, lq)
    b = rng.uniform(0.5, 3, lk)
    s = np.array([1, -1, 1, 1, -1, -1, 1.0])
    q = (a[:, None] * u)[:, None, :]
    k = (s[:, None] * b[:, None] * u)[:, None, :]
    v = rng.standard_normal((lk, 1, D))
    out = gdpa_forward(q, k, v, [0, lq], [0, lk], "cross", "gelu_tanh", 0, eps=0.0)
    g = F.gelu(torch.tensor([4.0, -4.0], dtype=torch.float64), approximate="tanh").numpy()
    expect = (np.where(s > 0, g[0], g[1])[:, None] * v[:, 0]).sum(0) / lk
    np.testing.assert_allclose(out[:, 0], np.broadcast_to(expect, (lq, D)), atol=1e-13)


def test_zero_queries_give_zero_output():
    qo, ko, q, k, v = random_jagged(5, [9, 4], [16, 64], 2, 32)
    out = gdpa_forward(np.zeros_like(q), k, v, qo, ko, "cross", "gelu_tanh", 0)
    np.testing.assert_array_equal(out, 0.0)


def test_query_scale_invariance():
    qo, ko, q, k, v = random_jagged(6, [9, 4], [16, 64], 2, 32)
    a = gdpa_forward(q, k, v, qo, ko, "cross", "gelu_tanh", 0, eps=0.0)
    b = gdpa_forward(q * 8.0, k * 0.25, v, qo, ko, "cross", "gelu_tanh", 0, eps=0.0)
    np.testing.assert_allclose(a, b, atol=1e-12)


def test_gelu_attention_matches_library_composition():
    qo, ko, q, k, v = random_jagged(7, [30, 1, 17], [16, 40, 64], 4, 64)
    out = gdpa_forward(q, k, v, qo, ko, "cross", "gelu_tanh", 0)
    for b in range(3):
        for h in range(4):
            Q = F.rms_norm(torch.from_numpy(q[qo[b]:qo[b + 1], h].astype(np.float64)), (64,), eps=1e-6)
            K = F.rms_norm(torch.from_numpy(k[ko[b]:ko[b + 1], h].astype(np.float64)), (64,), eps=1e-6)
            V = torch.from_numpy(v[ko[b]:ko[b + 1], h].astype(np.float64))
            S = Q @ K.T * 64 ** -0.5
            ref = (F.gelu(S, approximate="tanh") @ V / K.shape[0]).numpy()
            np.testing.assert_allclose(out[qo[b]:qo[b + 1], h], ref, atol=1e-13)


def test_gelu_key_permutation_invariance_and_empty_kv():
    qo, ko, q, k, v = random_jagged(8, [5, 6], [20, 0], 1, 32)
    out = gdpa_forward(q, k, v, qo, ko, "cross", "gelu_tanh", 0)
    np.testing.assert_array_equal(out[qo[1]:], 0.0)
    perm = rng_for(9).permutation(20)
    out2 = gdpa_forward(q, k[perm], v[perm], qo, ko, "cross", "gelu_tanh", 0)
    np.testing.assert_allclose(out2, out, atol=1e-14)


def test_gelu_rows_match_full():
    qo, ko, q, k, v = random_jagged(10, [40, 3], [33, 64], 2, 32)
    full = gdpa_forward(q, k, v, qo, ko, "cross", "gelu_tanh", 0)
    rows = [(0, 0), (39, 1), (41, 0), (42, 1)]
    got = gdpa_rows(q, k, v, qo, ko, rows, "cross", "gelu_tanh", 0)
    for r, (t, h) in enumerate(rows):
        np.testing.assert_allclose(got[r], full[t, h], atol=1e-14)
