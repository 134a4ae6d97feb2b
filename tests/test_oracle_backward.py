"""Pins for the oracle's backward: torch autograd through its own
scaled_dot_product_attention (softmax) or F.rms_norm + F.gelu(approximate='tanh')
(GELU scores) in float64 (independent library paths), central finite
differences of the oracle's forward, and closed forms."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import (gdpa_backward, gdpa_forward, sliding_window_allowed, block_window_allowed, gelu_tanh,
                    gelu_tanh_grad, rms_normalise_bwd)
from recsys_jagged_attention_amd.inputs import random_jagged


def autograd_ref(q, k, v, dout, qo, ko, mask_fn):
    """Per sample and head: SDPA with a boolean mask, gradients by autograd."""
    dq, dk, dv = (np.zeros(a.shape) for a in (q, k, v))
    for b in range(len(qo) - 1):
        qs, ks = slice(qo[b], qo[b + 1]), slice(ko[b], ko[b + 1])
        lq, lk = qo[b + 1] - qo[b], ko[b + 1] - ko[b]
        if lq == 0 or lk == 0:
            continue
        Q = torch.tensor(q[qs].astype(np.float64).transpose(1, 0, 2), requires_grad=True)
        K = torch.tensor(k[ks].astype(np.float64).transpose(1, 0, 2), requires_grad=True)
        V = torch.tensor(v[ks].astype(np.float64).transpose(1, 0, 2), requires_grad=True)
        mask = None if mask_fn is None else torch.from_numpy(mask_fn(lq, lk))
        O = F.scaled_dot_product_attention(Q, K, V, attn_mask=mask)
        O.backward(torch.tensor(dout[qs].astype(np.float64).transpose(1, 0, 2)))
        dq[qs] = Q.grad.numpy().transpose(1, 0, 2)
        dk[ks] = K.grad.numpy().transpose(1, 0, 2)
        dv[ks] = V.grad.numpy().transpose(1, 0, 2)
    return dq, dk, dv


CASES = [
    ("self", 0, None),
    ("self", 64, lambda lq, lk: block_window_allowed(lq, lk, 64)),
    ("self", 128, lambda lq, lk: block_window_allowed(lq, lk, 128)),
    ("sliding", 5, lambda lq, lk: sliding_window_allowed(lq, lk, 5)),
    ("sliding", 70, lambda lq, lk: sliding_window_allowed(lq, lk, 70)),
    ("cross", 0, None),
    ("pma", 0, None),
]


@pytest.mark.parametrize("variant,window,mask_fn", CASES)
def test_matches_torch_autograd(variant, window, mask_fn):
    if variant in ("self", "sliding"):
        L = [130, 1, 64, 0, 77]
        qo, ko, q, k, v = random_jagged(31 + window, L, L, 2, 16)
    elif variant == "cross":
        qo, ko, q, k, v = random_jagged(32, [50, 3, 0, 9], [7, 1, 4, 0], 2, 16)
    else:
        qo, ko, q, k, v = random_jagged(33, [32, 32, 32], [100, 1, 0], 2, 16)
    dout = np.random.default_rng(34).standard_normal(q.shape)
    got = gdpa_backward(q, k, v, dout, qo, ko, variant, "softmax", window)
    ref = autograd_ref(q, k, v, dout, qo, ko, mask_fn)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, rtol=0, atol=1e-12)


def test_matches_finite_differences_of_the_forward():
    """d<dout, O>/dx by central differences of the oracle's own forward."""
    L = [6, 3]
    qo, ko, q, k, v = random_jagged(35, L, L, 1, 4)
    q, k, v = (a.astype(np.float64) for a in (q, k, v))
    dout = np.random.default_rng(36).standard_normal(q.shape)
    for variant, window in (("self", 0), ("sliding", 2), ("self", 64)):
        dq, dk, dv = gdpa_backward(q, k, v, dout, qo, ko, variant, "softmax", window)
        f = lambda qq, kk, vv: float((gdpa_forward(qq, kk, vv, qo, ko, variant, "softmax", window) * dout).sum())
        h = 1e-6
        for arr, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
            for idx in [(0, 0, 1), (4, 0, 3), (7, 0, 0)]:
                args = [q.copy(), k.copy(), v.copy()]
                args[which][idx] += h
                fp = f(*args)
                args[which][idx] -= 2 * h
                fm = f(*args)
                assert abs((fp - fm) / (2 * h) - grad[idx]) < 1e-7


def test_closed_forms():
    """One key: P = 1, so dV = sum of dO over the queries and dQ = dK = 0.
    Window 1 (sliding): each query sees only its own key: dV = dO, dQ = dK = 0."""
    qo, ko, q, k, v = random_jagged(37, [32], [1], 2, 8)
    dout = np.random.default_rng(38).standard_normal(q.shape)
    dq, dk, dv = gdpa_backward(q, k, v, dout, qo, ko, "pma")
    np.testing.assert_allclose(dv[0], dout.sum(axis=0), atol=1e-12)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13
    qo, ko, q, k, v = random_jagged(39, [9], [9], 2, 8)
    dout = np.random.default_rng(40).standard_normal(q.shape)
    dq, dk, dv = gdpa_backward(q, k, v, dout, qo, ko, "sliding", "softmax", 1)
    np.testing.assert_allclose(dv, dout, atol=1e-13)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13


def gelu_autograd_ref(q, k, v, dout, qo, ko, eps=1e-6):
    """Per sample: RMSNorm, scores, tanh GELU and the 1/Lk mean by torch ops, gradients by autograd."""
    dq, dk, dv = (np.zeros(a.shape) for a in (q, k, v))
    d = q.shape[-1]
    for b in range(len(qo) - 1):
        qs, ks = slice(qo[b], qo[b + 1]), slice(ko[b], ko[b + 1])
        lq, lk = qo[b + 1] - qo[b], ko[b + 1] - ko[b]
        if lq == 0 or lk == 0:
            continue
        Q = torch.tensor(q[qs].astype(np.float64).transpose(1, 0, 2), requires_grad=True)
        K = torch.tensor(k[ks].astype(np.float64).transpose(1, 0, 2), requires_grad=True)
        V = torch.tensor(v[ks].astype(np.float64).transpose(1, 0, 2), requires_grad=True)
        Qn = F.rms_norm(Q, (d,), eps=eps)
        Kn = F.rms_norm(K, (d,), eps=eps)
        S = torch.matmul(Qn, Kn.transpose(1, 2).contiguous()) / d ** 0.5
        O = torch.matmul(F.gelu(S, approximate="tanh"), V) / lk
        O.backward(torch.tensor(dout[qs].astype(np.float64).transpose(1, 0, 2)))
        dq[qs] = Q.grad.numpy().transpose(1, 0, 2)
        dk[ks] = K.grad.numpy().transpose(1, 0, 2)
        dv[ks] = V.grad.numpy().transpose(1, 0, 2)
    return dq, dk, dv


@pytest.mark.parametrize("variant", ["cross", "pma", "self"])
def test_gelu_matches_torch_autograd(variant):
    if variant == "cross":
        qo, ko, q, k, v = random_jagged(41, [50, 3, 0, 9], [7, 1, 4, 0], 2, 16)
    elif variant == "pma":
        qo, ko, q, k, v = random_jagged(42, [32, 32, 32], [100, 1, 0], 2, 16)
    else:
        L = [70, 1, 0, 13]
        qo, ko, q, k, v = random_jagged(43, L, L, 2, 32)
    dout = np.random.default_rng(44).standard_normal(q.shape)
    got = gdpa_backward(q, k, v, dout, qo, ko, variant, "gelu_tanh")
    ref = gelu_autograd_ref(q, k, v, dout, qo, ko)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, rtol=0, atol=1e-12)


def test_gelu_matches_finite_differences_of_the_forward():
    qo, ko, q, k, v = random_jagged(45, [5, 2], [3, 4], 1, 4)
    q, k, v = (a.astype(np.float64) for a in (q, k, v))
    dout = np.random.default_rng(46).standard_normal(q.shape)
    dq, dk, dv = gdpa_backward(q, k, v, dout, qo, ko, "cross", "gelu_tanh")
    f = lambda qq, kk, vv: float((gdpa_forward(qq, kk, vv, qo, ko, "cross", "gelu_tanh") * dout).sum())
    h = 1e-6
    for arr, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        for idx in [(0, 0, 1), (4, 0, 3), (arr.shape[0] - 1, 0, 0)]:
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += h
            fp = f(*args)
            args[which][idx] -= 2 * h
            fm = f(*args)
            assert abs((fp - fm) / (2 * h) - grad[idx]) < 1e-7


def test_gelu_grad_closed_forms():
    """gelu(x) - gelu(-x) = x gives gelu'(x) + gelu'(-x) = 1; gelu'(0) = 1/2;
    gelu' -> 1 above and -> 0 below; and it is the slope of gelu_tanh."""
    x = np.linspace(-9, 9, 721)
    np.testing.assert_allclose(gelu_tanh_grad(x) + gelu_tanh_grad(-x), 1.0, atol=1e-14)
    assert gelu_tanh_grad(0.0) == 0.5
    assert abs(gelu_tanh_grad(12.0) - 1) < 1e-15 and abs(gelu_tanh_grad(-12.0)) < 1e-15
    h = 1e-5
    np.testing.assert_allclose((gelu_tanh(x + h) - gelu_tanh(x - h)) / (2 * h), gelu_tanh_grad(x), atol=1e-9)


def test_rms_normalise_bwd_closed_form():
    """rms(x) is invariant to scaling x as eps -> 0, so the gradient is nearly
    orthogonal to x: x . dx = r (x . dy) eps / (mean(x^2) + eps) exactly."""
    rng = np.random.default_rng(47)
    x, dy = rng.standard_normal((6, 32)), rng.standard_normal((6, 32))
    eps = 1e-3
    ms = np.mean(x * x, axis=1)
    r = 1 / np.sqrt(ms + eps)
    got = np.sum(x * rms_normalise_bwd(x, dy, eps), axis=1)
    np.testing.assert_allclose(got, r * np.sum(x * dy, axis=1) * eps / (ms + eps), rtol=1e-12)
