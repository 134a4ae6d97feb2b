"""Pins for the oracle's softmax paths (full, block window, cross, PMA).

Each test checks the oracle against something fixed outside it: torch's
scaled_dot_product_attention in float64 (an independent library routine),
scalar brute force, closed forms, or invariants of the definition."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import gdpa_forward, gdpa_rows, attention_dense
from recsys_jagged_attention_amd.inputs import random_jagged, rng_for, offsets_from_lengths


def sdpa_padded(q, k, v, qo, ko, allowed_fn=None):
    """Pad every sample to the max length and run torch SDPA (float64) with a boolean mask."""
    B, H, D = len(qo) - 1, q.shape[1], q.shape[2]
    lq = np.diff(qo)
    lk = np.diff(ko)
    Mq, Mk = int(lq.max()), int(lk.max())
    Qp = torch.zeros(B, H, Mq, D, dtype=torch.float64)
    Kp = torch.zeros(B, H, Mk, D, dtype=torch.float64)
    Vp = torch.zeros(B, H, Mk, D, dtype=torch.float64)
    mask = torch.zeros(B, 1, Mq, Mk, dtype=torch.bool)
    for b in range(B):
        Qp[b, :, :lq[b]] = torch.from_numpy(q[qo[b]:qo[b + 1]].astype(np.float64)).transpose(0, 1)
        Kp[b, :, :lk[b]] = torch.from_numpy(k[ko[b]:ko[b + 1]].astype(np.float64)).transpose(0, 1)
        Vp[b, :, :lk[b]] = torch.from_numpy(v[ko[b]:ko[b + 1]].astype(np.float64)).transpose(0, 1)
        m = torch.zeros(Mq, Mk, dtype=torch.bool)
        m[:lq[b], :lk[b]] = True if allowed_fn is None else torch.from_numpy(allowed_fn(lq[b], lk[b]))
        mask[b, 0] = m
    O = F.scaled_dot_product_attention(Qp, Kp, Vp, attn_mask=mask)
    out = np.zeros(q.shape, dtype=np.float64)
    for b in range(B):
        out[qo[b]:qo[b + 1]] = O[b, :, :lq[b]].transpose(0, 1).numpy()
    return out


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_full_self_matches_library_sdpa(seed):
    rng = rng_for(seed)
    L = rng.integers(1, 40, size=5)
    qo, ko, q, k, v = random_jagged(seed, L, L, 3, 16)
    k, v = q.copy() * 0 + k, v
    got = gdpa_forward(q, k, v, qo, ko, "self", "softmax", 0)
    ref = sdpa_padded(q, k, v, qo, ko)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("variant", ["cross", "pma"])
def test_cross_and_pma_match_library_sdpa(variant):
    rng = rng_for(7)
    lq = rng.integers(1, 20, size=4) if variant == "cross" else np.full(4, 32)
    lk = rng.integers(1, 90, size=4)
    qo, ko, q, k, v = random_jagged(8, lq, lk, 2, 32)
    got = gdpa_forward(q, k, v, qo, ko, variant, "softmax", 0)
    ref = sdpa_padded(q, k, v, qo, ko)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("window", [64, 128, 256])
def test_block_window_reduces_to_full_attention_on_slices(window):
    """Query block i attends exactly key blocks i-W/64+1..i: its rows equal unmasked
    SDPA of that query block against the concatenated key blocks (a slice, no mask)."""
    L = [300, 64, 65, 1, 200]
    qo, ko, q, k, v = random_jagged(11, L, L, 2, 16)
    got = gdpa_forward(q, k, v, qo, ko, "self", "softmax", window)
    nb = window // 64
    for b in range(len(L)):
        s = qo[b]
        for blk in range((L[b] + 63) // 64):
            q0, q1 = s + 64 * blk, min(s + 64 * (blk + 1), qo[b + 1])
            k0 = s + 64 * max(0, blk - nb + 1)
            Q = torch.from_numpy(q[q0:q1].astype(np.float64)).transpose(0, 1)
            K = torch.from_numpy(k[k0:q1].astype(np.float64)).transpose(0, 1)
            V = torch.from_numpy(v[k0:q1].astype(np.float64)).transpose(0, 1)
            ref = F.scaled_dot_product_attention(Q, K, V).transpose(0, 1).numpy()
            np.testing.assert_allclose(got[q0:q1], ref, rtol=0, atol=1e-12)


def test_window_64_is_independent_blocks():
    """W=64: every 64-token block is its own full-attention problem."""
    L = [200]
    qo, ko, q, k, v = random_jagged(12, L, L, 1, 8)
    got = gdpa_forward(q, k, v, qo, ko, "self", "softmax", 64)
    blocks = [64, 64, 64, 8]
    bo = offsets_from_lengths(blocks)
    ref = gdpa_forward(q, k, v, bo, bo, "self", "softmax", 0)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)


def test_window_covering_short_sample_is_full_attention():
    """L <= 64 and W >= 64: the window is the whole sample (non-causal full attention)."""
    L = [64, 17, 1]
    qo, ko, q, k, v = random_jagged(13, L, L, 2, 8)
    for w in (64, 256):
        np.testing.assert_allclose(gdpa_forward(q, k, v, qo, ko, "self", "softmax", w),
                                   gdpa_forward(q, k, v, qo, ko, "self", "softmax", 0), atol=1e-14)


def test_brute_force_scalar_loops():
    """Tiny inputs against scalar loops with math.exp (no numpy vector ops)."""
    L = [3, 6, 1]
    qo, ko, q, k, v = random_jagged(14, L, L, 2, 4)
    got = gdpa_forward(q, k, v, qo, ko, "self", "softmax", 0)
    for b in range(3):
        for h in range(2):
            for i in range(qo[b], qo[b + 1]):
                sc = []
                for j in range(ko[b], ko[b + 1]):
                    sc.append(sum(float(q[i, h, d]) * float(k[j, h, d]) for d in range(4)) / 2.0)
                mx = max(sc)
                w = [math.exp(s - mx) for s in sc]
                tot = sum(w)
                for d in range(4):
                    o = sum(w[jj] * float(v[ko[b] + jj, h, d]) for jj in range(len(w))) / tot
                    assert abs(got[i, h, d] - o) < 1e-12


def test_one_key_returns_that_value():
    qo, ko, q, k, v = random_jagged(15, [32, 32], [1, 1], 3, 16)
    out = gdpa_forward(q, k, v, qo, ko, "pma", "softmax", 0)
    for b in range(2):
        np.testing.assert_allclose(out[qo[b]:qo[b + 1]], np.broadcast_to(v[ko[b]], (32, 3, 16)), atol=1e-15)
    qo, ko, q, k, v = random_jagged(16, [1, 1, 1], [1, 1, 1], 2, 8)
    np.testing.assert_allclose(gdpa_forward(q, k, v, qo, ko, "self", "softmax", 0), v, atol=1e-15)


def test_uniform_scores_give_mean_of_values():
    qo, ko, q, k, v = random_jagged(17, [5, 9], [7, 3], 2, 8)
    zero_q = np.zeros_like(q)
    out = gdpa_forward(zero_q, k, v, qo, ko, "cross", "softmax", 0)
    same_k = np.broadcast_to(k[:1], k.shape).copy()
    out2 = gdpa_forward(q, same_k, v, qo, ko, "cross", "softmax", 0)
    for b in range(2):
        mean = v[ko[b]:ko[b + 1]].astype(np.float64).mean(axis=0)
        np.testing.assert_allclose(out[qo[b]:qo[b + 1]], np.broadcast_to(mean, out[qo[b]:qo[b + 1]].shape), atol=1e-14)
        np.testing.assert_allclose(out2[qo[b]:qo[b + 1]], np.broadcast_to(mean, out2[qo[b]:qo[b + 1]].shape), atol=1e-14)


def test_pma_invariant_to_key_permutation():
    lk = [40, 100, 7]
    qo, ko, q, k, v = random_jagged(18, [32] * 3, lk, 2, 16)
    base = gdpa_forward(q, k, v, qo, ko, "pma", "softmax", 0)
    rng = rng_for(19)
    perm = np.concatenate([ko[b] + rng.permutation(lk[b]) for b in range(3)])
    np.testing.assert_allclose(gdpa_forward(q, k[perm], v[perm], qo, ko, "pma", "softmax", 0), base, atol=1e-13)


def test_full_self_equivariant_under_joint_permutation():
    L = [20, 33]
    qo, ko, q, k, v = random_jagged(20, L, L, 2, 8)
    base = gdpa_forward(q, k, v, qo, ko, "self", "softmax", 0)
    rng = rng_for(21)
    perm = np.concatenate([qo[b] + rng.permutation(L[b]) for b in range(2)])
    np.testing.assert_allclose(gdpa_forward(q[perm], k[perm], v[perm], qo, ko, "self", "softmax", 0),
                               base[perm], atol=1e-13)


def test_output_in_convex_hull_of_attended_values():
    L = [150]
    qo, ko, q, k, v = random_jagged(22, L, L, 1, 4)
    out = gdpa_forward(q * 3, k, v, qo, ko, "self", "softmax", 128)
    for i in range(150):
        blk = i // 64
        lo = 64 * max(0, blk - 1)
        hi = min(150, 64 * (blk + 1))
        vv = v[lo:hi, 0]
        assert np.all(out[i, 0] >= vv.min(axis=0) - 1e-12) and np.all(out[i, 0] <= vv.max(axis=0) + 1e-12)


def test_empty_samples():
    qo, ko, q, k, v = random_jagged(23, [0, 5, 3], [4, 0, 2], 2, 8)
    out = gdpa_forward(q, k, v, qo, ko, "cross", "softmax", 0)
    assert out.shape == q.shape
    np.testing.assert_array_equal(out[qo[1]:qo[2]], 0.0)
    ref = sdpa_padded(q[qo[2]:], k[ko[2]:], v[ko[2]:], np.array([0, 3]), np.array([0, 2]))
    np.testing.assert_allclose(out[qo[2]:], ref, atol=1e-12)


def test_rows_match_full_output():
    L = [130, 70]
    qo, ko, q, k, v = random_jagged(24, L, L, 2, 16)
    for w in (0, 128):
        full = gdpa_forward(q, k, v, qo, ko, "self", "softmax", w)
        rows = [(0, 0), (64, 1), (129, 0), (130, 1), (199, 0)]
        got = gdpa_rows(q, k, v, qo, ko, rows, "self", "softmax", w)
        for r, (t, h) in enumerate(rows):
            np.testing.assert_allclose(got[r], full[t, h], atol=1e-13)


def test_rejects_bad_arguments():
    qo, ko, q, k, v = random_jagged(25, [3], [4], 1, 8)
    with pytest.raises(ValueError):
        gdpa_forward(q, k, v, qo, ko, "self", "softmax", 0)          # self needs equal offsets
    with pytest.raises(ValueError):
        gdpa_forward(q, k, v, qo, ko, "cross", "softmax", 64)        # window only for self
    with pytest.raises(ValueError):
        attention_dense(q[:, 0], k[:, 0], v[:, 0], "softmax", 100)  # not a multiple of 64
