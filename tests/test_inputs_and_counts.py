"""Seeded input recipes and the attended-pair count used for useful FLOPs."""
import numpy as np

from oracle import attended_pairs
from recsys_jagged_attention_amd.inputs import (make_workload, pma_lengths, rng_for,
                                                lengths_loguniform, offsets_from_lengths)
from recsys_jagged_attention_amd import workload as wl


def test_loguniform_range_and_median():
    L = lengths_loguniform(rng_for(1), 20000, 100, 4096)
    assert L.min() >= 100 and L.max() <= 4096
    # median of a log-uniform on [100, 4097) is sqrt(100*4097) ~ 640
    assert 600 < np.median(L) < 680


def test_pma_lengths_skew():
    L = pma_lengths(rng_for(2), 512)
    assert (L > 8192).sum() == 26 and L.min() >= 64 and L.max() <= 16384


def test_workloads_are_seeded_and_shaped():
    a = make_workload("block_window", scale=0.1)
    b = make_workload("block_window", scale=0.1)
    np.testing.assert_array_equal(a.q, b.q)
    assert a.q.shape == (a.total_q, 8, 128) and a.window == 256
    p = make_workload("pma", scale=0.05)
    assert np.all(np.diff(p.q_offsets) == 32) and p.D == 64
    c = make_workload("cross_gelu", scale=0.05)
    lk = np.diff(c.kv_offsets)
    assert lk.min() >= 16 and lk.max() <= 64 and c.act == "gelu_tanh"


def brute_pairs(qo, ko, window):
    tot = 0
    for b in range(len(qo) - 1):
        lq, lk = qo[b + 1] - qo[b], ko[b + 1] - ko[b]
        for i in range(lq):
            for j in range(lk):
                if window == 0 or (i // 64 - window // 64 < j // 64 <= i // 64):
                    tot += 1
    return tot


def test_attended_pairs_count():
    L = [1, 63, 64, 65, 300]
    off = offsets_from_lengths(L)
    for w in (0, 64, 256):
        n = brute_pairs(off, off, w)
        assert attended_pairs(off, off, "softmax", w) == n
        assert wl.attended_pairs(np.diff(off), np.diff(off), w) == n
    qo, ko = offsets_from_lengths([3, 0, 5]), offsets_from_lengths([7, 2, 0])
    assert wl.attended_pairs(np.diff(qo), np.diff(ko), 0) == attended_pairs(qo, ko) == 21


def test_sliding_pairs_count():
    """The closed form for the sliding window against a brute-force count."""
    L = [1, 5, 64, 300, 0]
    off = offsets_from_lengths(L)
    for w in (1, 7, 64, 256, 1000):
        n = sum(1 for Ls in L for i in range(Ls) for j in range(Ls) if i - w < j <= i)
        assert wl.attended_pairs(np.diff(off), np.diff(off), w, "sliding") == n
        assert attended_pairs(off, off, "softmax", w, "sliding") == n
