"""The device-side work enumeration, read back from the workspace.

The plan kernel writes the work items of a call into the workspace (a 256-byte
header -- status, item count, partial slots, byte offset of the item list --
then 32-byte records {b, h, q0, split, qbeg, lq, kbeg, lk}).  These tests copy
that list back after a forward call and compare it with a brute-force host
enumeration of the same schedule: every (sample, head, query tile, key split)
with at least one query row appears exactly once, samples without query rows
give none, and each record carries its sample's offsets.  Where the items are
placed in cost order (tile stream, key split, MX window), the key tiles each
item walks never increase along the list (the techfeed.io summary of "GEM
Training: ...", section "Generalized Dot-Product Attention（GDPA）": only valid
tiles, empty ones skipped, skewed work balanced)."""
import numpy as np
import pytest
import torch

from recsys_jagged_attention_amd import forward, Workspace
from recsys_jagged_attention_amd.inputs import Workload, random_jagged, device_tensors, mx_encode_e4m3

pytestmark = pytest.mark.gpu
BLOCK = 64


def adhoc(variant, act, dtype, lq, lk, H, D, window=0, seed=0):
    qo, ko, q, k, v = random_jagged(seed, lq, lk, H, D)
    w = Workload("sched", variant, act, dtype, len(lq), H, D, window, qo, ko, q, k, v, seed)
    if dtype == "mxfp8":
        w.mx = {n: mx_encode_e4m3(x) for n, x in (("q", q), ("k", k), ("v", v))}
    return w


def key_chunk(H, total_kv):
    """The key chunk of the key-split (PMA) schedule: the smallest power of two
    from 512 to 8192 keys that gives at most about 2048 items."""
    target = -(-H * total_kv // 2048)
    kvc = 512
    while kvc < target and kvc < 8192:
        kvc *= 2
    return kvc


def schedule(w):
    """(query rows per item, key chunk or 0, cost-ordered) of the library's schedule."""
    if w.dtype == "f32":
        return 64, 0, False
    if w.variant == "pma":
        return 32, key_chunk(w.H, w.total_kv), True
    tile_stream = w.dtype == "bf16" or (w.D == 128 and w.variant == "self" and w.act == "softmax"
                                        and w.window <= 4 * BLOCK)
    if tile_stream:
        if w.variant == "self" and 0 < w.window <= 4 * BLOCK:
            return 1024, 0, True       # block-window pipeline: runs of 16 query blocks
        return 256, 0, True            # tile stream
    if w.window > 0:
        return 128, 0, True            # MX window kernel, dealt by cost
    if w.variant == "self" and w.act == "softmax":
        return 256, 0, False
    return 128, 0, False


def expected_items(w, bm, kvc):
    qo, ko = w.q_offsets.astype(np.int64), w.kv_offsets.astype(np.int64)
    items = []
    for b in range(w.B):
        lq, lk = int(qo[b + 1] - qo[b]), int(ko[b + 1] - ko[b])
        if lq == 0:
            continue
        nqt = -(-lq // bm)
        ns = -(-lk // kvc) if (kvc and nqt == 1 and lk > kvc) else 1
        for h in range(w.H):
            for t in range(nqt):
                for sp in range(ns):
                    items.append((b, h, t * bm, sp, int(qo[b]), lq, int(ko[b]), lk))
    return items


def walked_tiles(w, it, bm, kvc):
    """Key tiles an item walks (the cost the plan sorts by; costs of 1023
    tiles and more share the top bucket)."""
    return min(_walked_tiles(w, it, bm, kvc), 1023)


def _walked_tiles(w, it, bm, kvc):
    b, h, q0, sp, qbeg, lq, kbeg, lk = it
    if kvc and -(-lq // bm) == 1 and lk > kvc:
        keys = min(kvc, lk - sp * kvc)
        return -(-keys // BLOCK)
    te, tl = -(-lk // BLOCK), 0
    if w.window > 0 and w.variant == "self":
        te = min(te, -(-min(q0 + bm, lq) // BLOCK))
        tl = max(0, q0 // BLOCK - w.window // BLOCK + 1)
    elif w.variant == "sliding":
        te = min(te, -(-min(q0 + bm, lq) // BLOCK))
        tl = max(0, q0 - w.window + 1) // BLOCK
    return max(te - tl, 0)


def device_items(w):
    q, k, v, qo, ko, scales = device_tensors(w, "cuda")
    ws = Workspace("cuda")
    forward(q, k, v, qo, ko, variant=w.variant, act=w.act, window=w.window, dtype=w.dtype, scales=scales,
            workspace=ws, check=True)
    torch.cuda.synchronize()
    raw = ws.buf.cpu().numpy()
    hdr = raw[:256].view(np.int32)
    status, n_items, items_off = int(hdr[0]), int(hdr[1]), int(hdr[3])
    assert status == 0
    rec = raw[items_off:items_off + 32 * n_items].view(np.int32).reshape(n_items, 8)
    return [tuple(int(x) for x in r) for r in rec]


CASES = {
    # name: (variant, act, dtype, lq, lk, H, D, window)
    "tile_stream_cross": ("cross", "gelu_tanh", "bf16", [0, 1, 300, 700, 0, 256, 2000, 5],
                          [10, 0, 64, 3, 7, 70, 1, 0], 3, 64, 0),
    "tile_stream_self": ("self", "softmax", "bf16", [0, 1, 255, 256, 257, 2049, 0, 64], None, 2, 32, 0),
    "block_pipeline": ("self", "softmax", "bf16", [0, 1, 64, 65, 1024, 1025, 3000, 0, 200], None, 2, 32, 256),
    "block_window_long": ("self", "softmax", "bf16", [0, 700, 1500, 64, 0, 300], None, 2, 32, 512),
    "sliding": ("sliding", "softmax", "bf16", [0, 1, 300, 1000, 0, 513], None, 2, 32, 100),
    "key_split": ("pma", "softmax", "bf16", [32, 32, 0, 7, 32, 32], [0, 513, 100, 70000, 20000, 64], 4, 64, 0),
    "mx_window": ("self", "softmax", "mxfp8", [0, 1, 128, 129, 700, 0, 64], None, 2, 128, 256),
    "mx_window_long": ("self", "softmax", "mxfp8", [0, 1, 128, 129, 700, 0, 64], None, 2, 128, 512),
    "mx_window_d64": ("self", "softmax", "mxfp8", [0, 1, 128, 129, 700, 0, 64], None, 2, 64, 128),
    "mx_full": ("self", "softmax", "mxfp8", [0, 1, 300, 256, 0], None, 2, 128, 0),
    "mx_cross": ("cross", "softmax", "mxfp8", [0, 1, 300, 256, 9], [5, 0, 70, 200, 1], 2, 128, 0),
    "f32": ("self", "softmax", "f32", [0, 1, 63, 64, 65, 200, 0], None, 2, 32, 0),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_device_items_equal_host_enumeration(case):
    variant, act, dtype, lq, lk, H, D, window = CASES[case]
    w = adhoc(variant, act, dtype, lq, lk if lk is not None else lq, H, D, window=window, seed=len(case))
    bm, kvc, cost_ordered = schedule(w)
    want = expected_items(w, bm, kvc)
    got = device_items(w)
    print(f"{case}: {len(got)} items (expected {len(want)})", flush=True)
    assert len(got) == len(set(got)), "an item appears twice"
    assert sorted(got) == sorted(want)
    empty = {b for b in range(w.B) if w.q_offsets[b + 1] == w.q_offsets[b]}
    assert not any(it[0] in empty for it in got)
    if cost_ordered:
        cost = [walked_tiles(w, it, bm, kvc) for it in got]
        assert all(a >= b for a, b in zip(cost, cost[1:])), "items are not in decreasing cost order"


def test_device_items_many_samples():
    """More samples than the plan kernel has threads (1024): chunked scans and
    carried item counts, in cost order."""
    rng = np.random.Generator(np.random.PCG64(33))
    B = 2600
    L = rng.integers(0, 300, size=B).tolist()
    w = adhoc("self", "softmax", "bf16", L, L, 2, 32, window=128, seed=34)
    bm, kvc, _ = schedule(w)
    got = device_items(w)
    assert sorted(got) == sorted(expected_items(w, bm, kvc))
    cost = [walked_tiles(w, it, bm, kvc) for it in got]
    assert all(a >= b for a, b in zip(cost, cost[1:]))


@pytest.mark.parametrize("window", [0, 256])
def test_device_items_in_kernel_enumeration_at_its_sample_limit(window):
    """511 samples (the most the tile stream enumerates in its own prologue):
    every wave holds samples, and with a block window a sample has up to three
    runs of equal cost.  Skewed lengths put items in many cost buckets; the
    item list must still equal the host enumeration, in cost order."""
    rng = np.random.Generator(np.random.PCG64(41 + window))
    B = 511
    L = np.floor(np.exp(rng.uniform(0.0, np.log(3001.0), size=B))).astype(int)
    L[rng.integers(0, B, size=40)] = 0  # empty samples among them
    L = L.tolist()
    w = adhoc("self", "softmax", "bf16", L, L, 2, 32, window=window, seed=42 + window)
    bm, kvc, _ = schedule(w)
    got = device_items(w)
    want = expected_items(w, bm, kvc)
    assert len(got) == len(set(got)), "an item appears twice"
    assert sorted(got) == sorted(want)
    cost = [walked_tiles(w, it, bm, kvc) for it in got]
    assert all(a >= b for a, b in zip(cost, cost[1:])), "items are not in decreasing cost order"
