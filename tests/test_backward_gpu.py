"""GPU parity of the backward (jagged_attn_bwd) against the float64 oracle
(oracle.gdpa_backward) on the same inputs: every variant, window kind, head
dim and input dtype, softmax and GELU scores, with empty and ragged samples."""
import sys

import numpy as np
import pytest
import torch

import oracle
from recsys_jagged_attention_amd import backward
from recsys_jagged_attention_amd.inputs import random_jagged, make_workload

pytestmark = pytest.mark.gpu

# max |grad - ref| <= tol * max(max |ref|, 1) per tensor; the inputs are unit
# normal.  fp32 inputs run in fp32 arithmetic throughout (1e-5).  bf16 inputs
# run on bf16 MFMA with the score weights (P, or gelu(S)/Lk) and dS rounded to
# bf16 (relative error up to 2^-8 per element, as P in the bf16 forward), so
# they take the bf16 forward's 1e-2.
def tol(dtype, act):
    return 1e-5 if dtype == "f32" else 1e-2


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run(variant, window, dtype, qo, ko, q, k, v, seed=0, act="softmax"):
    dout = np.random.default_rng(seed).standard_normal(q.shape).astype(np.float32)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    tq, tk, tv, tg = (torch.from_numpy(x).to(dt) for x in (q, k, v, dout))
    exact = [t.to(torch.float64).numpy() for t in (tq, tk, tv, tg)]
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    dq, dk, dv = backward(tq.cuda(), tk.cuda(), tv.cuda(), tg.cuda(), to(qo), to(ko), variant=variant,
                          act=act, window=window, dtype=dtype, check=True)
    torch.cuda.synchronize()
    ref = oracle.gdpa_backward(exact[0], exact[1], exact[2], exact[3], qo, ko, variant, act, window)
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        g = g.cpu().numpy().astype(np.float64)
        # (a gradient that is exactly zero -- dQ, dK with one key per query --
        # is compared against the inputs' unit scale instead)
        if r.size == 0:  # (no rows: an empty gradient)
            assert g.size == 0, name
            continue
        scale = max(np.abs(r).max(), 1.0)
        err = np.abs(g - r).max() / scale
        assert np.isfinite(g).all(), name
        log(f"  {name}: rel err {err:.3e}")
        assert err <= tol(dtype, act), f"{name}: rel err {err:.3e}"
    return dq


EDGE = [0, 1, 31, 64, 65, 129, 200]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("variant,window", [("self", 0), ("self", 64), ("self", 256), ("sliding", 1),
                                            ("sliding", 40), ("sliding", 300)])
def test_self_variants(variant, window, D, dtype):
    qo, ko, q, k, v = random_jagged(D + window, EDGE, EDGE, 2, D)
    log(f"backward {variant} W={window} D={D} {dtype}")
    run(variant, window, dtype, qo, ko, q, k, v, seed=window)


@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("variant,act", [("self", "softmax"), ("cross", "softmax"), ("cross", "gelu_tanh")])
def test_long_key_runs(variant, act, D):
    """Key runs of 128 or more on average: the MFMA dK/dV kernel's 4-wave,
    128-key-item shape (shorter runs and windows take the 2-wave shape, which
    the edge-length cases cover)."""
    lq = [300, 129, 0, 200, 513]
    lk = lq if variant == "self" else [260, 1, 0, 190, 400]
    qo, ko, q, k, v = random_jagged(60 + D, lq, lk, 2, D)
    log(f"backward long key runs {variant} {act} D={D}")
    run(variant, 0, "bf16", qo, ko, q, k, v, seed=9, act=act)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_empty_key_or_query_tensors(dtype):
    """No key rows at all (dQ is zero, dK and dV are empty) and no query rows
    at all (dK and dV are zero): empty tensors, whose data pointers may be
    null, are accepted as in the forward."""
    qo, ko, q, k, v = random_jagged(71, [5, 40], [0, 0], 2, 64)
    log(f"backward cross without keys {dtype}")
    run("cross", 0, dtype, qo, ko, q, k, v, seed=11)
    qo, ko, q, k, v = random_jagged(72, [0, 0], [10, 70], 2, 64)
    log(f"backward cross without queries {dtype}")
    run("cross", 0, dtype, qo, ko, q, k, v, seed=12)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_cross_and_pma(dtype):
    qo, ko, q, k, v = random_jagged(41, [300, 0, 17, 64], [40, 9, 0, 1], 2, 64)
    run("cross", 0, dtype, qo, ko, q, k, v, seed=1)
    qo, ko, q, k, v = random_jagged(42, [32, 32, 32], [500, 1, 0], 2, 64)
    run("pma", 0, dtype, qo, ko, q, k, v, seed=2)


def test_block_window_workload_slice():
    """A slice of the block-window workload (long samples, D = 128, bf16)."""
    w = make_workload("block_window", scale=0.06)
    log(f"backward block_window slice B={w.B} N={w.total_q}")
    run("self", w.window, "bf16", w.q_offsets, w.kv_offsets, w.q, w.k, w.v, seed=3)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [32, 64, 128])
def test_gelu_cross_pma_self(D, dtype):
    """GELU scores with QK-RMSNorm: cross (long Q, short K/V), PMA and full self."""
    qo, ko, q, k, v = random_jagged(50 + D, [300, 0, 17, 64, 129], [40, 9, 0, 1, 64], 2, D)
    log(f"backward gelu cross D={D} {dtype}")
    run("cross", 0, dtype, qo, ko, q, k, v, seed=4, act="gelu_tanh")
    qo, ko, q, k, v = random_jagged(51 + D, [32, 32, 32], [500, 1, 0], 2, D)
    log(f"backward gelu pma D={D} {dtype}")
    run("pma", 0, dtype, qo, ko, q, k, v, seed=5, act="gelu_tanh")
    qo, ko, q, k, v = random_jagged(52 + D, EDGE, EDGE, 2, D)
    log(f"backward gelu self D={D} {dtype}")
    run("self", 0, dtype, qo, ko, q, k, v, seed=6, act="gelu_tanh")


def test_cross_gelu_workload_slice():
    """A slice of the cross-GELU workload (long Q, 16-64 keys, D = 128, bf16)."""
    w = make_workload("cross_gelu", scale=0.02)
    log(f"backward cross_gelu slice B={w.B} Nq={w.total_q} Nk={w.total_kv}")
    run("cross", 0, "bf16", w.q_offsets, w.kv_offsets, w.q, w.k, w.v, seed=7, act="gelu_tanh")


@pytest.mark.parametrize("name", ["block_window", "full_self", "cross_gelu", "sliding_window", "pma"])
def test_full_size_sampled(name):
    """The whole workload at its full size, in the launch configuration the
    benchmark times; the oracle recomputes dQ, dK, dV of a few (sample, head)
    pairs -- the longest sample among them -- and every element of those is
    compared."""
    from recsys_jagged_attention_amd.inputs import cast_values

    w = make_workload(name)
    lq, lk = np.diff(w.q_offsets), np.diff(w.kv_offsets)
    rng = np.random.default_rng(11)
    picks = {(int(np.argmax(lq * np.maximum(lk, 1))), int(rng.integers(w.H)))}
    while len(picks) < 3:
        picks.add((int(rng.integers(w.B)), int(rng.integers(w.H))))
    log(f"backward full-size {name}: B={w.B} Nq={w.total_q} Nk={w.k.shape[0]} pairs {sorted(picks)}")
    dout = np.random.default_rng(12).standard_normal(w.q.shape).astype(np.float32)
    dt = torch.bfloat16
    tq, tk, tv, tg = (torch.from_numpy(x).to(dt).cuda() for x in (w.q, w.k, w.v, dout))
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    dq, dk, dv = backward(tq, tk, tv, tg, to(w.q_offsets), to(w.kv_offsets), variant=w.variant, act=w.act,
                          window=w.window, dtype="bf16", check=True)
    torch.cuda.synchronize()
    dq, dk, dv = (t.cpu().numpy().astype(np.float64) for t in (dq, dk, dv))
    q, k, v, g = (cast_values(x, "bf16").astype(np.float64) for x in (w.q, w.k, w.v, dout))
    for b, h in sorted(picks):
        qs = slice(w.q_offsets[b], w.q_offsets[b + 1])
        ks = slice(w.kv_offsets[b], w.kv_offsets[b + 1])
        if w.act == "softmax":
            ref = oracle.attention_dense_bwd(q[qs, h], k[ks, h], v[ks, h], g[qs, h], w.window, w.variant)
        else:
            ref = oracle.attention_dense_gelu_bwd(q[qs, h], k[ks, h], v[ks, h], g[qs, h])
        for nm, got, r in zip(("dq", "dk", "dv"), (dq[qs, h], dk[ks, h], dv[ks, h]), ref):
            err = np.abs(got - r).max() / max(np.abs(r).max(), 1.0) if r.size else 0.0
            log(f"  sample {b} head {h} {nm}: rel err {err:.3e}")
            assert np.isfinite(got).all() and err <= tol("bf16", w.act), f"{nm} b={b} h={h}: {err:.3e}"


@pytest.mark.parametrize("variant,act,window,dtype", [
    ("self", "softmax", 256, "bf16"), ("self", "softmax", 0, "bf16"), ("sliding", "softmax", 100, "bf16"),
    ("cross", "gelu_tanh", 0, "bf16"), ("pma", "softmax", 0, "bf16"), ("self", "softmax", 128, "f32"),
    ("cross", "softmax", 0, "f32")])
def test_every_gradient_element_written_once_and_repeatable(variant, act, window, dtype):
    """dQ, dK and dV in NaN-filled buffers with NaN guard bands on both sides:
    every element is written (rows of samples without keys, and keys no query
    sees, get zeros), nothing is written outside, and two calls give bitwise
    equal gradients (no atomics, a fixed order)."""
    lq = [0, 1, 65, 200, 3] if variant != "pma" else [32, 32, 32, 32, 32]
    lk = [5, 0, 130, 64, 1] if variant in ("cross", "pma") else lq
    qo, ko, q, k, v = random_jagged(17, lq, lk, 2, 64)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    tq, tk, tv = (torch.from_numpy(x).to(dt).cuda() for x in (q, k, v))
    tg = torch.from_numpy(np.random.default_rng(5).standard_normal(q.shape).astype(np.float32)).to(dt).cuda()
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    pad = 4096
    runs = []
    for rep in range(2):
        bigs = [torch.full((t.numel() + 2 * pad,), float("nan"), dtype=torch.float32, device="cuda")
                for t in (tq, tk, tv)]
        outs = tuple(b[pad:pad + t.numel()].view(t.shape) for b, t in zip(bigs, (tq, tk, tv)))
        backward(tq, tk, tv, tg, to(qo), to(ko), variant=variant, act=act, window=window, dtype=dtype,
                 check=True, out=outs)
        torch.cuda.synchronize()
        for name, b, o in zip(("dq", "dk", "dv"), bigs, outs):
            assert torch.isnan(b[:pad]).all() and torch.isnan(b[-pad:]).all(), f"{name}: write outside"
            assert not torch.isnan(o).any(), f"{name}: an element was not written"
        runs.append([o.clone() for o in outs])
    log(f"{variant} {act} W={window} {dtype}: every element written, repeatable")
    for a, b in zip(*runs):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
