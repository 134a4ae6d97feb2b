"""Seeded random shapes through the whole path: the forward, its log-sum-exp
and the backward (with the forward's statistics handed in, and recomputed),
each against the float64 oracle on the same inputs.

Every case draws a variant (self with or without a block window, sliding,
cross, PMA), a head dim, an input dtype, the number of heads and ragged
sample lengths that include empty samples, single rows and lengths either
side of the 64-row tile.  The shapes are small enough for the oracle to
finish in seconds; the bounds are the per-path ones used elsewhere: output
1e-5 (fp32) / 1e-2 (bf16) of max|O_ref|, log-sum-exp 2e-4 absolute,
gradients 1e-5 / 1e-2 of max(max|ref|, 1)."""
import sys

import numpy as np
import pytest
import torch

import oracle
from recsys_jagged_attention_amd import forward, backward
from recsys_jagged_attention_amd.inputs import random_jagged, rng_for
from parity_util import TOL

pytestmark = pytest.mark.gpu

LENGTHS = [0, 1, 2, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 200, 257, 300]


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def draw(seed):
    rng = rng_for(1000 + seed)
    variant = ["self", "self_window", "sliding", "cross", "pma"][int(rng.integers(5))]
    D = int(rng.choice([32, 64, 128]))
    dtype = ["bf16", "f32"][int(rng.integers(2))]
    H = int(rng.integers(1, 4))
    B = int(rng.integers(1, 9))
    window = 0
    if variant == "pma":
        lq = [32] * B
        lk = [int(rng.choice(LENGTHS + [700, 1500])) for _ in range(B)]
    elif variant == "cross":
        lq = [int(rng.choice(LENGTHS)) for _ in range(B)]
        lk = [int(rng.choice([0, 1, 16, 40, 64, 65])) for _ in range(B)]
    else:
        lq = [int(rng.choice(LENGTHS)) for _ in range(B)]
        lk = lq
        if variant == "self_window":
            window = 64 * int(rng.integers(1, 6))
        elif variant == "sliding":
            window = int(rng.choice([1, 7, 64, 100, 300]))
    if sum(lq) == 0:
        lq[0] = 33
        if variant in ("self_window", "sliding", "self"):
            lk = lq
    v = "self" if variant == "self_window" else variant
    return v, window, D, dtype, H, lq, lk


def rel(got, ref, floor=0.0):
    if ref.size == 0:
        assert got.size == 0
        return 0.0
    scale = max(float(np.abs(ref).max()), floor)
    if scale == 0.0:
        return float(np.abs(got).max()) if got.size else 0.0
    return float(np.abs(got - ref).max()) / scale


@pytest.mark.parametrize("seed", range(16))
def test_random_shape_forward_lse_backward(seed):
    variant, window, D, dtype, H, lq, lk = draw(seed)
    log(f"seed {seed}: {variant} W={window} D={D} {dtype} H={H} lq={lq} lk={lk}")
    qo, ko, q, k, v = random_jagged(seed + 77, lq, lk, H, D)
    dout = rng_for(seed + 5).standard_normal(q.shape).astype(np.float32)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    tq, tk, tv, tg = (torch.from_numpy(x).to(tdt) for x in (q, k, v, dout))
    exact = [t.to(torch.float64).numpy() for t in (tq, tk, tv, tg)]
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    dq_, dk_, dv_, dg, dqo, dko = tq.cuda(), tk.cuda(), tv.cuda(), tg.cuda(), to(qo), to(ko)

    lse = torch.empty((q.shape[0], H), dtype=torch.float32, device="cuda")
    out = forward(dq_, dk_, dv_, dqo, dko, variant=variant, act="softmax", window=window, dtype=dtype,
                  check=True, lse=lse)
    g_saved = backward(dq_, dk_, dv_, dg, dqo, dko, variant=variant, window=window, dtype=dtype, check=True,
                       lse=lse, fwd_out=out)
    g_recomp = backward(dq_, dk_, dv_, dg, dqo, dko, variant=variant, window=window, dtype=dtype, check=True)
    torch.cuda.synchronize()

    ref = oracle.gdpa_forward(exact[0], exact[1], exact[2], qo, ko, variant, "softmax", window)
    err = rel(out.float().cpu().numpy().astype(np.float64), ref)
    log(f"  out rel err {err:.3e}")
    assert err <= TOL[dtype]

    ref_lse = oracle.gdpa_lse(exact[0], exact[1], qo, ko, variant, window)
    got_lse = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(got_lse == -np.inf, ref_lse == -np.inf), "-inf rows differ"
    fin = ref_lse != -np.inf
    lerr = float(np.abs(got_lse[fin] - ref_lse[fin]).max()) if fin.any() else 0.0
    log(f"  lse abs err {lerr:.3e}")
    assert lerr <= 2e-4 + 1e-6 * float(np.abs(ref_lse[fin]).max() if fin.any() else 0.0)

    gref = oracle.gdpa_backward(exact[0], exact[1], exact[2], exact[3], qo, ko, variant, "softmax", window)
    gtol = 1e-5 if dtype == "f32" else 1e-2
    for form, grads in (("saved", g_saved), ("recomputed", g_recomp)):
        for name, g, r in zip(("dq", "dk", "dv"), grads, gref):
            e = rel(g.cpu().numpy().astype(np.float64), r, floor=1.0)
            log(f"  {form} {name} rel err {e:.3e}")
            assert np.isfinite(g.cpu().numpy()).all(), f"{form} {name} not finite"
            assert e <= gtol, f"{form} {name}: {e:.3e}"


def draw_other(seed):
    """GELU scores (no window) and MXFP8 inputs."""
    rng = rng_for(2000 + seed)
    kind = ["gelu", "mx"][seed % 2]
    kinds = ["self", "cross", "pma"] if kind == "gelu" else ["self", "self_window", "cross", "pma"]
    variant = kinds[int(rng.integers(len(kinds)))]
    D = int(rng.choice([32, 64, 128]))
    H = int(rng.integers(1, 4))
    B = int(rng.integers(1, 9))
    window = 64 * int(rng.integers(1, 9)) if variant == "self_window" else 0
    if variant == "pma":
        lq = [32] * B
        lk = [int(rng.choice(LENGTHS + [700, 1500])) for _ in range(B)]
    elif variant == "cross":
        lq = [int(rng.choice(LENGTHS)) for _ in range(B)]
        lk = [int(rng.choice([0, 1, 16, 40, 64, 65])) for _ in range(B)]
        if sum(lq) == 0:
            lq[0] = 33
    else:
        lq = [int(rng.choice(LENGTHS)) for _ in range(B)]
        if sum(lq) == 0:
            lq[0] = 33
        lk = lq
    act = "gelu_tanh" if kind == "gelu" else ["softmax", "gelu_tanh"][int(rng.integers(2))]
    if window:
        act = "softmax"
    dtype = ["bf16", "f32"][int(rng.integers(2))] if kind == "gelu" else "mxfp8"
    return ("self" if variant == "self_window" else variant), window, D, dtype, act, H, lq, lk


@pytest.mark.parametrize("seed", range(12))
def test_random_shape_gelu_and_mxfp8(seed):
    """GELU scores (forward and backward) and MXFP8 inputs (forward, and the
    log-sum-exp where the shape gives it) on seeded random shapes."""
    from recsys_jagged_attention_amd import JaggedAttnError, JA_EUNSUPPORTED
    from recsys_jagged_attention_amd.inputs import Workload, mx_encode_e4m3, device_tensors
    from parity_util import full_parity, oracle_values

    variant, window, D, dtype, act, H, lq, lk = draw_other(seed)
    log(f"seed {seed}: {variant} W={window} D={D} {dtype} {act} H={H} lq={lq} lk={lk}")
    qo, ko, q, k, v = random_jagged(seed + 177, lq, lk, H, D)
    w = Workload("random", variant, act, dtype, len(lq), H, D, window, qo, ko, q, k, v, seed)
    if dtype == "mxfp8":
        w.mx = {n: mx_encode_e4m3(x) for n, x in (("q", q), ("k", k), ("v", v))}
    log(f"  out rel err {full_parity(w):.3e}")
    if dtype == "mxfp8" and act == "softmax":
        tq, tk, tv, tqo, tko, scales = device_tensors(w, "cuda")
        lse = torch.empty((w.total_q, H), dtype=torch.float32, device="cuda")
        try:
            forward(tq, tk, tv, tqo, tko, variant=variant, act=act, window=window, dtype=dtype, scales=scales,
                    check=True, lse=lse)
        except JaggedAttnError as e:
            assert e.status == JA_EUNSUPPORTED
            log("  (no log-sum-exp for this MXFP8 shape)")
        else:
            oq, ok_, _ = oracle_values(w)
            ref = oracle.gdpa_lse(oq, ok_, qo, ko, variant, window)
            got = lse.cpu().numpy().astype(np.float64)
            assert np.array_equal(got == -np.inf, ref == -np.inf)
            fin = ref != -np.inf
            lerr = float(np.abs(got[fin] - ref[fin]).max()) if fin.any() else 0.0
            log(f"  lse abs err {lerr:.3e}")
            assert lerr <= 2e-4 + 1e-6 * float(np.abs(ref[fin]).max() if fin.any() else 0.0)
    if act == "gelu_tanh" and dtype != "mxfp8":
        dout = rng_for(seed + 9).standard_normal(q.shape).astype(np.float32)
        tdt = torch.float32 if dtype == "f32" else torch.bfloat16
        tq, tk, tv, tg = (torch.from_numpy(x).to(tdt) for x in (q, k, v, dout))
        exact = [t.to(torch.float64).numpy() for t in (tq, tk, tv, tg)]
        to = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
        grads = backward(tq.cuda(), tk.cuda(), tv.cuda(), tg.cuda(), to(qo), to(ko), variant=variant, act=act,
                         dtype=dtype, check=True)
        torch.cuda.synchronize()
        gref = oracle.gdpa_backward(exact[0], exact[1], exact[2], exact[3], qo, ko, variant, act, 0)
        gtol = 1e-5 if dtype == "f32" else 1e-2
        for name, g, r in zip(("dq", "dk", "dv"), grads, gref):
            e = rel(g.cpu().numpy().astype(np.float64), r, floor=1.0)
            log(f"  {name} rel err {e:.3e}")
            assert np.isfinite(g.cpu().numpy()).all() and e <= gtol, f"{name}: {e:.3e}"
