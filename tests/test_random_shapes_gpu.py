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
