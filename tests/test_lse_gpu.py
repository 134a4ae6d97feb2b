"""GPU parity of the forward's log-sum-exp output (ja_io.lse) against the
oracle's (oracle.gdpa_lse, pinned in test_oracle_lse.py), on the same
dequantised inputs.

Tolerance: both sides see the same input values, so the difference is fp32
arithmetic only: scores accumulated in fp32, exp2 within 1 ulp, a row sum of
at most a few thousand fp32 terms (relative error below 2^-24 per term added,
well under 1e-4 in total) and log2 within 1 ulp.  |lse_gpu - lse_ref| <= 2e-4
(+ 1e-6 |lse_ref|) bounds that with margin.  Rows without keys are -inf on
both sides, nothing is written outside the buffer (NaN guard bands), and
asking for the log-sum-exp leaves the output bit for bit as it is without
it."""
import sys

import numpy as np
import pytest
import torch

import oracle
from recsys_jagged_attention_amd import forward
from recsys_jagged_attention_amd.inputs import Workload, make_workload, random_jagged, device_tensors, mx_encode_e4m3
from parity_util import oracle_values

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-4, 1e-6


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def adhoc(variant, dtype, lq, lk, H, D, window=0, seed=0):
    qo, ko, q, k, v = random_jagged(seed, lq, lk, H, D)
    w = Workload(f"lse_{variant}", variant, "softmax", dtype, len(lq), H, D, window, qo, ko, q, k, v, seed)
    if dtype == "mxfp8":
        w.mx = {n: mx_encode_e4m3(x) for n, x in (("q", q), ("k", k), ("v", v))}
    return w


PAD = 4096  # NaN guard band on each side of the log-sum-exp buffer


def run(w, with_lse=True):
    q, k, v, qo, ko, scales = device_tensors(w, "cuda")
    lse = None
    if with_lse:
        n = w.total_q * w.H
        big = torch.full((n + 2 * PAD,), float("nan"), dtype=torch.float32, device="cuda")
        lse = big[PAD:PAD + n].view(w.total_q, w.H)
    out = forward(q, k, v, qo, ko, variant=w.variant, act=w.act, window=w.window, dtype=w.dtype,
                  scales=scales, check=True, lse=lse)
    torch.cuda.synchronize()
    if with_lse:
        assert torch.isnan(big[:PAD]).all() and torch.isnan(big[-PAD:]).all(), "log-sum-exp written outside"
    return out.cpu(), (lse.cpu().numpy().astype(np.float64) if with_lse else None)


def check_lse(w):
    out, got = run(w)
    q, k, _ = oracle_values(w)
    ref = oracle.gdpa_lse(q, k, w.q_offsets, w.kv_offsets, w.variant, w.window)
    assert got.shape == ref.shape
    assert not np.any(np.isnan(got)), "rows left unwritten"
    empty = ref == -np.inf
    assert np.array_equal(got == -np.inf, empty), "-inf rows differ"
    fin = ~empty
    assert np.all(np.isfinite(got[fin]))
    err = np.abs(got[fin] - ref[fin])
    bound = ATOL + RTOL * np.abs(ref[fin])
    worst = float(err.max()) if err.size else 0.0
    assert np.all(err <= bound), f"{w.name}: max |lse err| {worst:.3e}"
    # the output does not change when the log-sum-exp is asked for
    out0, _ = run(w, with_lse=False)
    assert torch.equal(out, out0)
    return worst


SELF_LENS = [0, 1, 31, 65, 129, 200, 300]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [32, 64, 128])
def test_lse_self_full(dtype, D):
    w = adhoc("self", dtype, SELF_LENS, SELF_LENS, 2, D, seed=D)
    log(f"lse self full {dtype} D={D}")
    log(f"  max err {check_lse(w):.3e}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("window", [64, 128, 256, 512])
def test_lse_self_block_window(dtype, window):
    """Windows of 1 to 4 blocks (the tile stream's pipeline) and 8 blocks."""
    w = adhoc("self", dtype, [0, 1, 70, 300, 513, 64], [0, 1, 70, 300, 513, 64], 2, 128, window, seed=window)
    log(f"lse self window {dtype} W={window}")
    log(f"  max err {check_lse(w):.3e}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("window", [1, 37, 200])
def test_lse_sliding(dtype, window):
    w = adhoc("sliding", dtype, [0, 1, 70, 300, 129], [0, 1, 70, 300, 129], 2, 64, window, seed=window + 3)
    log(f"lse sliding {dtype} W={window}")
    log(f"  max err {check_lse(w):.3e}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
def test_lse_cross_with_keyless_samples(dtype, D):
    """Samples without keys give -inf rows (the tile stream's zero-row path)."""
    w = adhoc("cross", dtype, [3, 0, 90, 200, 65, 40], [70, 5, 0, 300, 1, 0], 2, D, seed=D + 5)
    log(f"lse cross {dtype} D={D}")
    log(f"  max err {check_lse(w):.3e}")


@pytest.mark.parametrize("dtype", ["bf16", "mxfp8"])
@pytest.mark.parametrize("D", [64, 128])
def test_lse_pma_key_split(dtype, D):
    """The key-split shape: samples long enough to be split (the merge writes
    the log-sum-exp), short ones taken whole (the attention kernel writes it),
    and a sample without keys (-inf)."""
    w = adhoc("pma", dtype, [32, 32, 32, 32, 32], [0, 100, 1500, 4100, 33], 2, D, seed=D + 13)
    log(f"lse pma {dtype} D={D}")
    log(f"  max err {check_lse(w):.3e}")


def test_lse_f32_pma():
    w = adhoc("pma", "f32", [32, 32, 32, 32], [0, 100, 700, 33], 2, 64, seed=11)
    log("lse f32 pma")
    log(f"  max err {check_lse(w):.3e}")


@pytest.mark.parametrize("window", [0, 128, 256])
def test_lse_mxfp8_self(window):
    w = adhoc("self", "mxfp8", [0, 1, 70, 300, 513], [0, 1, 70, 300, 513], 2, 128, window, seed=window + 1)
    log(f"lse mxfp8 self W={window}")
    log(f"  max err {check_lse(w):.3e}")


@pytest.mark.parametrize("name", ["block_window", "full_self", "sliding_window", "pma"])
def test_lse_full_size(name):
    """The softmax workloads at their full sizes, every row against the oracle."""
    w = make_workload(name)
    log(f"lse full size {name} B={w.B} Nq={w.total_q}")
    log(f"  max err {check_lse(w):.3e}")
