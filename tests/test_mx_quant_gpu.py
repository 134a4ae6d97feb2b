"""GPU parity of the device MX quantiser (jagged_attn_mx_quantize) against the
oracle's encoder: codes and scales bit-exact."""
import sys

import numpy as np
import pytest
import torch

import oracle
from recsys_jagged_attention_amd import mx_quantize, forward
from recsys_jagged_attention_amd.inputs import make_workload, device_tensors

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check(x32: np.ndarray, dtype: str):
    """x32 float32 [..., D]: quantise on the GPU (as float32 or bf16) and compare
    with the oracle on the exact input values."""
    t = torch.from_numpy(np.ascontiguousarray(x32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    exact = t.to(torch.float64).numpy()
    codes, scales = mx_quantize(t.cuda())
    torch.cuda.synchronize()
    rc, rs = oracle.mx_encode(exact)
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    bad_s = np.argwhere(got_s != rs)
    assert bad_s.size == 0, f"scales differ at {bad_s[:5].tolist()}: {got_s[tuple(bad_s[0])]} vs {rs[tuple(bad_s[0])]}"
    bad = np.argwhere(got_c != rc)
    assert bad.size == 0, (f"codes differ at {bad[:5].tolist()}: got {got_c[tuple(bad[0])]:#x} "
                           f"want {rc[tuple(bad[0])]:#x} for x={exact[tuple(bad[0])]!r}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(1, 1, 32), (37, 3, 64), (1000, 2, 128), (513, 96)])
def test_random_blocks(dtype, shape):
    rng = np.random.default_rng(hash(shape) % 1000 + (dtype == "f32"))
    x = rng.standard_normal(shape).astype(np.float32)
    x *= np.exp2(rng.integers(-30, 30, size=shape[:-1] + (1,))).astype(np.float32)
    log(f"mx quantise {dtype} {shape}")
    check(x, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_special_blocks(dtype):
    """All-zero and negative-zero blocks, saturating blocks (scaled max in
    (448, 512)), huge and tiny scales, and values exactly halfway between e4m3
    steps (ties to even) and between subnormal steps."""
    rows = []
    rows.append(np.zeros(32))
    rows.append(-np.zeros(32))
    r = np.full(32, 1.0); r[0] = 500.0; rows.append(r)                # 500 -> scale 2^0, saturates
    r = np.linspace(-511, 511, 32); rows.append(r)
    r = np.full(32, 3.0e38); rows.append(r)                            # largest scales
    r = np.full(32, 2.0 ** -100); r[3] = 2.0 ** -110; rows.append(r)  # tiny but normal
    grid = oracle.e4m3_grid()
    mids = (grid[1:] + grid[:-1]) / 2
    for i in range(0, len(mids), 31):
        r = np.zeros(32)
        r[0] = 256.0                                                   # scale 2^0: values are e4m3 steps
        r[1:1 + len(mids[i:i + 31])] = mids[i:i + 31]
        rows.append(r)
        rows.append(-r)
    x = np.array(rows, dtype=np.float32).reshape(len(rows), 1, 32)
    if dtype == "bf16":
        # bf16 cannot hold every midpoint; keep the rows whose values survive the cast
        keep = [i for i in range(len(x)) if np.array_equal(
            torch.from_numpy(x[i]).to(torch.bfloat16).to(torch.float32).numpy(), x[i])]
        x = x[keep]
    check(x, dtype)


def test_subnormal_inputs_f32():
    """Blocks whose values (and max) are float32 subnormals get scale 2^-127;
    their codes come from x * 2^127."""
    x = np.zeros((4, 1, 32), dtype=np.float32)
    x[0, 0, :] = np.float32(2.0 ** -130)
    x[1, 0, :] = np.float32(2.0 ** -149) * np.arange(32, dtype=np.float32)
    x[2, 0, 5] = np.float32(-(2.0 ** -127))
    x[3, 0, :] = np.float32(2.0 ** -126) * 1.5
    check(x, "f32")


def test_device_quantised_inputs_drive_the_mxfp8_forward():
    """The mxfp8 forward on device-quantised q/k/v equals the forward on the
    host-encoded inputs (the codes are identical)."""
    w = make_workload("mxfp8_window", scale=0.05)
    q, k, v, qo, ko, sc = device_tensors(w, "cuda")
    out_host = forward(q, k, v, qo, ko, variant=w.variant, act=w.act, window=w.window, dtype="mxfp8", scales=sc)
    qs, ks, vs = (torch.from_numpy(x).cuda() for x in (w.q, w.k, w.v))
    (q2, s2), (k2, t2), (v2, u2) = mx_quantize(qs), mx_quantize(ks), mx_quantize(vs)
    out_dev = forward(q2, k2, v2, qo, ko, variant=w.variant, act=w.act, window=w.window, dtype="mxfp8",
                      scales=(s2, t2, u2))
    torch.cuda.synchronize()
    assert torch.equal(q2, q) and torch.equal(s2, sc[0])
    assert torch.equal(out_dev, out_host)


def test_full_size_block_window_tensors():
    w = make_workload("block_window")
    for name, x in (("q", w.q), ("k", w.k), ("v", w.v)):
        log(f"mx quantise full-size {name} {x.shape}")
        check(x, "bf16")
