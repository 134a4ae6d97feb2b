"""Debug mode (environment variable JA_DEBUG=1): every entry point synchronises
its stream and returns the device status itself, so offset errors reported by
the device come back from jagged_attn_fwd / jagged_attn_bwd /
jagged_attn_fwd_noalloc directly instead of through jagged_attn_check.

The flag is read once per process, so the checks run in a child process with
JA_DEBUG set; each case prints one line the parent checks."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import ctypes, sys
sys.path.insert(0, "tests")
import numpy as np, torch
import oracle
from recsys_jagged_attention_amd import forward, backward, JaggedAttnError, JA_EOFFSETS
from recsys_jagged_attention_amd import _lib
from recsys_jagged_attention_amd.inputs import random_jagged, device_tensors, Workload
from parity_util import rel_err

def line(msg):
    print(msg, flush=True)

qo, ko, q, k, v = random_jagged(3, [5, 70], [9, 40], 2, 32)
w = Workload("debug", "cross", "softmax", "bf16", 2, 2, 32, 0, qo, ko, q, k, v, 3)
tq, tk, tv, dqo, dko, _ = device_tensors(w, "cuda")
bad_q = torch.tensor([0, 9, 80], dtype=torch.int32, device="cuda")  # does not end at total_q (75)

# a valid call returns OK with the right output (no check needed)
out = forward(tq, tk, tv, dqo, dko, variant="cross", act="softmax", check=False)
ref = oracle.gdpa_forward(tq.float().cpu().numpy(), tk.float().cpu().numpy(), tv.float().cpu().numpy(),
                          qo, ko, variant="cross", act="softmax")
line(f"fwd_ok {rel_err(out.float().cpu().numpy(), ref):.3e}")

# bad offsets: the forward itself returns JA_EOFFSETS
try:
    forward(tq, tk, tv, bad_q, dko, variant="cross", act="softmax", check=False)
    line("fwd_bad none")
except JaggedAttnError as e:
    line(f"fwd_bad {e.status} {'jagged_attn_fwd' in str(e)}")

# the backward: both of its plans check the offsets
dout = torch.ones_like(tq)
try:
    backward(tq, tk, tv, dout, bad_q, dko, variant="cross", act="softmax", check=False)
    line("bwd_bad none")
except JaggedAttnError as e:
    line(f"bwd_bad {e.status} {'jagged_attn_bwd' in str(e)}")

# the no-allocation entry point
lib = _lib.load()
io = _lib.JaIo()
io.dtype = _lib.DTYPES["bf16"]
io.total_q = tq.shape[0]
io.total_kv = tk.shape[0]
io.stream = torch.cuda.current_stream().cuda_stream
o2 = torch.empty_like(tq)
rc = lib.jagged_attn_fwd_noalloc(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), bad_q.data_ptr(), dko.data_ptr(),
                                 2, 2, 32, _lib.VARIANTS["cross"], _lib.ACTS["softmax"], 0, o2.data_ptr(),
                                 ctypes.byref(io))
line(f"noalloc_bad {rc}")
rc = lib.jagged_attn_fwd_noalloc(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), dqo.data_ptr(), dko.data_ptr(),
                                 2, 2, 32, _lib.VARIANTS["cross"], _lib.ACTS["softmax"], 0, o2.data_ptr(),
                                 ctypes.byref(io))
line(f"noalloc_ok {rc} {rel_err(o2.float().cpu().numpy(), ref):.3e}")
"""


def test_debug_mode_returns_device_status():
    env = dict(os.environ, JA_DEBUG="1")
    r = subprocess.run([sys.executable, "-c", CHILD], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    print(r.stdout, r.stderr[-2000:], flush=True)
    assert r.returncode == 0
    got = {ln.split()[0]: ln.split()[1:] for ln in r.stdout.splitlines() if ln.strip()}
    assert float(got["fwd_ok"][0]) < 1e-2
    assert got["fwd_bad"] == [str(-5), "True"]
    assert got["bwd_bad"] == [str(-5), "True"]
    assert got["noalloc_bad"] == [str(-5)]
    assert got["noalloc_ok"][0] == "0" and float(got["noalloc_ok"][1]) < 1e-2
