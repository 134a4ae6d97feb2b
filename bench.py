#!/usr/bin/env python3
"""Benchmark of the jagged GDPA forward on one MI355X.

One step = one jagged_attn_fwd call (device-side plan + attention kernel
[+ split merge]) over one batch of seeded synthetic input already resident in
HBM.  Several copies of the batch are cycled so that no step reads data a
previous step left in the 256 MB last-level cache.

Prints ONE JSON line: useful (unpadded) TFLOPS of the whole job, the
roofline of the dominant (attention) kernel timed live with HIP events that
its own dispatch writes (start and end), the step period between consecutive
steps, the float64 CPU oracle timed on a bounded sample of the same workload,
and the error of the last timed step's output against the oracle on that
sample.

  python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload block_window]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_TFLOPS = {"bf16": 2500.0, "mxfp8": 5000.0, "f32": 157.3}  # dense MFMA/vector peaks
PEAK_HBM_GBS = 8000.0
METRIC = "useful TFLOPS (unpadded) & % bf16 MFMA peak, jagged GDPA fwd, 1 MI355X"
KERNEL_NAME = {  # dominant kernel per workload (template instance)
    "tiny_full": "attn_f32_kernel<32,softmax,nowindow>",
    "block_window": "attn_pp_kernel<128,softmax,block_pipeline>",
    "full_self": "attn_pp_kernel<128,softmax>",
    "cross_gelu": "attn_pp_kernel<128,gelu>",
    "pma": "attn_kernel<64,NWQ=1,NWK=4,softmax,bf16,split>",
    "mxfp8_window": "attn_pp_kernel<128,softmax,block_pipeline,mx8>",
    "mxfp8_full": "attn_pp_kernel<128,softmax,mx8>",
    "sliding_window": "attn_pp_kernel<128,softmax,sliding>",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles, created through the HIP runtime."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self) -> int:
        e = ctypes.c_void_p()
        if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, e: int):
        self.hip.hipEventDestroy(ctypes.c_void_p(e))

    def record(self, e: int, stream: int):
        if self.hip.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")


def device_info() -> dict:
    """Compute units and the engine clock the HIP runtime reports (kHz -> MHz)."""
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipDeviceGetAttribute.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.c_int, ctypes.c_int]
    hip.hipGetDevice.argtypes = [ctypes.POINTER(ctypes.c_int)]
    dev = ctypes.c_int()
    hip.hipGetDevice(ctypes.byref(dev))
    info = {}
    # hipDeviceAttribute_t values of the ROCm headers
    for name, attr in (("compute_units", "hipDeviceAttributeMultiprocessorCount"),
                       ("clock_mhz", "hipDeviceAttributeClockRate")):
        v = ctypes.c_int()
        code = HIP_ATTR.get(attr)
        if code is not None and hip.hipDeviceGetAttribute(ctypes.byref(v), code, dev.value) == 0:
            info[name] = v.value // 1000 if name == "clock_mhz" else v.value
    return info


def _hip_attr_codes() -> dict:
    """Enum values of hipDeviceAttribute_t, read from the installed HIP header."""
    import re
    try:
        src = open("/opt/rocm/include/hip/hip_runtime_api.h").read()
    except OSError:
        return {}
    body = src[src.index("typedef enum hipDeviceAttribute_t {") + len("typedef enum hipDeviceAttribute_t {"):]
    body = body[:body.index("} hipDeviceAttribute_t;")]
    body = re.sub(r"//[^\n]*", "", body)
    codes, idx = {}, -1
    for entry in body.split(","):
        entry = entry.strip()
        if not entry:
            continue
        m = re.fullmatch(r"(\w+)\s*(?:=\s*(\w+))?", entry)
        if not m:
            continue
        if m.group(2) is not None:
            g = m.group(2)
            idx = int(g, 0) if g[0].isdigit() else codes[g]
        else:
            idx += 1
        codes[m.group(1)] = idx
    return codes


HIP_ATTR = _hip_attr_codes()


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas"]
        return int(max(n)) if n else 1
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline(w, budget_s: float, gpu_out=None):
    """Time the float64 oracle on whole samples of the workload (seeded order)
    until about budget_s seconds of CPU work; report useful TFLOPS.  With the
    output of a timed GPU step (``gpu_out``, float64 [total_q, H, D]), also
    report max|O_gpu - O_ref| / max|O_ref| over the samples the oracle ran."""
    import oracle
    from recsys_jagged_attention_amd.inputs import cast_values
    from recsys_jagged_attention_amd import workload as wl

    rng = np.random.Generator(np.random.PCG64(w.seed + 7))
    order = rng.permutation(w.B)
    spent, flops, used = 0.0, 0, []
    err_num, ref_max = 0.0, 0.0
    for b in order:
        q0, q1 = int(w.q_offsets[b]), int(w.q_offsets[b + 1])
        k0, k1 = int(w.kv_offsets[b]), int(w.kv_offsets[b + 1])
        if w.dtype == "mxfp8":
            q = oracle.mx_dequantise(w.mx["q"][0][q0:q1], w.mx["q"][1][q0:q1])
            k = oracle.mx_dequantise(w.mx["k"][0][k0:k1], w.mx["k"][1][k0:k1])
            v = oracle.mx_dequantise(w.mx["v"][0][k0:k1], w.mx["v"][1][k0:k1])
        else:
            q, k, v = (cast_values(x, w.dtype).astype(np.float64)
                       for x in (w.q[q0:q1], w.k[k0:k1], w.v[k0:k1]))
        qo, ko = np.array([0, q1 - q0]), np.array([0, k1 - k0])
        t0 = time.perf_counter()
        ref = oracle.gdpa_forward(q, k, v, qo, ko, w.variant, w.act, w.window)
        spent += time.perf_counter() - t0
        if gpu_out is not None and ref.size:
            err_num = max(err_num, float(np.abs(gpu_out[q0:q1] - ref).max()))
            ref_max = max(ref_max, float(np.abs(ref).max()))
        flops += wl.useful_flops([q1 - q0], [k1 - k0], w.H, w.D, w.window, w.variant)
        used.append(int(b))
        if spent >= budget_s:
            break
    res = {
        "value": flops / spent / 1e12 if spent > 0 else None,
        "unit": "TFLOPS",
        "cores": blas_threads(),
        "kind": "oracle",
        "sample": f"{len(used)} of {w.B} samples of the {w.name} batch (seeded order), "
                  f"{flops / 1e9:.2f} useful GFLOP in {spent:.1f} s, numpy float64",
    }
    parity = None
    if gpu_out is not None and ref_max > 0:
        parity = {"max_abs_err_over_max_ref": err_num / ref_max, "samples": len(used),
                  "rows": int(sum(int(w.q_offsets[b + 1] - w.q_offsets[b]) for b in used)) * w.H}
    return res, parity


# Source file of each forward kernel, and the headers every kernel file includes.
KERNEL_SOURCE = {"attn_pp_kernel": "ja_attn_pp.hip", "attn_kernel": "ja_attn_mfma.hip",
                 "attn_f32_kernel": "ja_attn_f32.hip", "bwd_mfma_kernels": "ja_attn_bwd_mfma.hip",
                 "mx_quant_kernel": "ja_mx_quant.hip"}
KERNEL_HEADERS = ("ja_internal.h", "ja_device.h", "ja_mfma_util.h", "ja_gelu_poly.h", "ja_sched.h")


def kernel_source_hash(kernel_tag: str) -> str:
    """sha256 over the dominant kernel's source file and the shared headers: a
    counter summary is valid for exactly that code."""
    import hashlib

    csrc = os.path.join(ROOT, "recsys_jagged_attention_amd", "csrc")
    h = hashlib.sha256()
    for f in (KERNEL_SOURCE[kernel_tag.split("<")[0]],) + KERNEL_HEADERS:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


def profile_path(kernel_tag: str, workload: str) -> str:
    """The committed rocprofv3 summary of a kernel on a workload."""
    return os.path.join(ROOT, "profiles", f"{kernel_tag.split('<')[0]}_{workload}.txt")


def load_traffic(kernel_tag: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, only if
    they were taken on the current kernel source (matching source hash)."""
    path = profile_path(kernel_tag, workload)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            a, b = line.split(":", 1)
            kv[a.strip()] = b.strip()
    if kv.get("source_sha256") != kernel_source_hash(kernel_tag) or kv.get("kernel") != kernel_tag:
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def run_mx_quantize(args):
    """Time the device MX quantiser on the block-window tensors (q, k, v in bf16,
    three launches per step) and print one JSON line in GB/s of compulsory
    bytes (2 read + 1 written per element, plus one scale byte per 32)."""
    import torch

    from recsys_jagged_attention_amd import mx_quantize
    from recsys_jagged_attention_amd.inputs import make_workload

    w = make_workload("block_window", seed=args.seed)
    dev = torch.device("cuda:0")
    xs = [torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in (w.q, w.k, w.v)]
    n_el = sum(x.numel() for x in xs)
    alg_bytes = n_el * 2 + n_el + n_el // 32
    n_copies = int(max(2, min(8, math.ceil(args.rotate_bytes / alg_bytes))))
    sets = [xs] + [[x.clone() for x in xs] for _ in range(n_copies - 1)]
    outs = [[(torch.empty(x.shape, dtype=torch.uint8, device=dev),
              torch.empty(x.shape[:-1] + (x.shape[-1] // 32,), dtype=torch.uint8, device=dev)) for x in xs]
            for _ in range(n_copies)]
    from recsys_jagged_attention_amd import _lib
    stream = torch.cuda.current_stream(dev).cuda_stream

    def step(i):
        for x, (c, sc) in zip(sets[i % n_copies], outs[i % n_copies]):
            st = _lib.jagged_attn_mx_quantize(x.data_ptr(), _lib.JA_BF16, x.numel() // x.shape[-1], x.shape[-1],
                                              c.data_ptr(), sc.data_ptr(), stream)
            if st != _lib.JA_OK:
                raise _lib.JaggedAttnError(st, "jagged_attn_mx_quantize")

    mx_quantize(xs[0])
    ev = HipEvents()
    K, W = args.steps, args.warmup
    starts = [ev.create() for _ in range(K)]
    stops = [ev.create() for _ in range(K)]
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev.record(starts[i], stream)
        step(i)
        ev.record(stops[i], stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern_s = float(np.mean([ev.elapsed_ms(starts[i], stops[i]) for i in range(K)])) * 1e-3
    for e in starts + stops:
        ev.destroy(e)
    ms_per_step = (t1 - t0) * 1e3 / K
    value = alg_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = alg_bytes / kern_s / 1e9
    log(f"[bench] mx quantise: {ms_per_step * 1e3:.1f} us/step, kernels {kern_s * 1e6:.1f} us, "
        f"{achieved:.0f} GB/s ({100 * achieved / PEAK_HBM_GBS:.1f}% of HBM)")
    cpu = None
    if not args.no_cpu_baseline:
        import os as _os
        import oracle
        rows = w.q.reshape(-1, w.D)
        n = min(len(rows), 20000)
        t = time.perf_counter()
        reps = 0
        while time.perf_counter() - t < min(args.cpu_seconds, 10.0) or reps == 0:
            oracle.mx_encode(rows[:n].astype(np.float64))
            reps += 1
        dt = time.perf_counter() - t
        cpu = {"value": round(reps * n * w.D * (2 + 1 + 1 / 32) / dt / 1e9, 4), "unit": "GB/s",
               "cores": len(_os.sched_getaffinity(0)), "kind": "oracle",
               "sample": f"{n} rows of D={w.D} (block_window q), repeated {reps}x"}
    line = {
        "metric": "MX quantisation throughput (bf16 -> e4m3 + E8M0 per 32 along D), 1 MI355X",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "mx_quantize", "tensors": "block_window q, k, v", "elements": int(n_el),
                   "D": w.D, "seed": w.seed},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": "mx_quant_kernel<bf16>", "kernel_avg_us": round(kern_s * 1e6, 2),
                     "algorithmic_bytes_per_launch": int(alg_bytes)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


PEAK_VALU_F32 = 157.3  # TFLOP/s, fp32 vector (packed FMA); non-packed FMA issue gives half


def run_backward(args):
    """Time the backward (dQ, dK, dV) on a workload's tensors with a seeded
    dout and print one JSON line.  Softmax workloads hand the backward the
    forward's output and log-sum-exp (computed once, untimed) unless
    --recompute-stats.  Useful FLOPs: 8 D per attended pair and head (dV, dP,
    dQ and dK); the kernels also recompute the scores."""
    import torch

    from recsys_jagged_attention_amd import backward, forward, Workspace
    from recsys_jagged_attention_amd import workload as wl
    from recsys_jagged_attention_amd.inputs import make_workload, device_tensors

    w = make_workload(args.workload, seed=args.seed)
    if w.dtype not in ("f32", "bf16") or w.act not in ("softmax", "gelu_tanh"):
        raise SystemExit("the backward covers softmax and gelu_tanh workloads with f32 or bf16 inputs")
    dev = torch.device("cuda:0")
    q, k, v, qo, ko, _ = device_tensors(w, dev)
    dout = torch.from_numpy(np.random.default_rng(w.seed + 1).standard_normal(w.q.shape, dtype=np.float32)).to(
        q.dtype).to(dev)
    lq, lk = np.diff(w.q_offsets), np.diff(w.kv_offsets)
    pairs = wl.attended_pairs(lq, lk, w.window, w.variant)
    flops = 8 * w.D * w.H * pairs
    wsp = Workspace(dev)
    ev = HipEvents()
    K, W = args.steps, args.warmup
    starts = [ev.create() for _ in range(K)]
    stops = [ev.create() for _ in range(K)]
    saved = {}
    if w.act == "softmax" and not args.recompute_stats:
        # the forward's output and log-sum-exp, as a training step keeps them
        # (computed once, outside the timed region)
        # (bf16 PMA's key-split forward gives no log-sum-exp: recomputed there)
        from recsys_jagged_attention_amd import JaggedAttnError, JA_EUNSUPPORTED
        lse = torch.empty((w.total_q, w.H), dtype=torch.float32, device=dev)
        try:
            o = forward(q, k, v, qo, ko, variant=w.variant, act=w.act, window=w.window, dtype=w.dtype, check=True,
                        lse=lse)
            saved = {"lse": lse, "fwd_out": o}
        except JaggedAttnError as e:
            if e.status != JA_EUNSUPPORTED:
                raise
    run = lambda e=None: backward(q, k, v, dout, qo, ko, variant=w.variant, act=w.act, window=w.window,
                                  dtype=w.dtype, workspace=wsp, events=e, **saved)
    run()
    backward(q, k, v, dout, qo, ko, variant=w.variant, act=w.act, window=w.window, dtype=w.dtype, workspace=wsp,
             check=True, **saved)
    for _ in range(W):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        run((starts[i], stops[i]))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern_s = float(np.mean([ev.elapsed_ms(starts[i], stops[i]) for i in range(K)])) * 1e-3
    for e in starts + stops:
        ev.destroy(e)
    ms_per_step = (t1 - t0) * 1e3 / K
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / kern_s / 1e12
    # bf16 inputs run on bf16 MFMA; fp32 inputs on the fp32 VALU
    on_mfma = w.dtype == "bf16"
    bound, peak = ("mfma", PEAK_TFLOPS["bf16"]) if on_mfma else ("alu", PEAK_VALU_F32)
    kernels = (("bwd_rms_kernel + " if w.act != "softmax" else "") +
               ("bwd_dq_mfma_kernel + bwd_dkv_pair_kernel"
                if on_mfma else "bwd_q_kernel + bwd_kv_kernel"))
    log(f"[bench] backward {w.name}: {ms_per_step * 1e3:.1f} us/step, kernels {kern_s * 1e6:.1f} us, "
        f"{achieved:.2f} useful TFLOP/s ({100 * achieved / peak:.1f}% of the {bound} peak {peak})")
    cpu = None
    if not args.no_cpu_baseline:
        import os as _os
        import oracle
        # whole samples, shortest first, until about the time budget is used
        order = np.argsort(lq, kind="stable")
        t = time.perf_counter()
        done = 0
        for b in order:
            sl = slice(w.q_offsets[b], w.q_offsets[b + 1])
            sk = slice(w.kv_offsets[b], w.kv_offsets[b + 1])
            oracle.gdpa_backward(w.q[sl], w.k[sk], w.v[sk], dout[sl].float().cpu().numpy(),
                                 [0, lq[b]], [0, lk[b]], w.variant, w.act, w.window)
            done += 8 * w.D * w.H * wl.attended_pairs([lq[b]], [lk[b]], w.window, w.variant)
            if time.perf_counter() - t > min(args.cpu_seconds, 10.0):
                break
        dt = time.perf_counter() - t
        cpu = {"value": round(done / dt / 1e12, 6), "unit": "TFLOPS", "cores": len(_os.sched_getaffinity(0)),
               "kind": "oracle", "sample": f"{done / 8 / w.D / w.H:.0f} attended pairs x {w.H} heads"}
    line = {
        "metric": "useful TFLOPS of the attention backward (dQ, dK, dV), jagged, 1 MI355X",
        "value": round(value, 3), "unit": "TFLOPS", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "variant": w.variant, "act": w.act, "B": w.B, "H": w.H, "D": w.D,
                   "window": w.window, "total_q": w.total_q, "useful_gflop": round(flops / 1e9, 3), "seed": w.seed,
                   "row_stats": "from the forward" if saved else "recomputed"},
        "roofline": {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": None,
                     "kernel": kernels, "kernel_avg_us": round(kern_s * 1e6, 2),
                     "useful_flops_per_launch": int(flops)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="block_window")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rotate-bytes", type=float, default=1.2e9,
                    help="bytes of input copies cycled through (defeats cache reuse across steps)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes 5 times (the reference "
                         "for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE counters) and exit")
    ap.add_argument("--event-every", type=int, default=5,
                    help="time the attention kernel (dispatch events) on every N-th timed step")
    ap.add_argument("--fp8-pv", action="store_true",
                    help="MXFP8 workloads: O += P V on the fp8 MFMA too (P and V requantised along the keys)")
    ap.add_argument("--backward", action="store_true",
                    help="time the softmax backward on the workload instead of the forward")
    ap.add_argument("--recompute-stats", action="store_true",
                    help="with --backward on a softmax workload: recompute the row statistics instead of "
                         "handing the backward the forward's output and log-sum-exp (the default)")
    ap.add_argument("--mx-quantize", action="store_true",
                    help="time the device MX quantiser instead of the attention forward")
    args = ap.parse_args()

    if args.backward:
        if args.gpus != 1:
            raise SystemExit("bench.py measures one GPU only")
        run_backward(args)
        return

    if args.mx_quantize:
        if args.gpus != 1:
            raise SystemExit("bench.py measures one GPU only")
        run_mx_quantize(args)
        return

    if args.copy_calibration:
        import torch
        n = args.copy_calibration
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {n} bytes 5 times")
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the forward kernel runs on one device); "
              f"--gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)

    import torch

    from recsys_jagged_attention_amd import forward, Workspace
    from recsys_jagged_attention_amd import workload as wl
    from recsys_jagged_attention_amd.inputs import make_workload, device_tensors, WORKLOADS

    if args.workload not in WORKLOADS:
        raise SystemExit(f"unknown workload {args.workload}; choose from {WORKLOADS}")
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    w = make_workload(args.workload, seed=args.seed)
    log(f"[bench] workload {w.name}: B={w.B} H={w.H} D={w.D} window={w.window} "
        f"tokens q={w.total_q} kv={w.total_kv} dtype={w.dtype} (generated in {time.perf_counter() - t_gen:.1f}s)")
    q, k, v, qo, ko, scales = device_tensors(w, dev)
    in_bytes = {"f32": 4, "bf16": 2, "mxfp8": 1}[w.dtype]
    out_bytes = 4 if w.dtype == "f32" else 2
    alg_bytes = wl.compulsory_bytes(w.total_q, w.total_kv, w.H, w.D, in_bytes, out_bytes,
                                    mx_scales=w.dtype == "mxfp8")
    lq, lk = np.diff(w.q_offsets), np.diff(w.kv_offsets)
    flops = wl.useful_flops(lq, lk, w.H, w.D, w.window, w.variant)
    n_copies = int(max(2, min(8, math.ceil(args.rotate_bytes / max(alg_bytes, 1)))))
    sets = [(q, k, v, scales)]
    for _ in range(n_copies - 1):
        sets.append((q.clone(), k.clone(), v.clone(),
                     None if scales is None else tuple(s.clone() for s in scales)))
    outs = [torch.empty(q.shape, dtype=torch.float32 if w.dtype == "f32" else torch.bfloat16, device=dev)
            for _ in range(n_copies)]
    wsp = Workspace(dev)
    ev = HipEvents()
    K, W = args.steps, args.warmup
    # the attention kernel's dispatch writes start/stop events on every
    # `event_every`-th timed step (each timed dispatch costs a few us of
    # stream time, so timing every step would slow the steps it measures)
    E = max(1, args.event_every)
    timed = list(range(0, K, E))
    starts = {i: ev.create() for i in timed}
    stops = {i: ev.create() for i in timed}

    def step(i, events=None):
        qq, kk, vv, ss = sets[i % n_copies]
        forward(qq, kk, vv, qo, ko, variant=w.variant, act=w.act, window=w.window, dtype=w.dtype,
                scales=ss, out=outs[i % n_copies], workspace=wsp, events=events, fp8_pv=args.fp8_pv)

    forward(q, k, v, qo, ko, variant=w.variant, act=w.act, window=w.window, dtype=w.dtype,
            scales=scales, out=outs[0], workspace=wsp, check=True, fp8_pv=args.fp8_pv)  # validates offsets once
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({W} steps), timing {K} steps over {n_copies} input copies")
    t0 = time.perf_counter()
    for i in range(K):
        step(i, (starts[i], stops[i]) if i in starts else None)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # kernel durations (start and end stamps of the sampled attention
    # dispatches), and the step period: the time between the ends of two
    # sampled steps' attention kernels over the steps between them (every
    # kernel of a step, back to back)
    kern_ms = np.array([ev.elapsed_ms(starts[i], stops[i]) for i in timed])
    period_ms = np.array([ev.elapsed_ms(stops[a], stops[b]) / (b - a) for a, b in zip(timed, timed[1:])])
    for e in list(starts.values()) + list(stops.values()):
        ev.destroy(e)
    ms_per_step = (t1 - t0) * 1e3 / K
    value = flops / (ms_per_step * 1e-3) / 1e12
    kern_avg_s = float(np.mean(kern_ms)) * 1e-3
    intensity = flops / alg_bytes
    ridge = PEAK_TFLOPS[w.dtype] * 1e12 / (PEAK_HBM_GBS * 1e9)
    kernel_tag = KERNEL_NAME[w.name]
    if args.fp8_pv:
        if not kernel_tag.endswith(",mx8>"):
            raise SystemExit("--fp8-pv applies to the MXFP8 self-attention workloads")
        kernel_tag = kernel_tag[:-1] + ",fp8pv>"
    if intensity < ridge:
        achieved = alg_bytes / kern_avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    else:
        achieved = flops / kern_avg_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_TFLOPS[w.dtype],
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS[w.dtype], 4)}
    roof["traffic"] = load_traffic(kernel_tag, w.name)
    roof["kernel"] = kernel_tag
    roof["kernel_avg_us"] = round(kern_avg_s * 1e6, 2)
    roof["kernel_us"] = {"median": round(float(np.median(kern_ms)) * 1e3, 2),
                         "min": round(float(np.min(kern_ms)) * 1e3, 2),
                         "p90": round(float(np.percentile(kern_ms, 90)) * 1e3, 2)}
    roof["algorithmic_bytes_per_launch"] = int(alg_bytes)
    roof["useful_flops_per_launch"] = int(flops)
    roof["frac_of_peak_flops"] = round(flops / kern_avg_s / 1e12 / PEAK_TFLOPS[w.dtype], 4)
    log(f"[bench] {ms_per_step * 1e3:.1f} us/step, kernel {kern_avg_s * 1e6:.1f} us, "
        f"{value:.1f} useful TFLOPS, {roof['achieved']} {roof['unit']} ({roof['frac'] * 100:.1f}% of peak)")

    # launch diagnostics (after the timed region): the host's time to enqueue K
    # steps, and the time per step of K steps launched without events
    t_e0 = time.perf_counter()
    for i in range(K):
        step(i)
    t_e1 = time.perf_counter()
    torch.cuda.synchronize()
    t_e2 = time.perf_counter()
    launch_diag = {"host_enqueue_us_per_step": round((t_e1 - t_e0) * 1e6 / K, 2),
                   "no_event_us_per_step": round((t_e2 - t_e0) * 1e6 / K, 2)}
    # one more (untimed) call with the softmax's diagnostic counters: how often
    # the lazy reference max had to move after a query block's first tile
    softmax_stats = None
    if w.act == "softmax" and kernel_tag.startswith("attn_pp_kernel"):
        st = torch.zeros(3, dtype=torch.int64, device=dev)
        forward(q, k, v, qo, ko, variant=w.variant, act=w.act, window=w.window, dtype=w.dtype,
                scales=scales, out=outs[0], workspace=wsp, softmax_stats=st, fp8_pv=args.fp8_pv)
        torch.cuda.synchronize()
        tiles, first, later = (int(x) for x in st.cpu())
        softmax_stats = {"wave_tiles": tiles, "first_tile_max_passes": first, "later_rescales": later,
                         "later_rescale_frac": round(later / max(tiles, 1), 6)}
    cpu, parity = None, None
    if not args.no_cpu_baseline:
        t_cpu = time.perf_counter()
        last = outs[(K - 1) % n_copies].float().cpu().numpy().astype(np.float64)  # output of the last timed step
        cpu, parity = cpu_baseline(w, args.cpu_seconds, gpu_out=last)
        log(f"[bench] cpu oracle baseline {cpu['value']:.4g} TFLOPS on {cpu['cores']} threads "
            f"({time.perf_counter() - t_cpu:.1f}s); timed output vs oracle {parity}")
    dev_info = device_info()
    padded = wl.padded_dense_flops(lq, lk, w.H, w.D, w.window)

    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "pct_bf16_peak": round(100 * value / PEAK_TFLOPS["bf16"], 2),
        "step_us": {"median": round(float(np.median(period_ms)) * 1e3, 2) if len(period_ms) else None,
                    "min": round(float(np.min(period_ms)) * 1e3, 2) if len(period_ms) else None,
                    "p90": round(float(np.percentile(period_ms, 90)) * 1e3, 2) if len(period_ms) else None,
                    "kernel_events_every": E},
        "config": {"workload": w.name, "variant": w.variant, "act": w.act, "B": w.B, "H": w.H, "D": w.D,
                   "window": w.window, "total_q": w.total_q, "total_kv": w.total_kv, "seed": w.seed,
                   "useful_gflop": round(flops / 1e9, 3), "padded_dense_gflop": round(padded / 1e9, 3),
                   "fp8_pv": bool(args.fp8_pv), "parallelism": "single GPU"},
        "device": dev_info,
        "parity": parity,
        "softmax_stats": softmax_stats,
        "launch": launch_diag,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
