"""Seeded synthetic inputs for jagged attention.

This module is shared by the GPU path's tests/bench and by the float64 oracle.
It draws lengths and values only; it contains none of the attention arithmetic.

Workloads (sizes of the jagged user-history batches the pages describe:
"hundreds to tens of thousands of tokens" per history, [GEM Training summary,
techfeed.io, "なぜLLM向けのインフラをそのまま使えないのか"]):

* ``tiny_full``      : B=4, L~U{1..128}, H=2, D=32, fp32, full self-attention
* ``block_window``   : B=64, L~logU[100,4096], H=8, D=128, bf16, 64-token blocks, window 256
* ``full_self``      : the block_window tensors with no window (full self-attention)
* ``cross_gelu``     : B=256, Lq~logU[256,8192], Lkv~U{16..64}, H=4, D=128, bf16, RMSNorm+GELU
* ``pma``            : B=512, 32 seeds/sample, Lkv: 5% logU[8193,16384], rest logU[64,8192], H=8, D=64
* ``mxfp8_window``   : block_window lengths/values quantised to e4m3 + E8M0 (one scale per 32 along D)
* ``mxfp8_full``     : the mxfp8_window inputs with no window (full self-attention on MX inputs)
* ``sliding_window`` : the block_window tensors under a 256-token sliding window

Every generator takes an explicit integer seed and uses numpy's PCG64.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

BLOCK = 64  # token block of block-aligned attention


def rng_for(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def lengths_loguniform(rng: np.random.Generator, n: int, lo: int, hi: int) -> np.ndarray:
    """Discrete log-uniform lengths: floor(exp(U(ln lo, ln(hi+1)))) clipped to [lo, hi]."""
    u = rng.uniform(math.log(lo), math.log(hi + 1), size=n)
    return np.clip(np.floor(np.exp(u)).astype(np.int64), lo, hi)


def lengths_uniform(rng: np.random.Generator, n: int, lo: int, hi: int) -> np.ndarray:
    return rng.integers(lo, hi + 1, size=n, dtype=np.int64)


def pma_lengths(rng: np.random.Generator, n: int, lo: int = 64, hi: int = 16384,
                long_frac: float = 0.05, split: int = 8192) -> np.ndarray:
    """Skewed K/V lengths: round(long_frac*n) samples log-uniform in (split, hi],
    the rest log-uniform in [lo, split], in a seeded random order."""
    n_long = int(round(long_frac * n))
    long_l = lengths_loguniform(rng, n_long, split + 1, hi)
    short_l = lengths_loguniform(rng, n - n_long, lo, split)
    lens = np.concatenate([long_l, short_l])
    return lens[rng.permutation(n)]


def offsets_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    off = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=off[1:])
    if off[-1] >= 2**31:
        raise ValueError("total length exceeds int32 offsets")
    return off.astype(np.int32)


def normal_values(rng: np.random.Generator, n: int, h: int, d: int) -> np.ndarray:
    return rng.standard_normal(size=(n, h, d), dtype=np.float32)


# --------------------------------------------------------------------------
# MX (microscaling) encoding of generated values: e4m3 codes + one E8M0 scale
# per 32 contiguous elements along D.  This is input preparation: the kernels
# and the oracle both receive the codes and scales and decode them themselves.
# --------------------------------------------------------------------------
MX_BLOCK = 32
E4M3_MAX = 448.0
E4M3_EMAX = 8  # exponent of the largest power of two representable in e4m3


def mx_encode_e4m3(x: np.ndarray):
    """float32 [N,H,D] -> (codes uint8 [N,H,D], scales uint8 [N,H,D/32]).

    Scale exponent E = floor(log2(max|x| over the 32-block)) - 8, clamped to the
    E8M0 range; the element is x / 2^E saturated to +-448 and rounded to nearest
    even in e4m3 (torch's float8_e4m3fn cast).  An all-zero block gets the
    smallest scale and zero codes.
    """
    import torch

    n, h, d = x.shape
    if d % MX_BLOCK:
        raise ValueError("D must be a multiple of 32 for MX encoding")
    xb = x.reshape(n, h, d // MX_BLOCK, MX_BLOCK).astype(np.float32)
    amax = np.abs(xb).max(axis=-1)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - E4M3_EMAX, -127)
    e = np.clip(e, -127, 127).astype(np.int32)
    scaled = xb / np.exp2(e.astype(np.float64))[..., None]
    scaled = np.clip(scaled, -E4M3_MAX, E4M3_MAX).astype(np.float32)
    codes = torch.from_numpy(np.ascontiguousarray(scaled)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    scales = (e + 127).astype(np.uint8)
    return codes.reshape(n, h, d), scales


# --------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Workload:
    name: str
    variant: str            # "self" | "cross" | "pma" | "sliding"
    act: str                # "softmax" | "gelu_tanh"
    dtype: str              # "f32" | "bf16" | "mxfp8"
    B: int
    H: int
    D: int
    window: int
    q_offsets: np.ndarray   # int32 [B+1]
    kv_offsets: np.ndarray  # int32 [B+1]
    q: np.ndarray           # float32 [Nq,H,D]   (values before any cast)
    k: np.ndarray           # float32 [Nkv,H,D]
    v: np.ndarray           # float32 [Nkv,H,D]
    seed: int
    mx: Optional[dict] = None  # for mxfp8: codes/scales per tensor

    @property
    def total_q(self) -> int:
        return int(self.q_offsets[-1])

    @property
    def total_kv(self) -> int:
        return int(self.kv_offsets[-1])


WORKLOADS = ("tiny_full", "block_window", "full_self", "cross_gelu", "pma", "mxfp8_window", "mxfp8_full",
             "sliding_window")
DEFAULT_SEED = {"tiny_full": 1001, "block_window": 1002, "full_self": 1002,
                "cross_gelu": 1003, "pma": 1004, "mxfp8_window": 1002, "mxfp8_full": 1002, "sliding_window": 1002}


def make_workload(name: str, seed: Optional[int] = None, scale: float = 1.0) -> Workload:
    """Build a named workload.  ``scale`` < 1 shrinks the batch size B (for tests)."""
    if seed is None:
        seed = DEFAULT_SEED[name]
    rng = rng_for(seed)

    def nb(b):
        return max(1, int(round(b * scale)))

    if name == "tiny_full":
        B, H, D = nb(4), 2, 32
        L = lengths_uniform(rng, B, 1, 128)
        off = offsets_from_lengths(L)
        q = normal_values(rng, int(off[-1]), H, D)
        k = normal_values(rng, int(off[-1]), H, D)
        v = normal_values(rng, int(off[-1]), H, D)
        return Workload(name, "self", "softmax", "f32", B, H, D, 0, off, off, q, k, v, seed)
    if name in ("block_window", "full_self", "mxfp8_window", "mxfp8_full", "sliding_window"):
        B, H, D = nb(64), 8, 128
        L = lengths_loguniform(rng, B, 100, 4096)
        off = offsets_from_lengths(L)
        n = int(off[-1])
        q = normal_values(rng, n, H, D)
        k = normal_values(rng, n, H, D)
        v = normal_values(rng, n, H, D)
        window = 0 if name in ("full_self", "mxfp8_full") else 256  # (sliding_window: 256 tokens)
        dtype = "mxfp8" if name in ("mxfp8_window", "mxfp8_full") else "bf16"
        variant = "sliding" if name == "sliding_window" else "self"
        w = Workload(name, variant, "softmax", dtype, B, H, D, window, off, off, q, k, v, seed)
        if dtype == "mxfp8":
            w.mx = {}
            for nm, x in (("q", q), ("k", k), ("v", v)):
                codes, scales = mx_encode_e4m3(x)
                w.mx[nm] = (codes, scales)
        return w
    if name == "cross_gelu":
        B, H, D = nb(256), 4, 128
        Lq = lengths_loguniform(rng, B, 256, 8192)
        Lkv = lengths_uniform(rng, B, 16, 64)
        qo, ko = offsets_from_lengths(Lq), offsets_from_lengths(Lkv)
        q = normal_values(rng, int(qo[-1]), H, D)
        k = normal_values(rng, int(ko[-1]), H, D)
        v = normal_values(rng, int(ko[-1]), H, D)
        return Workload(name, "cross", "gelu_tanh", "bf16", B, H, D, 0, qo, ko, q, k, v, seed)
    if name == "pma":
        B, H, D = nb(512), 8, 64
        Lkv = pma_lengths(rng, B)
        qo = offsets_from_lengths(np.full(B, 32))
        ko = offsets_from_lengths(Lkv)
        q = normal_values(rng, int(qo[-1]), H, D)
        k = normal_values(rng, int(ko[-1]), H, D)
        v = normal_values(rng, int(ko[-1]), H, D)
        return Workload(name, "pma", "softmax", "bf16", B, H, D, 0, qo, ko, q, k, v, seed)
    raise KeyError(name)


def random_jagged(seed: int, lengths_q, lengths_kv, H: int, D: int):
    """Small ad-hoc jagged inputs (for edge-case tests): returns offsets and float32 values."""
    rng = rng_for(seed)
    qo = offsets_from_lengths(lengths_q)
    ko = offsets_from_lengths(lengths_kv)
    q = normal_values(rng, int(qo[-1]), H, D)
    k = normal_values(rng, int(ko[-1]), H, D)
    v = normal_values(rng, int(ko[-1]), H, D)
    return qo, ko, q, k, v


def device_tensors(w: Workload, device):
    """Move a workload to the GPU in its input dtype (casts only; RNE for bf16).

    Returns (q, k, v, q_offsets, kv_offsets, scales) as torch tensors; scales is
    None except for mxfp8 (then (q_scale, k_scale, v_scale) uint8)."""
    import torch

    qo = torch.from_numpy(np.ascontiguousarray(w.q_offsets, dtype=np.int32)).to(device)
    ko = torch.from_numpy(np.ascontiguousarray(w.kv_offsets, dtype=np.int32)).to(device)
    if w.dtype == "mxfp8":
        t = [torch.from_numpy(np.ascontiguousarray(w.mx[n][0])).to(device) for n in "qkv"]
        s = tuple(torch.from_numpy(np.ascontiguousarray(w.mx[n][1])).to(device) for n in "qkv")
        return t[0], t[1], t[2], qo, ko, s
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    t = [torch.from_numpy(x).to(dt).to(device) for x in (w.q, w.k, w.v)]
    return t[0], t[1], t[2], qo, ko, None


def cast_values(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values as the device receives them for f32/bf16 inputs (exact, float32)."""
    import torch

    if dtype == "f32":
        return x
    if dtype == "bf16":
        return torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    raise ValueError(dtype)
