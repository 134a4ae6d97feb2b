"""MX (microscaling) FP8 decoding in float64 (oracle side; test infrastructure only).

[GEM-T] "MXFP8による超低精度トレーニング": attention runs on Microscaling FP8.
Reading used: OCP-MX layout -- e4m3 ("fn" variant: no infinities, S.1111.111 is
NaN, max 448) elements with one E8M0 power-of-two scale per 32 contiguous
elements along the head dimension D.  Decoding is exact in float64.
"""
import numpy as np


def decode_e4m3(codes) -> np.ndarray:
    """uint8 e4m3fn codes -> float64.  Bits: s eeee mmm, exponent bias 7.
    exponent 0 is subnormal: (m/8) * 2^-6; s.1111.111 is NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    val = np.where(e == 0, sub, normal) * sign
    return np.where((e == 15) & ((c & 0x7) == 7), np.nan, val)


def decode_e8m0(scales) -> np.ndarray:
    """uint8 E8M0 -> float64 power of two 2^(E-127); 0xFF is NaN."""
    s = np.asarray(scales, dtype=np.uint8).astype(np.int64)
    return np.where(s == 255, np.nan, np.exp2(s.astype(np.float64) - 127.0))


def mx_dequantise(codes, scales, block: int = 32) -> np.ndarray:
    """codes uint8 [..., D], scales uint8 [..., D/block] -> float64 [..., D]."""
    x = decode_e4m3(codes)
    sc = decode_e8m0(scales)
    d = x.shape[-1]
    if d % block or sc.shape[-1] != d // block:
        raise ValueError("scale shape does not match one scale per 32 elements along D")
    return (x.reshape(*x.shape[:-1], d // block, block) * sc[..., None]).reshape(x.shape)
