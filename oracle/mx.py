"""MX (microscaling) FP8 decoding in float64 (oracle side; test infrastructure only).

[GEM-T] "MXFP8による超低精度トレーニング": attention runs on Microscaling FP8.
Reading used: OCP-MX layout -- e4m3 ("fn" variant: no infinities, S.1111.111 is
NaN, max 448) elements with one E8M0 power-of-two scale per 32 contiguous
elements along the head dimension D.  Decoding is exact in float64.

Encoding (the pages give no rule; reading used): the scale exponent of a
32-block is E = floor(log2(max |x|)) - 8 (8 = the exponent of e4m3's largest
power of two), clamped to [-127, 127], and -127 for an all-zero block; an
element becomes the e4m3 value nearest to x / 2^E, ties to the even code,
after saturating to +-448.
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


def e4m3_grid() -> np.ndarray:
    """The 127 non-negative finite e4m3fn values, index = code (0 .. 126)."""
    return decode_e4m3(np.arange(127, dtype=np.uint8))


def encode_e4m3(y) -> np.ndarray:
    """float -> uint8 e4m3fn code: the nearest representable value (ties to the
    even code, i.e. the even mantissa), magnitudes above 448 saturated to 448."""
    y = np.asarray(y, dtype=np.float64)
    grid = e4m3_grid()
    a = np.minimum(np.abs(y), 448.0)
    hi = np.clip(np.searchsorted(grid, a, side="left"), 0, 126)   # first grid value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo = a - grid[lo]
    d_hi = grid[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(y), code | 0x80, code).astype(np.uint8)


def mx_encode(x, block: int = 32):
    """float [..., D] -> (codes uint8 [..., D], scales uint8 [..., D/block])."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d % block:
        raise ValueError("D must be a multiple of the block size")
    xb = x.reshape(*x.shape[:-1], d // block, block)
    amax = np.abs(xb).max(axis=-1)
    # floor(log2 amax) exactly: frexp gives amax = f * 2^e with f in [0.5, 1)
    _, e2 = np.frexp(np.where(amax > 0, amax, 1.0))
    e = np.where(amax > 0, e2 - 1 - 8, -127)
    e = np.clip(e, -127, 127)
    codes = encode_e4m3(xb / np.exp2(e.astype(np.float64))[..., None])
    return codes.reshape(x.shape), (e + 127).astype(np.uint8)
