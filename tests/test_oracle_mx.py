"""Pins for the MX (e4m3 + E8M0) decoding used by the oracle, and for the
input encoder that produces MX inputs."""
import numpy as np
import torch

from oracle import decode_e4m3, decode_e8m0, mx_dequantise
from recsys_jagged_attention_amd.inputs import mx_encode_e4m3, rng_for


def test_e4m3_decode_matches_library_cast_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = decode_e4m3(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])


def test_e4m3_closed_forms():
    vals = decode_e4m3(np.array([0x38, 0xB8, 0x7E, 0xFE, 0x01, 0x08, 0x00, 0x80, 0x7F, 0xFF, 0x3C], dtype=np.uint8))
    np.testing.assert_array_equal(vals[:8], [1.0, -1.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -6, 0.0, -0.0])
    assert np.isnan(vals[8]) and np.isnan(vals[9])
    assert vals[10] == 1.5


def test_e8m0_closed_forms():
    s = decode_e8m0(np.array([127, 0, 254, 128, 255], dtype=np.uint8))
    np.testing.assert_array_equal(s[:4], [1.0, 2.0 ** -127, 2.0 ** 127, 2.0])
    assert np.isnan(s[4])


def test_mx_round_trip_bounds():
    rng = rng_for(11)
    x = rng.standard_normal((64, 2, 128)).astype(np.float32)
    x[0, 0, :32] = 0.0                      # an all-zero block
    x[1, 0, 5] = 1000.0                     # a block with a large outlier
    codes, scales = mx_encode_e4m3(x)
    assert codes.shape == x.shape and scales.shape == (64, 2, 4)
    y = mx_dequantise(codes, scales)
    assert np.all(np.isfinite(y))
    np.testing.assert_array_equal(y[0, 0, :32], 0.0)
    # every block's max element lands in [256, 448] after scaling (scale = floor(log2 amax) - 8)
    amax = np.abs(x.reshape(64, 2, 4, 32)).max(-1)
    nz = amax > 0
    e = scales.astype(np.int64) - 127
    r = amax[nz] / np.exp2(e[nz].astype(float))
    assert np.all(r >= 256) and np.all(r < 512)
    # normal-range, unsaturated elements carry 4 significant bits: relative error <= 2^-4;
    # elements whose scaled magnitude exceeds 448 saturate to +-448
    dec_codes = np.abs(decode_e4m3(codes))
    scaled = np.abs(x) / np.exp2(np.repeat(e, 32, axis=-1).astype(float))
    normal = (dec_codes >= 2.0 ** -6) & (scaled <= 448)
    rel = np.abs(y - x)[normal] / np.abs(x)[normal]
    assert rel.max() <= 2.0 ** -4 + 1e-12
    assert np.all(dec_codes <= 448)
    np.testing.assert_array_equal(dec_codes[scaled > 448], 448.0)


def test_mx_dequantise_applies_scale_per_32_along_d():
    codes = np.full((1, 1, 64), 0x38, dtype=np.uint8)  # all 1.0
    scales = np.array([[[127 + 3, 127 - 2]]], dtype=np.uint8)
    y = mx_dequantise(codes, scales)
    np.testing.assert_array_equal(y[0, 0, :32], 8.0)
    np.testing.assert_array_equal(y[0, 0, 32:], 0.25)


# ---- encoder ---------------------------------------------------------------
from oracle import encode_e4m3, mx_encode


def test_e4m3_encode_matches_library_cast():
    """Nearest e4m3fn value, ties to even: torch's float8_e4m3fn cast on float32
    (a library routine) for values on, between and halfway between grid points."""
    grid = decode_e4m3(np.arange(127, dtype=np.uint8))
    mids = (grid[1:] + grid[:-1]) / 2
    rng = np.random.default_rng(3)
    vals = np.concatenate([grid, mids, rng.uniform(0, 448, 4000), rng.uniform(0, 2 ** -6, 500)])
    vals = np.concatenate([vals, -vals]).astype(np.float32)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = encode_e4m3(vals)
    np.testing.assert_array_equal(got, ref)


def test_e4m3_encode_saturates_and_closed_forms():
    assert encode_e4m3([448.0, 449.0, 1e9, -1e9]).tolist() == [0x7E, 0x7E, 0x7E, 0xFE]
    assert encode_e4m3([0.0, 1.0, 2 ** -9, 3 * 2 ** -10]).tolist() == [0, 0x38, 1, 2]   # 1.5 ulp -> 2 (even)
    assert encode_e4m3([1.0625]).tolist() == [0x38]      # halfway 1 and 1.125: even mantissa 0
    assert encode_e4m3([1.1875]).tolist() == [0x3A]      # halfway 1.125 and 1.25: even mantissa 2


def test_mx_encode_scale_rule_and_round_trip():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((7, 3, 64)) * np.exp2(rng.integers(-20, 20, (7, 3, 1)))
    x[0, 0, :32] = 0.0                                   # all-zero block
    x[1, 1, :32] = 0.0
    x[1, 1, 5] = 2.0 ** -130                              # tiny block
    x[2, 2, 32:] = 1.0
    x[2, 2, 40] = 448.0 * 2 ** 3                          # amax 3584 = 1.75 * 2^11 -> E = 3
    codes, scales = mx_encode(x)
    assert scales[0, 0, 0] == 0 and not codes[0, 0, :32].any()
    assert scales[1, 1, 0] == 0                           # E clamped to -127
    assert scales[2, 2, 1] == 127 + 3
    # the scale puts the block max in [2^8, 2^9): elements up to 448 steps are
    # within half an e4m3 step (relative 2^-4, or half the subnormal step),
    # larger ones saturate to +-448 steps
    xr = mx_dequantise(codes, scales)
    sc = np.repeat(np.exp2(scales.astype(np.float64) - 127), 32, axis=-1)
    inside = np.abs(x) <= 448 * sc
    err = np.abs(xr - x)
    assert np.all(err[inside] <= np.maximum(np.abs(x) * 2 ** -4, sc * 2 ** -10)[inside])
    np.testing.assert_array_equal(xr[~inside], np.sign(x[~inside]) * 448 * sc[~inside])
    assert (~inside).any()
    # and the oracle encoder agrees with the input generator's (torch-cast) encoder
    from recsys_jagged_attention_amd.inputs import mx_encode_e4m3
    c2, s2 = mx_encode_e4m3(x.astype(np.float32))
    c1, s1 = mx_encode(x.astype(np.float32))
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(s1, s2)
