"""Pins for the oracle's W4A4 (OCP MX FP4 on both operands) product, CPU only.

Checked against: a hand-written table of block scales (tests/golden/mx_scales.txt),
the hand-written E2M1 rounding table, exact agreement with the exact NVFP4
product when both operands are already MX-representable, and zero blocks.
"""
import os

import numpy as np

import oracle
from bit_quantized_decode_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def table(name, cols):
    out = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            out.append(tuple(t(v) for t, v in zip(cols, line.split())))
    return out


def bf16_bits(values):
    """Exact bf16 bit patterns of values that bf16 holds exactly."""
    f = np.asarray(values, np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), f)
    return bits


def test_block_scales_match_the_table():
    rows = table("mx_scales.txt", (float, int, int))
    x = np.zeros((len(rows), 32), np.float32)
    for i, (amax, _, _) in enumerate(rows):
        x[i, 5] = amax
        x[i, 9] = -amax / 4
    x = (x.view(np.uint32) >> 16).astype(np.uint16)          # these values are bf16-exact except 7.99 / 3.99
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    _, s = oracle.mx_from_bf16(x)
    for i, (amax, ex, byte) in enumerate(rows):
        # 7.99 and 3.99 truncate to bf16 values still on the same side of the power of two
        assert np.floor(np.log2(xf[i, 5])) == np.floor(np.log2(amax)) or amax == 0
        assert s[i, 0] == byte, (amax, s[i, 0], byte)


def test_element_rounding_matches_the_e2m1_table():
    rows = [(v, c) for v, c in table("e2m1_rounding.txt", (float, int)) if abs(v) < 8.0]
    x = np.zeros((len(rows), 32), np.float32)
    for i, (v, _) in enumerate(rows):
        x[i, 0] = v
        x[i, 1] = 6.0                                          # block scale 2^0: codes are the rounded values
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)        # truncation; values it changes are skipped below
    xf = (bits.astype(np.uint32) << 16).view(np.float32)
    codes, scales = oracle.mx_from_bf16(bits)
    assert np.all(scales[:, 0] == 127)
    for i, (v, want) in enumerate(rows):
        if xf[i, 0] != np.float32(v):
            continue                                           # not bf16-exact (e.g. 0.26): skipped
        assert (codes[i, 0] & 15) == want, (v, codes[i, 0] & 15, want)


def test_mx_representable_operands_give_the_exact_product():
    """Weights whose every 32-block holds a code of magnitude 4 or 6 under block
    scale 1.0, and activations that are E2M1 values with a 4 or 6 in every block:
    the W4A4 product equals the exact NVFP4 product."""
    rng = np.random.default_rng(3)
    n, k, m = 40, 128, 5
    codes = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    codes[:, ::32] = 7                                         # a 6.0 in every block
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    scales = np.full((n, k // 16), 0x38, np.uint8)             # E4M3 1.0
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6], np.float32)
    xv = grid[rng.integers(0, 16, size=(m, k))]
    xv[:, 3::32] = -4.0                                        # a 4 in every block (scale 2^0)
    xv[:, 4::32] = 6.0
    xb = bf16_bits(xv)
    mc, ms = oracle.mx_from_nvfp4(packed, scales)
    xc, xs = oracle.mx_from_bf16(xb)
    assert np.array_equal(mc, packed) and np.all(ms == 127)
    y, s = oracle.mx_gemm(mc, ms, I.TENSOR_SCALE, xc, xs)
    ye, se = oracle.gemm(packed, scales, I.TENSOR_SCALE, xb)
    assert np.array_equal(y, ye) and np.array_equal(s, se)


def test_zero_blocks():
    x = np.zeros((2, 64), np.uint16)
    x[1, 40] = bf16_bits([1.5])[0]
    c, s = oracle.mx_from_bf16(x)
    assert s[0, 0] == 0 and s[0, 1] == 0 and s[1, 0] == 0 and not c[0].any() and not c[1, :16].any()
    assert s[1, 1] == 125                                      # 1.5: exponent 0 - 2
