"""Pins for the oracle's NVFP4 quantiser (CPU only).

Each check compares the oracle with something other than itself: a hand-written
rounding table (tests/golden/e2m1_rounding.txt), torch's float32 -> float8_e4m3fn
cast for the block scales, exact round trips of NVFP4 data, and properties the
encoding fixes (half-step error bound, zero blocks).
"""
import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ONE_OVER_448 = np.float32(1.0 / 448.0)   # 448 * this rounds to 1.0 in fp32: block scale 448 divides by exactly 1


def read_table(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            v, c = line.split()
            rows.append((np.float32(v), int(c)))
    return rows


def codes_of(packed_codes):
    """[n][k/2] bytes -> [n][k] 4-bit codes (element 2i in the low nibble)."""
    lo = packed_codes & 15
    hi = packed_codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(packed_codes.shape[0], -1)


def test_element_rounding_matches_the_table():
    table = read_table("e2m1_rounding.txt")
    # One block per value: the value, then 6.0 (so the block's largest magnitude
    # is 6 and its scale 448 -- or saturated at 448 above 6), then zeros.
    w = np.zeros((len(table), 16), np.float32)
    for i, (v, _) in enumerate(table):
        w[i, 0] = v
        w[i, 1] = 6.0
    c, s, st = oracle.quantize(w, tensor_scale=ONE_OVER_448)
    assert np.all(s == 0x7E)
    got = codes_of(c)[:, 0]
    want = np.array([code for _, code in table])
    assert np.array_equal(got, want), list(zip([v for v, _ in table], got, want))
    assert np.all(codes_of(c)[:, 1] == 7)


def test_block_scale_rounding_matches_torch_e4m3fn_cast():
    # tensor scale fp32(1/6): 6 * s_t rounds to exactly 1.0, so the scale byte is
    # the E4M3 rounding of the block's largest magnitude itself.
    st = np.float32(1.0 / 6.0)
    assert np.float32(6.0) * st == np.float32(1.0)
    rng = np.random.default_rng(5)
    amax = np.concatenate([
        np.exp2(rng.uniform(-12, 8.8, size=3000)).astype(np.float32),     # below 460: no NaN from torch's cast
        oracle.e4m3(np.arange(0, 0x7F)).astype(np.float32),               # every finite E4M3 value exactly
        ((oracle.e4m3(np.arange(0, 0x7E)) + oracle.e4m3(np.arange(1, 0x7F))) / 2).astype(np.float32),  # midpoints
    ])
    amax = amax[amax <= 460.0]
    w = np.zeros((amax.size, 16), np.float32)
    w[:, 3] = amax
    _, s, _ = oracle.quantize(w, tensor_scale=st)
    ref = torch.from_numpy(amax).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(s[:, 0], ref)


def test_block_scale_saturates_at_448():
    st = np.float32(1.0 / 6.0)
    w = np.zeros((3, 16), np.float32)
    w[:, 0] = [470.0, 1e6, 3e38]
    _, s, _ = oracle.quantize(w, tensor_scale=st)
    assert np.all(s[:, 0] == 0x7E)


def test_round_trip_of_nvfp4_data_is_exact():
    """quantize(dequant(q)) == q for NVFP4 data in the encoder's own form: every
    block holds a code of magnitude 6, one block has scale 448, and s_t is a power
    of two (so amax / 2688 recovers it exactly)."""
    rng = np.random.default_rng(9)
    n, k = 37, 96
    codes = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    blocks = codes.reshape(n, k // 16, 16)
    pos = rng.integers(0, 16, size=(n, k // 16))
    np.put_along_axis(blocks, pos[..., None], (7 + 8 * rng.integers(0, 2, size=(n, k // 16)))[..., None], axis=2)
    scales = rng.integers(0, 0x7F, size=(n, k // 16), dtype=np.uint8)   # every finite non-negative byte
    scales[0, 0] = 0x7E
    scales[scales == 0] = 1                                                # a zero scale has no codes to recover
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    st = np.float32(2.0 ** -8)
    w = oracle.dequant(packed, scales, st).astype(np.float32)
    assert np.array_equal(w.astype(np.float64), oracle.dequant(packed, scales, st))   # exact in fp32
    c2, s2, st2 = oracle.quantize(w)
    assert st2 == st
    assert np.array_equal(s2, scales)
    assert np.array_equal(c2, packed)


def test_bf16_input_equals_fp32_input_of_the_same_values():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((20, 64)).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)          # truncation: some bf16 values
    xf = (bits.astype(np.uint32) << 16).view(np.float32)
    a = oracle.quantize(bits)
    b = oracle.quantize(xf)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]


def test_error_is_at_most_half_a_grid_step():
    """|w - dequant(quantize(w))| <= half the local E2M1 step times the block's
    scale (and the saturated part beyond 6)."""
    rng = np.random.default_rng(13)
    w = (rng.standard_normal((64, 256)) * np.exp2(rng.uniform(-4, 4, size=(64, 1)))).astype(np.float32)
    c, s, st = oracle.quantize(w)
    d = oracle.e4m3(s).astype(np.float64) * float(st)
    dq = oracle.dequant(c, s, st)
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    step = np.diff(grid)
    dd = np.repeat(d, 16, axis=1)
    a = np.abs(w.astype(np.float64)) / dd
    idx = np.clip(np.searchsorted(grid, a, side="right") - 1, 0, 6)
    half = np.where(a >= 6.0, a - 6.0, step[idx] / 2)
    # 2^-20 relative slack covers the fp32 rounding of the quotient and of the scale product
    assert np.all(np.abs(w - dq) <= (half + 2.0 ** -20 * a) * dd)
    # The largest block scale is 448: the tensor scale maps amax onto 6 * 448.
    assert s.max() == 0x7E


def test_zero_matrix_and_underflowing_blocks():
    c, s, st = oracle.quantize(np.zeros((3, 32), np.float32))
    assert st == np.float32(1.0) and not c.any() and not s.any()
    w = np.zeros((1, 32), np.float32)
    w[0, 0] = 1.0
    w[0, 16:] = -1e-9                      # second block: scale rounds to 0 -> codes 0
    c, s, st = oracle.quantize(w)
    assert s[0, 1] == 0 and not c[0, 8:].any()
    assert s[0, 0] == 0x7E and (c[0, 0] & 15) == 7
