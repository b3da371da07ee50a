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


# Maps of an E2M1 magnitude code (0..7) to the code of half its value, where
# half of it is on the grid: 0->0, 1.0->0.5, 2->1, 3->1.5, 4->2, 6->3.
HALF_CODE = {0: 0, 2: 1, 4: 2, 5: 3, 6: 4, 7: 5}


def test_mx_scales_vary_by_row_and_block():
    """MX-representable operands whose power-of-two scales differ per row and per
    32-block, and per 16-half inside a weight block.

    Weights: in each 32-block, one 16-half has E4M3 scale 2^a (a byte from
    0x08..0x48, mantissa 0) and a magnitude-6 code; the other half either shares
    that byte or has scale 2^(a-1) with codes whose halves are on the grid.  So
    the MX scale is 2^a, E8M0 byte 127 + a, the first half's codes are
    unchanged and the other half's codes are those of its values / 2^a.
    Activations: E2M1 values times 2^e with e drawn per (row, block) and a 4 or
    6 in every block, so the E8M0 byte is 127 + e and the codes are the grid codes.
    A requantiser that drops the E4M3 scale or reads another 16-half's, or an MX
    product that reads a scale at the wrong row or block, gives other bytes or
    another product.  The product then equals the exact NVFP4 one bit for bit
    (s_t = 1, so every partial sum is exact in fp64)."""
    rng = np.random.default_rng(17)
    n, k, m = 24, 256, 7
    nb = k // 32
    codes = rng.integers(0, 16, size=(n, k)).astype(np.uint8)
    scales = np.zeros((n, k // 16), np.uint8)
    want_mc = np.zeros((n, k), np.uint8)
    want_ms = np.zeros((n, nb), np.uint8)
    for r in range(n):
        for b in range(nb):
            ebyte = int(rng.integers(1, 10))              # E4M3 exponent field: 2^(ebyte - 7), 2^-6 .. 2^2
            a = ebyte - 7
            top = int(rng.integers(0, 2))                 # which 16-half holds the block's largest value
            lo = int(rng.integers(0, 3))                  # 0: both halves share 2^a; else the other has 2^(a-1)
            half = [32 * b, 32 * b + 16]
            big, other = half[top], half[1 - top]
            codes[r, big + int(rng.integers(0, 16))] = 7 | (8 if rng.integers(0, 2) else 0)
            scales[r, big // 16] = ebyte << 3
            want_mc[r, big:big + 16] = codes[r, big:big + 16]
            if lo == 0 or ebyte == 1:
                scales[r, other // 16] = ebyte << 3
                want_mc[r, other:other + 16] = codes[r, other:other + 16]
            else:
                mags = rng.choice(np.array(list(HALF_CODE), np.uint8), size=16)
                signs = rng.integers(0, 2, size=16).astype(np.uint8) << 3
                codes[r, other:other + 16] = mags | signs
                scales[r, other // 16] = (ebyte - 1) << 3
                want_mc[r, other:other + 16] = np.array([HALF_CODE[int(c)] for c in mags], np.uint8) | signs
            want_ms[r, b] = 127 + a
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    want_packed = (want_mc[:, 0::2] | (want_mc[:, 1::2] << 4)).astype(np.uint8)

    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6], np.float64)
    xcode = rng.integers(0, 16, size=(m, k)).astype(np.uint8)
    xexp = rng.integers(-6, 7, size=(m, nb))
    for r in range(m):
        for b in range(nb):
            xcode[r, 32 * b + int(rng.integers(0, 32))] = int(rng.choice([6, 7, 14, 15]))
    xv = grid[xcode] * np.exp2(np.repeat(xexp, 32, axis=1))
    xb = bf16_bits(xv.astype(np.float32))
    want_xc = (xcode[:, 0::2] | (xcode[:, 1::2] << 4)).astype(np.uint8)

    mc, ms = oracle.mx_from_nvfp4(packed, scales)
    xc, xs = oracle.mx_from_bf16(xb)
    assert np.array_equal(ms, want_ms)
    assert np.array_equal(mc, want_packed)
    assert np.array_equal(xs, (127 + xexp).astype(np.uint8))
    assert np.array_equal(xc, want_xc)
    one = np.float32(1.0)
    y, s = oracle.mx_gemm(mc, ms, one, xc, xs)
    ye, se = oracle.gemm(packed, scales, one, xb)
    assert np.array_equal(y, ye) and np.array_equal(s, se)
    # A row subset reads the same rows' scales.
    rows = np.array([n - 1, 3, 3, 0], np.int64)
    yr, sr = oracle.mx_gemm(mc, ms, one, xc, xs, rows=rows)
    assert np.array_equal(yr, y[:, rows]) and np.array_equal(sr, s[:, rows])


def test_mx_product_is_s_t_times_the_unscaled_sum():
    """The per-tensor scale multiplies the exact fp64 sum once (s_t after accumulation)."""
    rng = np.random.default_rng(19)
    n, k, m = 9, 96, 3
    wc = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    ws = rng.integers(110, 140, size=(n, k // 32), dtype=np.uint8)
    xc = rng.integers(0, 256, size=(m, k // 2), dtype=np.uint8)
    xs = rng.integers(110, 140, size=(m, k // 32), dtype=np.uint8)
    y1, s1 = oracle.mx_gemm(wc, ws, np.float32(1.0), xc, xs)
    st = I.TENSOR_SCALE
    y2, s2 = oracle.mx_gemm(wc, ws, st, xc, xs)
    assert np.array_equal(y2, float(st) * y1) and np.array_equal(s2, float(st) * s1)
    # and the unscaled sum is the plain definition over decoded operands
    def dec(c, s):
        codes = np.stack([c & 15, c >> 4], axis=-1).reshape(c.shape[0], -1)
        mag = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)[codes & 7]
        val = np.where(codes & 8, -mag, mag)
        return val * np.exp2(np.repeat(s.astype(np.float64) - 127, 32, axis=1))
    W, X = dec(wc, ws), dec(xc, xs)
    assert np.allclose(y1, X @ W.T, rtol=0, atol=1e-12 * (np.abs(X) @ np.abs(W).T).max())
    assert np.allclose(s1, np.abs(X) @ np.abs(W).T, rtol=1e-15)


def test_lone_subnormal_blocks_use_the_clamped_scale():
    """A block holding one bf16 subnormal: the scale exponent clamps to -127
    (byte 0), so the element's code is the E2M1 value nearest v / 2^-127."""
    cases = [(2.0 ** -128, 1), (3 * 2.0 ** -128, 3), (2.0 ** -127, 2), (2.0 ** -130, 0), (-(2.0 ** -129), 8),      # -0.25: a tie, to the even code (-0)
             (5 * 2.0 ** -128, 4)]                              # 2.5 ties to the even code 4 (2.0)
    x = np.zeros((len(cases), 32), np.float32)
    for i, (v, _) in enumerate(cases):
        x[i, 17] = v
    c, s = oracle.mx_from_bf16(bf16_bits(x))
    assert np.all(s[:, 0] == 0)
    for i, (_, code) in enumerate(cases):
        assert (c[i, 8] >> 4) == code, (cases[i], c[i, 8] >> 4)
        assert not np.delete(c[i], 8).any() and (c[i, 8] & 15) == 0
