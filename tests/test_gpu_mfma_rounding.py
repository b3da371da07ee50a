"""GPU: how one matrix instruction rounds -- the premise of the products'
accumulation error bounds.

The bounds charge each matrix instruction D = A B + C an error of at most
alpha * 2^-24 * (|C| + sum |a b|).  These tests measure that error for
v_mfma_f32_32x32x16_bf16 (the exact path's) and for
v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 operands (the W4A4 path's), on
random operands, on sums that nearly cancel, on accumulators far larger or
smaller than the products, and on same-sign sums.  The FP4 instruction
behaves as one rounding of the exact sum (alpha <= 1); the bf16 one does not
(its worst measured case is about 3.5, on same-sign sums; 60-80 % of its
results are correctly rounded), so the bounds take alpha = 4 for it.
Operand ranges keep every exact sum representable in fp64 (reference: numpy
in fp64)."""
import ctypes
import os

import numpy as np
import pytest
import torch

from helpers import device

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
U = 2.0 ** -24
ALPHA_BF16 = 4.0   # the per-instruction error the accumulation bounds charge the bf16 instruction
ALPHA_FP4 = 1.0
ALPHA_DOT2 = 3.0   # v_dot2_f32_bf16 (the GEMV's): two products and an fp32 addend, not fused


def probes():
    path = os.path.join(ROOT, "bit_quantized_decode_amd", "libnvfp4_probes.so")
    if not os.path.exists(path):
        pytest.fail("libnvfp4_probes.so is not built")
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    L.probe_mfma_bf16_once.argtypes = [P, P, P, P, ctypes.c_int, P]
    L.probe_mfma_fp4_once.argtypes = [P, P, P, P, P, P, ctypes.c_int, P]
    L.probe_dot2_once.argtypes = [P, P, P, P, ctypes.c_int, P]
    return L


def bf16_values(rng, shape, emin, emax):
    """Random bf16 bit patterns (sign, 8-bit significand, exponent in [emin, emax]) and their values."""
    sign = rng.integers(0, 2, size=shape)
    mant = rng.integers(128, 256, size=shape)
    e = rng.integers(emin, emax + 1, size=shape)
    val = np.where(sign == 1, -1.0, 1.0) * mant * np.exp2(e - 7.0)
    bits = (val.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64), val)
    return bits, val


def f32_values(rng, shape, emin, emax):
    sign = np.where(rng.integers(0, 2, size=shape) == 1, -1.0, 1.0)
    mant = rng.integers(1 << 23, 1 << 24, size=shape)
    e = rng.integers(emin, emax + 1, size=shape)
    return (sign * mant * np.exp2(e - 23.0)).astype(np.float32)


def report(d, exact, mag, what):
    err = np.abs(d.astype(np.float64) - exact)
    alpha = float(np.max(err / (U * np.maximum(mag, 1e-300))))
    rounded = float(np.mean(d == exact.astype(np.float32)))
    print(f"{what}: max error {alpha:.4f} x 2^-24 (|C| + sum|ab|); correctly rounded in {100 * rounded:.2f} %")
    return alpha


def test_bf16_mfma_error_per_instruction():
    dev = device()
    L = probes()
    rng = np.random.default_rng(1616)
    count = 4096
    a_bits, a = bf16_values(rng, (count, 32, 16), -4, 4)
    b_bits, b = bf16_values(rng, (count, 32, 16), -4, 4)     # [problem][column][k]
    prod = np.einsum("prk,pck->prc", a, b)                   # exact: every partial sum fits 45 bits
    mag_p = np.einsum("prk,pck->prc", np.abs(a), np.abs(b))
    c = f32_values(rng, (count, 32, 32), -8, 8)
    q = count // 4
    # Sums that nearly cancel: C is minus the products' sum, rounded to fp32, plus a few of its ulps.
    c[:q] = (-prod[:q]).astype(np.float32) + np.float32(2.0 ** -20) * rng.integers(-3, 4, size=(q, 32, 32))
    # Accumulators far larger, then far smaller, than the products.
    c[q:2 * q] *= np.float32(2.0 ** 6)
    c[2 * q:3 * q] *= np.float32(2.0 ** -6)
    # Same-sign sums: every product and C >= 0 (the case of a long positive chain).
    a_bits[3 * q:] &= 0x7FFF
    b_bits[3 * q:] &= 0x7FFF
    a[3 * q:], b[3 * q:] = np.abs(a[3 * q:]), np.abs(b[3 * q:])
    prod[3 * q:] = np.einsum("prk,pck->prc", a[3 * q:], b[3 * q:])
    c[3 * q:] = np.abs(c[3 * q:])
    exact = c.astype(np.float64) + prod
    mag = np.abs(c.astype(np.float64)) + mag_p
    A = torch.from_numpy(a_bits.view(np.int16)).to(dev)
    B = torch.from_numpy(b_bits.view(np.int16)).to(dev)
    C = torch.from_numpy(c).to(dev)
    D = torch.empty_like(C)
    assert L.probe_mfma_bf16_once(A.data_ptr(), B.data_ptr(), C.data_ptr(), D.data_ptr(), count, None) == 0
    torch.cuda.synchronize()
    alpha = report(D.cpu().numpy(), exact, mag, "v_mfma_f32_32x32x16_bf16")
    assert alpha <= ALPHA_BF16


E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6], np.float64)


def test_fp4_scaled_mfma_is_one_rounding():
    dev = device()
    L = probes()
    rng = np.random.default_rng(464)
    count = 768
    codes_a = rng.integers(0, 16, size=(count, 32, 64))
    codes_b = rng.integers(0, 16, size=(count, 32, 64))     # [problem][column][k]
    sa = rng.integers(124, 131, size=(count, 32, 2))        # E8M0 exponents -3..3
    sb = rng.integers(124, 131, size=(count, 32, 2))
    va = E2M1[codes_a] * np.exp2(np.repeat(sa - 127.0, 32, axis=2))
    vb = E2M1[codes_b] * np.exp2(np.repeat(sb - 127.0, 32, axis=2))
    prod = np.einsum("prk,pck->prc", va, vb)
    mag_p = np.einsum("prk,pck->prc", np.abs(va), np.abs(vb))
    c = f32_values(rng, (count, 32, 32), -6, 6)
    third = count // 3
    c[:third] = (-prod[:third]).astype(np.float32) + np.float32(2.0 ** -16) * rng.integers(-3, 4, size=(third, 32, 32))
    c[third:2 * third] *= np.float32(2.0 ** 8)
    c[2 * third:] *= np.float32(2.0 ** -4)
    exact = c.astype(np.float64) + prod
    mag = np.abs(c.astype(np.float64)) + mag_p

    def pack(codes):
        return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    A = torch.from_numpy(pack(codes_a)).to(dev)
    B = torch.from_numpy(pack(codes_b)).to(dev)
    SA = torch.from_numpy(sa.astype(np.uint8)).to(dev)
    SB = torch.from_numpy(sb.astype(np.uint8)).to(dev)
    C = torch.from_numpy(c).to(dev)
    D = torch.empty_like(C)
    assert L.probe_mfma_fp4_once(A.data_ptr(), B.data_ptr(), SA.data_ptr(), SB.data_ptr(), C.data_ptr(),
                                 D.data_ptr(), count, None) == 0
    torch.cuda.synchronize()
    alpha = report(D.cpu().numpy(), exact, mag, "v_mfma_scale_f32_32x32x64_f8f6f4 (FP4)")
    assert alpha <= ALPHA_FP4


def test_dot2_error_per_instruction():
    """v_dot2_f32_bf16 (the GEMV's inner product): c + a0 b0 + a1 b1, with
    exact products, rounds more than once (worst measured case about 2.7,
    on near-cancelling and same-sign sums); the GEMV's bound charges it 3."""
    dev = device()
    L = probes()
    rng = np.random.default_rng(2222)
    n = 1 << 22
    a_bits, a = bf16_values(rng, (n, 2), -6, 6)
    b_bits, b = bf16_values(rng, (n, 2), -6, 6)
    c = f32_values(rng, (n,), -12, 12)
    q = n // 4
    prod = (a * b).sum(axis=1)
    c[:q] = (-prod[:q]).astype(np.float32)                       # near-cancelling
    same = slice(3 * q, n)                                       # same sign
    a_bits[same] &= 0x7FFF
    b_bits[same] &= 0x7FFF
    a[same], b[same] = np.abs(a[same]), np.abs(b[same])
    c[same] = np.abs(c[same])
    prod = (a * b).sum(axis=1)
    exact = c.astype(np.float64) + prod                          # exact: <= 52 significant bits
    mag = np.abs(c.astype(np.float64)) + np.abs(a * b).sum(axis=1)
    A = torch.from_numpy(a_bits.view(np.uint32).reshape(n).view(np.int32)).to(dev)
    B = torch.from_numpy(b_bits.view(np.uint32).reshape(n).view(np.int32)).to(dev)
    C = torch.from_numpy(c).to(dev)
    D = torch.empty_like(C)
    assert L.probe_dot2_once(A.data_ptr(), B.data_ptr(), C.data_ptr(), D.data_ptr(), n, None) == 0
    torch.cuda.synchronize()
    alpha = report(D.cpu().numpy(), exact, mag, "v_dot2_f32_bf16")
    assert alpha <= ALPHA_DOT2
