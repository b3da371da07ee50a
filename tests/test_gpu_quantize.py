"""GPU parity: the NVFP4 quantiser against the CPU oracle, bit-exact.

Codes, block scales and the tensor scale are integer decisions (taken in fp32
on both sides), so every byte must match.
"""
import numpy as np
import pytest
import torch

import oracle
from bit_quantized_decode_amd import binding as B
from helpers import device

pytestmark = pytest.mark.gpu


def bf16_bits_of(x):
    """fp32 -> bf16 bit patterns, round to nearest even (exact arithmetic on the bits)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def run(w_host, bf16, ldw=None):
    """Quantise on the GPU; w_host: fp32 values or uint16 bf16 bits [n][k]."""
    dev = device()
    n, k = w_host.shape
    ldw = k if ldw is None else ldw
    if bf16:
        buf = torch.zeros((n, ldw), dtype=torch.int16, device=dev)
        buf[:, :k] = torch.from_numpy(w_host.view(np.int16)).to(dev)
        w = buf.view(torch.bfloat16)[:, :k]
    else:
        buf = torch.zeros((n, ldw), dtype=torch.float32, device=dev)
        buf[:, :k] = torch.from_numpy(w_host).to(dev)
        w = buf[:, :k]
    c, s, st = B.quantize(w)
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy(), np.float32(st.cpu().numpy()[0])


def check(w_host, bf16, ldw=None, what=""):
    c, s, st = run(w_host, bf16, ldw)
    c_ref, s_ref, st_ref = oracle.quantize(w_host, bf16=bf16)
    assert st.view(np.uint32) == np.float32(st_ref).view(np.uint32), (what, st, st_ref)
    bad_s = np.argwhere(s != s_ref)
    assert bad_s.size == 0, (what, "scales", bad_s[:5], s[tuple(bad_s[0])], s_ref[tuple(bad_s[0])])
    bad_c = np.argwhere(c != c_ref)
    assert bad_c.size == 0, (what, "codes", bad_c[:5], c[tuple(bad_c[0])], c_ref[tuple(bad_c[0])])


def wide_range(rng, n, k):
    """N(0,1) rows spread over 2^-12 .. 2^12 (block scales from subnormal to 448),
    with some exact zeros and negative zeros."""
    w = rng.standard_normal((n, k)) * np.exp2(rng.uniform(-12, 12, size=(n, 1)))
    w[rng.random((n, k)) < 0.02] = 0.0
    w[rng.random((n, k)) < 0.02] = -0.0
    return w.astype(np.float32)


@pytest.mark.parametrize("bf16", [True, False], ids=["bf16", "f32"])
@pytest.mark.parametrize("n,k", [(1, 16), (7, 48), (65, 272), (300, 1040), (513, 4096)])
def test_quantize_matches_oracle(n, k, bf16):
    rng = np.random.default_rng(n * 31 + k + (7 if bf16 else 0))
    w = wide_range(rng, n, k)
    check(bf16_bits_of(w) if bf16 else w, bf16, what=f"{n}x{k}")


@pytest.mark.parametrize("bf16", [True, False], ids=["bf16", "f32"])
def test_quantize_strided_rows(bf16):
    rng = np.random.default_rng(77)
    w = wide_range(rng, 33, 160)
    check(bf16_bits_of(w) if bf16 else w, bf16, ldw=200, what="strided")


def test_quantize_exact_ties_and_saturation():
    """Values at every E2M1 midpoint of a block whose divisor is exact: s_t = 2^-8
    (the matrix's largest magnitude is 10.5 = 2688 * 2^-8) and block scale 448,
    so each element divides by 1.75 exactly."""
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 5.9, 0.0, -0.25, -0.75, -2.5, -5.0, -6.0, -0.0])
    w = np.zeros((4, 32), np.float32)
    w[:, :16] = (mids * 1.75).astype(np.float32)  # 6 * 1.75 = 10.5 is the matrix maximum
    w[1, 16:] = np.float32(2.0 ** -20)             # a block whose scale is subnormal or 0
    w[2, 16:] = np.linspace(-1, 1, 16).astype(np.float32)
    w[3, 16:] = np.float32(1e-30)                  # scale rounds to 0: codes 0
    check(w, False, what="ties")
    check(bf16_bits_of(w), True, what="ties bf16")
    c, s, st = run(w, False)
    assert st == np.float32(2.0 ** -8)


def test_quantize_zero_matrix():
    c, s, st = run(np.zeros((5, 64), np.float32), False)
    assert st == np.float32(1.0) and not c.any() and not s.any()


def test_quantize_full_size_gate_matrix():
    """A 17408 x 5120 bf16 matrix (the 27B-class layer's gate), every byte."""
    rng = np.random.default_rng(5)
    w = bf16_bits_of((rng.standard_normal((17408, 5120)) * 0.02).astype(np.float32))
    check(w, True, what="gate 17408x5120")


def test_quantize_then_pack_then_gemv_round_trip():
    """The quantiser's output feeds the repack and the GEMV: y equals the oracle's
    product of the same codes."""
    from helpers import assert_within, to_dev_bf16
    from bit_quantized_decode_amd import inputs as I
    dev = device()
    rng = np.random.default_rng(8)
    n, k = 384, 2048
    w = bf16_bits_of(rng.standard_normal((n, k)).astype(np.float32))
    c, s, st = run(w, True)
    packed = B.pack(torch.from_numpy(c).to(dev), torch.from_numpy(s).to(dev))
    x = I.activations(90, 0, 1, k)[0]
    y = B.gemv(packed, n, k, float(st), to_dev_bf16(x, dev))
    torch.cuda.synchronize()
    y_ref, sb = oracle.gemm(c, s, st, x[None, :])
    assert_within(y.cpu().numpy().astype(np.float64), y_ref[0], sb[0], what="quantise -> pack -> gemv")
