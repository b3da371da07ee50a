"""Pins of the CPU oracle against facts fixed outside it.

Each test checks the oracle against something it does not contain: the OCP
format tables (fixtures under tests/golden/), an independent library routine
(torch's float8_e4m3fn / bfloat16 decoding, torch float64 matmul, torch.topk,
numpy's stable argsort, scipy's softmax), a closed form written differently
from the oracle's lookup, or an exact integer computation.
"""
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from bit_quantized_decode_amd import inputs as I

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_fixture(name):
    rows = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def e2m1_closed_form(code):
    """Generic minifloat decode: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = (m / 2.0) if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1)
    return -mag if s else mag


E2M1_INDEPENDENT = np.array([e2m1_closed_form(c) for c in range(16)], dtype=np.float64)


def decode_independent(codes, scales, st):
    """W = s_t * e2m1 * e4m3 with numpy nibble split, the closed form above, torch's E4M3."""
    n, kh = codes.shape
    c = np.stack([codes & 15, codes >> 4], axis=-1).reshape(n, 2 * kh)
    sc = torch.from_numpy(np.ascontiguousarray(scales)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return E2M1_INDEPENDENT[c] * np.repeat(sc, 16, axis=1) * float(st)


def bf16_bits_to_f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


# ---- element decoders ------------------------------------------------------

def test_e2m1_matches_spec_table():
    rows = read_fixture("e2m1_values.txt")
    assert len(rows) == 16
    for code, bits, value in rows:
        c = int(code)
        assert int(bits, 2) == c
        got = oracle.e2m1(c).item()
        assert got == float(value)
        assert math.copysign(1.0, got) == math.copysign(1.0, float(value))


def test_e2m1_matches_closed_form():
    for c in range(16):
        assert oracle.e2m1(c).item() == e2m1_closed_form(c)


def test_e4m3_all_bytes_match_torch():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3(b)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_e4m3_spec_points():
    for byte, value in read_fixture("e4m3_values.txt"):
        got = oracle.e4m3(int(byte, 16)).item()
        if value == "nan":
            assert math.isnan(got)
        else:
            assert got == float(value), (byte, got, value)
            assert math.copysign(1.0, got) == math.copysign(1.0, float(value))


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 65536, size=4000, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # leave out Inf/NaN patterns
    assert np.array_equal(oracle.bf16_to_f64(bits), bf16_bits_to_f64(bits))


def test_every_weight_value_is_exact_in_bf16():
    """e2m1 * e4m3 (finite) needs <= 6 significant bits and lies in bf16's range."""
    e2 = E2M1_INDEPENDENT
    sc = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    prod = (e2[:, None] * sc[None, ~np.isnan(sc)]).ravel()
    as_bf16 = torch.from_numpy(prod).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(prod, as_bf16)


# ---- dense product -----------------------------------------------------------

def random_matrix(rng, n, k):
    codes = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    scales = I.e4m3_round(np.exp2(rng.uniform(-6, 2, size=(n, k // 16))))
    return codes, scales


@pytest.mark.parametrize("n", range(1, 9))
@pytest.mark.parametrize("k", [16, 32, 48])
def test_gemm_bruteforce_matches_torch_float64(n, k):
    rng = np.random.default_rng(1000 * n + k)
    codes, scales = random_matrix(rng, n, k)
    x = I.bf16_round(rng.standard_normal((3, k)).astype(np.float32))
    y, s = oracle.gemm(codes, scales, I.TENSOR_SCALE, x, nthreads=1)
    w = torch.from_numpy(decode_independent(codes, scales, I.TENSOR_SCALE))
    xt = torch.from_numpy(bf16_bits_to_f64(x))
    yref = (xt @ w.T).numpy()
    sref = (xt.abs() @ w.abs().T).numpy()
    assert np.all(np.abs(y - yref) <= 1e-13 * sref + 1e-300)
    assert np.allclose(s, sref, rtol=1e-13, atol=0)


def test_gemm_medium_generator_distributions():
    codes, scales = I.nvfp4_matrix(99, 0, 37, 160)
    x = I.activations(99, 0, 5, 160)
    y, s = oracle.gemm(codes, scales, I.TENSOR_SCALE, x, nthreads=2)
    w = torch.from_numpy(decode_independent(codes, scales, I.TENSOR_SCALE))
    xt = torch.from_numpy(bf16_bits_to_f64(x))
    assert np.all(np.abs(y - (xt @ w.T).numpy()) <= 1e-13 * s)


def test_dequant_matches_independent_decode():
    rng = np.random.default_rng(3)
    codes, scales = random_matrix(rng, 5, 64)
    assert np.array_equal(oracle.dequant(codes, scales, np.float32(0.375)),
                          decode_independent(codes, scales, np.float32(0.375)))


def test_identity_returns_x_exactly():
    n = k = 64
    codes = np.zeros((n, k // 2), np.uint8)
    for i in range(n):
        codes[i, i // 2] = (2 << 4) if (i & 1) else 2      # code 2 = 1.0 on the diagonal
    scales = np.full((n, k // 16), 0x38, np.uint8)         # E4M3 1.0
    x = I.activations(98, 0, 2, k)
    y, _ = oracle.gemm(codes, scales, np.float32(1.0), x)
    assert np.array_equal(y, bf16_bits_to_f64(x))


def test_one_hot_picks_one_scaled_activation():
    n, k = 4, 48
    rows = read_fixture("e2m1_values.txt")
    table = {int(c): float(v) for c, _, v in rows}
    x = I.activations(97, 0, 1, k)
    xv = bf16_bits_to_f64(x)[0]
    for k0 in range(k):
        for code, sbyte in ((1, 0x38), (7, 0x7E), (9, 0x01), (15, 0x3C), (5, 0x08)):
            n0 = k0 % n
            codes = np.zeros((n, k // 2), np.uint8)
            codes[n0, k0 // 2] = (code << 4) if (k0 & 1) else code
            scales = np.full((n, k // 16), 0x38, np.uint8)
            scales[n0, k0 // 16] = sbyte
            st = np.float32(0.75)
            y, _ = oracle.gemm(codes, scales, st, x)
            sc = torch.tensor([sbyte], dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).item()
            expect = np.zeros(n)
            expect[n0] = table[code] * sc * 0.75 * xv[k0]
            assert np.array_equal(y[0], expect), (k0, code, sbyte)


def test_integer_exact_regime():
    """Integer x, scales in {0.5, 1, 2}, s_t = 1: 4*W*x is an integer, so the sum is exact."""
    rng = np.random.default_rng(11)
    n, k = 16, 4096
    codes = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    scales = rng.choice(np.array([0x30, 0x38, 0x40], np.uint8), size=(n, k // 16))
    xi = rng.integers(-8, 9, size=(2, k))
    x = I.bf16_round(xi.astype(np.float32))
    y, _ = oracle.gemm(codes, scales, np.float32(1.0), x)
    c = np.stack([codes & 15, codes >> 4], axis=-1).reshape(n, k).astype(np.int64)
    # 4*e2m1 is an even integer and 2*sigma is in {1, 2, 4}, so 4*e2m1*sigma = (4*e2m1)*(2*sigma)/2 exactly
    two_sigma = np.repeat(np.select([scales == 0x30, scales == 0x38], [1, 2], 4), 16, axis=1)
    w4 = np.rint(4 * E2M1_INDEPENDENT[c]).astype(np.int64) * two_sigma // 2
    exact4 = xi @ w4.T                                           # = 4 * y exactly (integers)
    assert np.array_equal(y * 4, exact4.astype(np.float64))


def test_row_subset_matches_full():
    codes, scales = I.nvfp4_matrix(96, 0, 50, 64)
    x = I.activations(96, 0, 3, 64)
    y, s = oracle.gemm(codes, scales, I.TENSOR_SCALE, x)
    rows = np.array([49, 0, 17, 17, 3], np.int64)
    ys, ss = oracle.gemm(codes, scales, I.TENSOR_SCALE, x, rows=rows)
    assert np.array_equal(ys, y[:, rows]) and np.array_equal(ss, s[:, rows])


# ---- routing -------------------------------------------------------------------

def test_route_matches_bruteforce_sort_and_softmax():
    rng = np.random.default_rng(5)
    t, e, k = 7, 40, 5
    logits = rng.standard_normal((t, e)).astype(np.float32)
    logits[2, 10] = logits[2, 3]                      # a tie: the smaller id must rank first
    ids, g = oracle.route(logits, k)
    for r in range(t):
        order = np.lexsort((np.arange(e), -logits[r].astype(np.float64)))
        assert np.array_equal(ids[r], order[:k])
        ref = scipy.special.softmax(logits[r, order[:k]].astype(np.float64))
        assert np.allclose(g[r], ref, rtol=1e-14, atol=0)
        assert abs(g[r].sum() - 1.0) < 1e-14


def test_route_matches_torch_topk_without_ties():
    logits = I.router_logits(95, 32, 512)
    ids, g = oracle.route(logits, 10)
    vals, tids = torch.topk(torch.from_numpy(logits).double(), 10, dim=1)
    assert np.array_equal(ids, tids.numpy().astype(np.int32))
    assert np.allclose(g, torch.softmax(vals, dim=1).numpy(), rtol=1e-14)


def test_route_uniform_logits_pick_lowest_ids():
    logits = np.full((3, 64), 0.25, np.float32)
    ids, g = oracle.route(logits, 10)
    assert np.array_equal(ids, np.tile(np.arange(10, dtype=np.int32), (3, 1)))
    assert np.allclose(g, 0.1, rtol=1e-15)
    ids1, g1 = oracle.route(logits, 1)
    assert np.all(ids1 == 0) and np.all(g1 == 1.0)


def test_route_bias_only_picks_hottest_experts():
    e = 512
    r = I.generator(94, 0, 4).permutation(e) + 1
    bias = (-1.1 * np.log(r.astype(np.float64))).astype(np.float32)
    ids, _ = oracle.route(bias[None, :].copy(), 10)
    assert np.array_equal(ids[0], np.argsort(r)[:10])


def test_group_matches_numpy():
    logits = I.router_logits(93, 32, 512)
    ids, _ = oracle.route(logits, 10)
    counts, offsets, perm, pos = oracle.group(ids, 512)
    flat = ids.ravel()
    assert np.array_equal(counts, np.bincount(flat, minlength=512))
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=512))]))
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))
    assert np.array_equal(pos[perm], np.arange(flat.size))
    assert offsets[-1] == 320
    for row in ids:
        assert len(set(row.tolist())) == 10


def test_silu_matches_torch():
    z = np.linspace(-30, 30, 601)
    assert np.allclose(oracle.silu(z), torch.nn.functional.silu(torch.from_numpy(z)).numpy(), rtol=1e-15, atol=1e-300)
    assert oracle.silu(0.0).item() == 0.0


# ---- the expert layer ---------------------------------------------------------

def small_moe(seed, e, t, hidden, inter):
    shape = I.MoeShape(tokens=t, experts=e, top_k=1, hidden=hidden, inter=inter)
    w = I.moe_weights(seed, shape)
    x = I.activations(seed, 0, t, hidden)
    logits = I.router_logits(seed, t, e)
    return w, x, logits


@pytest.mark.parametrize("top_k", [1, 2, 4])
def test_moe_matches_torch_float64_chain(top_k):
    e, t, hidden, inter = 6, 5, 32, 16
    w, x, logits = small_moe(92, e, t, hidden, inter)
    ids, g, y, yb = oracle.moe((w.gate_codes, w.gate_scales, w.gate_st), (w.up_codes, w.up_scales, w.up_st),
                               (w.down_codes, w.down_scales, w.down_st), x, logits, top_k, nthreads=2)
    xt = torch.from_numpy(bf16_bits_to_f64(x))
    vals, tids = torch.topk(torch.from_numpy(logits).double(), top_k, dim=1)
    gt = torch.softmax(vals, dim=1)
    assert np.array_equal(ids, tids.numpy())
    assert np.allclose(g, gt.numpy(), rtol=1e-14)
    yref = torch.zeros(t, hidden, dtype=torch.float64)
    ybref = torch.zeros(t, hidden, dtype=torch.float64)
    for ti in range(t):
        for j in range(top_k):
            ex = int(tids[ti, j])
            wg = torch.from_numpy(decode_independent(w.gate_codes[ex], w.gate_scales[ex], w.gate_st[ex]))
            wu = torch.from_numpy(decode_independent(w.up_codes[ex], w.up_scales[ex], w.up_st[ex]))
            wd = torch.from_numpy(decode_independent(w.down_codes[ex], w.down_scales[ex], w.down_st[ex]))
            h = torch.nn.functional.silu(wg @ xt[ti]) * (wu @ xt[ti])
            yref[ti] += gt[ti, j] * (wd @ h)
            ybref[ti] += gt[ti, j] * (wd.abs() @ h.abs())
    # ybound is the magnitude sum the end-to-end bound scales with: sum_j g_j |Wd| |h_j|
    assert np.allclose(yb, ybref.numpy(), rtol=1e-12, atol=0)
    assert np.all(yb >= np.abs(y) * (1 - 1e-12))
    assert np.all(np.abs(y - yref.numpy()) <= 1e-12 * yb + 1e-300)


def test_moe_ybound_closed_form_on_signed_and_scaled_weights():
    """ybound on a hand-built layer: one expert, h known in closed form.

    Gate codes all 0 except one weight, so G = w*x exactly; up weights give U;
    down weights of alternating sign make |Wd h| differ from |Wd| |h|, so a
    bound computed from the signed sum (a dropped abs) fails here."""
    hidden, inter, t = 32, 16, 1
    gc = np.zeros((1, inter, hidden // 2), np.uint8)
    uc = np.zeros((1, inter, hidden // 2), np.uint8)
    gc[0, :, 0] = 2                               # G[i] = 1.0 * x[0]  (code 2 = 1.0 at k = 0)
    uc[0, :, 0] = 4                               # U[i] = 2.0 * x[0]  (code 4 = 2.0)
    gs = np.full((1, inter, hidden // 16), 0x38, np.uint8)   # E4M3 1.0
    us = gs.copy()
    dc = np.zeros((1, hidden, inter // 2), np.uint8)
    dc[0, :, :] = (10 << 4) | 2                   # codes 2 (+1.0) and 10 (-1.0) alternate along i
    ds = np.full((1, hidden, inter // 16), 0x40, np.uint8)   # E4M3 2.0
    one = np.ones(1, np.float32)
    xv = np.zeros((t, hidden), np.float32)
    xv[0, 0] = 1.5
    x = I.bf16_round(xv)
    logits = np.zeros((t, 1), np.float32)
    ids, g, y, yb = oracle.moe((gc, gs, one), (uc, us, one), (dc, ds, one), x, logits, 1)
    hval = (1.5 / (1.0 + math.exp(-1.5))) * 3.0   # silu(1.5) * (2 * 1.5)
    # d[o] = sum_i 2 * (+-1) * h = 0 (inter even); |d| bound = sum_i 2 * h = 2 * inter * h
    assert np.all(np.abs(y) <= 1e-15)
    assert np.allclose(yb, 2.0 * inter * hval, rtol=1e-15, atol=0)


def test_moe_single_expert_reduces_to_dense_chain():
    w, x, logits = small_moe(91, 1, 4, 48, 32)
    ids, g, y, _ = oracle.moe((w.gate_codes, w.gate_scales, w.gate_st), (w.up_codes, w.up_scales, w.up_st),
                              (w.down_codes, w.down_scales, w.down_st), x, logits, 1)
    assert np.all(ids == 0) and np.all(g == 1.0)
    xt = torch.from_numpy(bf16_bits_to_f64(x))
    wg = torch.from_numpy(decode_independent(w.gate_codes[0], w.gate_scales[0], w.gate_st[0]))
    wu = torch.from_numpy(decode_independent(w.up_codes[0], w.up_scales[0], w.up_st[0]))
    wd = torch.from_numpy(decode_independent(w.down_codes[0], w.down_scales[0], w.down_st[0]))
    ref = (torch.nn.functional.silu(xt @ wg.T) * (xt @ wu.T)) @ wd.T
    assert np.allclose(y, ref.numpy(), rtol=1e-12, atol=1e-14)
