"""GPU parity: offline repack and the batch-1 GEMV against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
from bit_quantized_decode_amd import binding as B
from bit_quantized_decode_amd import inputs as I
from helpers import (assert_within, device, oracle_threads, pack_to_device, random_matrix, sample_rows,
                     to_dev_bf16, to_dev_u8)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,k", [(1, 16), (100, 48), (65, 272), (64, 256), (1024, 1024), (300, 4112)])
def test_pack_unpack_round_trip(n, k):
    dev = device()
    rng = np.random.default_rng(n * 7 + k)
    codes, scales = random_matrix(rng, n, k)
    scales[0, 0] = 0x7F  # NaN byte survives untouched
    packed = pack_to_device(codes, scales, dev)
    assert packed.numel() == B.packed_bytes(n, k)
    c2, s2 = B.unpack(packed, n, k)
    torch.cuda.synchronize()
    assert np.array_equal(c2.cpu().numpy(), codes)
    assert np.array_equal(s2.cpu().numpy(), scales)
    # Packing is a permutation plus zero padding: the byte histogram only gains zeros.
    hp = np.bincount(packed.cpu().numpy(), minlength=256)
    hc = np.bincount(codes.ravel(), minlength=256) + np.bincount(scales.ravel(), minlength=256)
    assert np.array_equal(hp[1:], hc[1:])
    assert hp[0] == hc[0] + (packed.numel() - codes.size - scales.size)


def run_gemv(codes, scales, st, xbits, dev):
    n, k = codes.shape[0], codes.shape[1] * 2
    packed = pack_to_device(codes, scales, dev)
    x = to_dev_bf16(xbits, dev)
    y = B.gemv(packed, n, k, st, x)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("n,k", [(1, 16), (100, 48), (65, 272), (200, 1040), (333, 4112), (64, 256), (130, 8192)])
def test_gemv_ragged_shapes(n, k):
    dev = device()
    rng = np.random.default_rng(11 * n + k)
    codes, scales = random_matrix(rng, n, k)
    x = I.bf16_round(rng.standard_normal(k).astype(np.float32))
    y = run_gemv(codes, scales, I.TENSOR_SCALE, x, dev)
    y_ref, s = oracle.gemm(codes, scales, I.TENSOR_SCALE, x[None, :])
    assert_within(y, y_ref[0], s[0], what=f"gemv {n}x{k}")


def test_gemv_single_1024():
    """The 1024 x 1024 batch-1 GEMV, every output."""
    dev = device()
    codes, scales = I.nvfp4_matrix(I.GEMV_1K, 0, 1024, 1024)
    x = I.activations(I.GEMV_1K, 0, 1, 1024)[0]
    y = run_gemv(codes, scales, I.TENSOR_SCALE, x, dev)
    y_ref, s = oracle.gemm(codes, scales, I.TENSOR_SCALE, x[None, :])
    assert_within(y, y_ref[0], s[0], what="gemv 1024")


def test_gemv_identity_is_exact():
    dev = device()
    n = k = 512
    codes = np.zeros((n, k // 2), np.uint8)
    for i in range(n):
        codes[i, i // 2] = (2 << 4) if (i & 1) else 2
    scales = np.full((n, k // 16), 0x38, np.uint8)
    x = I.activations(98, 0, 1, k)[0]
    y = run_gemv(codes, scales, 1.0, x, dev)
    ref = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(y, ref)


def test_gemv_one_hot_addressing_is_exact():
    dev = device()
    n, k = 128, 512
    rng = np.random.default_rng(5)
    x = I.activations(97, 0, 1, k)[0]
    xv = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double().numpy()
    for trial in range(24):
        n0, k0 = int(rng.integers(n)), int(rng.integers(k))
        code = int(rng.integers(1, 16))
        sbyte = int(rng.choice([0x01, 0x08, 0x38, 0x3C, 0x7E, 0xB8]))
        codes = np.zeros((n, k // 2), np.uint8)
        codes[n0, k0 // 2] = (code << 4) if (k0 & 1) else code
        scales = np.full((n, k // 16), 0x38, np.uint8)
        scales[n0, k0 // 16] = sbyte
        y = run_gemv(codes, scales, 0.75, x, dev)
        expect = np.zeros(n)
        expect[n0] = oracle.e2m1(code).item() * oracle.e4m3(sbyte).item() * 0.75 * xv[k0]
        assert np.array_equal(y, expect), (trial, n0, k0, code, sbyte)


def test_gemv_integer_regime_is_exact():
    """Integer x, scales {0.5, 1, 2}, s_t = 1: all partial sums are exact in fp32."""
    dev = device()
    rng = np.random.default_rng(12)
    n, k = 256, 4096
    codes = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    scales = rng.choice(np.array([0x30, 0x38, 0x40], np.uint8), size=(n, k // 16))
    x = I.bf16_round(rng.integers(-8, 9, size=k).astype(np.float32))
    y = run_gemv(codes, scales, 1.0, x, dev)
    y_ref, _ = oracle.gemm(codes, scales, np.float32(1.0), x[None, :])
    assert np.array_equal(y, y_ref[0])


def test_gemv_nan_scale_propagates_only_to_its_row():
    dev = device()
    rng = np.random.default_rng(13)
    n, k = 70, 512
    codes, scales = random_matrix(rng, n, k)
    scales[3, 5] = 0x7F
    x = I.bf16_round(rng.standard_normal(k).astype(np.float32))
    y = run_gemv(codes, scales, I.TENSOR_SCALE, x, dev)
    assert np.isnan(y[3])
    assert np.isfinite(np.delete(y, 3)).all()


def test_gemv_repeat_is_bit_identical():
    dev = device()
    codes, scales = I.nvfp4_matrix(I.DECODE_B1, 2, 5120, 17408)
    packed = pack_to_device(codes, scales, dev)
    x = to_dev_bf16(I.activations(I.DECODE_B1, 2, 1, 17408)[0], dev)
    y1 = B.gemv(packed, 5120, 17408, I.TENSOR_SCALE, x).clone()
    y2 = B.gemv(packed, 5120, 17408, I.TENSOR_SCALE, x).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


@pytest.mark.parametrize("mat", I.DENSE_LAYER, ids=lambda m: m.name)
def test_gemv_dense_layer_full_size(mat):
    """The 27B-class layer's five GEMVs at full size, in the benchmark's launch configuration."""
    dev = device()
    codes, scales = I.nvfp4_matrix(I.DECODE_B1, mat.matrix_id, mat.n, mat.k)
    x = I.activations(I.DECODE_B1, mat.matrix_id, 1, mat.k)[0]
    y = run_gemv(codes, scales, I.TENSOR_SCALE, x, dev)
    rows = sample_rows(mat.n, 1500, mat.matrix_id)
    y_ref, s = oracle.gemm(codes, scales, I.TENSOR_SCALE, x[None, :], rows=rows, nthreads=oracle_threads())
    assert_within(y[rows], y_ref[0], s[0], what=f"gemv {mat.name}")


def test_gemm_m1_matches_gemv():
    dev = device()
    rng = np.random.default_rng(21)
    n, k = 300, 2064
    codes, scales = random_matrix(rng, n, k)
    packed = pack_to_device(codes, scales, dev)
    xb = I.bf16_round(rng.standard_normal((1, k)).astype(np.float32))
    x = to_dev_bf16(xb, dev)
    yv = B.gemv(packed, n, k, I.TENSOR_SCALE, x[0].contiguous())
    ym = B.gemm(packed, n, k, I.TENSOR_SCALE, x, y_dtype=torch.float32)
    torch.cuda.synchronize()
    y_ref, s = oracle.gemm(codes, scales, I.TENSOR_SCALE, xb)
    assert_within(yv.cpu().numpy(), y_ref[0], s[0], what="gemv")
    assert_within(ym.cpu().numpy()[0], y_ref[0], s[0], what="gemm m=1")


def test_shared_workspace_across_shapes():
    """Split-K calls of different shapes share one workspace in stream order: a skinny call
    with few row groups, then a GEMV with many row tiles, then the skinny call again."""
    dev = device()
    ws = torch.zeros(B.gemv_workspace_bytes(17408, 5120) + B.gemm_workspace_bytes(32, 5120, 17408) + (1 << 20),
                     dtype=torch.uint8, device=dev)
    cd, sd = I.nvfp4_matrix(I.DECODE_B1, 2, 5120, 17408)
    cg, sg = I.nvfp4_matrix(I.DECODE_B1, 0, 17408, 5120)
    pd, pg = pack_to_device(cd, sd, dev), pack_to_device(cg, sg, dev)
    xd = I.activations(I.DECODE_B32, 2, 32, 17408)
    xg = I.activations(I.DECODE_B1, 0, 1, 5120)[0]
    y_d1 = B.gemm(pd, 5120, 17408, I.TENSOR_SCALE, to_dev_bf16(xd, dev), y_dtype=torch.float32, ws=ws).clone()
    y_g = B.gemv(pg, 17408, 5120, I.TENSOR_SCALE, to_dev_bf16(xg, dev), ws=ws).clone()
    y_d2 = B.gemm(pd, 5120, 17408, I.TENSOR_SCALE, to_dev_bf16(xd, dev), y_dtype=torch.float32, ws=ws).clone()
    torch.cuda.synchronize()
    assert torch.equal(y_d1, y_d2)
    rows = sample_rows(17408, 600, 7)
    y_ref, s = oracle.gemm(cg, sg, I.TENSOR_SCALE, xg[None, :], rows=rows, nthreads=oracle_threads())
    assert_within(y_g.cpu().numpy()[rows], y_ref[0], s[0], what="gemv after skinny")
    assert int(ws[:262144].count_nonzero()) == 0   # counters back at zero
