"""GPU parity: the decode-batch skinny GEMM (m <= 32) and the prefill GEMM (m > 32)."""
import numpy as np
import pytest
import torch

import oracle
from bit_quantized_decode_amd import binding as B
from bit_quantized_decode_amd import inputs as I
from helpers import (assert_within, bf16_to_f64, device, oracle_threads, pack_to_device, random_matrix,
                     sample_rows, to_dev_bf16, ulp_bf16)

pytestmark = pytest.mark.gpu


def run_gemm(packed, n, k, st, xbits, dev, y_dtype):
    x = to_dev_bf16(xbits, dev)
    y = B.gemm(packed, n, k, st, x, y_dtype=y_dtype)
    torch.cuda.synchronize()
    return y


def check_both_dtypes(codes, scales, st, xbits, rows=None, what=""):
    """fp32 output: strict bound; bf16 output: bound + one bf16 ulp of the reference."""
    dev = device()
    n, k = codes.shape[0], codes.shape[1] * 2
    packed = pack_to_device(codes, scales, dev)
    y32 = run_gemm(packed, n, k, st, xbits, dev, torch.float32).cpu().numpy().astype(np.float64)
    y16 = bf16_to_f64(run_gemm(packed, n, k, st, xbits, dev, torch.bfloat16))
    y_ref, s = oracle.gemm(codes, scales, st, xbits, rows=rows, nthreads=oracle_threads())
    sel = slice(None) if rows is None else rows
    assert_within(y32[:, sel], y_ref, s, what=f"{what} fp32")
    assert_within(y16[:, sel], y_ref, s, extra=ulp_bf16(y_ref), what=f"{what} bf16")


@pytest.mark.parametrize("m", [1, 5, 17, 32])
@pytest.mark.parametrize("n,k", [(1, 16), (100, 48), (65, 272), (200, 1040), (130, 2320)])
def test_skinny_ragged(m, n, k):
    rng = np.random.default_rng(1000 * m + 7 * n + k)
    codes, scales = random_matrix(rng, n, k)
    x = I.bf16_round(rng.standard_normal((m, k)).astype(np.float32))
    check_both_dtypes(codes, scales, I.TENSOR_SCALE, x, what=f"skinny m={m} {n}x{k}")


@pytest.mark.parametrize("m", [33, 100, 128, 129, 300])
@pytest.mark.parametrize("n,k", [(100, 48), (65, 272), (200, 1040), (257, 2320)])
def test_prefill_ragged(m, n, k):
    rng = np.random.default_rng(2000 * m + 7 * n + k)
    codes, scales = random_matrix(rng, n, k)
    x = I.bf16_round(rng.standard_normal((m, k)).astype(np.float32))
    check_both_dtypes(codes, scales, I.TENSOR_SCALE, x, what=f"prefill m={m} {n}x{k}")


@pytest.mark.parametrize("m", [32, 200])
def test_integer_regime_is_exact(m):
    dev = device()
    rng = np.random.default_rng(31 + m)
    n, k = 130, 4096
    codes = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    scales = rng.choice(np.array([0x30, 0x38, 0x40], np.uint8), size=(n, k // 16))
    x = I.bf16_round(rng.integers(-8, 9, size=(m, k)).astype(np.float32))
    packed = pack_to_device(codes, scales, dev)
    y = run_gemm(packed, n, k, 1.0, x, dev, torch.float32).cpu().numpy().astype(np.float64)
    y_ref, _ = oracle.gemm(codes, scales, np.float32(1.0), x)
    assert np.array_equal(y, y_ref)


@pytest.mark.parametrize("m", [32, 64])
def test_identity_is_exact(m):
    dev = device()
    n = k = 256
    codes = np.zeros((n, k // 2), np.uint8)
    for i in range(n):
        codes[i, i // 2] = (2 << 4) if (i & 1) else 2
    scales = np.full((n, k // 16), 0x38, np.uint8)
    x = I.activations(98, 1, m, k)
    packed = pack_to_device(codes, scales, dev)
    y = run_gemm(packed, n, k, 1.0, x, dev, torch.bfloat16)
    assert np.array_equal(y.cpu().view(torch.int16).numpy().view(np.uint16), x)


def test_strided_rows_and_output():
    """ldx > k and ldy > n: only the first k / n columns are read / written."""
    dev = device()
    rng = np.random.default_rng(41)
    m, n, k = 20, 100, 272
    codes, scales = random_matrix(rng, n, k)
    xfull = I.bf16_round(rng.standard_normal((m, k + 24)).astype(np.float32))
    packed = pack_to_device(codes, scales, dev)
    x = to_dev_bf16(xfull, dev)[:, :k]
    y = torch.full((m, 112), 7.0, dtype=torch.float32, device=dev)
    B.gemm(packed, n, k, I.TENSOR_SCALE, x, y=y[:, :n])
    torch.cuda.synchronize()
    yc = y.cpu().numpy()
    assert np.all(yc[:, n:] == 7.0)
    y_ref, s = oracle.gemm(codes, scales, I.TENSOR_SCALE, np.ascontiguousarray(xfull[:, :k]))
    assert_within(yc[:, :n], y_ref, s, what="strided")


def test_repeat_is_bit_identical():
    dev = device()
    codes, scales = I.nvfp4_matrix(I.DECODE_B32, 2, 5120, 17408)
    packed = pack_to_device(codes, scales, dev)
    x = to_dev_bf16(I.activations(I.DECODE_B32, 2, 32, 17408), dev)
    y1 = B.gemm(packed, 5120, 17408, I.TENSOR_SCALE, x).clone()
    y2 = B.gemm(packed, 5120, 17408, I.TENSOR_SCALE, x).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("mat", I.DENSE_LAYER, ids=lambda m: m.name)
def test_skinny_dense_layer_full_size(mat):
    """The 27B-class layer at 32 decode tokens (the batch-1 layer's weights), sampled rows."""
    codes, scales = I.nvfp4_matrix(I.DECODE_B1, mat.matrix_id, mat.n, mat.k)
    x = I.activations(I.DECODE_B32, mat.matrix_id, 32, mat.k)
    rows = sample_rows(mat.n, 384, 100 + mat.matrix_id)
    check_both_dtypes(codes, scales, I.TENSOR_SCALE, x, rows=rows, what=f"skinny {mat.name}")


@pytest.mark.parametrize("mat", I.PREFILL_MATRICES, ids=lambda m: m.name)
def test_prefill_full_size(mat):
    """The 512-token prefill, every matrix at full size, sampled weight rows x all 512 tokens."""
    codes, scales = I.nvfp4_matrix(I.PREFILL_512, mat.matrix_id, mat.n, mat.k)
    x = I.activations(I.PREFILL_512, mat.matrix_id, 512, mat.k)
    rows = sample_rows(mat.n, 48, 200 + mat.matrix_id)
    check_both_dtypes(codes, scales, I.TENSOR_SCALE, x, rows=rows, what=f"prefill {mat.name}")


@pytest.mark.parametrize("m,n,k", [(64, 256, 16384), (100, 300, 8192), (520, 700, 4096)])
def test_prefill_tiles_cut_between_many_workgroups(m, n, k):
    """Few output tiles over a long k: each tile's k range is shared by many
    workgroups (up to 32 here), whose partial sums the last one adds in order."""
    rng = np.random.default_rng(m * 13 + n + k)
    codes, scales = random_matrix(rng, n, k)
    x = I.bf16_round(rng.standard_normal((m, k)).astype(np.float32))
    check_both_dtypes(codes, scales, I.TENSOR_SCALE, x, what=f"prefill cut m={m} {n}x{k}")


def test_prefill_repeat_is_bit_identical_and_counters_return_to_zero():
    """The fix-up order of cut tiles is fixed, so results do not depend on
    which workgroup finishes a tile; every call leaves the counters zero."""
    dev = device()
    mat = I.PREFILL_MATRICES[2]
    codes, scales = I.nvfp4_matrix(I.PREFILL_512, mat.matrix_id, mat.n, mat.k)
    packed = pack_to_device(codes, scales, dev)
    x = to_dev_bf16(I.activations(I.PREFILL_512, mat.matrix_id, 512, mat.k), dev)
    need = B.gemm_workspace_bytes(512, mat.n, mat.k)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    y1 = B.gemm(packed, mat.n, mat.k, I.TENSOR_SCALE, x, ws=ws).clone()
    y2 = B.gemm(packed, mat.n, mat.k, I.TENSOR_SCALE, x, ws=ws).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert int(torch.count_nonzero(ws[: 1 << 18])) == 0


@pytest.mark.parametrize("m", [1, 7, 40, 300])
def test_empty_k_writes_zero_outputs(m):
    """k = 0 is an empty sum: every output is 0 (GEMV at m = 1 too)."""
    dev = device()
    n = 130
    packed = torch.zeros(16, dtype=torch.uint8, device=dev)
    x = torch.zeros((m, 8), dtype=torch.bfloat16, device=dev)
    y = torch.full((m, n), 7.0, dtype=torch.float32, device=dev)
    B.gemm(packed, n, 0, I.TENSOR_SCALE, x[:, :0], y=y)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(y)) == 0
    if m == 1:
        yv = torch.full((n,), 7.0, dtype=torch.float32, device=dev)
        B.gemv(packed, n, 0, I.TENSOR_SCALE, x[0, :0], y=yv)
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(yv)) == 0


def same_sign_inputs(rng, m, n, k):
    """Codes 0-7 only (non-negative weights), the bench's block scales, and
    activations |N(0,1)|: every product is >= 0, so every partial sum only
    grows -- the worst case for the length of an fp32 accumulation chain."""
    c = rng.integers(0, 8, size=(n, k)).astype(np.uint8)
    codes = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    scales = I.e4m3_round(np.exp2(rng.uniform(-6, 2, size=(n, k // 16))))
    x = I.bf16_round(np.abs(rng.standard_normal((m, k))).astype(np.float32))
    return codes, scales, x


@pytest.mark.parametrize("m,n,k,nrows", [
    (512, 5120, 17408, 48),    # the prefill's down product at full size
    (64, 256, 16384, None),    # few tiles, each cut between many workgroups
    (256, 512, 32768, 64),     # the longest k the products take
    (32, 5120, 17408, 128),    # decode batch of 32
    (32, 1024, 32768, 128),
    (1, 5120, 17408, None),    # one row: the GEMV mapping
    (1, 1024, 32768, None),
])
def test_same_sign_long_k(m, n, k, nrows):
    """fp32 output, the strict bound |y - y_ref| <= 1e-5 sum|w x| with every product >= 0."""
    dev = device()
    rng = np.random.default_rng(m + n + k)
    codes, scales, x = same_sign_inputs(rng, m, n, k)
    packed = pack_to_device(codes, scales, dev)
    y = run_gemm(packed, n, k, I.TENSOR_SCALE, x, dev, torch.float32).cpu().numpy().astype(np.float64)
    rows = None if nrows is None else sample_rows(n, nrows, 700 + k)
    y_ref, s = oracle.gemm(codes, scales, I.TENSOR_SCALE, x, rows=rows, nthreads=oracle_threads())
    sel = slice(None) if rows is None else rows
    worst = assert_within(y[:, sel], y_ref, s, what=f"same sign m={m} {n}x{k}")
    if m == 1:
        yv = B.gemv(packed, n, k, I.TENSOR_SCALE, to_dev_bf16(x[0], dev))
        torch.cuda.synchronize()
        worst = max(worst, assert_within(yv.cpu().numpy().astype(np.float64)[None, sel], y_ref, s,
                                         what=f"same sign gemv {n}x{k}"))
    print(f"same sign m={m} {n}x{k}: worst error {worst:.3g} of sum|w x|")
