"""GPU parity for the decode widths 2..8 of a batch-wide round (the layer's
five products in one batched launch, as the benchmark runs them) and for the
output-head GEMV at a 248k-row vocabulary; sampled rows against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from bit_quantized_decode_amd import binding as B
from bit_quantized_decode_amd import inputs as I
from helpers import (assert_within, bf16_to_f64, device, oracle_threads, pack_to_device, sample_rows, to_dev_bf16,
                     ulp_bf16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def layer():
    dev = device()
    mats = []
    for mat in I.DENSE_LAYER:
        codes, scales = I.nvfp4_matrix(I.DECODE_B1, mat.matrix_id, mat.n, mat.k)
        mats.append((mat, codes, scales, pack_to_device(codes, scales, dev)))
    return dev, mats


@pytest.mark.parametrize("m", [2, 3, 4, 8])
def test_decode_width_layer_batched(layer, m):
    dev, mats = layer
    xs = [I.activations(I.DECODE_WIDTHS, mat.matrix_id, m, mat.k) for mat, _, _, _ in mats]
    ys = [torch.empty((m, mat.n), dtype=torch.bfloat16, device=dev) for mat, _, _, _ in mats]
    items = [(p, mat.n, mat.k, I.TENSOR_SCALE, to_dev_bf16(x, dev), y) for (mat, _, _, p), x, y in zip(mats, xs, ys)]
    B.gemm_batched(items)
    torch.cuda.synchronize()
    for (mat, codes, scales, _), x, y in zip(mats, xs, ys):
        rows = sample_rows(mat.n, 200, 300 + m + mat.matrix_id)
        y_ref, s = oracle.gemm(codes, scales, I.TENSOR_SCALE, x, rows=rows, nthreads=oracle_threads())
        got = bf16_to_f64(y)[:, rows]
        assert_within(got, y_ref, s, extra=ulp_bf16(y_ref), what=f"width {m} {mat.name}")


def test_output_head_gemv():
    """248000 x 5120 (715 MB packed), batch 1, sampled rows including the ragged last tile."""
    dev = device()
    mat = I.HEAD
    codes, scales = I.nvfp4_matrix(I.OUTPUT_HEAD, mat.matrix_id, mat.n, mat.k)
    packed = pack_to_device(codes, scales, dev)
    x = I.activations(I.OUTPUT_HEAD, 0, 1, mat.k)[0]
    y = B.gemv(packed, mat.n, mat.k, I.TENSOR_SCALE, to_dev_bf16(x, dev))
    torch.cuda.synchronize()
    rows = np.union1d(sample_rows(mat.n, 1000, 400), np.arange(mat.n - 100, mat.n))
    y_ref, s = oracle.gemm(codes, scales, I.TENSOR_SCALE, x[None, :], rows=rows, nthreads=oracle_threads())
    assert_within(y.cpu().numpy().astype(np.float64)[rows], y_ref[0], s[0], what="output head")


def test_one_and_two_rows_equal_gemv_bit_for_bit():
    """m <= 2 runs the GEMV's mapping: each row's fp32 outputs equal a GEMV of
    that row exactly (strided x and y, a ragged k and n)."""
    dev = device()
    rng = np.random.default_rng(23)
    n, k = 1000, 5136
    codes, scales = I.nvfp4_matrix(91, 0, n, k)
    packed = pack_to_device(codes, scales, dev)
    xb = I.activations(91, 1, 2, k)
    xs = torch.zeros((2, k + 24), dtype=torch.bfloat16, device=dev)
    xs[:, :k] = to_dev_bf16(xb, dev)
    ys = torch.zeros((2, n + 5), dtype=torch.float32, device=dev)
    B.gemm(packed, n, k, I.TENSOR_SCALE, xs[:, :k], y=ys[:, :n], y_dtype=torch.float32)
    y1 = B.gemm(packed, n, k, I.TENSOR_SCALE, xs[:1, :k], y_dtype=torch.float32)
    g0 = B.gemv(packed, n, k, I.TENSOR_SCALE, to_dev_bf16(xb[0], dev))
    g1 = B.gemv(packed, n, k, I.TENSOR_SCALE, to_dev_bf16(xb[1], dev))
    torch.cuda.synchronize()
    assert torch.equal(ys[0, :n], g0) and torch.equal(ys[1, :n], g1)
    assert torch.equal(y1[0], g0)
    assert not ys[:, n:].any()          # nothing written past n
    y_ref, s = oracle.gemm(codes, scales, I.TENSOR_SCALE, xb, nthreads=oracle_threads())
    assert_within(ys[:, :n].cpu().numpy().astype(np.float64), y_ref, s, what="two rows")
