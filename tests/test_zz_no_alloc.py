"""GPU: nvfp4_gemv_batched_noalloc (the batched GEMV on the library's static
device scratch) against nvfp4_gemv_batched with a caller workspace: bit-identical
outputs on two calls in a row, the second smaller, and the same sums the oracle
bounds."""
import numpy as np
import pytest
import torch

import oracle
from bit_quantized_decode_amd import binding as B
from bit_quantized_decode_amd import inputs as I
from helpers import assert_within, device, oracle_threads, pack_to_device, random_matrix, sample_rows, to_dev_bf16

pytestmark = pytest.mark.gpu


def run_both(items_host, dev):
    """items_host: (codes, scales, n, k, x bits).  Returns (noalloc y's, workspace y's)."""
    packed = [pack_to_device(c, s, dev) for c, s, _, _, _ in items_host]
    xs = [to_dev_bf16(x, dev) for _, _, _, _, x in items_host]
    y_na = [torch.full((n,), 7.0, dtype=torch.float32, device=dev) for _, _, n, _, _ in items_host]
    y_ws = [torch.full((n,), 7.0, dtype=torch.float32, device=dev) for _, _, n, _, _ in items_host]
    B.gemv_batched_noalloc([(p, n, k, I.TENSOR_SCALE, x, y)
                            for p, (_, _, n, k, _), x, y in zip(packed, items_host, xs, y_na)])
    B.gemv_batched([(p, n, k, I.TENSOR_SCALE, x, y) for p, (_, _, n, k, _), x, y in zip(packed, items_host, xs, y_ws)])
    torch.cuda.synchronize()
    return y_na, y_ws


def test_noalloc_equals_workspace_call_twice_second_smaller():
    dev = device()
    print("noalloc call 1: the 27B-class layer's five GEMVs", flush=True)
    first = []
    for m in I.DENSE_LAYER:
        c, s = I.nvfp4_matrix(I.DECODE_B1, m.matrix_id, m.n, m.k)
        first.append((c, s, m.n, m.k, I.activations(I.DECODE_B1, m.matrix_id, 1, m.k)[0]))
    y_na, y_ws = run_both(first, dev)
    for (c, s, n, k, x), a, b in zip(first, y_na, y_ws):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), (n, k)
        rows = sample_rows(n, 64, n + k)
        y_ref, sabs = oracle.gemm(c, s, I.TENSOR_SCALE, x, rows=rows, nthreads=oracle_threads())
        assert_within(a.cpu().numpy()[rows][None, :], y_ref, sabs, what=f"noalloc {n}x{k}")

    print("noalloc call 2: three smaller ragged GEMVs", flush=True)
    rng = np.random.default_rng(5)
    second = []
    for n, k in ((1000, 4096), (130, 2320), (65, 272)):
        c, s = random_matrix(rng, n, k)
        second.append((c, s, n, k, I.bf16_round(rng.standard_normal(k).astype(np.float32))))
    y_na, y_ws = run_both(second, dev)
    for (c, s, n, k, x), a, b in zip(second, y_na, y_ws):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), (n, k)
        y_ref, sabs = oracle.gemm(c, s, I.TENSOR_SCALE, x)
        assert_within(a.cpu().numpy()[None, :], y_ref, sabs, what=f"noalloc {n}x{k}")
