"""GPU parity at the largest row count a product call takes: 4194304 rows, i.e.
65536 row tiles of 64, which is every counter of the workspace's split-K
counter area for the GEMV.  The weights are generated on the device (seeded),
the checked rows are copied back and computed by the oracle."""
import numpy as np
import pytest
import torch

import oracle
from bit_quantized_decode_amd import binding as B
from bit_quantized_decode_amd import inputs as I
from helpers import assert_within, device, oracle_threads, sample_rows, to_dev_bf16

pytestmark = pytest.mark.gpu

MAX_N = 4194304


def device_matrix(n, k, seed, dev):
    """Codes uniform over all bytes; scales 2^u, u ~ U[-6, 2], rounded to E4M3 (RNE)."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    codes = torch.randint(0, 256, (n, k // 2), dtype=torch.uint8, device=dev, generator=gen)
    u = torch.rand((n, k // 16), dtype=torch.float32, device=dev, generator=gen) * 8.0 - 6.0
    scales = torch.exp2(u).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scales


@pytest.fixture(scope="module")
def big():
    dev = device()
    k = 1280
    codes, scales = device_matrix(MAX_N, k, 71, dev)
    packed = B.pack(codes, scales)
    mx = B.mx_pack(codes, scales)
    rows = sample_rows(MAX_N, 256, 72)
    rows = np.union1d(rows, np.arange(MAX_N - 64, MAX_N))   # the whole last row tile
    idx = torch.from_numpy(rows).to(dev)
    c_rows = codes.index_select(0, idx).cpu().numpy()
    s_rows = scales.index_select(0, idx).cpu().numpy()
    del codes, scales
    torch.cuda.synchronize()
    return dev, k, packed, rows, c_rows, s_rows, mx


def test_gemv_max_rows(big):
    """Split K in two workgroups per row tile: all 65536 counters in use, left zero afterwards."""
    dev, k, packed, rows, c_rows, s_rows, _ = big
    x = I.activations(73, 0, 1, k)[0]
    ws = torch.zeros(B.gemv_workspace_bytes(MAX_N, k), dtype=torch.uint8, device=dev)
    y = B.gemv(packed, MAX_N, k, I.TENSOR_SCALE, to_dev_bf16(x, dev), ws=ws)
    torch.cuda.synchronize()
    y_ref, s = oracle.gemm(c_rows, s_rows, I.TENSOR_SCALE, x[None, :], nthreads=oracle_threads())
    assert_within(y.cpu().numpy().astype(np.float64)[rows], y_ref[0], s[0], what="gemv at the row limit")
    assert int(ws[:262144].count_nonzero()) == 0


@pytest.mark.parametrize("m", [32, 64])
def test_gemm_max_rows(big, m):
    """The skinny path (m = 32) and the prefill path (m = 64) at the row limit, fp32 output."""
    dev, k, packed, rows, c_rows, s_rows, _ = big
    x = I.activations(74, m, m, k)
    y = B.gemm(packed, MAX_N, k, I.TENSOR_SCALE, to_dev_bf16(x, dev), y_dtype=torch.float32)
    torch.cuda.synchronize()
    idx = torch.from_numpy(rows).to(dev)
    got = y.index_select(1, idx).cpu().numpy().astype(np.float64)
    y_ref, s = oracle.gemm(c_rows, s_rows, I.TENSOR_SCALE, x, nthreads=oracle_threads())
    assert_within(got, y_ref, s, what=f"gemm m={m} at the row limit")


def test_w4a4_max_rows(big):
    """The W4A4 product at the row limit with 300 activation rows: two row slabs
    of 256, so the launch's 32768 output tiles use every tile counter and XCD
    mask of the stream-K area; fp32 output, sampled weight rows against the
    oracle's MX product."""
    dev, k, packed, rows, c_rows, s_rows, mx = big
    m = 300
    x = I.activations(75, m, m, k)
    ws = torch.zeros(B.w4a4_workspace_bytes(m, k), dtype=torch.uint8, device=dev)
    y = B.w4a4_gemm(mx, MAX_N, k, I.TENSOR_SCALE, to_dev_bf16(x, dev), y_dtype=torch.float32, ws=ws)
    torch.cuda.synchronize()
    idx = torch.from_numpy(rows).to(dev)
    got = y.index_select(1, idx).cpu().numpy().astype(np.float64)
    del y
    wc, wsc = oracle.mx_from_nvfp4(c_rows, s_rows)
    xc, xs = oracle.mx_from_bf16(x)
    y_ref, s = oracle.mx_gemm(wc, wsc, I.TENSOR_SCALE, xc, xs, nthreads=oracle_threads())
    assert_within(got, y_ref, s, what="w4a4 m=300 at the row limit")
    assert int(ws[:262144].count_nonzero()) == 0


def test_activation_rows_beyond_one_launch(big):
    """513 activation rows at the row limit: three slabs of 256 rows would need
    49152 tile counters, so the prefill and the W4A4 product each run rows
    0..511 and then row 512 as a second launch (activation and output offsets
    of a later launch)."""
    dev, k, packed, rows, c_rows, s_rows, mx = big
    m = 513
    x = I.activations(76, m, m, k)
    xd = to_dev_bf16(x, dev)
    idx = torch.from_numpy(rows).to(dev)
    y = B.gemm(packed, MAX_N, k, I.TENSOR_SCALE, xd, y_dtype=torch.float32)
    torch.cuda.synchronize()
    got = y.index_select(1, idx).cpu().numpy().astype(np.float64)
    del y
    y_ref, s = oracle.gemm(c_rows, s_rows, I.TENSOR_SCALE, x, nthreads=oracle_threads())
    assert_within(got, y_ref, s, what="prefill m=513 at the row limit")
    y = B.w4a4_gemm(mx, MAX_N, k, I.TENSOR_SCALE, xd, y_dtype=torch.float32)
    torch.cuda.synchronize()
    got = y.index_select(1, idx).cpu().numpy().astype(np.float64)
    del y
    wc, wsc = oracle.mx_from_nvfp4(c_rows, s_rows)
    xc, xs = oracle.mx_from_bf16(x)
    y_ref, s = oracle.mx_gemm(wc, wsc, I.TENSOR_SCALE, xc, xs, nthreads=oracle_threads())
    assert_within(got, y_ref, s, what="w4a4 m=513 at the row limit")
