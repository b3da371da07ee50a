"""GPU parity: the routed expert layer (a4-a8) against the CPU oracle.

Integer outputs (ids, counts, offsets, perm) must be bit-exact.  Each GEMM
stage is checked against the oracle fed that stage's GPU input; the whole
layer is also checked end to end against the pure-oracle chain.
"""
import numpy as np
import pytest
import torch

import oracle
from bit_quantized_decode_amd import binding as B
from bit_quantized_decode_amd import inputs as I
from helpers import (TOL, assert_within, bf16_bits, bf16_to_f64, device, oracle_threads, to_dev_bf16, to_dev_u8,
                     ulp_bf16)

pytestmark = pytest.mark.gpu


def pack_pool(codes, scales, dev):
    """Pack every expert of [E][rows][...] into one pool; returns (pool, stride)."""
    e, n, kh = codes.shape
    stride = B.packed_bytes(n, 2 * kh)
    pool = torch.empty(e * stride, dtype=torch.uint8, device=dev)
    for i in range(e):
        p = B.pack(to_dev_u8(codes[i], dev), to_dev_u8(scales[i], dev))
        pool[i * stride:(i + 1) * stride].copy_(p)
    return pool, stride


def run_moe(w, x, logits, top_k, dev, y_dtype=torch.float32, debug=True):
    e = w.gate_codes.shape[0]
    inter = w.gate_codes.shape[1]
    pg, sg = pack_pool(w.gate_codes, w.gate_scales, dev)
    pu, su = pack_pool(w.up_codes, w.up_scales, dev)
    pd, sd = pack_pool(w.down_codes, w.down_scales, dev)
    o = B.moe_grouped(to_dev_bf16(x, dev), torch.from_numpy(logits).to(dev), top_k, pg, pu, pd, sg, su, sd,
                      torch.from_numpy(w.gate_st).to(dev), torch.from_numpy(w.up_st).to(dev),
                      torch.from_numpy(w.down_st).to(dev), inter, y_dtype=y_dtype, debug=debug)
    torch.cuda.synchronize()
    assert o["expert_counts"].numel() == e
    return o


def check_moe(w, x, logits, top_k, y_dtype=torch.float32, end_to_end=True):
    dev = device()
    t, hidden = x.shape
    e = logits.shape[1]
    inter = w.gate_codes.shape[1]
    o = run_moe(w, x, logits, top_k, dev, y_dtype=y_dtype)
    nt = oracle_threads()

    # a4 / a5: routing and grouping, bit-exact.
    ids_ref, g_ref = oracle.route(logits, top_k)
    counts_ref, offsets_ref, perm_ref, pos_ref = oracle.group(ids_ref, e)
    ids = o["topk_ids"].cpu().numpy()
    assert np.array_equal(ids, ids_ref)
    assert np.array_equal(o["expert_counts"].cpu().numpy(), counts_ref)
    assert np.array_equal(o["expert_offsets"].cpu().numpy(), offsets_ref)
    assert np.array_equal(o["perm"].cpu().numpy(), perm_ref)
    g = o["topk_weights"].cpu().numpy().astype(np.float64)
    assert np.allclose(g, g_ref, rtol=1e-6, atol=0)

    # a6: gate / up per expert, fed the same activation rows.
    gate = o["dbg_gate"].cpu().numpy().astype(np.float64)
    up = o["dbg_up"].cpu().numpy().astype(np.float64)
    h = o["dbg_h"]
    h_f64 = bf16_to_f64(h)
    h_bits = bf16_bits(h)
    down = o["dbg_down"].cpu().numpy().astype(np.float64)
    y = (o["y"].cpu().numpy() if y_dtype == torch.float32 else bf16_to_f64(o["y"])).astype(np.float64)
    d_ref_gpu_h = np.zeros((t * top_k, hidden))
    s_down = np.zeros((t * top_k, hidden))
    for ex in np.nonzero(counts_ref)[0]:
        p0, p1 = offsets_ref[ex], offsets_ref[ex + 1]
        toks = perm_ref[p0:p1] // top_k
        xs = np.ascontiguousarray(x[toks])
        gy, gs = oracle.gemm(w.gate_codes[ex], w.gate_scales[ex], w.gate_st[ex], xs, nthreads=nt)
        uy, us = oracle.gemm(w.up_codes[ex], w.up_scales[ex], w.up_st[ex], xs, nthreads=nt)
        assert_within(gate[p0:p1], gy, gs, what=f"gate expert {ex}")
        assert_within(up[p0:p1], uy, us, what=f"up expert {ex}")
        # a7: down, fed the GPU's own h.
        dy, ds = oracle.gemm(w.down_codes[ex], w.down_scales[ex], w.down_st[ex],
                             np.ascontiguousarray(h_bits[p0:p1]), nthreads=nt)
        assert_within(down[p0:p1], dy, ds, what=f"down expert {ex}")
        d_ref_gpu_h[p0:p1] = dy
        s_down[p0:p1] = ds
    # h = bf16(silu(G) * U) from the GPU's own G and U, within one bf16 ulp.
    hz = oracle.silu(gate) * up
    assert np.all(np.abs(h_f64 - hz) <= ulp_bf16(hz) + 1e-300)

    # a8: scatter with the GPU's g over the oracle's d (of the GPU's h).
    pos = pos_ref.reshape(t, top_k)
    y_ref_stage = np.einsum("tj,tjo->to", g, d_ref_gpu_h[pos])
    bound_stage = np.einsum("tj,tjo->to", g, s_down[pos])
    extra = ulp_bf16(y_ref_stage) if y_dtype == torch.bfloat16 else 0.0
    assert_within(y, y_ref_stage, bound_stage, extra=extra, what="scatter")

    if end_to_end:
        ids2, g2, y_ref, yb = oracle.moe((w.gate_codes, w.gate_scales, w.gate_st), (w.up_codes, w.up_scales, w.up_st),
                                         (w.down_codes, w.down_scales, w.down_st), x, logits, top_k, nthreads=nt)
        assert np.array_equal(ids2, ids_ref)
        # One bf16 ulp per element of h is allowed on top of the accumulation bound.
        h_ref_ulp = np.zeros((t * top_k, inter))
        for ti in range(t):
            for j in range(top_k):
                ex = ids_ref[ti, j]
                xs = x[ti:ti + 1]
                gy, _ = oracle.gemm(w.gate_codes[ex], w.gate_scales[ex], w.gate_st[ex], xs)
                uy, _ = oracle.gemm(w.up_codes[ex], w.up_scales[ex], w.up_st[ex], xs)
                h_ref_ulp[ti * top_k + j] = 2.0 * ulp_bf16(oracle.silu(gy[0]) * uy[0])
        extra_e2e = np.zeros((t, hidden))
        for ti in range(t):
            for j in range(top_k):
                ex = ids_ref[ti, j]
                wd = np.abs(oracle.dequant(w.down_codes[ex], w.down_scales[ex], w.down_st[ex]))
                extra_e2e[ti] += g_ref[ti, j] * (wd @ h_ref_ulp[ti * top_k + j])
        if y_dtype == torch.bfloat16:
            extra_e2e += ulp_bf16(y_ref)
        assert_within(y, y_ref, yb, extra=extra_e2e, what="end to end")
    return o


def small_weights(seed, e, hidden, inter):
    return I.moe_weights(seed, I.MoeShape(tokens=1, experts=e, top_k=1, hidden=hidden, inter=inter))


@pytest.mark.parametrize("t,e,k,hidden,inter", [
    (5, 8, 2, 256, 64),
    (7, 6, 3, 272, 48),      # ragged against the 256-k and 64-row tiles
    (40, 12, 4, 512, 96),    # an expert can receive more than 32 rows
    (3, 64, 1, 128, 32),
    (130, 16, 8, 128, 32),   # tokens * top_k > 1024: separate routing and grouping launches
    (4, 1100, 2, 128, 32),   # more than 1024 experts: separate launches, 32 logits per lane
    (1536, 6, 4, 1024, 384),  # more work-list items than the persistent expert-GEMM grids hold
    (3, 2048, 64, 128, 32),   # the largest expert count and top-k the layer takes
])
def test_moe_small(t, e, k, hidden, inter):
    w = small_weights(50 + e, e, hidden, inter)
    x = I.activations(50 + e, 0, t, hidden)
    logits = I.router_logits(50 + e, t, e)
    check_moe(w, x, logits, k)


def test_moe_bf16_output():
    w = small_weights(61, 8, 256, 64)
    x = I.activations(61, 0, 6, 256)
    logits = I.router_logits(61, 6, 8)
    check_moe(w, x, logits, 3, y_dtype=torch.bfloat16)


def test_moe_tied_logits_rank_by_id():
    w = small_weights(62, 16, 128, 32)
    x = I.activations(62, 0, 4, 128)
    logits = np.zeros((4, 16), np.float32)
    logits[:, 5] = 1.0
    o = check_moe(w, x, logits, 4)
    assert np.array_equal(o["topk_ids"].cpu().numpy(), np.tile([5, 0, 1, 2], (4, 1)))


@pytest.fixture(scope="module")
def moe_full():
    shape = I.MoeShape()
    w = I.moe_weights(I.MOE_32T, shape)
    x = I.activations(I.MOE_32T, 0, shape.tokens, shape.hidden)
    logits = I.router_logits(I.MOE_32T, shape.tokens, shape.experts, shape.zipf_s)
    return shape, w, x, logits


def test_moe_full_size(moe_full):
    """32 tokens, 512 experts, top-10, hidden 2048, expert width 512."""
    shape, w, x, logits = moe_full
    o = check_moe(w, x, logits, shape.top_k, end_to_end=True)
    active = int((o["expert_counts"].cpu().numpy() > 0).sum())
    print(f"active experts: {active}")
    assert 20 <= active <= 320


def test_moe_full_size_repeat_is_bit_identical(moe_full):
    shape, w, x, logits = moe_full
    dev = device()
    o1 = run_moe(w, x, logits, shape.top_k, dev, debug=False)
    y1 = o1["y"].clone()
    o2 = run_moe(w, x, logits, shape.top_k, dev, debug=False)
    assert torch.equal(y1.view(torch.int32), o2["y"].view(torch.int32))
