"""Checks of the routed expert layer's outputs against the oracle, shared by
the resident (nvfp4_moe_grouped) and streamed (nvfp4_moe_streamed) tests.

Integer outputs (ids, counts, offsets, perm) must be bit-exact.  Each GEMM
stage is checked against the oracle fed that stage's GPU input; the whole
layer is also checked end to end against the pure-oracle chain.
"""
import numpy as np
import torch

import oracle
from bit_quantized_decode_amd import binding as B
from helpers import (assert_within, bf16_bits, bf16_to_f64, device, moe_end_to_end_extra, oracle_threads,
                     to_dev_bf16, to_dev_u8, ulp_bf16)


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


def check_moe(w, x, logits, top_k, y_dtype=torch.float32, end_to_end=True, o=None):
    """Run the layer (or take its outputs `o`, debug outputs included) and check
    every stage and the whole layer against the oracle."""
    dev = device()
    t, hidden = x.shape
    e = logits.shape[1]
    if o is None:
        o = run_moe(w, x, logits, top_k, dev, y_dtype=y_dtype)
    nt = oracle_threads()

    # Routing and grouping, bit-exact.
    ids_ref, g_ref = oracle.route(logits, top_k)
    counts_ref, offsets_ref, perm_ref, pos_ref = oracle.group(ids_ref, e)
    ids = o["topk_ids"].cpu().numpy()
    assert np.array_equal(ids, ids_ref)
    assert np.array_equal(o["expert_counts"].cpu().numpy(), counts_ref)
    assert np.array_equal(o["expert_offsets"].cpu().numpy(), offsets_ref)
    assert np.array_equal(o["perm"].cpu().numpy(), perm_ref)
    g = o["topk_weights"].cpu().numpy().astype(np.float64)
    assert np.allclose(g, g_ref, rtol=1e-6, atol=0)

    # Gate / up per expert, fed the same activation rows.
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
        # Down, fed the GPU's own h.
        dy, ds = oracle.gemm(w.down_codes[ex], w.down_scales[ex], w.down_st[ex],
                             np.ascontiguousarray(h_bits[p0:p1]), nthreads=nt)
        assert_within(down[p0:p1], dy, ds, what=f"down expert {ex}")
        d_ref_gpu_h[p0:p1] = dy
        s_down[p0:p1] = ds
    # h = bf16(silu(G) * U) from the GPU's own G and U, within one bf16 ulp.
    hz = oracle.silu(gate) * up
    assert np.all(np.abs(h_f64 - hz) <= ulp_bf16(hz) + 1e-300)

    # Scatter with the GPU's g over the oracle's d (of the GPU's h).
    pos = pos_ref.reshape(t, top_k)
    y_ref_stage = np.einsum("tj,tjo->to", g, d_ref_gpu_h[pos])
    bound_stage = np.einsum("tj,tjo->to", g, s_down[pos])
    extra = ulp_bf16(y_ref_stage) if y_dtype == torch.bfloat16 else 0.0
    assert_within(y, y_ref_stage, bound_stage, extra=extra, what="scatter")

    if end_to_end:
        ids2, g2, y_ref, yb = oracle.moe((w.gate_codes, w.gate_scales, w.gate_st), (w.up_codes, w.up_scales, w.up_st),
                                         (w.down_codes, w.down_scales, w.down_st), x, logits, top_k, nthreads=nt)
        assert np.array_equal(ids2, ids_ref)
        # h rounds to bf16 after an fp32 silu of the stages' fp32 sums: the
        # allowance propagates that through the down product (moe_end_to_end_extra).
        extra_e2e = moe_end_to_end_extra(w, x, ids_ref, g_ref, yb, nthreads=nt)
        if y_dtype == torch.bfloat16:
            extra_e2e += ulp_bf16(y_ref)
        assert_within(y, y_ref, yb, extra=extra_e2e, what="end to end")
    return o
