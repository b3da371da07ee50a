"""Shared test helpers: device transfer, bf16 views and the parity bounds."""
import os

import numpy as np
import pytest
import torch

from bit_quantized_decode_amd import inputs as I

TOL = 1e-5  # |y - y_ref| <= TOL * sum_k |w_k x_k| per output


def device():
    if not torch.cuda.is_available():
        pytest.fail("a GPU test ran without a visible GPU (these tests fail rather than skip)")
    from bit_quantized_decode_amd import binding as B
    B.lib()  # raises if the HIP library is not built
    return torch.device("cuda:0")


def to_dev_u8(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def to_dev_bf16(bits, dev):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev)
    return t.view(torch.bfloat16)


def bf16_to_f64(t):
    """torch bf16 tensor (any device) -> numpy float64."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def bf16_bits(t):
    return t.detach().to("cpu").view(torch.int16).numpy().view(np.uint16)


def ulp_bf16(v):
    """Spacing of bf16 at |v| (smallest subnormal spacing at 0)."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    _, e = np.frexp(v)
    u = np.ldexp(1.0, e - 8)
    return np.where(v > 0, np.maximum(u, 2.0 ** -133), 2.0 ** -133)


def assert_within(y, y_ref, s, extra=0.0, what=""):
    """Per-output bound |y - y_ref| <= TOL * s + extra; reports the worst ratio."""
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - y_ref)
    bound = TOL * s + extra
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        ratio = np.max(np.where(s > 0, err / np.maximum(s, 1e-300), np.inf))
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outputs outside the bound; "
                             f"worst err/S = {ratio:.3e}; first at {idx.tolist()}: "
                             f"y={y[tuple(idx[0])]!r} ref={y_ref[tuple(idx[0])]!r} S={s[tuple(idx[0])]!r}")
    return float(np.max(err / np.maximum(s, 1e-300))) if s.size else 0.0


def oracle_threads():
    try:
        return min(len(os.sched_getaffinity(0)), 16)
    except AttributeError:
        return 8


def pack_to_device(codes, scales, dev):
    from bit_quantized_decode_amd import binding as B
    return B.pack(to_dev_u8(codes, dev), to_dev_u8(scales, dev))


def sample_rows(n, count, seed):
    """First, last and random rows (sorted, unique)."""
    rng = np.random.default_rng(seed)
    rows = set(range(min(n, 8))) | set(range(max(0, n - 8), n))
    rows |= set(rng.choice(n, size=min(n, count), replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def random_matrix(rng, n, k):
    codes = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    scales = I.e4m3_round(np.exp2(rng.uniform(-6, 2, size=(n, k // 16))))
    return codes, scales


# Largest |silu'(z)| over all z (about 1.0998, near z = 2.4).
SILU_SLOPE = 1.1
# Relative error of the fp32 silu(G) * U the expert kernel evaluates before
# rounding h to bf16: expf within 1 ulp, then an add, a correctly rounded
# division and a multiply (about 5 * 2^-24), taken with margin.
SILU_FP32_REL = 2.0 ** -20
# Relative tolerance of the GPU's fp32 routing weights against the fp64 ones.
G_REL = 1e-6


def moe_end_to_end_extra(w, x, ids_ref, g_ref, ybound, nthreads=None):
    """What the fp64 chain's y may differ from a correct GPU layer's y by,
    beyond TOL * ybound, per output [t][hidden].

    The GPU layer rounds h to bf16 after an fp32 silu of fp32 gate and up sums,
    so its h differs from the fp64 chain's h by at most, per element,
      dh = P + ulp_bf16(|h| + P) / 2,
      P  = 1.1 * eG * (|U| + eU) + |silu(G)| * eU + 2^-20 * |h|,
    where eG = TOL * S_G and eU = TOL * S_U are the gate and up stages' own
    bounds, 1.1 bounds |silu'| and 2^-20 the fp32 evaluation.  That moves each
    down output by at most |Wd| dh (plus TOL of it, inside the down stage's
    bound), and the routing weights' tolerance G_REL moves y by G_REL of the
    bound's magnitude sum.  So:
      extra[t] = G_REL * (1 + TOL) * ybound[t] + (1 + TOL) * (1 + G_REL) * sum_j g_j |Wd_j| dh_j.
    """
    import oracle
    t, hidden = x.shape
    top_k = ids_ref.shape[1]
    extra = G_REL * (1 + TOL) * np.asarray(ybound, np.float64).copy()
    wd_abs = {}
    for ti in range(t):
        xs = np.ascontiguousarray(x[ti:ti + 1])
        for j in range(top_k):
            ex = int(ids_ref[ti, j])
            gy, gs = oracle.gemm(w.gate_codes[ex], w.gate_scales[ex], w.gate_st[ex], xs, nthreads=nthreads)
            uy, us = oracle.gemm(w.up_codes[ex], w.up_scales[ex], w.up_st[ex], xs, nthreads=nthreads)
            G, U = gy[0], uy[0]
            eG, eU = TOL * gs[0], TOL * us[0]
            sG = oracle.silu(G)
            h = sG * U
            p = SILU_SLOPE * eG * (np.abs(U) + eU) + np.abs(sG) * eU + SILU_FP32_REL * np.abs(h)
            dh = p + 0.5 * ulp_bf16(np.abs(h) + p)
            if ex not in wd_abs:
                wd_abs[ex] = np.abs(oracle.dequant(w.down_codes[ex], w.down_scales[ex], w.down_st[ex]))
            extra[ti] += (1 + TOL) * (1 + G_REL) * g_ref[ti, j] * (wd_abs[ex] @ dh)
    return extra
