"""Seeded synthetic inputs shared by the GPU path's tests and benchmark and by the oracle's tests.

This module only draws random numbers and rounds them into storage formats
with library casts (torch's float32 -> bfloat16 and float -> float8_e4m3fn,
both round-to-nearest-even).  It holds none of the product's arithmetic.

Every tensor has its own generator: numpy PCG64 seeded by
SeedSequence([workload_id, matrix_id, stream_id]), stream 0 = codes,
1 = scales, 2 = activations, 3 = router logits, 4 = expert-popularity permutation.

Distributions (the synthetic stand-in for the pages' 27B decode at one and at
32 users, the 10-of-512-experts MoE layer and the 512-token prompt):
  codes        each 4-bit code independently uniform over all 16 codes
               (each byte uniform over 0..255);
  block scales 2^u, u ~ U[-6, 2] drawn in fp64, rounded to E4M3FN (RNE);
  tensor scale float32(1/448);
  activations  N(0, 1) drawn in fp32, rounded to bf16 (RNE);
  router       N(0, 1) fp32 logits plus a per-expert bias -1.1 * ln(r_e),
               r a seeded random permutation of 1..E, so that expert
               popularity follows a Zipf(1.1) law with hot experts scattered
               over the expert ids.
"""
from dataclasses import dataclass, field

import numpy as np
import torch

TENSOR_SCALE = np.float32(1.0 / 448.0)

# Workload ids (the first seed word).
GEMV_1K = 0        # one 1024 x 1024 GEMV, batch 1
DECODE_B1 = 1      # 27B-class dense decode layer, batch 1
DECODE_B32 = 2     # the same layer at batch 32
MOE_32T = 3        # 512-expert MoE layer, 32 tokens, top-10
PREFILL_512 = 4    # 512-token prefill, gate/up/down
DECODE_WIDTHS = 5  # the dense layer at decode widths 2..8
OUTPUT_HEAD = 6    # the output head at a 248k-token vocabulary, batch 1


@dataclass(frozen=True)
class Matrix:
    name: str
    n: int          # output rows
    k: int          # input length (multiple of 16)
    matrix_id: int


# The five matrices of a 27B-class layer (hidden 5120, MLP 17408, QKV 7168).
DENSE_LAYER = (
    Matrix("gate", 17408, 5120, 0),
    Matrix("up", 17408, 5120, 1),
    Matrix("down", 5120, 17408, 2),
    Matrix("qkv", 7168, 5120, 3),
    Matrix("o", 5120, 5120, 4),
)
PREFILL_MATRICES = DENSE_LAYER[:3]
# The output head: a ~248k vocabulary (Ignis README, "Speculative decoding")
# over the layer's hidden size; 248000 rows leave a ragged last row tile.
HEAD = Matrix("head", 248000, 5120, 0)


@dataclass(frozen=True)
class MoeShape:
    tokens: int = 32
    experts: int = 512
    top_k: int = 10
    hidden: int = 2048
    inter: int = 512
    zipf_s: float = 1.1


def generator(workload_id, matrix_id, stream_id):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([workload_id, matrix_id, stream_id])))


def nvfp4_codes(workload_id, matrix_id, n, k):
    """uint8 [n][k/2]: two independent uniform 4-bit codes per byte."""
    assert k % 2 == 0
    return generator(workload_id, matrix_id, 0).integers(0, 256, size=(n, k // 2), dtype=np.uint8)


def e4m3_round(values):
    """Round float values to E4M3FN bytes with torch's cast (round-to-nearest-even)."""
    t = torch.from_numpy(np.ascontiguousarray(values, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def nvfp4_scales(workload_id, matrix_id, n, k):
    """uint8 E4M3FN [n][k/16]: 2^u, u ~ U[-6, 2]."""
    assert k % 16 == 0
    u = generator(workload_id, matrix_id, 1).uniform(-6.0, 2.0, size=(n, k // 16))
    return e4m3_round(np.exp2(u))


def bf16_round(values):
    """Round fp32 values to bf16, returned as uint16 bit patterns (torch cast, RNE)."""
    t = torch.from_numpy(np.ascontiguousarray(values, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def activations(workload_id, matrix_id, m, k):
    """bf16 bits [m][k], N(0, 1)."""
    z = generator(workload_id, matrix_id, 2).standard_normal(size=(m, k), dtype=np.float32)
    return bf16_round(z)


def nvfp4_matrix(workload_id, matrix_id, n, k):
    return nvfp4_codes(workload_id, matrix_id, n, k), nvfp4_scales(workload_id, matrix_id, n, k)


def router_logits(workload_id, tokens, experts, zipf_s=1.1, batch=0):
    """fp32 [tokens][experts] = N(0,1) + (-zipf_s * ln r_e).  `batch` draws other
    tokens' noise over the same expert popularity r."""
    z = generator(workload_id, batch, 3).standard_normal(size=(tokens, experts), dtype=np.float32)
    r = generator(workload_id, 0, 4).permutation(experts) + 1
    bias = (-zipf_s * np.log(r.astype(np.float64))).astype(np.float32)
    return (z + bias[None, :]).astype(np.float32)


@dataclass
class MoeWeights:
    """Canonical codes/scales of every expert: gate/up [E][I][H/2], down [E][H][I/2]."""
    gate_codes: np.ndarray
    gate_scales: np.ndarray
    up_codes: np.ndarray
    up_scales: np.ndarray
    down_codes: np.ndarray
    down_scales: np.ndarray
    gate_st: np.ndarray = field(default=None)
    up_st: np.ndarray = field(default=None)
    down_st: np.ndarray = field(default=None)


def moe_weights(workload_id, shape: MoeShape, experts=None):
    """Expert e's gate / up / down use matrix ids 3e, 3e+1, 3e+2."""
    e_count = shape.experts if experts is None else experts
    h, i = shape.hidden, shape.inter
    gc = np.empty((e_count, i, h // 2), np.uint8)
    gs = np.empty((e_count, i, h // 16), np.uint8)
    uc = np.empty_like(gc)
    us = np.empty_like(gs)
    dc = np.empty((e_count, h, i // 2), np.uint8)
    ds = np.empty((e_count, h, i // 16), np.uint8)
    for e in range(e_count):
        gc[e], gs[e] = nvfp4_matrix(workload_id, 3 * e, i, h)
        uc[e], us[e] = nvfp4_matrix(workload_id, 3 * e + 1, i, h)
        dc[e], ds[e] = nvfp4_matrix(workload_id, 3 * e + 2, h, i)
    st = np.full(e_count, TENSOR_SCALE, np.float32)
    return MoeWeights(gc, gs, uc, us, dc, ds, st.copy(), st.copy(), st.copy())
