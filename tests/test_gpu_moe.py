"""GPU parity: the routed expert layer against the CPU oracle.

Integer outputs (ids, counts, offsets, perm) must be bit-exact.  Each GEMM
stage is checked against the oracle fed that stage's GPU input; the whole
layer is also checked end to end against the pure-oracle chain.
"""
import numpy as np
import pytest
import torch

from bit_quantized_decode_amd import inputs as I
from helpers import device
from moe_checks import check_moe, run_moe

pytestmark = pytest.mark.gpu


def small_weights(seed, e, hidden, inter):
    return I.moe_weights(seed, I.MoeShape(tokens=1, experts=e, top_k=1, hidden=hidden, inter=inter))


@pytest.mark.parametrize("t,e,k,hidden,inter", [
    (5, 8, 2, 256, 64),
    (7, 6, 3, 272, 48),      # ragged against the 256-k and 64-row tiles
    (40, 12, 4, 512, 96),    # an expert can receive more than 32 rows
    (3, 64, 1, 128, 32),
    (128, 16, 8, 128, 32),   # tokens * top_k == 1024: still grouped inside the gate/up workgroups
    (130, 16, 8, 128, 32),   # tokens * top_k > 1024: the grouping launch
    (4, 1024, 3, 128, 32),   # 1024 experts: grouped inside the gate/up workgroups, 16 logits per lane
    (4, 1100, 2, 128, 32),   # more than 1024 experts: the grouping launch, 32 logits per lane
    (1536, 6, 4, 1024, 384),  # more work-list items than the persistent expert-GEMM grids hold
    (9, 10, 3, 1296, 608),    # several k rounds in both expert GEMMs, slots left without a tile in the last
    (3, 2048, 64, 128, 32),   # the largest expert count and top-k the layer takes
    (1, 1, 1, 16, 16),        # one token, one expert, the smallest hidden and inter
    (2, 3, 3, 48, 16),        # top_k == experts: every token reaches every expert
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
