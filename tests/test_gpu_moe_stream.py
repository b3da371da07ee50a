"""GPU: routed experts streamed from pinned host memory against the
oracle (every stage and the whole layer, as for the resident layer), against
the same layer with the experts device-resident (bit-identical outputs), and
the cache's bookkeeping (hits, least-recently-used eviction, the slot limit)."""
import numpy as np
import pytest
import torch

from bit_quantized_decode_amd import binding as B
from bit_quantized_decode_amd import inputs as I
from helpers import device, to_dev_bf16, to_dev_u8
from moe_checks import check_moe

pytestmark = pytest.mark.gpu


def pools(w, dev):
    out = []
    for codes, scales in ((w.gate_codes, w.gate_scales), (w.up_codes, w.up_scales), (w.down_codes, w.down_scales)):
        e, n, kh = codes.shape
        stride = B.packed_bytes(n, 2 * kh)
        pool = torch.empty(e * stride, dtype=torch.uint8, device=dev)
        for i in range(e):
            pool[i * stride:(i + 1) * stride].copy_(B.pack(to_dev_u8(codes[i], dev), to_dev_u8(scales[i], dev)))
        out.append((pool, stride))
    return out


@pytest.fixture(scope="module")
def setup():
    dev = device()
    shape = I.MoeShape(tokens=8, experts=48, top_k=3, hidden=256, inter=128)
    w = I.moe_weights(77, shape)
    (pg, sg), (pu, su), (pd, sd) = pools(w, dev)
    st = [torch.from_numpy(v).to(dev) for v in (w.gate_st, w.up_st, w.down_st)]
    return dev, shape, (pg, pu, pd, sg, su, sd), st, w


def call(dev, shape, x, logits, wts, st, stream_obj=None, debug=False):
    pg, pu, pd, sg, su, sd = wts
    args = (to_dev_bf16(x, dev), torch.from_numpy(logits).to(dev), shape.top_k)
    if stream_obj is None:
        o = B.moe_grouped(*args, pg, pu, pd, sg, su, sd, *st, shape.inter, debug=debug)
    else:
        o = B.moe_grouped(*args, stream_obj, None, None, None, None, None, *st, shape.inter, debug=debug)
    torch.cuda.synchronize()
    return {k: v.clone() for k, v in o.items()}


def test_streamed_equals_resident_over_calls(setup):
    dev, shape, wts, st, w = setup
    pg, pu, pd, sg, su, sd = wts
    es = B.ExpertStream(pg, pu, pd, sg, su, sd, shape.experts, 16, dev)
    seen = set()
    for r in range(6):
        x = I.activations(78, r, shape.tokens, shape.hidden)
        logits = I.router_logits(79 + r, shape.tokens, shape.experts)
        ref = call(dev, shape, x, logits, wts, st)
        got = call(dev, shape, x, logits, wts, st, es, debug=True)
        # The streamed layer against the oracle: routing, grouping, every stage, end to end.
        check_moe(w, x, logits, shape.top_k, o=got)
        for key in ("y", "topk_ids", "topk_weights", "expert_counts", "expert_offsets", "perm"):
            assert torch.equal(got[key].view(torch.int32) if got[key].dtype == torch.float32 else got[key],
                               ref[key].view(torch.int32) if ref[key].dtype == torch.float32 else ref[key]), (r, key)
        active = set(np.nonzero(ref["expert_counts"].cpu().numpy())[0].tolist())
        s = es.stats()
        assert s["active"] == len(active)
        # Every routed expert not already cached is fetched; with 16 slots and <= 16 routed experts per call.
        assert s["fetched"] <= len(active)
        if r == 0:
            assert s["fetched"] == len(active)
        seen |= active
        # The same call again: everything it routes to is cached now.
        again = call(dev, shape, x, logits, wts, st, es)
        assert torch.equal(again["y"].view(torch.int32), ref["y"].view(torch.int32))
        assert es.stats()["fetched"] == 0 and es.stats()["bytes"] == 0


def test_lru_eviction_and_slot_limit(setup):
    dev, shape, wts, st, w = setup
    pg, pu, pd, sg, su, sd = wts
    # Logits that route every token to experts {0, 1, 2}, then to {3, 4, 5}, then {0, 1, 2} again.
    def routed_to(ids):
        lg = np.full((shape.tokens, shape.experts), -5.0, np.float32)
        lg[:, ids] = [3.0, 2.0, 1.0]
        return lg
    x = I.activations(80, 0, shape.tokens, shape.hidden)
    es = B.ExpertStream(pg, pu, pd, sg, su, sd, shape.experts, 4, dev)
    call(dev, shape, x, routed_to([0, 1, 2]), wts, st, es)
    assert es.stats() == {"active": 3, "fetched": 3, "bytes": 3 * (2 * B.packed_bytes(128, 256) + B.packed_bytes(256, 128))}
    call(dev, shape, x, routed_to([3, 4, 5]), wts, st, es)   # one free slot, then the two least recently used
    assert es.stats()["fetched"] == 3
    assert sorted(es.expert_in.tolist()) == [2, 3, 4, 5] or sorted(es.expert_in.tolist()) == [0, 3, 4, 5] \
        or sorted(es.expert_in.tolist()) == [1, 3, 4, 5]
    ref = call(dev, shape, x, routed_to([0, 1, 2]), wts, st)
    got = call(dev, shape, x, routed_to([0, 1, 2]), wts, st, es, debug=True)
    assert es.stats()["fetched"] == 2                          # one of them survived
    check_moe(w, x, routed_to([0, 1, 2]), shape.top_k, o=got)  # refilled slots against the oracle
    assert torch.equal(got["y"].view(torch.int32), ref["y"].view(torch.int32))
    # More routed experts than slots: refused after routing.
    lg = I.router_logits(81, shape.tokens, shape.experts)
    with pytest.raises(B.Nvfp4Error, match="NVFP4_ERR_ARG"):
        call(dev, shape, x, lg, wts, st, B.ExpertStream(pg, pu, pd, sg, su, sd, shape.experts, 2, dev))
