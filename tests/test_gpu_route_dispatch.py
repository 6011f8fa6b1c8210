"""moe_route_dispatch (route then dispatch in one call; small batches
select and dispatch in one workgroup) gives exactly the outputs of
moe_route followed by moe_dispatch: indices, weights, logits, counts,
offsets, the permutation, pair positions and ready waves, bit for bit, on
both sides of the one-workgroup bound (T = 16 / 17) and of the dispatch's
one-workgroup path, for the fp32 router, the bf16 router with a bias, a
local window of 32 of 256 router experts, and the layer's forward through
it."""
import pytest
import torch

from combine_wave_level_amd import moe
from helpers import Layer
from workloads import make_inputs

pytestmark = pytest.mark.gpu


def _both(L):
    idx, w, lg = moe.route(L.p, L.x, L.packed, L.ws, bias=L.bias, want_logits=True)
    d = moe.dispatch(L.p, idx, L.ws)
    ref = (idx.clone(), w.clone(), lg.clone(), d.counts.clone(), d.offsets.clone(), d.sorted_token.clone(),
           d.pair_pos.clone(), d.ready_wave.clone())
    torch.cuda.synchronize()
    idx2, w2, lg2, d2 = moe.route_dispatch(L.p, L.x, L.packed, L.ws, bias=L.bias, want_logits=True)
    torch.cuda.synchronize()
    moe.check_error(L.ws)
    got = (idx2, w2, lg2, d2.counts, d2.offsets, d2.sorted_token, d2.pair_pos, d2.ready_wave)
    return ref, got, d2


@pytest.mark.parametrize("name,T", [("tiny", 64), ("tiny", 16), ("decode", 1), ("decode", 8), ("decode", 16),
                                    ("decode", 17), ("decode", 128), ("mid", 12), ("v4share", 9),
                                    ("v4share", 33), ("mid", 4096)])
def test_route_dispatch_equals_route_then_dispatch(name, T):
    L = Layer(make_inputs(name, T=T))
    print(f"[case] route_dispatch {name} T={T}", flush=True)
    ref, got, _ = _both(L)
    P = int(ref[4][-1])
    names = ("topk_idx", "topk_w", "logits", "counts", "offsets", "sorted_token", "pair_pos", "ready_wave")
    for nm, a, b in zip(names, ref, got):
        if nm == "sorted_token":
            a, b = a[:P], b[:P]
        assert torch.equal(a, b), nm


def test_forward_through_route_dispatch():
    """The FFN on route_dispatch's outputs gives the layer's bits (decode T = 8)."""
    L = Layer(make_inputs("decode", T=8))
    r = moe.forward(L.p, L.x, L.packed, L.ws, bias=L.bias)
    torch.cuda.synchronize()
    idx, w, _, d = moe.route_dispatch(L.p, L.x, L.packed, L.ws, bias=L.bias)
    y, out = moe.ffn_waved(L.p, L.x, L.packed, d, w, L.ws)
    torch.cuda.synchronize()
    moe.check_error(L.ws)
    assert torch.equal(out, r["out"])
