"""moe_route_noalloc through the C ABI: the router with its scratch in the
library's fixed per-GPU array gives the same indices, weights and logits,
bit for bit, as moe_route with a caller workspace, on two calls in a row
with the second on a smaller batch (the array keeps the first call's
contents), for the bf16 layers (mid, the decode sweep with its logit bias,
the V3/V4-scale share whose partial logits fill the array exactly) and the
fp32 tiny layer; a problem past the array's size is rejected before any
launch."""
import ctypes

import numpy as np
import pytest
import torch

from combine_wave_level_amd import moe
from helpers import Layer
from workloads import make_inputs

pytestmark = pytest.mark.gpu


def _both(L, T):
    p = L.p.replace(T=T)
    x = L.x[:T]
    ref = moe.route(p, x, L.packed, L.ws, bias=L.bias, want_logits=True)
    got = moe.route_noalloc(p, x, L.packed, bias=L.bias, want_logits=True)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    return ref


@pytest.mark.parametrize("name,T1,T2", [("mid", 4096, 300), ("decode", 128, 8), ("v4share", 8192, 1000),
                                        ("tiny", 64, 17)])
def test_noalloc_route_equals_route_on_two_calls(name, T1, T2):
    inp = make_inputs(name, T=T1)
    L = Layer(inp)
    print(f"[case] noalloc route {name} T={T1} then T={T2}", flush=True)
    _both(L, T1)
    idx, _, _ = _both(L, T2)
    assert idx.shape == (T2, L.p.k)


def test_noalloc_route_rejects_past_the_array():
    inp = make_inputs("v4share", T=8193, weights=False)
    p = moe.problem(T=8193, d=7168, I=2048, E_global=256, k=8, E_local=32)
    # 2 partial logit ranges x 8193 tokens x 256 experts x 4 B > 16 MiB
    assert 2 * 8193 * 256 * 4 > moe.ROUTE_NOALLOC_MAX_BYTES
    f = ctypes.c_void_p(0x10000)
    st = moe.lib().moe_route_noalloc(ctypes.byref(p), f, f, None, f, f, None, None)
    assert st == moe.MOE_ERR_UNSUPPORTED
    assert inp["x"].shape[0] == 8193
