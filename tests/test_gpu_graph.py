"""The layer step (route, dispatch, expert FFN with fused combine) captured
in a HIP graph and replayed: every replay gives the eager step's bits.

Decode loops launch the same small step over and over; a graph replays its
six kernels without the host in between.  Nothing in the step allocates
device memory or records a memset (the persistent kernel's counters are
cleared by kernels: moe_dispatch's fill and the kernel's own exit), so the
captured step needs no change.  Replays alternate with eager work and
synchronisations, and each one is checked against the eager result.
"""
import pytest
import torch

from combine_wave_level_amd import moe
from helpers import Layer
from workloads import make_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,T,forced", [("decode", 1, {}), ("decode", 32, {"persistent": True}),
                                           ("mid", 777, {"persistent": True}), ("mid", 777, {"serial": True})])
def test_graph_replays_equal_the_eager_step(name, T, forced):
    L = Layer(make_inputs(name, T=T))
    print(f"[case] graph {name} T={T} {forced}", flush=True)
    p = L.p
    y = torch.empty((max(1, moe.p_max(p)), p.d), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((p.T, p.d), dtype=torch.bfloat16, device="cuda")

    def step():
        idx, w, _ = moe.route(p, L.x, L.packed, L.ws, bias=L.bias)
        disp = moe.dispatch(p, idx, L.ws)
        moe.ffn_waved(p, L.x, L.packed, disp, w, L.ws, y=y, out=out, **forced)
        return idx, disp

    idx_e, disp_e = step()
    torch.cuda.synchronize()
    moe.check_error(L.ws)
    out_e, idx_e = out.clone(), idx_e.clone()
    P = int(disp_e.offsets[-1])
    y_e = y[:P].clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm the capture stream
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        idx_g, disp_g = step()
    torch.cuda.synchronize()
    for rep in range(4):
        out.view(torch.int16).fill_(0x7F7F)
        y.view(torch.int16).fill_(0x7F7F)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        moe.check_error(L.ws)
        assert torch.equal(idx_g, idx_e), rep
        assert torch.equal(out, out_e), rep
        assert torch.equal(y[:P], y_e), rep
        # eager work between replays
        step()
        torch.cuda.synchronize()
        assert torch.equal(out, out_e), rep
