"""GPU parity and determinism of the weight gradient.

dW1, dW3, dW2 of L = <dout, out> against the float64 oracle (full on the
tiny layer; sampled intermediate columns on the stress layer, where the hot
expert's rows exceed one reduction chunk and the isolated-partial path is
taken), and bitwise equality over ten runs.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_wave_level_amd import moe
from helpers import Layer, dev, f64, oracle_inputs
from workloads import make_inputs

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _rel(g, r):
    s = np.abs(r).max()
    return 0.0 if s == 0 else float(np.abs(g - r).max() / s)


def _run(inp, dout):
    L = Layer(inp)
    o = oracle_inputs(inp)
    wl = inp["workload"]
    l64 = oracle.router_logits(o["x"], o["Wg"], o["bias"])
    idx_o, w_o, _ = oracle.route(l64, wl.k)
    meta = oracle.dispatch(idx_o, wl.e_begin, wl.E_local, wl.G)
    disp, y, out, w_d = L.ffn_from_routing(idx_o, w_o)
    g = moe.wgrad(L.p, L.x, L.packed, disp, w_d, dev(dout), L.ws)
    torch.cuda.synchronize()
    moe.check_error(L.ws)
    return L, o, meta, w_d.cpu().numpy().astype(np.float64), g, disp


def test_wgrad_tiny_full():
    inp = make_inputs("tiny", need_dout=True)
    L, o, meta, w32, (dW1, dW3, dW2), _ = _run(inp, inp["dout"])
    r1, r3, r2 = oracle.wgrad(o["x"], o["W1"], o["W3"], o["W2"], meta, w32, f64(inp["dout"]))
    for e in range(8):
        assert _rel(dW1[e].cpu().numpy(), r1[e]) <= TOL, e
        assert _rel(dW3[e].cpu().numpy(), r3[e]) <= TOL, e
        assert _rel(dW2[e].cpu().numpy(), r2[e]) <= TOL, e


def test_wgrad_stress_sampled_columns_and_split_rows():
    inp = make_inputs("stress", T=8192, need_dout=True)
    print("[case] wgrad stress T=8192", flush=True)
    L, o, meta, w32, (dW1, dW3, dW2), disp = _run(inp, inp["dout"])
    counts = meta["counts"]
    hot = int(np.argmax(counts))
    assert counts[hot] > 2048          # more than one reduction chunk
    rng = np.random.default_rng(3)
    cols = np.sort(rng.choice(1536, 6, replace=False))
    experts = [hot, int(np.argmin(counts)), int(rng.integers(64))]
    r1, r3, r2 = oracle.wgrad(o["x"], o["W1"], o["W3"], o["W2"], meta, w32, f64(inp["dout"]),
                              experts=experts, cols=cols)
    for e in experts:
        assert _rel(dW1[e][:, cols].cpu().numpy(), r1[e]) <= TOL, e
        assert _rel(dW3[e][:, cols].cpu().numpy(), r3[e]) <= TOL, e
        assert _rel(dW2[e][cols, :].cpu().numpy(), r2[e]) <= TOL, e


def test_wgrad_determinism_ten_runs():
    inp = make_inputs("stress", T=16384, need_dout=True)
    print("[case] wgrad determinism T=16384", flush=True)
    L, o, meta, w32, first, disp = _run(inp, inp["dout"])
    dout = dev(inp["dout"])
    w_d = torch.from_numpy(w32.astype(np.float32)).cuda()
    for _ in range(9):
        g = moe.wgrad(L.p, L.x, L.packed, disp, w_d, dout, L.ws)
        torch.cuda.synchronize()
        for a, b in zip(g, first):
            assert torch.equal(a, b)
