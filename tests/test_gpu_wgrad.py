"""GPU parity and determinism of the weight gradient.

dW1, dW3, dW2 of L = <dout, out> against the float64 oracle, every matrix
compared per intermediate index i: column i of dW1_e and dW3_e ([d, I]) and
row i of dW2_e ([I, d]) is scaled by its own largest reference entry, so a
small column cannot hide behind a large one of the same expert.  Full
comparisons at the tiny layer, a ragged cut of the mid layer and a ragged
cut of the V3/V4-scale share (E_local = 32 of 256 router experts); at the
stress layer (T = 8192, the hot expert's rows exceed one reduction chunk, so
the isolated-partial path runs) 96 intermediate indices of 12 experts,
the hot one and the emptiest among them.  Bitwise equality over ten runs.
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


def _rel_cols(g, r):
    """max over columns c of max_i |g[i, c] - r[i, c]| / max_i |r[i, c]|;
    columns whose reference is exactly zero must be exactly zero."""
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    scale = np.abs(r).max(axis=0)
    zero = scale == 0
    assert (g[:, zero] == 0).all(), "columns with an exactly zero reference must be zero"
    if (~zero).sum() == 0:
        return 0.0
    return float((np.abs(g[:, ~zero] - r[:, ~zero]).max(axis=0) / scale[~zero]).max())


def _check_expert(e, dW1, dW3, dW2, r1, r3, r2, cols=None):
    """Per-index comparison of expert e (cols: the intermediate indices the
    oracle computed, default all)."""
    sel = slice(None) if cols is None else cols
    g1 = dW1[e][:, sel].cpu().numpy()
    g3 = dW3[e][:, sel].cpu().numpy()
    g2 = dW2[e][sel, :].cpu().numpy()
    errs = (_rel_cols(g1, r1[e]), _rel_cols(g3, r3[e]), _rel_cols(g2.T, r2[e].T))
    assert max(errs) <= TOL, (e, errs)
    return max(errs)


def _run(inp, dout):
    L = Layer(inp, backward=True)
    o = oracle_inputs(inp)
    wl = inp["workload"]
    l64 = oracle.router_logits(o["x"], o["Wg"], o["bias"])
    idx_o, w_o, _ = oracle.route(l64, wl.k)
    meta = oracle.dispatch(idx_o, wl.e_begin, wl.E_local, wl.G)
    disp, y, out, w_d = L.ffn_from_routing(idx_o, w_o)
    packed_bwd = moe.pack_weights_bwd(L.p, L.Wg, dev(inp["W1"]), dev(inp["W3"]), dev(inp["W2"]))
    g = moe.wgrad(L.p, L.x, L.packed, packed_bwd, disp, w_d, dev(dout), L.ws)
    torch.cuda.synchronize()
    moe.check_error(L.ws)
    return L, o, meta, w_d.cpu().numpy().astype(np.float64), g, disp, packed_bwd


def _full_compare(inp):
    """Every local expert, every intermediate index, one expert at a time
    (the oracle's float64 matrices of a wide layer do not all fit at once)."""
    wl = inp["workload"]
    L, o, meta, w32, (dW1, dW3, dW2), _, _ = _run(inp, inp["dout"])
    print(f"[case] wgrad {wl.name} T={L.T} full", flush=True)
    worst = 0.0
    for e in range(wl.E_local):
        r1, r3, r2 = oracle.wgrad(o["x"], o["W1"], o["W3"], o["W2"], meta, w32, f64(inp["dout"]), experts=[e])
        worst = max(worst, _check_expert(e, dW1, dW3, dW2, r1, r3, r2))
    print(f"  worst per-index rel err {worst:.3g}", flush=True)
    return meta


def test_wgrad_tiny_full():
    _full_compare(make_inputs("tiny", need_dout=True))


def test_wgrad_mid_ragged_cut_full():
    _full_compare(make_inputs("mid", T=301, need_dout=True))


def test_wgrad_v4_share_ragged_cut_full():
    """Picks of other GPUs' experts contribute nothing here."""
    _full_compare(make_inputs("v4share", T=203, need_dout=True))


def test_wgrad_stress_sampled_columns_and_split_rows():
    inp = make_inputs("stress", T=8192, need_dout=True)
    print("[case] wgrad stress T=8192", flush=True)
    L, o, meta, w32, (dW1, dW3, dW2), disp, _ = _run(inp, inp["dout"])
    counts = meta["counts"]
    hot = int(np.argmax(counts))
    assert counts[hot] > 2048          # more than one reduction chunk
    rng = np.random.default_rng(3)
    cols = np.sort(rng.choice(1536, 96, replace=False))
    others = [e for e in rng.permutation(64) if e not in (hot, int(np.argmin(counts)))][:10]
    experts = [hot, int(np.argmin(counts))] + [int(e) for e in others]
    r1, r3, r2 = oracle.wgrad(o["x"], o["W1"], o["W3"], o["W2"], meta, w32, f64(inp["dout"]),
                              experts=experts, cols=cols)
    worst = max(_check_expert(e, dW1, dW3, dW2, r1, r3, r2, cols) for e in experts)
    print(f"  {len(experts)} experts x {cols.size} indices, worst per-index rel err {worst:.3g}", flush=True)


def test_wgrad_determinism_ten_runs():
    inp = make_inputs("stress", T=16384, need_dout=True)
    print("[case] wgrad determinism T=16384", flush=True)
    L, o, meta, w32, first, disp, packed_bwd = _run(inp, inp["dout"])
    dout = dev(inp["dout"])
    w_d = torch.from_numpy(w32.astype(np.float32)).cuda()
    for _ in range(9):
        g = moe.wgrad(L.p, L.x, L.packed, packed_bwd, disp, w_d, dout, L.ws)
        torch.cuda.synchronize()
        for a, b in zip(g, first):
            assert torch.equal(a, b)
