"""The saved pre-activation path through the C ABI: moe_expert_ffn_waved_save_h
keeps the first GEMM's fp32 accumulators h (h1 | h3 per routed row, packed
column order), moe_backward_saved_h reads them instead of recomputing.

Pins: the forward's out and y are bitwise those of moe_expert_ffn_waved;
the saved rows equal the oracle's h1 and h3 (oracle.expert_ffn on the same
bf16 operands) to fp32-accumulation accuracy, which fixes the column order;
every backward output (dx, dtopk_w, dlogits, dWg, dW1, dW3, dW2) is bitwise
that of moe_backward, whose parity with the oracle the backward tests
establish.  Cases: the tiny layer (fp32 x), a ragged cut of the mid layer,
widths that run the 128-wide tiles, the ungated layer, and the mid layer at
its benchmark size.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_wave_level_amd import moe
from helpers import Layer, dev, f64, oracle_inputs
from workloads import Workload, bf16_bits, make_inputs, ungated

pytestmark = pytest.mark.gpu

RELU2 = moe.MOE_ACT_RELU2
H_TOL = 1e-4   # fp32 accumulation of bf16 products against float64


def _odd():
    return Workload("odd", T=157, d=384, I=192, E_global=7, E_local=3, k=3, G=1, e_begin=2, seed=11)


CASES = {
    "tiny": lambda: make_inputs("tiny", need_dout=True),
    "mid301": lambda: make_inputs("mid", T=301, need_dout=True),
    "odd": lambda: make_inputs(_odd(), need_dout=True),
    "relu2_mid301": lambda: make_inputs(ungated("mid"), T=301, need_dout=True),
    "mid4096": lambda: make_inputs("mid", need_dout=True),
}


def _setup(inp, relu2):
    wl = inp["workload"]
    kw = {"activation": RELU2} if relu2 else {}
    L = Layer(inp, backward=True, **kw)
    W3 = None if relu2 else dev(inp["W3"])
    packed_bwd = moe.pack_weights_bwd(L.p, L.Wg, dev(inp["W1"]), W3, dev(inp["W2"]))
    o = oracle_inputs(inp)
    l64 = oracle.router_logits(o["x"], o["Wg"], o["bias"])
    idx_o, w_o, _ = oracle.route(l64, wl.k)
    idx_d = torch.from_numpy(idx_o.astype(np.int32)).cuda()
    w_d = torch.from_numpy(w_o.astype(np.float32)).cuda()
    disp = moe.dispatch(L.p, idx_d, L.ws)
    torch.cuda.synchronize()
    return L, packed_bwd, idx_d, w_d, disp


def _ffn_x(inp):
    """x as the expert GEMMs see it (fp32 inputs are rounded to bf16)."""
    x = inp["x"]
    return f64(x) if x.dtype == np.uint16 else f64(bf16_bits(x))


def _saved_rows(h, offsets, rows, ncol):
    """Rows (sorted-row order) of the saved buffer as [len(rows), ncol],
    decoded from its documented layout: routed row r of local expert e at
    padded row s = seg[e] + r - offsets[e] (seg: row counts rounded up to 64),
    element (s, c) at float ((s // 16) * (ncol // 16) + c // 16) * 256 +
    ((s % 16) + 16 * ((c % 16) // 4)) * 4 + c % 4."""
    counts = np.diff(offsets)
    seg = np.concatenate([[0], np.cumsum((counts + 63) // 64 * 64)])
    flat = h.reshape(-1).cpu().numpy()
    c = np.arange(ncol)
    out = np.empty((len(rows), ncol), np.float64)
    for n, r in enumerate(rows):
        e = int(np.searchsorted(offsets, r, "right") - 1)
        s = int(seg[e] + r - offsets[e])
        off = ((s // 16) * (ncol // 16) + c // 16) * 256 + ((s % 16) + 16 * ((c % 16) // 4)) * 4 + c % 4
        out[n] = flat[off]
    return out


def _check_saved_rows(inp, L, disp, h, relu2, nrows=24):
    """Sampled routed rows of h against the oracle's h1 | h3, unpacked from
    the packed column order (gated: 16 columns of h1, then the same 16
    indices of h3)."""
    offsets = disp.offsets.cpu().numpy()
    sorted_token = disp.sorted_token.cpu().numpy()
    P = int(offsets[-1])
    if P == 0:
        return
    rows = np.unique(np.concatenate([np.random.default_rng(3).choice(P, min(nrows, P), replace=False),
                                     [0, P - 1]]))
    x = _ffn_x(inp)
    r64 = lambda a: f64(bf16_bits(a)) if a.dtype != np.uint16 else f64(a)  # noqa: E731
    W1, W2 = r64(inp["W1"]), r64(inp["W2"])
    W3 = None if relu2 else r64(inp["W3"])
    I = L.p.I
    hg = _saved_rows(h, offsets, rows, (1 if relu2 else 2) * I)
    for n, r in enumerate(rows):
        e = int(np.searchsorted(offsets, r, "right") - 1)  # local expert (the weights are the local ones)
        _, h1, h3, _ = oracle.expert_ffn(x[sorted_token[r]][None], W1[e], None if relu2 else W3[e], W2[e],
                                         activation="relu2" if relu2 else "swiglu")
        if relu2:
            ref = h1[0]
        else:
            ref = np.empty(2 * I)
            q = np.arange(I) // 16
            j = np.arange(I) % 16
            ref[32 * q + j] = h1[0]
            ref[32 * q + 16 + j] = h3[0]
        scale = max(np.abs(ref).max(), 1e-30)
        err = np.abs(hg[n] - ref).max() / scale
        assert err <= H_TOL, f"saved row {r} (expert {e}) off by {err:.3g}"


@pytest.mark.parametrize("name", list(CASES))
def test_saved_pre_activations_forward_and_backward(name):
    relu2 = name.startswith("relu2")
    inp = CASES[name]()
    L, packed_bwd, idx_d, w_d, disp = _setup(inp, relu2)
    print(f"[case] saved h {name} T={L.T}", flush=True)
    # forward: the plain call, then the saving one (same routing)
    y0, out0 = moe.ffn_waved(L.p, L.x, L.packed, disp, w_d, L.ws)
    y0, out0 = y0.clone(), out0.clone()
    h = torch.full(moe.saved_h_shape(L.p), float("nan"), dtype=torch.float32, device="cuda")
    y1, out1 = moe.ffn_waved(L.p, L.x, L.packed, disp, w_d, L.ws, save_h=h)
    torch.cuda.synchronize()
    moe.check_error(L.ws)
    P = int(disp.offsets[-1])
    assert torch.equal(out0, out1)
    assert torch.equal(y0[:P], y1[:P])
    offsets = disp.offsets.cpu().numpy()
    ncol = h.shape[1]
    assert not np.isnan(_saved_rows(h, offsets, np.arange(P), ncol)).any(), "every routed row is written"
    _check_saved_rows(inp, L, disp, h, relu2)
    # backward: recompute against saved, every output bit for bit
    dout = dev(inp["dout"])
    kw = dict(want_dtopk_w=True, want_dlogits=True, want_dwg=True, want_dw=True)
    g0 = moe.backward(L.p, L.x, L.packed, packed_bwd, idx_d, w_d, disp, dout, L.ws, **kw)
    g0 = {k: (v.clone() if v is not None else None) for k, v in g0.items()}
    g1 = moe.backward(L.p, L.x, L.packed, packed_bwd, idx_d, w_d, disp, dout, L.ws, saved_h=h, **kw)
    torch.cuda.synchronize()
    moe.check_error(L.ws)
    for k, v in g0.items():
        if v is None:
            assert g1[k] is None, k
            continue
        assert torch.equal(v, g1[k]), f"{k} differs between the recompute and the saved pre-activations"


def test_saved_path_rejects_a_wrong_buffer():
    inp = make_inputs("tiny", need_dout=True)
    L, packed_bwd, idx_d, w_d, disp = _setup(inp, False)
    bad = torch.empty((moe.saved_h_shape(L.p)[0], 3), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        moe.ffn_waved(L.p, L.x, L.packed, disp, w_d, L.ws, save_h=bad)
