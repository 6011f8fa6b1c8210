"""GPU parity, determinism and batch invariance of the backward (data
gradient dx, combine-weight gradient, logits gradient, router-weight
gradient dWg) through the C ABI, against the float64 oracle.

The GPU runs on the oracle's routing (indices and the fp32 weights the GPU
is given), so both sides differentiate the same routed layer.  Sizes: the
tiny layer (fp32 x) and ragged cuts of the mid layer and of the V3/V4-scale
share (E_local = 32 of 256 router experts, so some picks are owned by other
GPUs) are compared in full; the stress layer at its full size (T = 16384,
hot expert) on sampled tokens, dWg there as the product x^T dlogits of the
checked logits gradient, and bitwise over repeated runs and across batch
sizes.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_wave_level_amd import moe
from helpers import OUT_TOL, Layer, dev, f64, host_f64, oracle_inputs, rel_err_rows
from workloads import Workload, bf16_bits, make_inputs

pytestmark = pytest.mark.gpu


def _setup(inp):
    """Layer on the GPU, backward weights, and the oracle's routing."""
    wl = inp["workload"]
    L = Layer(inp, backward=True)
    o = oracle_inputs(inp)
    packed_bwd = moe.pack_weights_bwd(L.p, L.Wg, dev(inp["W1"]), dev(inp["W3"]), dev(inp["W2"]))
    l64 = oracle.router_logits(o["x"], o["Wg"], o["bias"])
    idx_o, w_o, _ = oracle.route(l64, wl.k)
    meta = oracle.dispatch(idx_o, wl.e_begin, wl.E_local, wl.G)
    idx_d = torch.from_numpy(idx_o.astype(np.int32)).cuda()
    w_d = torch.from_numpy(w_o.astype(np.float32)).cuda()
    disp = moe.dispatch(L.p, idx_d, L.ws)
    torch.cuda.synchronize()
    return L, o, packed_bwd, idx_o, meta, idx_d, w_d, disp


# dl_j = w_j (dw_j - sum_m w_m dw_m) is a difference of a token's combine-
# weight gradients; where one pick carries almost all the weight the other
# picks' w_j fall to the bottom of fp32's range (the stress layer's hot router
# column gives weights near exp(-100)) and dl is far below the token's dw
# scale.  Logits gradients are therefore compared per token relative to
# max(max_j |dl_j|, DL_FLOOR * max_j |dw_j|).
DL_FLOOR = 1e-3


def _dl_err(g, r, dw_ref):
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    scale = np.maximum(np.abs(r).max(axis=1), DL_FLOOR * np.abs(dw_ref).max(axis=1))
    zero = scale == 0
    assert (g[zero] == 0).all(), "tokens without a gradient must get exact zeros"
    if (~zero).sum() == 0:
        return 0.0
    return float((np.abs(g[~zero] - r[~zero]).max(axis=1) / scale[~zero]).max())


def _ffn_operands(inp, o):
    """Expert weights and FFN input as the expert GEMMs see them: for fp32
    inputs the GPU rounds both to bf16 (RNE) for the FFN only, the router
    keeps fp32 x.  The combine-weight and logits gradients are differences
    of a few FFN outputs per token, so that rounding must be on both sides
    of the comparison."""
    if inp["x"].dtype == np.uint16:
        return o["W1"], o["W3"], o["W2"], None
    r = lambda a: f64(bf16_bits(a))  # noqa: E731
    return r(inp["W1"]), r(inp["W3"]), r(inp["W2"]), r(inp["x"])


def _backward(L, packed_bwd, idx_d, w_d, disp, dout_d, **kw):
    kw.setdefault("want_dlogits", True)
    g = moe.backward(L.p, L.x, L.packed, packed_bwd, idx_d, w_d, disp, dout_d, L.ws, **kw)
    torch.cuda.synchronize()
    moe.check_error(L.ws)
    return g


def _compare_full(inp):
    wl = inp["workload"]
    L, o, packed_bwd, idx_o, meta, idx_d, w_d, disp = _setup(inp)
    print(f"[case] backward {wl.name} T={L.T}", flush=True)
    g = _backward(L, packed_bwd, idx_d, w_d, disp, dev(inp["dout"]))
    w32 = w_d.cpu().numpy().astype(np.float64)
    W1, W3, W2, x_ffn = _ffn_operands(inp, o)
    ref = oracle.backward(o["x"], o["Wg"], W1, W3, W2, idx_o, w32, meta, f64(inp["dout"]), x_ffn=x_ffn)
    errs = {
        "dx": rel_err_rows(host_f64(g["dx"]), ref["dx"]),
        "dtopk_w": rel_err_rows(host_f64(g["dtopk_w"]), ref["dw"]),
        "dlogits": _dl_err(host_f64(g["dlogits"]), ref["dl"], ref["dw"]),
        "dWg": rel_err_rows(host_f64(g["dWg"]).T, ref["dWg"].T),
    }
    print("  " + ", ".join(f"{k} {v:.3g}" for k, v in errs.items()), flush=True)
    for k, v in errs.items():
        assert v <= OUT_TOL, k
    return L, g, ref


def test_backward_tiny_full():
    _compare_full(make_inputs("tiny", need_dout=True))


def test_backward_mid_ragged_cut_full():
    _compare_full(make_inputs("mid", T=301, need_dout=True))


def test_backward_v4_share_ragged_cut_full():
    """Picks owned by other GPUs have an exactly zero combine-weight gradient
    but a non-zero logits gradient; tokens with no local pick get dx from the
    router alone."""
    inp = make_inputs("v4share", T=203, need_dout=True)
    L, g, ref = _compare_full(inp)
    wl = inp["workload"]
    l64 = oracle.router_logits(f64(inp["x"]), f64(inp["Wg"]))
    idx_o, _, _ = oracle.route(l64, wl.k)
    nonlocal_pick = (idx_o < wl.e_begin) | (idx_o >= wl.e_begin + wl.E_local)
    assert nonlocal_pick.any() and (~nonlocal_pick).any()
    assert (g["dtopk_w"].cpu().numpy()[nonlocal_pick] == 0).all()
    no_local = nonlocal_pick.all(axis=1)
    assert no_local.any()
    assert rel_err_rows(host_f64(g["dx"])[no_local], ref["dx_router"][no_local]) <= OUT_TOL


def test_backward_odd_intermediate_width_and_local_window():
    """I = 192 (not a multiple of 128: the 64-wide stage-1 product), d = 384
    (not a multiple of 256: the 128-wide tiles), a window of 3 local experts
    of 7 starting at 2, k = 3, a ragged batch."""
    wl = Workload("odd", T=157, d=384, I=192, E_global=7, E_local=3, k=3, G=1, e_begin=2, seed=11)
    _compare_full(make_inputs(wl, need_dout=True))


def test_backward_weight_gradient_matches_wgrad_entry_point():
    inp = make_inputs("mid", T=257, need_dout=True)
    L, o, packed_bwd, idx_o, meta, idx_d, w_d, disp = _setup(inp)
    dout = dev(inp["dout"])
    g = _backward(L, packed_bwd, idx_d, w_d, disp, dout, want_dw=True)
    ref = moe.wgrad(L.p, L.x, L.packed, packed_bwd, disp, w_d, dout, L.ws)
    torch.cuda.synchronize()
    for a, b in zip((g["dW1"], g["dW3"], g["dW2"]), ref):
        assert torch.equal(a, b)


def _stress_inputs(T, probe_dout):
    """Stress layer at batch size T with the probe tokens' dout fixed (the
    generator draws dout per T; batch invariance needs it per token)."""
    inp = make_inputs("stress", T=T, need_dout=True)
    dout = inp["dout"].copy()
    pos = inp["probe_pos"]
    dout[pos] = probe_dout[:pos.size]
    inp["dout"] = dout
    return inp


def _probe_dout(d):
    rng = np.random.default_rng([2024, 5])
    return bf16_bits(rng.standard_normal((256, d), dtype=np.float32))


def test_backward_stress_full_size_sampled_and_determinism():
    inp = _stress_inputs(16384, _probe_dout(4096))
    wl = inp["workload"]
    L, o, packed_bwd, idx_o, meta, idx_d, w_d, disp = _setup(inp)
    print("[case] backward stress T=16384", flush=True)
    dout = dev(inp["dout"])
    g = _backward(L, packed_bwd, idx_d, w_d, disp, dout, want_dw=True)
    w32 = w_d.cpu().numpy().astype(np.float64)
    hot = inp["hot_expert"]
    rng = np.random.default_rng(9)
    picks_hot = np.nonzero((idx_o == hot).any(axis=1))[0]
    toks = np.unique(np.concatenate([rng.choice(L.T, 6, replace=False), rng.choice(picks_hot, 4, replace=False),
                                     [0, L.T - 1]]))
    dx_r, dw_r, dl_r = oracle.backward_tokens(o["x"][toks], o["x"][toks], idx_o[toks], w32[toks],
                                              f64(inp["dout"])[toks], o["Wg"], o["W1"], o["W3"], o["W2"],
                                              wl.e_begin, wl.E_local)
    e_dx = rel_err_rows(host_f64(g["dx"])[toks], dx_r)
    e_dw = rel_err_rows(host_f64(g["dtopk_w"])[toks], dw_r)
    dl_g = np.take_along_axis(host_f64(g["dlogits"])[toks], idx_o[toks].astype(np.int64), 1)
    e_dl = _dl_err(dl_g, dl_r, dw_r)
    # dWg at full size: the product of x and the logits gradient (an identity
    # between outputs, compared per expert column in float64)
    dlg = host_f64(g["dlogits"])
    e_wg = rel_err_rows(host_f64(g["dWg"]).T, (o["x"].T @ dlg).T)
    print(f"  sampled dx {e_dx:.3g}, dtopk_w {e_dw:.3g}, dlogits {e_dl:.3g}; dWg vs x^T dlogits {e_wg:.3g}",
          flush=True)
    assert e_dx <= OUT_TOL and e_dw <= OUT_TOL and e_dl <= OUT_TOL and e_wg <= OUT_TOL
    # dlogits are zero off the picks
    mask = np.zeros(dlg.shape, dtype=bool)
    mask[np.repeat(np.arange(L.T), wl.k), idx_o.reshape(-1)] = True
    assert (dlg[~mask] == 0).all()
    # bitwise over repeated runs
    for _ in range(4):
        h = _backward(L, packed_bwd, idx_d, w_d, disp, dout, want_dw=True)
        for key in ("dx", "dtopk_w", "dlogits", "dWg", "dW1", "dW3", "dW2"):
            assert torch.equal(h[key], g[key]), key


def test_backward_batch_invariance_of_probe_tokens():
    probe_dout = _probe_dout(4096)
    first = None
    for T in (256, 4096, 16384):
        inp = _stress_inputs(T, probe_dout)
        L, o, packed_bwd, idx_o, meta, idx_d, w_d, disp = _setup(inp)
        print(f"[case] backward batch invariance T={T}", flush=True)
        g = _backward(L, packed_bwd, idx_d, w_d, disp, dev(inp["dout"]))
        pos = torch.from_numpy(inp["probe_pos"]).cuda()
        rows = {k: g[k].index_select(0, pos).cpu() for k in ("dx", "dtopk_w", "dlogits")}
        if first is None:
            first = rows
        else:
            for k in rows:
                assert torch.equal(rows[k], first[k]), (T, k)
        del L, g


def test_backward_edge_empty_batch():
    inp = make_inputs("mid", T=0, need_dout=True)
    L = Layer(inp, backward=True)
    packed_bwd = moe.pack_weights_bwd(L.p, L.Wg, dev(inp["W1"]), dev(inp["W3"]), dev(inp["W2"]))
    idx = torch.zeros((0, L.p.k), dtype=torch.int32, device="cuda")
    w = torch.zeros((0, L.p.k), dtype=torch.float32, device="cuda")
    disp = moe.dispatch(L.p, idx, L.ws)
    dout = torch.zeros((0, L.p.d), dtype=torch.bfloat16, device="cuda")
    g = _backward(L, packed_bwd, idx, w, disp, dout, want_dw=True)
    assert g["dx"].shape == (0, L.p.d)
    assert (g["dWg"] == 0).all() and (g["dW1"] == 0).all() and (g["dW2"] == 0).all()
