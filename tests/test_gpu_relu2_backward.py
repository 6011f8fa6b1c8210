"""GPU parity, determinism and batch invariance of the backward of the
ungated squared-ReLU expert (a = max(x W1, 0)^2, no W3) through the C ABI,
against the float64 oracle (oracle.backward / oracle.wgrad with
activation="relu2").

Layers are the workloads' ungated variants (intermediate size 3I/2 rounded
up to a multiple of 128).  The tiny layer (fp32 x; the expert GEMMs see x and
the weights rounded to bf16, on both sides) and a ragged cut of the mid
layer are compared in full: dx, the combine-weight and logits gradients,
dWg, and dW1, dW2 per intermediate index; moe_backward's weight gradient
equals moe_expert_wgrad's bit for bit and repeats bitwise; the stress
layer's probe tokens get bitwise identical dx and combine-weight gradients
at T = 256 and 4096.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_wave_level_amd import moe
from helpers import OUT_TOL, Layer, dev, f64, host_f64, oracle_inputs, rel_err_rows
from workloads import bf16_bits, make_inputs, ungated

pytestmark = pytest.mark.gpu

RELU2 = moe.MOE_ACT_RELU2
DL_FLOOR = 1e-3
W_TOL = 2e-2


def _dl_err(g, r, dw_ref):
    """Logits gradients per token relative to max(max_j |dl_j|, DL_FLOOR
    max_j |dw_j|) (dl is a difference of a token's combine-weight gradients)."""
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    scale = np.maximum(np.abs(r).max(axis=1), DL_FLOOR * np.abs(dw_ref).max(axis=1))
    zero = scale == 0
    assert (g[zero] == 0).all()
    if (~zero).sum() == 0:
        return 0.0
    return float((np.abs(g[~zero] - r[~zero]).max(axis=1) / scale[~zero]).max())


def _rel_cols(g, r):
    """max over columns of max_i |g - r| / max_i |r| (exact zeros stay zero)."""
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    scale = np.abs(r).max(axis=0)
    zero = scale == 0
    assert (g[:, zero] == 0).all()
    if (~zero).sum() == 0:
        return 0.0
    return float((np.abs(g[:, ~zero] - r[:, ~zero]).max(axis=0) / scale[~zero]).max())


def _operands(inp, o):
    """W1, W2 and the FFN input as the expert GEMMs see them (bf16)."""
    if inp["x"].dtype == np.uint16:
        return o["W1"], o["W2"], None
    r = lambda a: f64(bf16_bits(a))  # noqa: E731
    return r(inp["W1"]), r(inp["W2"]), r(inp["x"])


def _setup(inp):
    wl = inp["workload"]
    L = Layer(inp, backward=True, activation=RELU2)
    o = oracle_inputs(inp)
    packed_bwd = moe.pack_weights_bwd(L.p, L.Wg, dev(inp["W1"]), None, dev(inp["W2"]))
    l64 = oracle.router_logits(o["x"], o["Wg"], o["bias"])
    idx_o, w_o, _ = oracle.route(l64, wl.k)
    meta = oracle.dispatch(idx_o, wl.e_begin, wl.E_local, wl.G)
    idx_d = torch.from_numpy(idx_o.astype(np.int32)).cuda()
    w_d = torch.from_numpy(w_o.astype(np.float32)).cuda()
    disp = moe.dispatch(L.p, idx_d, L.ws)
    torch.cuda.synchronize()
    return L, o, packed_bwd, idx_o, meta, idx_d, w_d, disp


def _run(L, packed_bwd, idx_d, w_d, disp, dout_d):
    g = moe.backward(L.p, L.x, L.packed, packed_bwd, idx_d, w_d, disp, dout_d, L.ws, want_dlogits=True,
                     want_dw=True)
    torch.cuda.synchronize()
    moe.check_error(L.ws)
    assert g["dW3"] is None
    return g


def _compare_full(inp):
    wl = inp["workload"]
    L, o, packed_bwd, idx_o, meta, idx_d, w_d, disp = _setup(inp)
    print(f"[case] relu2 backward {wl.name} I={wl.I} T={L.T}", flush=True)
    dout = f64(inp["dout"])
    g = _run(L, packed_bwd, idx_d, w_d, disp, dev(inp["dout"]))
    w32 = w_d.cpu().numpy().astype(np.float64)
    W1, W2, x_ffn = _operands(inp, o)
    ref = oracle.backward(o["x"], o["Wg"], W1, None, W2, idx_o, w32, meta, dout, x_ffn=x_ffn, activation="relu2")
    errs = {
        "dx": rel_err_rows(host_f64(g["dx"]), ref["dx"]),
        "dtopk_w": rel_err_rows(host_f64(g["dtopk_w"]), ref["dw"]),
        "dlogits": _dl_err(host_f64(g["dlogits"]), ref["dl"], ref["dw"]),
        "dWg": rel_err_rows(host_f64(g["dWg"]).T, ref["dWg"].T),
    }
    xw = o["x"] if x_ffn is None else x_ffn
    worst = 0.0
    for e in range(wl.E_local):
        r1, r3, r2 = oracle.wgrad(xw, W1, None, W2, meta, w32, dout, experts=[e], activation="relu2")
        assert r3 == {}
        worst = max(worst, _rel_cols(g["dW1"][e].cpu().numpy(), r1[e]),
                    _rel_cols(g["dW2"][e].cpu().numpy().T, r2[e].T))
    errs["dW (per index)"] = worst
    print("  " + ", ".join(f"{k} {v:.3g}" for k, v in errs.items()), flush=True)
    for k, v in errs.items():
        assert v <= (W_TOL if k.startswith("dW ") else OUT_TOL), k
    return L, packed_bwd, idx_d, w_d, disp, g


def test_relu2_backward_tiny_full():
    _compare_full(make_inputs(ungated("tiny"), need_dout=True))


def test_relu2_backward_mid_ragged_cut_full_and_repeat():
    inp = make_inputs(ungated("mid"), T=301, need_dout=True)
    L, packed_bwd, idx_d, w_d, disp, g = _compare_full(inp)
    dout = dev(inp["dout"])
    ref = moe.wgrad(L.p, L.x, L.packed, packed_bwd, disp, w_d, dout, L.ws)
    torch.cuda.synchronize()
    assert ref[1] is None
    assert torch.equal(g["dW1"], ref[0]) and torch.equal(g["dW2"], ref[2])
    for _ in range(2):
        h = _run(L, packed_bwd, idx_d, w_d, disp, dout)
        for key in ("dx", "dtopk_w", "dlogits", "dWg", "dW1", "dW2"):
            assert torch.equal(h[key], g[key]), key


def test_relu2_backward_probe_tokens_bitwise_across_batch_sizes():
    """The stress layer's 256 probe tokens (fixed rows and dout) get the same
    dx and combine-weight gradient bits at T = 256 and 4096."""
    wl = ungated("stress")
    rng = np.random.default_rng([2024, 6])
    probe_dout = bf16_bits(rng.standard_normal((256, wl.d), dtype=np.float32))
    got = []
    for T in (256, 4096):
        inp = make_inputs(wl, T=T, need_dout=True)
        pos = inp["probe_pos"]
        dout = inp["dout"].copy()
        dout[pos] = probe_dout[:pos.size]
        inp["dout"] = dout
        print(f"[case] relu2 backward probes T={T}", flush=True)
        L, o, packed_bwd, idx_o, meta, idx_d, w_d, disp = _setup(inp)
        g = moe.backward(L.p, L.x, L.packed, packed_bwd, idx_d, w_d, disp, dev(dout), L.ws)
        torch.cuda.synchronize()
        moe.check_error(L.ws)
        got.append((g["dx"][torch.from_numpy(pos).cuda()].clone(),
                    g["dtopk_w"][torch.from_numpy(pos).cuda()].clone()))
        del L, g, packed_bwd
    assert torch.equal(got[0][0], got[1][0]) and torch.equal(got[0][1], got[1][1])
