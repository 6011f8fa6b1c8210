"""GPU parity of the ungated squared-ReLU expert (the cheap element-wise
activation: a = max(x W1, 0)^2, no gating projection W3) through the C ABI,
against the float64 oracle.

Layers are the workloads' layers with an ungated expert at about the same
parameter count (intermediate size 3I/2, rounded up to a multiple of 128).
The tiny layer (fp32 x; the expert GEMMs see x and the weights rounded to
bf16, on both sides of the comparison) and a ragged cut of the mid layer are
compared in full; the mid layer at its benchmark size and the decode shapes
on all or sampled tokens; the persistent kernel equals the phase-by-phase
path bit for bit; the wave size does not change bits; the stress layer's
probe tokens are bitwise identical across batch sizes; the FP8-dispatch FFN
equals the bf16 path on the dequantized rows bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_wave_level_amd import moe
from helpers import (OUT_TOL, Layer, check_dispatch_exact, check_routing, dev, f64, host_bf16_bits, host_f64,
                     oracle_inputs, rel_err_rows)
from workloads import bf16_bits, make_inputs, ungated

pytestmark = pytest.mark.gpu

RELU2 = moe.MOE_ACT_RELU2
_cache = {}


def _inputs(name, T=None):
    """Inputs of the ungated variant; weights are drawn once per workload and
    reused for every batch size (they do not depend on T)."""
    wl = ungated(name)
    if name not in _cache:
        _cache[name] = make_inputs(wl)
    base = _cache[name]
    if T is None or T == base["x"].shape[0]:
        return base
    inp = dict(base)
    inp.update(make_inputs(wl, T=T, weights=False))
    return inp


def _ffn_operands(inp, o):
    """W1, W2 and the FFN input as the expert GEMMs see them (bf16)."""
    if inp["x"].dtype == np.uint16:
        return o["W1"], o["W2"], o["x"]
    r = lambda a: f64(bf16_bits(a))  # noqa: E731
    return r(inp["W1"]), r(inp["W2"]), r(inp["x"])


def _compare(inp, sample=None, seed=0, serial=False):
    wl = inp["workload"]
    L = Layer(inp, activation=RELU2)
    o = oracle_inputs(inp)
    T = L.T
    print(f"[case] relu2 {wl.name} I={wl.I} T={T} serial={serial}", flush=True)
    r = L.forward(serial=serial)
    l64 = oracle.router_logits(o["x"], o["Wg"], o["bias"])
    tie, m = check_routing(r["logits"].cpu().numpy(), r["idx"].cpu().numpy(), r["w"].cpu().numpy(), l64, wl.k)
    idx_o, w_o, _ = oracle.route(l64, wl.k)
    meta = oracle.dispatch(idx_o, wl.e_begin, L.p.E_local, L.p.experts_per_wave)
    disp, y, out, w_d = L.ffn_from_routing(idx_o, w_o, serial=serial)
    check_dispatch_exact(disp, meta, T)
    w32 = w_d.cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(seed)
    toks = np.arange(T) if sample is None or sample >= T else np.sort(rng.choice(T, sample, replace=False))
    W1, W2, xf = _ffn_operands(inp, o)
    ref = oracle.forward_tokens(xf[toks], idx_o[toks], w32[toks], W1, None, W2, wl.e_begin, L.p.E_local,
                                activation="relu2")
    err = rel_err_rows(host_f64(out)[toks], ref)
    # routed rows of the sampled tokens against the oracle's expert
    pos = meta["pair_pos"][toks]
    rows = pos[pos >= 0][:64]
    err_y = 0.0
    if rows.size:
        experts = np.searchsorted(meta["offsets"], rows, "right") - 1
        yo = np.stack([oracle.expert_ffn(xf[meta["sorted_token"][rr]][None], W1[e], None, W2[e], "relu2")[0][0]
                       for rr, e in zip(rows, experts)])
        err_y = rel_err_rows(host_f64(y)[rows], yo)
    # the GPU's own routing end to end, outside the tie class
    ok = ~tie[toks]
    ref_e2e = oracle.forward_tokens(xf[toks][ok], idx_o[toks][ok], w_o[toks][ok], W1, None, W2, wl.e_begin,
                                    L.p.E_local, activation="relu2")
    err_e2e = rel_err_rows(host_f64(r["out"])[toks][ok], ref_e2e)
    print(f"  logits max err {m:.3g}, out rel err {err:.3g}, y rows {err_y:.3g}, end to end {err_e2e:.3g}",
          flush=True)
    assert err <= OUT_TOL and err_y <= OUT_TOL and err_e2e <= OUT_TOL
    return L, r


def test_relu2_tiny_full():
    L, r = _compare(_inputs("tiny"))
    assert r["out"].dtype == torch.float32


@pytest.mark.parametrize("serial", [False, True])
def test_relu2_mid_ragged_cut_full(serial):
    _compare(_inputs("mid", T=300), serial=serial)


def test_relu2_mid_benchmark_size_sampled():
    _compare(_inputs("mid"), sample=48)


@pytest.mark.parametrize("T", [1, 8, 128])
def test_relu2_decode_shapes(T):
    _compare(_inputs("decode", T=T), sample=None if T <= 32 else 32)


def test_relu2_persistent_equals_serial_and_standalone_combine():
    L = Layer(_inputs("mid", T=777), activation=RELU2)
    a = L.forward(serial=False)
    b = L.forward(serial=True)
    assert torch.equal(a["out"], b["out"])
    P = int(a["disp"].offsets[-1])
    assert torch.equal(a["y"][:P], b["y"][:P])
    c = moe.combine(L.p, a["y"], a["disp"].pair_pos, a["w"])
    torch.cuda.synchronize()
    assert torch.equal(c, a["out"])


@pytest.mark.parametrize("G", [1, 16])
def test_relu2_output_bits_do_not_depend_on_wave_size(G):
    inp = _inputs("mid", T=500)
    base = Layer(inp, G=4, activation=RELU2).forward()
    other = Layer(inp, G=G, activation=RELU2).forward()
    assert torch.equal(base["out"], other["out"])


def test_relu2_probe_tokens_bitwise_identical_across_batch_sizes():
    L0 = Layer(_inputs("stress"), activation=RELU2)
    res = {}
    for T in (1, 17, 256, 4096, 16384):
        inp = _inputs("stress", T=T)
        print(f"[case] relu2 stress T={T}", flush=True)
        r = L0.with_tokens(inp["x"]).forward()
        res[T] = host_bf16_bits(r["out"])[inp["probe_pos"]]   # probe i at the i-th smallest position
    full = res[16384]
    for T, got in res.items():
        assert (got == full[:got.shape[0]]).all(), T


@pytest.mark.parametrize("name,T", [("mid", 500), ("decode", 8)])
@pytest.mark.parametrize("serial", [False, True])
def test_relu2_fp8_dispatch_equals_bf16_path_on_dequantized_rows(name, T, serial):
    inp = _inputs(name, T=T)
    wl = inp["workload"]
    L = Layer(inp, activation=RELU2)
    o = oracle_inputs(inp)
    print(f"[case] relu2 fp8 {wl.name} T={T} serial={serial}", flush=True)
    x8, sc = moe.quantize_fp8(L.p, L.x)
    torch.cuda.synchronize()
    codes = x8.cpu().numpy()
    scale = sc.cpu().numpy().astype(np.float64)
    x_deq = oracle.e4m3_decode(codes) * scale[:, None]
    l64 = oracle.router_logits(o["x"], o["Wg"], o["bias"])
    idx_o, w_o, _ = oracle.route(l64, wl.k)
    idx_d = torch.from_numpy(idx_o.astype(np.int32)).cuda()
    w_d = torch.from_numpy(w_o.astype(np.float32)).cuda()
    disp = moe.dispatch(L.p, idx_d, L.ws)
    y8, out8 = moe.ffn_waved_fp8(L.p, x8, sc, L.packed, disp, w_d, L.ws, serial=serial, persistent=not serial)
    torch.cuda.synchronize()
    moe.check_error(L.ws)
    xq = bf16_bits(x_deq.astype(np.float32))
    yb, outb = moe.ffn_waved(L.p, dev(xq), L.packed, disp, w_d, L.ws, serial=serial, persistent=not serial)
    torch.cuda.synchronize()
    moe.check_error(L.ws)
    P = int(disp.offsets[-1].item())
    assert torch.equal(y8[:P], yb[:P]) and torch.equal(out8, outb)
    w32 = w_d.cpu().numpy().astype(np.float64)
    ref = oracle.forward_tokens(x_deq, idx_o, w32, o["W1"], None, o["W2"], wl.e_begin, wl.E_local,
                                activation="relu2")
    err = rel_err_rows(host_f64(out8), ref)
    print(f"  out rel err vs oracle on dequantized rows {err:.3g}", flush=True)
    assert err <= OUT_TOL


def test_relu2_edge_empty_batch():
    L = Layer(_inputs("mid", T=300), activation=RELU2).with_tokens(np.zeros((0, 4096), dtype=np.uint16))
    r = L.forward()
    assert r["out"].shape == (0, 4096)
