"""GPU parity of the forward path (router, dispatch, waved expert FFN,
combine) against the float64 oracle, through the C ABI.

Sizes: the tiny layer and a ragged cut of the mid layer are compared in
full; the mid layer at its benchmark size (T=4096, the launch configuration
bench.py times), the V3/V4-scale share and the decode sweep are compared on
all routing/dispatch outputs and on sampled tokens' output rows.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_wave_level_amd import moe
from helpers import (OUT_TOL, Layer, check_dispatch_exact, check_dispatch_valid, check_routing,
                     host_f64, oracle_inputs, rel_err_rows)
from workloads import Workload, get, make_inputs

pytestmark = pytest.mark.gpu

_cache = {}


def inputs(name, T=None):
    key = (name, T)
    if key not in _cache:
        _cache[key] = make_inputs(name, T=T)
    return _cache[key]


def _full_compare(inp, G=None, sample=None, seed=0, extra=()):
    """Runs the layer on the GPU and compares every stage with the oracle.
    sample: number of tokens whose output rows are compared (None = all);
    extra: tokens compared in addition to the sample."""
    wl = inp["workload"]
    L = Layer(inp, G=G)
    o = oracle_inputs(inp)
    T = L.T
    print(f"[case] {wl.name} T={T} G={L.p.experts_per_wave}", flush=True)
    # 1. router, end to end on the GPU
    r = L.forward()
    l64 = oracle.router_logits(o["x"], o["Wg"], o["bias"])
    idx_g = r["idx"].cpu().numpy()
    w_g = r["w"].cpu().numpy()
    tie, m = check_routing(r["logits"].cpu().numpy(), idx_g, w_g, l64, wl.k)
    check_dispatch_valid(r["disp"], idx_g, wl.e_begin, L.p.E_local, L.p.experts_per_wave)
    # 2. dispatch + FFN + combine on the oracle's routing
    idx_o, w_o, _ = oracle.route(l64, wl.k)
    meta = oracle.dispatch(idx_o, wl.e_begin, L.p.E_local, L.p.experts_per_wave)
    disp, y, out, w_d = L.ffn_from_routing(idx_o, w_o)
    check_dispatch_exact(disp, meta, T)
    w32 = w_d.cpu().numpy().astype(np.float64)   # the weights the GPU was given
    rng = np.random.default_rng(seed)
    toks = np.arange(T) if sample is None or sample >= T else np.sort(rng.choice(T, sample, replace=False))
    toks = np.unique(np.concatenate([toks, np.asarray(extra, dtype=np.int64)]))
    ref = oracle.forward_tokens(o["x"][toks], idx_o[toks], w32[toks], o["W1"], o["W3"], o["W2"],
                                wl.e_begin, L.p.E_local)
    got = host_f64(out)[toks]
    err = rel_err_rows(got, ref)
    print(f"  logits max err {m:.3g}, tie tokens {int(tie.sum())}, out rel err {err:.3g}", flush=True)
    assert err <= OUT_TOL
    # y rows of the sampled tokens' local pairs
    pos = meta["pair_pos"][toks]
    rows = pos[pos >= 0]
    if rows.size:
        yr = host_f64(y)[rows]
        yo = np.stack([oracle.expert_ffn(o["x"][meta["sorted_token"][rr]][None],
                                         o["W1"][np.searchsorted(meta["offsets"], rr, "right") - 1],
                                         o["W3"][np.searchsorted(meta["offsets"], rr, "right") - 1],
                                         o["W2"][np.searchsorted(meta["offsets"], rr, "right") - 1])[0][0]
                       for rr in rows[:64]])
        assert rel_err_rows(yr[:64], yo) <= OUT_TOL
    # 3. the GPU's own routing end to end: compare tokens outside the tie class
    ok = ~tie[toks]
    ref_e2e = oracle.forward_tokens(o["x"][toks][ok], idx_o[toks][ok], w_o[toks][ok], o["W1"], o["W3"],
                                    o["W2"], wl.e_begin, L.p.E_local)
    assert rel_err_rows(host_f64(r["out"])[toks][ok], ref_e2e) <= OUT_TOL
    return L, r, (disp, y, out)


def test_tiny_layer_full():
    L, r, _ = _full_compare(inputs("tiny"))
    # fp32 output dtype for the fp32 layer
    assert r["out"].dtype == torch.float32


def test_mid_layer_ragged_cut_full():
    _full_compare(inputs("mid", T=300))


def test_mid_layer_benchmark_size_sampled():
    _full_compare(inputs("mid"), sample=48)


def test_odd_widths_run_the_128_wide_tiles():
    """d = 384 and 2I = 384 are not multiples of 256, so both expert GEMMs
    run the 128-wide tile shape; 3 local experts of 7 starting at 2, k = 3,
    a ragged batch; full comparison, then the phase kernels against the
    persistent kernel bit for bit."""
    wl = Workload("odd", T=157, d=384, I=192, E_global=7, E_local=3, k=3, G=1, e_begin=2, seed=11)
    inp = make_inputs(wl)
    L, r, _ = _full_compare(inp)
    a = L.forward(serial=False)
    b = L.forward(serial=True)
    assert torch.equal(a["out"], b["out"])
    P = int(a["disp"].offsets[-1])
    assert torch.equal(a["y"][:P], b["y"][:P])


@pytest.mark.parametrize("T", [1, 8, 32, 128])
def test_decode_sweep(T):
    _full_compare(inputs("decode", T=T), sample=None if T <= 32 else 32)


def test_v4_scale_share_sampled():
    L, r, _ = _full_compare(inputs("v4share"), sample=32)
    # tokens without a local pick get exact zeros
    idx = r["idx"].cpu().numpy()
    none = ~((idx >= 0) & (idx < 32)).any(axis=1)
    assert none.any()
    assert (host_f64(r["out"])[none] == 0).all()


def test_stress_layer_full_size_sampled():
    """The stress layer at its largest batch (T = 16384; one expert chosen
    by about half of the tokens, so the whole-expert deal splits it over
    XCDs): routing and dispatch in full, output rows of 32 sampled tokens
    plus token 0, token T - 1 and 8 tokens that pick the hot expert, and y
    rows of their pairs."""
    inp = inputs("stress", T=16384)
    wl = inp["workload"]
    o = oracle_inputs(inp)
    idx_o, _, _ = oracle.route(oracle.router_logits(o["x"], o["Wg"], o["bias"]), wl.k)
    hot_toks = np.nonzero((idx_o == inp["hot_expert"]).any(axis=1))[0]
    assert hot_toks.size > 0.3 * wl.T
    pick = np.random.default_rng(7).choice(hot_toks, 8, replace=False)
    _full_compare(inp, sample=32, seed=1, extra=np.concatenate([[0, 16383], pick]))


@pytest.mark.parametrize("name,T", [("mid", 777), ("decode", 8)])
def test_forward_stays_inside_the_forward_workspace(name, T):
    """A workspace of exactly the forward size (moe_workspace_size with no
    flags) followed by guard bytes: route, dispatch, the expert FFN
    (persistent and phases) and the FP8-dispatch FFN write nothing past it,
    and give the same bits as on a backward-sized workspace."""
    inp = inputs(name, T=T)
    L = Layer(inp)
    print(f"[case] forward-only workspace {name} T={T}", flush=True)
    n = moe.workspace_size(L.p)
    assert n == L.ws.numel() and n < moe.workspace_size(L.p, backward=True)
    buf = torch.full((n + 65536,), 0xA5, dtype=torch.uint8, device="cuda")
    buf[:n].zero_()
    ws = buf[:n]
    big = moe.workspace(L.p, backward=True)
    for serial in (False, True):
        a = moe.forward(L.p, L.x, L.packed, ws, bias=L.bias, serial=serial, persistent=not serial)
        b = moe.forward(L.p, L.x, L.packed, big, bias=L.bias, serial=serial, persistent=not serial)
        torch.cuda.synchronize()
        moe.check_error(ws)
        moe.check_error(big)
        assert torch.equal(a["out"], b["out"]) and torch.equal(a["idx"], b["idx"])
        x8, sc = moe.quantize_fp8(L.p, L.x)
        moe.ffn_waved_fp8(L.p, x8, sc, L.packed, a["disp"], a["w"], ws, serial=serial, persistent=not serial)
        torch.cuda.synchronize()
        moe.check_error(ws)
    assert (buf[n:] == 0xA5).all()


def test_persistent_equals_serial_and_standalone_combine():
    inp = inputs("mid", T=777)
    L = Layer(inp)
    a = L.forward(serial=False)
    b = L.forward(serial=True)
    assert torch.equal(a["out"], b["out"])
    P = int(a["disp"].offsets[-1])
    assert torch.equal(a["y"][:P], b["y"][:P])
    c = moe.combine(L.p, a["y"], a["disp"].pair_pos, a["w"])
    torch.cuda.synchronize()
    assert torch.equal(c, a["out"])


@pytest.mark.parametrize("T", [8, 32, 100, 128])
def test_small_batch_persistent_equals_serial_over_runs(T):
    """Decode shapes: m-tiles that do not divide evenly over the 8 XCDs
    make the persistent kernel spread every m-tile's output tiles over all
    XCDs (the GEMM1 -> GEMM2 hand-off then crosses XCDs); its bits equal
    the phase-by-phase path's on every one of several runs."""
    L = Layer(inputs("decode", T=T))
    b = L.forward(serial=True)
    P = int(b["disp"].offsets[-1])
    for _ in range(5):
        a = L.forward(serial=False)
        assert torch.equal(a["out"], b["out"])
        assert torch.equal(a["y"][:P], b["y"][:P])


@pytest.mark.parametrize("T", [1024, 1025])
def test_dispatch_exact_on_both_sides_of_the_one_workgroup_path(T):
    """moe_dispatch runs its count, scan and scatter in one workgroup for
    T <= 1024 and as three kernels above: on the mid layer's routing at
    T = 1024 and 1025 both give the oracle's permutation exactly, and the
    persistent and phase-by-phase FFNs on them the same bits."""
    inp = inputs("mid", T=T)
    wl = inp["workload"]
    L = Layer(inp)
    o = oracle_inputs(inp)
    l64 = oracle.router_logits(o["x"], o["Wg"], o["bias"])
    idx_o, w_o, _ = oracle.route(l64, wl.k)
    meta = oracle.dispatch(idx_o, wl.e_begin, L.p.E_local, L.p.experts_per_wave)
    disp, y, out, _ = L.ffn_from_routing(idx_o, w_o)
    check_dispatch_exact(disp, meta, T)
    disp_s, y_s, out_s, _ = L.ffn_from_routing(idx_o, w_o, serial=True)
    check_dispatch_exact(disp_s, meta, T)
    P = int(meta["offsets"][-1])
    assert torch.equal(out, out_s)
    assert torch.equal(y[:P], y_s[:P])


@pytest.mark.parametrize("name,T", [("mid", 777), ("decode", 1), ("decode", 128)])
def test_persistent_back_to_back_on_one_dispatch(name, T):
    """The persistent kernel's tickets and hand-off counters need no fill of
    their own: moe_dispatch clears them and every launch clears them as it
    ends.  On a workspace poisoned before the dispatch, repeated persistent
    calls on one dispatch (outputs poisoned before each call) all give the
    phase-by-phase path's bits."""
    L = Layer(inputs(name, T=T))
    L.ws.fill_(0xA5)
    idx, w, _ = moe.route(L.p, L.x, L.packed, L.ws, bias=L.bias)
    disp = moe.dispatch(L.p, idx, L.ws)
    y_ref, out_ref = moe.ffn_waved(L.p, L.x, L.packed, disp, w, L.ws, serial=True)
    torch.cuda.synchronize()
    moe.check_error(L.ws)
    P = int(disp.offsets[-1])
    y = torch.empty_like(y_ref)
    out = torch.empty_like(out_ref)
    for _ in range(4):
        y.view(torch.int16).fill_(0x7F7F)
        out.view(torch.int16).fill_(0x7F7F)
        moe.ffn_waved(L.p, L.x, L.packed, disp, w, L.ws, y=y, out=out, persistent=True)
        torch.cuda.synchronize()
        moe.check_error(L.ws)
        assert torch.equal(out, out_ref)
        assert torch.equal(y[:P], y_ref[:P])


@pytest.mark.parametrize("G", [1, 2, 8, 16])
def test_output_bits_do_not_depend_on_wave_size(G):
    inp = inputs("mid", T=500)
    base = Layer(inp, G=4).forward()
    other = Layer(inp, G=G).forward()
    assert torch.equal(base["out"], other["out"])
    assert torch.equal(base["idx"], other["idx"]) and torch.equal(base["w"], other["w"])


def test_edge_empty_batch():
    inp = inputs("mid", T=300)
    L = Layer(inp).with_tokens(np.zeros((0, 4096), dtype=np.uint16))
    r = L.forward()
    assert r["out"].shape == (0, 4096)
    assert r["disp"].counts.sum().item() == 0


def test_edge_single_token_and_local_window():
    # a window of 4 local experts of the mid layer's 16, top-4, one wave each
    inp = dict(inputs("mid", T=300))
    inp["W1"], inp["W3"], inp["W2"] = inp["W1"][4:8], inp["W3"][4:8], inp["W2"][4:8]
    for T in (1, 300):
        sub = dict(inp)
        sub["x"] = inp["x"][:T]
        L = Layer(sub, G=1, e_begin=4, E_local=4)
        o = oracle_inputs(sub)
        l64 = oracle.router_logits(o["x"], o["Wg"], None)
        idx_o, w_o, _ = oracle.route(l64, 4)
        meta = oracle.dispatch(idx_o, 4, 4, 1)
        disp, y, out, w_d = L.ffn_from_routing(idx_o, w_o)
        check_dispatch_exact(disp, meta, T)
        ref = oracle.forward_tokens(o["x"], idx_o, w_d.cpu().numpy().astype(np.float64), o["W1"], o["W3"],
                                    o["W2"], 4, 4)
        assert rel_err_rows(host_f64(out), ref) <= OUT_TOL


def test_edge_k_equals_E_and_single_expert():
    inp = inputs("tiny")
    # k = E: every token visits every expert
    L = Layer(inp, k=8)
    o = oracle_inputs(inp)
    l64 = oracle.router_logits(o["x"], o["Wg"], None)
    idx_o, w_o, _ = oracle.route(l64, 8)
    disp, y, out, w_d = L.ffn_from_routing(idx_o, w_o)
    assert disp.counts.cpu().numpy().tolist() == [64] * 8
    ref = oracle.forward_tokens(o["x"], idx_o, w_d.cpu().numpy().astype(np.float64), o["W1"], o["W3"], o["W2"], 0, 8)
    assert rel_err_rows(host_f64(out), ref) <= OUT_TOL
    # one local expert, top-1, one wave: a dense SwiGLU for the tokens routed to it
    sub = dict(inp)
    sub["W1"], sub["W3"], sub["W2"] = inp["W1"][2:3], inp["W3"][2:3], inp["W2"][2:3]
    L1 = Layer(sub, G=1, k=1, e_begin=2, E_local=1)
    idx1, w1, _ = oracle.route(l64, 1)
    disp, y, out, w_d = L1.ffn_from_routing(idx1, w1)
    ref = oracle.forward_tokens(o["x"], idx1, w_d.cpu().numpy().astype(np.float64), sub["W1"].astype(np.float64),
                                sub["W3"].astype(np.float64), sub["W2"].astype(np.float64), 2, 1)
    assert rel_err_rows(host_f64(out), ref) <= OUT_TOL


@pytest.mark.parametrize("name,T,want", [("mid", 4096, "phases"), ("stress", 4096, "phases"),
                                         ("stress", 16384, "phases"), ("decode", 1, "phases"),
                                         ("v4share", 2048, "phases")])
def test_default_schedule_choice_gives_the_same_bits(name, T, want):
    """With no flag the library runs its default schedule (moe_ffn_path on
    the device's CU count: the phase kernels); the call gives the bits of
    both forced schedules."""
    L = Layer(inputs(name, T=T))
    print(f"[case] default schedule {name} T={T}", flush=True)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    path = moe.ffn_path(L.p, cus)
    if cus == 256:
        assert path == (moe.MOE_PATH_PERSISTENT if want == "persistent" else moe.MOE_PATH_PHASES)
    a = moe.forward(L.p, L.x, L.packed, L.ws, bias=L.bias)
    torch.cuda.synchronize()
    moe.check_error(L.ws)
    P = int(a["disp"].offsets[-1])
    for forced in ({"serial": True}, {"persistent": True}):
        b = moe.forward(L.p, L.x, L.packed, L.ws, bias=L.bias, **forced)
        torch.cuda.synchronize()
        moe.check_error(L.ws)
        assert torch.equal(a["out"], b["out"]), forced
        assert torch.equal(a["y"][:P], b["y"][:P]), forced
