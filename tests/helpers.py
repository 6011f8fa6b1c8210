"""Shared helpers of the GPU tests: moving seeded inputs to the device,
running the library through its binding, and the comparison rules.

Comparison rules (written out once here, used by every GPU test):
  * routing indices, expert counts, permutation: bit-exact;
  * router logits: max |gpu - fp64| <= LOGIT_TOL; selection is then compared
    exactly for every token whose fp64 consecutive-score margins among the
    first k+1 ranks exceed twice the measured logit error (the "tie class"
    below that is checked for validity instead: the GPU's picks are a top-k
    of its own logits and within that error of a top-k of the fp64 logits);
  * layer outputs: per row, max|gpu - ref| / max|ref| <= OUT_TOL (2e-2);
    rows whose reference is exactly zero must be exactly zero.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from combine_wave_level_amd import moe
from workloads import Workload, bf16_value

LOGIT_TOL = 1e-4
OUT_TOL = 2e-2


def dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def host_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.detach().cpu().float().numpy().astype(np.float64)
    return t.detach().cpu().numpy().astype(np.float64)


def f64(a: np.ndarray) -> np.ndarray:
    """Exact float64 value of a generated input (bf16 bits or float32)."""
    return oracle.decode_bf16(a) if a.dtype == np.uint16 else a.astype(np.float64)


def problem_for(wl: Workload, T: int, G: int | None = None, **kw) -> moe.Problem:
    xdt = moe.MOE_F32 if wl.dtype == "f32" else moe.MOE_BF16
    return moe.problem(T=T, d=wl.d, I=wl.I, E_global=wl.E_global, k=kw.get("k", wl.k),
                       e_begin=kw.get("e_begin", wl.e_begin), E_local=kw.get("E_local", wl.E_local),
                       experts_per_wave=wl.G if G is None else G, x_dtype=xdt, w_dtype=xdt,
                       out_dtype=xdt, activation=kw.get("activation", moe.MOE_ACT_SWIGLU))


class Layer:
    """Device copies of one workload's inputs plus packed weights and workspace."""

    def __init__(self, inp: dict, G: int | None = None, backward: bool = False, **kw):
        """backward: size the workspace for the backward entry points too
        (otherwise it holds exactly the forward entry points' size)."""
        wl: Workload = inp["workload"]
        self.wl = wl
        self.T = inp["x"].shape[0]
        self.p = problem_for(wl, self.T, G, **kw)
        self.x = dev(inp["x"])
        self.Wg = dev(inp["Wg"])
        self.bias = dev(inp["bias"]) if inp.get("bias") is not None else None
        W3 = dev(inp["W3"]) if self.p.activation == moe.MOE_ACT_SWIGLU else None
        self.packed = moe.pack_weights(self.p, self.Wg, dev(inp["W1"]), W3, dev(inp["W2"]))
        self.backward = backward
        self.ws = moe.workspace(self.p, backward=backward)
        torch.cuda.synchronize()

    def with_tokens(self, x_np: np.ndarray, bias=None) -> "Layer":
        """Same weights, another batch."""
        other = object.__new__(Layer)
        other.wl = self.wl
        other.T = x_np.shape[0]
        other.p = self.p.replace(T=other.T)
        other.x = dev(x_np)
        other.Wg = self.Wg
        other.bias = self.bias
        other.packed = self.packed
        other.backward = self.backward
        other.ws = moe.workspace(other.p, backward=self.backward)
        return other

    def forward(self, serial=False, want_logits=True):
        """The layer on the phase kernels (serial) or the persistent kernel
        (forced, whatever schedule the library would pick)."""
        r = moe.forward(self.p, self.x, self.packed, self.ws, bias=self.bias, serial=serial,
                        want_logits=want_logits, persistent=not serial)
        torch.cuda.synchronize()
        moe.check_error(self.ws)
        return r

    def ffn_from_routing(self, idx: np.ndarray, w: np.ndarray, serial=False, fused=True):
        """Dispatch + FFN (+ combine) of a routing given on the host."""
        idx_d = torch.from_numpy(idx.astype(np.int32)).cuda()
        w_d = torch.from_numpy(w.astype(np.float32)).cuda()
        disp = moe.dispatch(self.p, idx_d, self.ws)
        y, out = moe.ffn_waved(self.p, self.x, self.packed, disp, w_d, self.ws, fused_combine=fused,
                               serial=serial, persistent=not serial)
        torch.cuda.synchronize()
        moe.check_error(self.ws)
        return disp, y, out, w_d


def oracle_inputs(inp: dict):
    """float64 views of the generated inputs: x for the router, x for the FFN
    (the same values), router weights, bias and expert weights."""
    x = f64(inp["x"])
    return dict(x=x, Wg=f64(inp["Wg"]), bias=None if inp.get("bias") is None else inp["bias"].astype(np.float64),
                W1=f64(inp["W1"]), W3=f64(inp["W3"]), W2=f64(inp["W2"]))


def check_routing(logits_gpu: np.ndarray, idx_gpu: np.ndarray, w_gpu: np.ndarray, l64: np.ndarray, k: int):
    """Returns (tie_mask, max_logit_err).  Asserts everything outside the tie class."""
    err = np.abs(logits_gpu - l64)
    m = float(err.max()) if err.size else 0.0
    assert m <= LOGIT_TOL, f"router logits off by {m}"
    idx_o, w_o, _ = oracle.route(l64, k)
    T, E = l64.shape
    srt = -np.sort(-l64, axis=1)[:, :min(k + 1, E)]
    margins = srt[:, :-1] - srt[:, 1:] if srt.shape[1] > 1 else np.full((T, 1), np.inf)
    tie = (margins < 2 * m + 1e-12).any(axis=1) if k < E or srt.shape[1] > 1 else np.zeros(T, bool)
    ok = ~tie
    assert (idx_gpu[ok] == idx_o[ok]).all(), "routing differs outside the tie class"
    rel = np.abs(w_gpu[ok] - w_o[ok]) / np.maximum(w_o[ok], 1e-30)
    assert (rel <= 4 * m + 1e-5).all(), f"router weights off: {rel.max()}"
    for t in np.nonzero(tie)[0]:
        check_topk_valid(logits_gpu[t], idx_gpu[t], w_gpu[t], l64[t], k, 2 * m)
    return tie, m


def check_topk_valid(lg, idx, w, l64, k, slack):
    """The picks are a top-k of the GPU logits (descending, ties to lower id)
    and, within `slack`, a top-k of the fp64 logits; weights form a
    distribution in rank order.  A weight may be exactly zero: a pick whose
    logit trails the top one by more than about 103 has exp(l - l_max) below
    fp32's smallest subnormal (the stress layer's hot router column puts the
    other picks near exp(-100))."""
    order = sorted(range(lg.size), key=lambda e: (-lg[e], e))
    assert list(idx) == order[:k]
    chosen = set(int(e) for e in idx)
    rest = [e for e in range(lg.size) if e not in chosen]
    if rest:
        assert min(l64[list(chosen)]) >= max(l64[rest]) - slack
    assert abs(float(w.sum()) - 1.0) < 1e-5 and (np.diff(w) <= 0).all() and (w >= 0).all() and w[0] > 0


def rel_err_rows(g: np.ndarray, r: np.ndarray) -> float:
    """max over rows of max|g - r| / max|r|; exact-zero rows must match exactly."""
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    scale = np.abs(r).max(axis=1)
    zero = scale == 0
    assert (g[zero] == 0).all(), "rows with an exactly zero reference must be zero"
    if (~zero).sum() == 0:
        return 0.0
    return float((np.abs(g[~zero] - r[~zero]).max(axis=1) / scale[~zero]).max())


def check_dispatch_exact(disp: moe.Dispatch, meta: dict, T: int):
    P = int(meta["offsets"][-1])
    assert disp.counts.cpu().numpy().tolist() == meta["counts"].tolist()
    assert disp.offsets.cpu().numpy().tolist() == meta["offsets"].tolist()
    assert (disp.sorted_token.cpu().numpy()[:P] == meta["sorted_token"]).all()
    assert (disp.pair_pos.cpu().numpy() == meta["pair_pos"]).all()
    assert (disp.ready_wave.cpu().numpy() == meta["token_ready_wave"]).all()


def check_dispatch_valid(disp: moe.Dispatch, idx: np.ndarray, e_begin: int, E_local: int, G: int):
    """Properties of any correct dispatch of `idx` (used on GPU-made routings)."""
    counts = disp.counts.cpu().numpy()
    off = disp.offsets.cpu().numpy()
    pos = disp.pair_pos.cpu().numpy()
    st = disp.sorted_token.cpu().numpy()
    local = (idx >= e_begin) & (idx < e_begin + E_local)
    P = int(local.sum())
    assert counts.sum() == P and off[-1] == P and (np.diff(off) == counts).all()
    assert ((pos >= 0) == local).all()
    rows = np.sort(pos[local])
    assert (rows == np.arange(P)).all()
    ts, js = np.nonzero(local)
    assert (st[pos[ts, js]] == ts).all()
    for le in range(E_local):
        seg = st[off[le]:off[le + 1]]
        assert (np.diff(seg) > 0).all()
        assert (idx[seg] == e_begin + le).any(axis=1).all()
