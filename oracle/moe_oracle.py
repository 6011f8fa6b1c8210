"""Plain, slow, float64 CPU oracle for one GPU's share of a fine-grained
expert-parallel MoE layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
helper with the HIP library and imports nothing from it.

Sources (the method as the pages state it; each function cites its passage):

* [V4-TH]  "DeepSeek-V4 launch digest" (itsolotime.com, Thai translation of
  the DeepSeek-V4 report's infrastructure chapter): §1.1 (an MoE layer is
  dispatch, first linear, second linear, combine), §1.2 (experts are split
  into waves of a few experts each), §1.4 "compute/communication ratio"
  bullet (per token-expert pair the expert FFN is SwiGLU gating, up and down
  projection), §3 (batch-invariant, deterministic kernel library).
* [ZH-10100] 10100.com commentary on the report (sections "fine-grained
  compute/communication overlap of the EP all-to-all" and "high-performance
  batch-invariant and deterministic operators"): the three stages dispatch /
  Linear + activation + Linear / combine; determinism by pre-sorting,
  isolated buffers and a fixed-order final reduction.
* The tiny-layer workload definition that fixes the router and FFN formula:
  softmax over all experts, top-k, weights renormalised over the k picks,
  out = sum_k w_k * W2(silu(W1 x) * (W3 x)).

Readings where the pages are silent (each is also listed in the design
notes of this repository):

* top-k ties go to the lower expert id; rank order (descending probability)
  is also the combine order;
* inside one expert's segment, pairs are ordered by ascending token id
  (a stable counting sort: "pre-sorting");
* expert waves are consecutive local expert ids, ``G`` per wave, ascending;
* no capacity limit and no token dropping: every routed pair is processed
  exactly once;
* the oracle computes everything in float64 from the exact input values
  (bf16 inputs decoded exactly); it rounds no intermediate;
* FP8 dispatch (the "FP8 scatter" of [V4-TH] §1.4): the token rows the
  experts pull are OCP e4m3 values with one power-of-two scale per token,
  the smallest one that brings the row's largest magnitude to at most 448
  (the pages name neither the format details nor the scale granularity);
  e4m3 values times a power of two are exact in bf16, so the experts see
  exactly the dequantized rows; the router keeps the unquantized x;
* the backward holds the routing fixed: the top-k selection is piecewise
  constant in the logits, so gradients flow only through the k renormalised
  weights; on an expert-parallel share (some picks owned by other GPUs) the
  loss is <dout, out> of this GPU's partial output, whose gradient is this
  GPU's additive share of the full layer's gradient.

Every function here is pinned by ``tests/test_oracle_pins.py`` against
closed forms, library routines, brute force and finite differences.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "decode_bf16",
    "router_logits",
    "route",
    "dispatch",
    "expert_ffn",
    "combine",
    "forward",
    "forward_tokens",
    "wgrad",
    "backward",
    "backward_tokens",
    "e4m3_decode",
    "e4m3_encode",
    "quantize_fp8_per_token",
]


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of bf16 numbers given as their uint16 bit patterns.

    A bf16 number is the upper half of an IEEE-754 binary32 number, so the
    value is recovered exactly by placing the 16 bits in the high half of a
    32-bit word.
    """
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError("decode_bf16 expects uint16 bit patterns")
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def router_logits(x: np.ndarray, Wg: np.ndarray, bias: np.ndarray | None = None) -> np.ndarray:
    """Router scores l[t, e] = sum_i x[t, i] * Wg[i, e] (+ bias[e]), float64.

    The router is the gate of the tiny-layer workload definition ("softmax
    then top-k"); the pages name it only as the "MoE Routing" kernel of
    TileKernels ([V4-TH] §1.3).  ``bias`` is an additive per-expert logit
    offset (used to skew expert popularity in the small-batch workload).
    """
    x64 = np.asarray(x, dtype=np.float64)
    w64 = np.asarray(Wg, dtype=np.float64)
    l = x64 @ w64
    if bias is not None:
        l = l + np.asarray(bias, dtype=np.float64)[None, :]
    return l


def route(logits: np.ndarray, k: int):
    """Softmax over all experts, top-k, renormalise the k weights.

    Steps in the order the workload definition states them:
      1. p = softmax(l) over all E experts (the row max is subtracted first;
         this does not change p).
      2. rank experts by descending p, ties to the lower expert id; keep the
         first k -> idx[t, 0..k-1] in rank order.
      3. w[t, j] = p[t, idx[t, j]] / sum_j' p[t, idx[t, j']].

    Returns (idx int32 [T, k], w float64 [T, k], p float64 [T, E]).
    """
    l = np.asarray(logits, dtype=np.float64)
    T, E = l.shape
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    z = np.exp(l - l.max(axis=1, keepdims=True))
    p = z / z.sum(axis=1, keepdims=True)
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    ids = np.arange(E)
    for t in range(T):
        # lexsort sorts by the last key first: primary -p (descending p),
        # secondary expert id (ascending) for exact ties.
        order = np.lexsort((ids, -p[t]))
        sel = order[:k]
        idx[t] = sel
        w[t] = p[t, sel] / p[t, sel].sum()
    return idx, w, p


def dispatch(idx: np.ndarray, e_begin: int, E_local: int, G: int):
    """Deterministic permutation of routed pairs by local expert.

    [ZH-10100] "deterministic operators": pairs are pre-sorted so that no
    position is ever assigned by an unordered atomic.  Reading: local
    experts in ascending id; inside an expert, ascending token id.
    [V4-TH] §1.2: experts are grouped into waves of a few experts; reading:
    wave(e) = (e - e_begin) // G.

    Returns a dict with
      counts [E_local], offsets [E_local + 1] (exclusive scan),
      sorted_token [P] (row -> source token), sorted_slot [P] (row -> rank j),
      pair_pos [T, k] (pair -> row, -1 when the expert is not local),
      token_ready_wave [T] (last wave holding one of the token's local
      experts, -1 when it has none), wave_rows [W + 1] (first row of each
      wave, then P).
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    if E_local <= 0 or G <= 0 or E_local % G:
        raise ValueError("need E_local > 0 and E_local % G == 0")
    W = E_local // G
    counts = np.zeros(E_local, dtype=np.int64)
    sorted_token: list[np.ndarray] = []
    sorted_slot: list[np.ndarray] = []
    pair_pos = np.full((T, k), -1, dtype=np.int64)
    row = 0
    for le in range(E_local):
        # nonzero scans row-major, so the pairs of expert e come out in
        # ascending token order (a token picks an expert at most once).
        ts, js = np.nonzero(idx == e_begin + le)
        n = ts.size
        pair_pos[ts, js] = row + np.arange(n)
        sorted_token.append(ts)
        sorted_slot.append(js)
        counts[le] = n
        row += n
    offsets = np.zeros(E_local + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    ready = np.full(T, -1, dtype=np.int64)
    for j in range(k):
        le = idx[:, j].astype(np.int64) - e_begin
        local = (le >= 0) & (le < E_local)
        ready = np.where(local, np.maximum(ready, le // G), ready)
    wave_rows = np.array([offsets[w * G] for w in range(W)] + [offsets[E_local]], dtype=np.int64)
    return {
        "counts": counts,
        "offsets": offsets,
        "sorted_token": np.concatenate(sorted_token).astype(np.int64),
        "sorted_slot": np.concatenate(sorted_slot).astype(np.int64),
        "pair_pos": pair_pos,
        "token_ready_wave": ready,
        "wave_rows": wave_rows,
    }


def _silu(h: np.ndarray) -> np.ndarray:
    return h / (1.0 + np.exp(-h))


def expert_ffn(X: np.ndarray, W1e: np.ndarray, W3e: np.ndarray, W2e: np.ndarray, activation: str = "swiglu"):
    """One expert's FFN on the rows X [M, d], float64.

    [V4-TH] §1.4 (compute/communication bullet): each token-expert pair costs
    the gating, up and down projections.  With the workload formula:
      h1 = X W1, h3 = X W3, a = silu(h1) * h3, y = a W2,
    silu(h) = h / (1 + exp(-h)).
    activation "relu2": the cheap element-wise activation of [V4-TH] §1.4
    (activation-function bullet: no exponential, no division, no gating
    projection; the function is not named there, the reading is squared
    ReLU): a = max(h1, 0)^2, W3 unused (h3 is returned as None).
    Returns (y [M, d], h1, h3, a).
    """
    X = np.asarray(X, dtype=np.float64)
    h1 = X @ np.asarray(W1e, dtype=np.float64)
    if activation == "relu2":
        a = np.maximum(h1, 0.0) ** 2
        h3 = None
    elif activation == "swiglu":
        h3 = X @ np.asarray(W3e, dtype=np.float64)
        a = _silu(h1) * h3
    else:
        raise ValueError(f"unknown activation {activation!r}")
    y = a @ np.asarray(W2e, dtype=np.float64)
    return y, h1, h3, a


def combine(y_rows: np.ndarray, pair_pos: np.ndarray, w: np.ndarray, d: int) -> np.ndarray:
    """Router-weighted sum back to token order.

    [ZH-10100] and [V4-TH] §1.1: combine collects the expert outputs back to
    their tokens.  out[t] = sum over ranks j with a local expert of
    w[t, j] * y[pair_pos[t, j]]; tokens with no local pick get zeros.
    """
    T, k = pair_pos.shape
    out = np.zeros((T, d), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            r = pair_pos[t, j]
            if r >= 0:
                out[t] += w[t, j] * y_rows[r]
    return out


def forward(x, Wg, bias, W1, W3, W2, k, e_begin, E_local, G, x_ffn=None, activation="swiglu"):
    """Whole layer share: route -> dispatch -> expert FFN per expert -> combine.

    ``x`` feeds the router; ``x_ffn`` (default ``x``) feeds the experts.
    W1, W3 are [E_local, d, I] and W2 is [E_local, I, d] for the local
    experts e_begin .. e_begin + E_local - 1.

    The expert FFN runs expert by expert on the expert's sorted rows; the
    wave grouping changes the schedule, never the values, so the oracle
    evaluates experts in ascending order ([V4-TH] §1.2).
    """
    x_ffn = x if x_ffn is None else x_ffn
    xf = np.asarray(x_ffn, dtype=np.float64)
    T, d = xf.shape
    logits = router_logits(x, Wg, bias)
    idx, w, p = route(logits, k)
    meta = dispatch(idx, e_begin, E_local, G)
    P = int(meta["offsets"][-1])
    y = np.zeros((P, d), dtype=np.float64)
    off = meta["offsets"]
    for le in range(E_local):
        r0, r1 = int(off[le]), int(off[le + 1])
        if r1 > r0:
            rows = meta["sorted_token"][r0:r1]
            y[r0:r1] = expert_ffn(xf[rows], W1[le], None if W3 is None else W3[le], W2[le], activation)[0]
    out = combine(y, meta["pair_pos"], w, d)
    return {"logits": logits, "idx": idx, "w": w, "p": p, "meta": meta, "y": y, "out": out}


def forward_tokens(x_ffn_rows, idx_rows, w_rows, W1, W3, W2, e_begin, E_local, activation="swiglu"):
    """Layer output for a subset of tokens, one token at a time.

    out[t] depends only on token t's own row, its picks and its weights
    ([ZH-10100]: batch invariance is a property of the math), so a sample of
    tokens can be checked at any batch size without running the whole batch.
    ``x_ffn_rows`` [n, d], ``idx_rows`` [n, k], ``w_rows`` [n, k].
    """
    xs = np.asarray(x_ffn_rows, dtype=np.float64)
    n, d = xs.shape
    out = np.zeros((n, d), dtype=np.float64)
    for i in range(n):
        for j in range(idx_rows.shape[1]):
            le = int(idx_rows[i, j]) - e_begin
            if 0 <= le < E_local:
                y = expert_ffn(xs[i:i + 1], W1[le], None if W3 is None else W3[le], W2[le], activation)[0][0]
                out[i] += w_rows[i, j] * y
    return out


def wgrad(x_ffn, W1, W3, W2, meta, w, dout, experts=None, cols=None, activation="swiglu"):
    """Weight gradient of L = <dout, out> for the local experts, float64.

    For every routed row r = (t, j) of expert e (dy_r = w[t, j] * dout[t]):
      h1 = x_t W1_e, h3 = x_t W3_e, s = sigmoid(h1), a = h1 s h3,
      dA  = dy_r W2_e^T,
      dH3 = dA * h1 s,
      dH1 = dA * h3 * s (1 + h1 (1 - s)),
      dW2_e += a^T dy_r, dW1_e += x_t^T dH1, dW3_e += x_t^T dH3.
    activation "relu2" (a = max(h1, 0)^2, no W3): dH1 = dA * 2 max(h1, 0),
    dW3 is not formed (the dict stays empty).
    Determinism ([ZH-10100], [V4-TH] §3) is a property of the GPU reduction
    order; the oracle sums in float64 with matmuls.

    ``experts``: local expert ids to compute (default all); ``cols``: subset
    of intermediate columns i (default all).  Returns dicts keyed by local
    expert: dW1[e] [d, n_cols], dW3[e] [d, n_cols], dW2[e] [n_cols, d].
    """
    xf = np.asarray(x_ffn, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    E_local = W1.shape[0]
    I = W1.shape[2]
    experts = range(E_local) if experts is None else experts
    cols = np.arange(I) if cols is None else np.asarray(cols)
    off = meta["offsets"]
    dW1, dW3, dW2 = {}, {}, {}
    for le in experts:
        r0, r1 = int(off[le]), int(off[le + 1])
        toks = meta["sorted_token"][r0:r1]
        slots = meta["sorted_slot"][r0:r1]
        X = xf[toks]                                   # [M, d]
        dY = w[toks, slots][:, None] * dout[toks]      # [M, d]
        W1c = np.asarray(W1[le], dtype=np.float64)[:, cols]
        W2c = np.asarray(W2[le], dtype=np.float64)[cols, :]
        h1 = X @ W1c
        dA = dY @ W2c.T
        if activation == "relu2":
            r = np.maximum(h1, 0.0)
            a = r * r
            dH1 = dA * 2.0 * r
        else:
            W3c = np.asarray(W3[le], dtype=np.float64)[:, cols]
            h3 = X @ W3c
            s = 1.0 / (1.0 + np.exp(-h1))
            a = h1 * s * h3
            dH3 = dA * h1 * s
            dH1 = dA * h3 * s * (1.0 + h1 * (1.0 - s))
            dW3[le] = X.T @ dH3
        dW2[le] = a.T @ dY
        dW1[le] = X.T @ dH1
    return dW1, dW3, dW2


def _gate_backward(w: np.ndarray, dw: np.ndarray) -> np.ndarray:
    """Gradient of the k renormalised weights with respect to the picked
    logits.  w_j = exp(l_j) / sum_j' exp(l_j') over the picks (softmax then
    renormalisation, the workload definition), so
    dl_j = sum_m dw_m dw_m/dl_j = w_j (dw_j - sum_m w_m dw_m)."""
    s = (w * dw).sum(axis=1, keepdims=True)
    return w * (dw - s)


def backward(x, Wg, W1, W3, W2, idx, w, meta, dout, x_ffn=None, activation="swiglu"):
    """Data and router gradients of L = <dout, out>, float64.

    Chain rule through the layer of the workload definition ([V4-TH] §1.1
    and §1.4: route, dispatch, SwiGLU expert FFN, router-weighted combine),
    with the routing held fixed:
      per routed row r = (t, j) of local expert e:
        h1 = x_t W1_e, h3 = x_t W3_e, s = sigmoid(h1), a = h1 s h3, y = a W2_e,
        dw[t, j] = <dout_t, y>                       (combine: out += w y)
        dA  = w[t, j] dout_t W2_e^T,
        dH3 = dA h1 s,  dH1 = dA h3 s (1 + h1 (1 - s)),
        dx_ffn[t] += dH1 W1_e^T + dH3 W3_e^T;
      picks of non-local experts contribute nothing to out, so their dw is 0;
      per token: dl[t, idx_j] = w_j (dw_j - sum_m w_m dw_m), 0 off the picks;
      router (l = x Wg + b): dWg = x^T dl, dx_router = dl Wg^T;
      dx = dx_router + dx_ffn.
    activation "relu2" (a = max(h1, 0)^2, no W3): dH1 = dA * 2 max(h1, 0),
    dx_ffn[t] += dH1 W1_e^T (the derivative of max(h, 0)^2 is 0 at h = 0
    from both sides).
    ``x`` feeds the router and ``x_ffn`` (default ``x``) the experts; a cast
    between them passes the gradient through unchanged.  [ZH-10100]
    (deterministic operators): the GPU's fixed reduction orders are its own
    property; the oracle sums in float64 with matmuls.

    Returns a dict with dw [T, k], dl [T, E], dWg [d, E], dx_router,
    dx_ffn and dx [T, d].
    """
    xr = np.asarray(x, dtype=np.float64)
    xf = xr if x_ffn is None else np.asarray(x_ffn, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    Wg64 = np.asarray(Wg, dtype=np.float64)
    T, k = idx.shape
    d = xf.shape[1]
    E = Wg64.shape[1]
    dw = np.zeros((T, k), dtype=np.float64)
    dx_ffn = np.zeros((T, d), dtype=np.float64)
    off = meta["offsets"]
    for le in range(len(off) - 1):
        r0, r1 = int(off[le]), int(off[le + 1])
        if r1 == r0:
            continue
        toks = meta["sorted_token"][r0:r1]
        slots = meta["sorted_slot"][r0:r1]
        W1e = np.asarray(W1[le], dtype=np.float64)
        W2e = np.asarray(W2[le], dtype=np.float64)
        X = xf[toks]
        h1 = X @ W1e
        if activation == "relu2":
            r = np.maximum(h1, 0.0)
            a = r * r
        else:
            W3e = np.asarray(W3[le], dtype=np.float64)
            h3 = X @ W3e
            s = 1.0 / (1.0 + np.exp(-h1))
            a = h1 * s * h3
        y = a @ W2e
        dw[toks, slots] = (dout[toks] * y).sum(axis=1)
        dA = (w[toks, slots][:, None] * dout[toks]) @ W2e.T
        # a token picks an expert at most once: toks has no repeats here
        if activation == "relu2":
            dx_ffn[toks] += (dA * 2.0 * r) @ W1e.T
        else:
            dH3 = dA * h1 * s
            dH1 = dA * h3 * s * (1.0 + h1 * (1.0 - s))
            dx_ffn[toks] += dH1 @ W1e.T + dH3 @ W3e.T
    dl_picks = _gate_backward(np.asarray(w, dtype=np.float64), dw)
    dl = np.zeros((T, E), dtype=np.float64)
    rows = np.repeat(np.arange(T), k)
    dl[rows, np.asarray(idx).reshape(-1)] = dl_picks.reshape(-1)
    dWg = xr.T @ dl
    dx_router = dl @ Wg64.T
    return {"dw": dw, "dl": dl, "dWg": dWg, "dx_router": dx_router, "dx_ffn": dx_ffn,
            "dx": dx_router + dx_ffn}


def backward_tokens(x_rows, x_ffn_rows, idx_rows, w_rows, dout_rows, Wg, W1, W3, W2, e_begin, E_local,
                    activation="swiglu"):
    """dx, dw and the picked dl of a subset of tokens, one token at a time.

    A token's data gradient depends only on its own row, picks, weights and
    dout (the layer is token-local apart from the weights), so a sample of
    tokens can be checked at any batch size.  Same formulas as ``backward``.
    Returns (dx [n, d], dw [n, k], dl [n, k]) with dl in rank order.
    """
    xr = np.asarray(x_rows, dtype=np.float64)
    xf = np.asarray(x_ffn_rows, dtype=np.float64)
    dout = np.asarray(dout_rows, dtype=np.float64)
    w = np.asarray(w_rows, dtype=np.float64)
    Wg64 = np.asarray(Wg, dtype=np.float64)
    n, k = idx_rows.shape
    dx = np.zeros_like(xf)
    dw = np.zeros((n, k), dtype=np.float64)
    for i in range(n):
        for j in range(k):
            le = int(idx_rows[i, j]) - e_begin
            if not 0 <= le < E_local:
                continue
            W1e = np.asarray(W1[le], dtype=np.float64)
            W2e = np.asarray(W2[le], dtype=np.float64)
            h1 = xf[i] @ W1e
            dA = W2e @ (w[i, j] * dout[i])
            if activation == "relu2":
                r = np.maximum(h1, 0.0)
                dw[i, j] = dout[i] @ ((r * r) @ W2e)
                dx[i] += W1e @ (dA * 2.0 * r)
                continue
            W3e = np.asarray(W3[le], dtype=np.float64)
            h3 = xf[i] @ W3e
            s = 1.0 / (1.0 + np.exp(-h1))
            dw[i, j] = dout[i] @ ((h1 * s * h3) @ W2e)
            dx[i] += W1e @ (dA * h3 * s * (1.0 + h1 * (1.0 - s))) + W3e @ (dA * h1 * s)
    dl = _gate_backward(w, dw)
    for i in range(n):
        for j in range(k):
            dx[i] += dl[i, j] * Wg64[:, int(idx_rows[i, j])]
    return dx, dw, dl


# ---------------------------------------------------------------- FP8 dispatch

_E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of OCP FP8 E4M3 codes (uint8), float64.

    1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0
    holds subnormals m * 2^-9; S.1111.111 is NaN (there is no infinity), so
    the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code of float64 values with |v| <= 448, ties to the even
    code (the spacing is 2^-9 below 2^-6 and 2^(e-3) in the binade
    [2^e, 2^(e+1)); rounding up out of a binade lands on its next power of
    two, which is representable)."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(np.abs(v) > _E4M3_MAX) or np.any(np.isnan(v)):
        raise ValueError("e4m3_encode expects finite values with |v| <= 448")
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.where(a >= 2.0 ** -6, e, -6.0)          # subnormal range shares the 2^-9 spacing
    q = 2.0 ** (e - 3)
    n = a / q                                        # exact: a power-of-two division
    r = np.floor(n)
    frac = n - r
    r = r + ((frac > 0.5) | ((frac == 0.5) & (r % 2 == 1)))
    mag = r * q
    # encode mag (now exactly representable) back to bits
    codes = np.zeros(v.shape, dtype=np.int64)
    nz = mag > 0
    me = np.floor(np.log2(np.where(nz, mag, 1.0)))
    normal = nz & (me >= -6)
    sub = nz & ~normal
    codes = np.where(normal, ((me + 7).astype(np.int64) << 3) | ((mag / 2.0 ** me - 1.0) * 8).astype(np.int64), codes)
    codes = np.where(sub, (mag / 2.0 ** -9).astype(np.int64), codes)
    codes = np.where(np.signbit(v), codes | 0x80, codes)  # a negative value that rounds to zero is -0
    return codes.astype(np.uint8)


def quantize_fp8_per_token(x: np.ndarray):
    """Per-token FP8 copy of x [T, d] (float64 values): scale_t = 2^k_t with
    k_t the smallest integer for which max_i |x[t, i]| <= 448 * 2^k_t (scale
    1 for an all-zero row), codes = e4m3_encode(x[t] / scale_t).
    Returns (codes uint8 [T, d], scale float64 [T], dequantized float64 [T, d])."""
    x = np.asarray(x, dtype=np.float64)
    amax = np.abs(x).max(axis=1) if x.shape[1] else np.zeros(x.shape[0])
    k = np.zeros(x.shape[0], dtype=np.int64)
    for t in range(x.shape[0]):
        if amax[t] > 0:
            kk = int(np.ceil(np.log2(amax[t] / _E4M3_MAX)))
            # guard the floating log2 against an off-by-one at exact powers
            while amax[t] > _E4M3_MAX * 2.0 ** kk:
                kk += 1
            while amax[t] <= _E4M3_MAX * 2.0 ** (kk - 1):
                kk -= 1
            k[t] = kk
    scale = np.exp2(k.astype(np.float64))
    codes = e4m3_encode(x / scale[:, None])
    deq = e4m3_decode(codes) * scale[:, None]
    return codes, scale, deq
