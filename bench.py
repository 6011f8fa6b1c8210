"""Benchmark of one GPU's share of the expert-parallel MoE layer.

Default workload (the mid layer): T=4096 tokens, d=4096, I=1024, 16 experts,
top-4, 4 experts per wave, bf16 with fp32 accumulation; synthetic seeded
inputs (x ~ N(0,1), weights ~ N(0, 0.02)).  A step is one pass of the layer's
hot path over the batch: router, dispatch, and the expert FFN in waves (pull,
GEMM1 + SwiGLU, GEMM2, combine) on the library's default schedule (the
phase kernels; --serial and --persistent force the phase kernels or the
persistent expert-wave kernel), all inputs resident in HBM.  One JSON line
is printed on stdout.

    python bench.py [--steps K] [--warmup W] [--workload mid|v4share|decode|stress]
                    [--T T] [--no-cpu] [--serial | --persistent] [--no-backward]

The step is the forward (the metric's configuration is a forward).  The same
run also times the layer's backward on the same batch (data gradient,
combine-weight and logits gradients, dWg and the expert weight gradient, one
moe_backward call) and reports it under "extra.backward" (--no-backward
skips it), with the expert FFN that keeps the first GEMM's pre-activations
and the backward that reads them instead of recomputing under
"extra.backward.saved_h", and the forward with FP8 dispatch (per-token e4m3 staging, then
the expert FFN pulling it) under "extra.fp8_dispatch" (--no-fp8 skips it).

Only one GPU is used: --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s + grouped-GEMM TFLOP/s (% MFMA peak), 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="mid")
    ap.add_argument("--T", type=int, default=None)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--serial", action="store_true", help="time the phase-by-phase path")
    ap.add_argument("--persistent", action="store_true",
                    help="time the persistent expert-wave kernel wherever it fits")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-backward", action="store_true", help="skip timing the backward")
    ap.add_argument("--no-fp8", action="store_true", help="skip timing the FP8-dispatch forward")
    ap.add_argument("--no-ungated", action="store_true",
                    help="skip timing the layer with the ungated squared-ReLU expert")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the other workloads' rows (decode sweep, V3/V4-scale share, stress)")
    ap.add_argument("--ramp-ms", type=float, default=200.0,
                    help="untimed run of the layer before the warmup steps, in ms of wall time")
    return ap.parse_args()


def cpu_baseline(inp, wl, target_s):
    """The float64 oracle, as it stands, on a bounded sample of the same
    workload: the first n tokens of the batch through route, dispatch,
    expert FFN and combine; n grows until about target_s seconds."""
    import numpy as np

    import oracle

    def f64(a):
        return oracle.decode_bf16(a) if a.dtype == np.uint16 else a.astype(np.float64)

    x, Wg, W1, W3, W2 = (f64(inp[n]) for n in ("x", "Wg", "W1", "W3", "W2"))
    bias = inp.get("bias")
    n, spent, done = 32, 0.0, 0
    while True:
        n = min(n, x.shape[0])
        t0 = time.perf_counter()
        oracle.forward(x[:n], Wg, bias, W1, W3, W2, wl.k, wl.e_begin, wl.E_local, wl.G)
        dt = time.perf_counter() - t0
        spent += dt
        done = n
        if spent >= target_s or n == x.shape[0]:
            break
        n = int(min(x.shape[0], max(2 * n, n * (target_s - spent) / max(dt, 1e-3))))
    # when the whole batch takes less than the budget, repeat it and report
    # the mean over the repetitions
    reps, total = 1, dt
    while n == x.shape[0] and spent < target_s:
        t0 = time.perf_counter()
        oracle.forward(x[:n], Wg, bias, W1, W3, W2, wl.k, wl.e_begin, wl.E_local, wl.G)
        d1 = time.perf_counter() - t0
        spent += d1
        total += d1
        reps += 1
    dt = total / reps
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # noqa: BLE001
        cores = os.cpu_count()
    return {"value": done / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {done} tokens of the {wl.name} batch, float64 numpy oracle "
                      f"(route, dispatch, expert FFN, combine), {dt:.2f} s per run, mean of {reps}"}


def time_fp8_dispatch(args, p, x, bias, packed, idx, w, disp, ws, stream, out, y, L, P, check, pp, sp, nws, T):
    """Times the forward with FP8 dispatch: router, dispatch, the per-token
    e4m3 quantization of x and the expert-wave kernel pulling it."""
    import torch

    from combine_wave_level_amd import moe

    x8 = torch.empty((p.T, p.d), dtype=torch.uint8, device=x.device)
    sc = torch.empty(p.T, dtype=torch.float32, device=x.device)

    def step():
        check(L.moe_route_dispatch(pp, P(x), P(packed), P(bias), P(idx), P(w), None, P(disp.counts),
                                   P(disp.offsets), P(disp.sorted_token), P(disp.pair_pos), P(disp.ready_wave),
                                   P(ws), nws, sp), "route_dispatch")
        check(L.moe_quantize_fp8(pp, P(x), P(x8), P(sc), sp), "quantize")
        check(L.moe_expert_ffn_waved_fp8(pp, P(x8), P(sc), P(packed), P(disp.offsets), P(disp.sorted_token),
                                         P(disp.pair_pos), P(w), P(disp.ready_wave), P(y), P(out), 0,
                                         P(ws), nws, sp), "ffn_fp8")

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    n = max(3, args.steps)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(n):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    moe.check_error(ws)
    ms = t0.elapsed_time(t1) / n
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
            "pulled_bytes_per_pair": p.d, "pulled_bytes_per_pair_bf16": 2 * p.d}


def time_ungated(args, wl, T, d, stream):
    """Times the forward of the same layer with the ungated squared-ReLU
    expert at about the same parameter count (intermediate size 3I/2):
    router, dispatch and the expert-wave kernel on its own buffers."""
    import torch

    from combine_wave_level_amd import moe
    from workloads import make_inputs, ungated

    uw = ungated(wl)
    inp = make_inputs(uw, T=T, need_dout=not args.no_backward)
    xdt = moe.MOE_F32 if uw.dtype == "f32" else moe.MOE_BF16
    p = moe.problem(T=T, d=uw.d, I=uw.I, E_global=uw.E_global, k=uw.k, e_begin=uw.e_begin,
                    E_local=uw.E_local, experts_per_wave=uw.G, x_dtype=xdt, w_dtype=xdt, out_dtype=xdt,
                    activation=moe.MOE_ACT_RELU2)
    x = d(inp["x"])
    bias = d(inp["bias"]) if inp.get("bias") is not None else None
    packed = moe.pack_weights(p, d(inp["Wg"]), d(inp["W1"]), None, d(inp["W2"]))
    packed_bwd = None if args.no_backward else moe.pack_weights_bwd(p, d(inp["Wg"]), d(inp["W1"]), None,
                                                                    d(inp["W2"]))
    dout = None if args.no_backward else d(inp["dout"])
    ws = moe.workspace(p)
    del inp
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    y = torch.empty((max(1, moe.p_max(p)), p.d), dtype=torch.bfloat16, device=x.device)
    out = torch.empty((T, p.d), dtype=x.dtype, device=x.device)

    def step(timed_ffn=False):
        idx, w, _, disp = moe.route_dispatch(p, x, packed, ws, bias=bias)
        if timed_ffn:
            ev[2].record(stream)
        moe.ffn_waved(p, x, packed, disp, w, ws, y=y, out=out)
        if timed_ffn:
            ev[3].record(stream)
        return disp

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    n = max(3, args.steps)
    ffn = 0.0
    ev[0].record(stream)
    for _ in range(n):
        step()
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / n
    for _ in range(n):
        disp = step(timed_ffn=True)
        torch.cuda.synchronize()
        ffn += ev[2].elapsed_time(ev[3])
    moe.check_error(ws)
    ffn /= n
    P_local = int(disp.offsets[-1].item())
    tflops = 4.0 * uw.d * uw.I * P_local / (ffn * 1e-3) / 1e12
    res = {"activation": "relu2", "I": uw.I, "ms_per_step": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
           "ffn_ms": round(ffn, 4), "grouped_gemm_tflops": round(tflops, 2),
           "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4)}
    if packed_bwd is not None:
        # its backward (dx, dtopk_w, dWg, dW1, dW2) on the last step's routing,
        # on a backward-sized workspace
        wsb = moe.workspace(p, backward=True)
        idx, w_, _ = moe.route(p, x, packed, wsb, bias=bias)
        dispb = moe.dispatch(p, idx, wsb)

        def run():
            return moe.backward(p, x, packed, packed_bwd, idx, w_, dispb, dout, wsb, want_dtopk_w=True,
                                want_dlogits=False, want_dwg=True, want_dw=True)

        for _ in range(max(1, args.warmup // 10)):
            run()
        torch.cuda.synchronize()
        nb = max(3, args.steps // 2)
        ev[0].record(stream)
        for _ in range(nb):
            run()
        ev[1].record(stream)
        torch.cuda.synchronize()
        moe.check_error(wsb)
        bms = ev[0].elapsed_time(ev[1]) / nb
        P_b = int(dispb.offsets[-1].item())
        # recompute h1 (2 d I') + dA (2 d I') + dx rows (2 d I') + dW (4 d I') per
        # routed pair, plus the dense dWg product (2 d E per token)
        bfl = 10.0 * uw.d * uw.I * P_b + 2.0 * T * uw.d * uw.E_global
        res["backward"] = {"ms": round(bms, 4), "tflops": round(bfl / (bms * 1e-3) / 1e12, 2),
                           "mfma_frac": round(bfl / (bms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    return res


def time_backward(args, wl, T, p, inp, d, x, packed, idx, w, disp, stream, P_local):
    """Times moe_backward (all outputs) on the forward's routing, on a
    workspace of the backward size; returns the figures reported under
    extra.backward."""
    import torch

    from combine_wave_level_amd import moe

    packed_bwd = moe.pack_weights_bwd(p, d(inp["Wg"]), d(inp["W1"]), d(inp["W3"]), d(inp["W2"]))
    dout = d(inp["dout"])
    ws = moe.workspace(p, backward=True)
    disp = moe.dispatch(p, idx, ws)

    def run():
        return moe.backward(p, x, packed, packed_bwd, idx, w, disp, dout, ws, want_dtopk_w=True,
                            want_dlogits=False, want_dwg=True, want_dw=True)

    for _ in range(max(1, args.warmup)):
        run()
    torch.cuda.synchronize()
    n = max(3, args.steps // 2)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(n):
        run()
    t1.record(stream)
    torch.cuda.synchronize()
    moe.check_error(ws)
    ms = t0.elapsed_time(t1) / n
    # recompute of h1, h3 (4 d I) + dA (2 d I) + dx rows (4 d I) + dW (6 d I)
    # per routed pair, plus the dense dWg product (2 d E per token)
    flops = 16.0 * wl.d * wl.I * P_local + 2.0 * T * wl.d * wl.E_global
    tf = flops / (ms * 1e-3) / 1e12
    res = {"ms": round(ms, 4), "tflops": round(tf, 2), "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4),
           "flops_per_step": flops, "tokens_per_s": round(T / (ms * 1e-3), 1)}
    # the saved pre-activation path: the expert FFN that keeps h1 | h3
    # (fp32, P x 2I) and the backward that reads them instead of recomputing
    h = torch.empty(moe.saved_h_shape(p), dtype=torch.float32, device=x.device)

    def fwd_save():
        return moe.ffn_waved(p, x, packed, disp, w, ws, save_h=h)

    def bwd_saved():
        return moe.backward(p, x, packed, packed_bwd, idx, w, disp, dout, ws, want_dtopk_w=True,
                            want_dlogits=False, want_dwg=True, want_dw=True, saved_h=h)

    def timed(fn):
        for _ in range(max(1, args.warmup // 2)):
            fn()
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(n):
            fn()
        t1.record(stream)
        torch.cuda.synchronize()
        moe.check_error(ws)
        return t0.elapsed_time(t1) / n

    fms = timed(fwd_save)
    sms = timed(bwd_saved)
    sflops = flops - 4.0 * wl.d * wl.I * P_local
    stf = sflops / (sms * 1e-3) / 1e12
    res["saved_h"] = {"ffn_save_ms": round(fms, 4), "ms": round(sms, 4), "tflops": round(stf, 2),
                      "mfma_frac": round(stf / PEAK_BF16_TFLOPS, 4), "flops_per_step": sflops,
                      "tokens_per_s": round(T / (sms * 1e-3), 1),
                      "h_bytes": int(h.numel() * 4)}
    return res


MALL_FLUSH_BYTES = 512 << 20   # twice the MI355X's 256 MB last-level cache

# Other workloads, timed as rows of "extra.rows": the small-batch decode
# sweep and the V3/V4-scale share stream their experts' weights (HBM bound;
# the last-level cache is flushed before every timed step), the stress
# layer at T = 4096 is compute bound.
ROWS = (("decode", 1), ("decode", 8), ("decode", 32), ("decode", 128), ("v4share", 8192), ("stress", 4096))
STREAMING = ("decode", "v4share")


def roofline_of(d, I, T, counts):
    """Algorithmic work of the expert FFN for one batch: FLOPs 6 d I per
    routed pair; bytes = the touched experts' weights once + x read, y
    written and read, out written."""
    P_local = int(counts.sum())
    flops = 6.0 * d * I * P_local
    nbytes = int((counts > 0).sum()) * 3.0 * d * I * 2 + 2.0 * d * (2 * T + 2 * P_local)
    mfma = flops / (PEAK_BF16_TFLOPS * 1e12) >= nbytes / (PEAK_HBM_GBS * 1e9)
    return flops, nbytes, mfma, P_local


def measure_peaks(stream):
    """The roofline denominators measured on this device with the library's
    probes: a matrix-core loop (bf16 16x16x32 MFMA on register operands, 8
    wavefronts per CU) and a plain 1 GiB device copy, each launched 10 times
    between one event pair on the launch stream after 3 untimed launches."""
    import torch

    from combine_wave_level_amd import moe

    def timed(fn, n=10):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e-3

    out, flops = moe.probe_mfma(4096)
    t_mfma = timed(lambda: moe.probe_mfma(4096, out))
    nbytes = 1 << 30
    src = torch.ones(nbytes, dtype=torch.uint8, device=out.device)
    dst = torch.empty_like(src)
    t_copy = timed(lambda: moe.probe_copy(dst, src))
    del src, dst
    return {"mfma_bf16_tflops": round(flops / t_mfma / 1e12, 1), "copy_gbs": round(2.0 * nbytes / t_copy / 1e9, 1),
            "mfma_probe": "8 wavefronts per CU, 16 independent 16x16x32 bf16 MFMAs per step, 4096 steps",
            "copy_probe": "1 GiB device to device, read + written bytes"}


def time_graph_step(step, stream, flush, out, n):
    """The row's whole step (route, dispatch, FFN) captured once in a HIP
    graph and replayed n times, each replay timed alone between events on
    the launch stream (after the cache flush when one is given); the replays'
    output must equal the eager step's bits."""
    import numpy as np
    import torch

    try:
        step()
        torch.cuda.synchronize()
        ref = out.clone()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):   # warm the capture stream
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize()
        ts = []
        for i in range(n):
            if flush is not None:
                flush.fill_(i & 0xff)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        if not torch.equal(out, ref):
            return {"graph_error": "replayed output differs from the eager step"}
        return {"step_ms_graph": round(float(np.median(ts)), 4)}
    except RuntimeError as exc:   # capture refused: reported, the eager figures stand
        return {"graph_error": str(exc)[:200]}


def time_rows(args, stream, peaks=None):
    """Each row: the workload's router, dispatch and expert FFN (on the
    schedule the library picks), timed per step between events (median of
    the steps), and the expert FFN call alone the same way; for the weight-streaming rows a
    512 MiB buffer is written before every timed step and call, outside the
    events.  The step is also captured in a HIP graph and its replays timed
    the same way (step_ms_graph).  The expert weights are drawn on the device (seeded, N(0, 0.02),
    bf16): only the routing depends on values, and x, Wg and the bias come
    from the workload generator."""
    import numpy as np
    import torch

    from combine_wave_level_amd import moe
    from workloads import get, make_inputs

    dev = torch.device("cuda:0")
    flush = torch.empty(MALL_FLUSH_BYTES, dtype=torch.uint8, device=dev)
    rows, weights = [], {}

    def d(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    for name, T in ROWS:
        wl = get(name)
        inp = make_inputs(wl, T=T, weights=False)
        p = moe.problem(T=T, d=wl.d, I=wl.I, E_global=wl.E_global, k=wl.k, e_begin=wl.e_begin,
                        E_local=wl.E_local, experts_per_wave=wl.G)
        if name not in weights:
            weights.clear()
            g = torch.Generator(device=dev)
            g.manual_seed(1000 + len(rows))
            W = [torch.empty(s, dtype=torch.bfloat16, device=dev) for s in
                 ((wl.E_local, wl.d, wl.I), (wl.E_local, wl.d, wl.I), (wl.E_local, wl.I, wl.d))]
            for w_ in W:
                for e in range(w_.shape[0]):
                    w_[e].copy_(torch.randn(w_.shape[1:], generator=g, device=dev) * 0.02)
            weights[name] = W
        W1, W3, W2 = weights[name]
        x = d(inp["x"])
        bias = d(inp["bias"]) if inp.get("bias") is not None else None
        packed = moe.pack_weights(p, d(inp["Wg"]), W1, W3, W2)
        ws = moe.workspace(p)
        y = torch.empty((max(1, moe.p_max(p)), wl.d), dtype=torch.bfloat16, device=dev)
        out = torch.empty((T, wl.d), dtype=torch.bfloat16, device=dev)
        cache = {}

        def step(ffn_only=False):
            if not ffn_only:
                idx, w, _, cache["disp"] = moe.route_dispatch(p, x, packed, ws, bias=bias)
                cache["w"] = w
            moe.ffn_waved(p, x, packed, cache["disp"], cache["w"], ws, y=y, out=out)

        for _ in range(max(10, args.warmup // 5)):
            step()
        torch.cuda.synchronize()
        stream_w = name in STREAMING
        res = {}
        for kind in ("step", "ffn"):
            ts = []
            for _ in range(max(10, args.steps)):
                if stream_w:
                    flush.fill_(len(ts) & 0xff)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                step(ffn_only=kind == "ffn")
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            res[kind] = float(np.median(ts))
        moe.check_error(ws)
        counts = cache["disp"].counts.cpu().numpy().astype(np.int64)
        graph = time_graph_step(step, stream, flush if stream_w else None, out, max(10, args.steps))
        moe.check_error(ws)
        flops, nbytes, mfma, P_local = roofline_of(wl.d, wl.I, T, counts)
        path = moe.ffn_path(p, torch.cuda.get_device_properties(dev).multi_processor_count)
        row = {"workload": name, "T": T, "ffn_path": "persistent" if path == moe.MOE_PATH_PERSISTENT else "phases",
               "step_ms": round(res["step"], 4), "ffn_ms": round(res["ffn"], 4),
               "tokens_per_s": round(T / (res["step"] * 1e-3), 1), "local_pairs": P_local,
               "experts_touched": int((counts > 0).sum()), "bound": "mfma" if mfma else "hbm",
               "mall_flushed": stream_w, **graph}
        for lvl, ms in (("ffn", res["ffn"]), ("step", res["step"])):
            row[f"{lvl}_hbm_frac"] = round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
            row[f"{lvl}_mfma_frac"] = round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
        if peaks:
            row["ffn_frac_of_measured_peak"] = round(
                (flops / (res["ffn"] * 1e-3) / 1e12 / peaks["mfma_bf16_tflops"]) if mfma
                else (nbytes / (res["ffn"] * 1e-3) / 1e9 / peaks["copy_gbs"]), 4)
        rows.append(row)
        del packed, ws, y, out, x
    return rows


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the layer; --gpus {args.gpus} is not supported "
              "(one process drives one MI355X; there are no collectives)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from combine_wave_level_amd import moe
    from workloads import get, make_inputs

    wl = get(args.workload)
    T = args.T if args.T is not None else wl.T
    inp = make_inputs(wl, T=T, need_dout=not args.no_backward)
    dev = torch.device("cuda:0")

    def d(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    xdt = moe.MOE_F32 if wl.dtype == "f32" else moe.MOE_BF16
    p = moe.problem(T=T, d=wl.d, I=wl.I, E_global=wl.E_global, k=wl.k, e_begin=wl.e_begin,
                    E_local=wl.E_local, experts_per_wave=wl.G, x_dtype=xdt, w_dtype=xdt, out_dtype=xdt)
    x = d(inp["x"])
    bias = d(inp["bias"]) if inp.get("bias") is not None else None
    packed = moe.pack_weights(p, d(inp["Wg"]), d(inp["W1"]), d(inp["W3"]), d(inp["W2"]))
    ws = moe.workspace(p)
    idx = torch.empty((T, wl.k), dtype=torch.int32, device=dev)
    w = torch.empty((T, wl.k), dtype=torch.float32, device=dev)
    disp = moe.Dispatch(
        counts=torch.empty(wl.E_local, dtype=torch.int32, device=dev),
        offsets=torch.empty(wl.E_local + 1, dtype=torch.int32, device=dev),
        sorted_token=torch.empty(max(1, moe.p_max(p)), dtype=torch.int32, device=dev),
        pair_pos=torch.empty((T, wl.k), dtype=torch.int32, device=dev),
        ready_wave=torch.empty(T, dtype=torch.int32, device=dev))
    y = torch.empty((max(1, moe.p_max(p)), wl.d), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, wl.d), dtype=torch.bfloat16 if xdt == moe.MOE_BF16 else torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    L = moe.lib()
    import ctypes
    pp = ctypes.byref(p)
    sp = ctypes.c_void_p(stream.cuda_stream)

    def P(t):
        return None if t is None else ctypes.c_void_p(t.data_ptr())

    def check(st, where):
        if st != moe.MOE_OK:
            raise moe.MoEError(st, where)

    nws = ws.numel()
    if args.serial and args.persistent:
        raise SystemExit("--serial and --persistent exclude each other")
    flags = moe.MOE_FLAG_SERIAL if args.serial else (moe.MOE_FLAG_PERSISTENT if args.persistent else 0)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    path = moe.ffn_path(p, cus, serial=args.serial, persistent=args.persistent)
    persistent_path = path == moe.MOE_PATH_PERSISTENT

    def step(ev=None, fl=flags):
        if ev is not None:
            ev[0].record(stream)
        check(L.moe_route_dispatch(pp, P(x), P(packed), P(bias), P(idx), P(w), None, P(disp.counts),
                                   P(disp.offsets), P(disp.sorted_token), P(disp.pair_pos), P(disp.ready_wave),
                                   P(ws), nws, sp), "route_dispatch")
        if ev is not None:
            ev[2].record(stream)
        check(L.moe_expert_ffn_waved(pp, P(x), P(packed), P(disp.offsets), P(disp.sorted_token),
                                     P(disp.pair_pos), P(w), P(disp.ready_wave), P(y), P(out), fl,
                                     P(ws), nws, sp), "ffn")
        if ev is not None:
            ev[3].record(stream)

    def timed(nsteps, fl):
        """Wall time of nsteps whole steps between one event pair on the
        launch stream: nothing else is recorded inside the region."""
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(nsteps):
            step(None, fl)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / nsteps

    def ffn_launches(nsteps, fl):
        """Average duration of the expert-FFN call (the dominant kernel),
        nsteps launches back to back on the last step's routing, between one
        event pair on the launch stream."""
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(nsteps):
            check(L.moe_expert_ffn_waved(pp, P(x), P(packed), P(disp.offsets), P(disp.sorted_token),
                                         P(disp.pair_pos), P(w), P(disp.ready_wave), P(y), P(out), fl,
                                         P(ws), nws, sp), "ffn")
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / nsteps

    def instrumented(nsteps, fl):
        """Per-step breakdown from a separate pass with events between the
        calls (the events themselves add to these steps)."""
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(nsteps)]
        torch.cuda.synchronize()
        for i in range(nsteps):
            step(evs[i], fl)
        torch.cuda.synchronize()
        per_step = sorted(e[0].elapsed_time(e[3]) for e in evs)
        return {"route_dispatch_ms": sum(e[0].elapsed_time(e[2]) for e in evs) / nsteps,
                "ffn_ms": sum(e[2].elapsed_time(e[3]) for e in evs) / nsteps,
                "step_ms_median": per_step[len(per_step) // 2], "step_ms_min": per_step[0],
                "step_ms_max": per_step[-1]}

    # the clocks ramp up over the first ~10 ms of launches: run the layer
    # untimed for --ramp-ms of wall time, then the W warmup steps
    torch.cuda.synchronize()
    r0 = time.perf_counter()
    while (time.perf_counter() - r0) * 1e3 < args.ramp_ms:
        for _ in range(8):
            step()
        torch.cuda.synchronize()
    for _ in range(max(0, args.warmup)):
        step()
    torch.cuda.synchronize()
    moe.check_error(ws)
    ms = timed(args.steps, flags)
    moe.check_error(ws)
    ffn_ms = ffn_launches(args.steps, flags)
    moe.check_error(ws)
    inst = {k: round(v, 4) for k, v in instrumented(args.steps, flags).items()}
    moe.check_error(ws)

    # host side of the C ABI (side metric): wall time to validate and enqueue
    # one step's three calls, ctypes marshalling included, and of a call that
    # validation rejects before any launch
    n_host = max(10, args.steps)
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    for _ in range(n_host):
        step()
    h1 = time.perf_counter()
    torch.cuda.synchronize()
    bad = ctypes.c_void_p(out.data_ptr() + 8)  # misaligned out: rejected by validation
    h2 = time.perf_counter()
    for _ in range(1000):
        L.moe_combine(pp, P(y), P(disp.pair_pos), P(w), bad, sp)
    h3 = time.perf_counter()
    host_us_per_call = (h1 - h0) / (2 * n_host) * 1e6
    host_us_rejected = (h3 - h2) / 1000 * 1e6

    counts = disp.counts.cpu().numpy().astype(np.int64)
    P_local = int(counts.sum())
    flops_ffn = 6.0 * wl.d * wl.I * P_local
    touched = int((counts > 0).sum())
    weight_bytes = touched * 3.0 * wl.d * wl.I * 2
    act_bytes = 2.0 * wl.d * (T + 2 * P_local + T)  # x read, y written and read, out written
    tflops = flops_ffn / (ffn_ms * 1e-3) / 1e12
    gbs = (weight_bytes + act_bytes) / (ffn_ms * 1e-3) / 1e9
    mfma_bound = flops_ffn / (PEAK_BF16_TFLOPS * 1e12) >= (weight_bytes + act_bytes) / (PEAK_HBM_GBS * 1e9)
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / PEAK_BF16_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4)}
    roof["kernel"] = ("ffn_waved_kernel" if persistent_path
                      else "gemm1_phase_kernel+gemm2_phase_kernel+combine_kernel")
    # HBM bytes per launch from the committed rocprofv3 counter runs
    # (FETCH_SIZE + WRITE_SIZE, calibrated by a plain copy; on the phase
    # schedule the sum over its three kernels), reported only while the
    # kernel sources are the ones that were measured
    from combine_wave_level_amd import profiling
    tname = "ffn_waved_kernel" if persistent_path else "phase_kernels"
    trec = profiling.load_traffic(os.path.join(ROOT, "profiles", f"traffic_{tname}_{wl.name}_T{T}.json"), wl.name, T)
    roof["traffic"] = trec["traffic_bytes"] if trec else None
    peaks = measure_peaks(stream)
    meas = peaks["mfma_bf16_tflops"] if roof["bound"] == "mfma" else peaks["copy_gbs"]
    roof["frac_of_measured_peak"] = round(roof["achieved"] / meas, 4)

    extra = {"measured_peaks": peaks,
             "ffn_path": "persistent" if persistent_path else "phases", "ffn_ms": round(ffn_ms, 4),
             "grouped_gemm_tflops": round(tflops, 2), "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
             "ffn_hbm_gbs_min_bytes": round(gbs, 1), "local_pairs": P_local, "experts_touched": touched,
             "host_us_per_abi_call": round(host_us_per_call, 2), "host_us_rejected_call": round(host_us_rejected, 2),
             "instrumented_pass": inst}
    if not args.serial and not args.persistent:
        # both schedules forced (same bits): the phase kernels, and the
        # persistent kernel wherever it fits
        n_s = max(3, args.steps // 4)
        extra["serial_ms_per_step"] = round(timed(n_s, moe.MOE_FLAG_SERIAL), 4)
        s_ffn = ffn_launches(n_s, moe.MOE_FLAG_SERIAL)
        extra["serial_ffn_ms"] = round(s_ffn, 4)
        if moe.ffn_path(p, cus, persistent=True) == moe.MOE_PATH_PERSISTENT:
            p_ffn = ffn_launches(n_s, moe.MOE_FLAG_PERSISTENT)
            extra["persistent_ffn_ms"] = round(p_ffn, 4)
            extra["overlap_speedup_ffn"] = round(s_ffn / p_ffn, 3)
        extra["speedup_vs_phases_ffn"] = round(s_ffn / ffn_ms, 3)

    if not args.no_fp8:
        extra["fp8_dispatch"] = time_fp8_dispatch(args, p, x, bias, packed, idx, w, disp, ws, stream, out, y, L,
                                                  P, check, pp, sp, nws, T)
    if not args.no_ungated:
        extra["relu2_same_params"] = time_ungated(args, wl, T, d, stream)
    if not args.no_backward:
        extra["backward"] = time_backward(args, wl, T, p, inp, d, x, packed, idx, w, disp, stream, P_local)
    if not args.no_rows:
        extra["rows"] = time_rows(args, stream, peaks)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(inp, wl, args.cpu_seconds)

    rec = {
        "metric": METRIC,
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if xdt == moe.MOE_BF16 else "f32",
        "data": "synthetic (seeded x ~ N(0,1), weights ~ N(0,0.02), random-init)",
        "config": {"workload": f"{wl.name}: T={T} d={wl.d} I={wl.I} experts {wl.E_local} local of "
                               f"{wl.E_global}, top-{wl.k}, {wl.G} experts per wave, "
                               f"{'persistent expert-wave kernel' if persistent_path else 'phase kernels'}",
                   "T": T, "d": wl.d, "I": wl.I, "E_global": wl.E_global, "E_local": wl.E_local,
                   "k": wl.k, "experts_per_wave": wl.G},
        "roofline": roof,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
