"""FP8 dispatch on the GPU, through the C ABI.

* The quantizer's codes and scales equal the float64 oracle's bit for bit
  (random rows of every workload's dtype, and crafted rows that hit rounding
  ties, the subnormal range, values that round to zero, -0 and all-zero rows).
* The expert FFN pulling the FP8 staging buffer equals, bit for bit, the bf16
  path run on the dequantized rows (which are exact in bf16), persistent and
  phase-by-phase, for every tile shape (tiny fp32 layer, small-batch decode
  shapes, the mid layer), and matches the oracle's layer on the dequantized
  rows within the 2e-2 row tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_wave_level_amd import moe
from helpers import OUT_TOL, Layer, dev, f64, host_f64, oracle_inputs, rel_err_rows
from workloads import bf16_bits, make_inputs

pytestmark = pytest.mark.gpu


def _quantize(L, x_np):
    x8, sc = moe.quantize_fp8(L.p, dev(x_np))
    torch.cuda.synchronize()
    return x8.cpu().numpy(), sc.cpu().numpy().astype(np.float64)


def _check_codes(L, x_np):
    codes, scale = _quantize(L, x_np)
    r_codes, r_scale, _ = oracle.quantize_fp8_per_token(f64(x_np))
    assert (scale == r_scale).all(), np.nonzero(scale != r_scale)
    bad = np.nonzero(codes != r_codes)
    assert bad[0].size == 0, (bad[0][:5], bad[1][:5], codes[bad][:5], r_codes[bad][:5])
    return codes, scale


@pytest.mark.parametrize("name,T", [("tiny", 64), ("mid", 301), ("decode", 32)])
def test_quantize_matches_oracle_on_workload_rows(name, T):
    inp = make_inputs(name, T=T)
    print(f"[case] fp8 quantize {name} T={T}", flush=True)
    _check_codes(Layer(inp), inp["x"])


def test_quantize_crafted_rounding_cases():
    inp = make_inputs("mid", T=7)
    L = Layer(inp)
    d = L.p.d
    rows = np.zeros((7, d), dtype=np.float32)
    rows[0, 0] = 448.0                                      # scale 1
    ties = [1 + 1 / 16, 1 + 3 / 16, 2.0 ** -10, 3 * 2.0 ** -10, 13 * 2.0 ** -10, 432.0, 200.0, 2.0 ** -7 * 1.0625]
    rows[0, 1:1 + len(ties)] = ties
    rows[0, 20:20 + len(ties)] = [-v for v in ties]
    rows[0, 40] = -2.0 ** -12                               # rounds to -0
    rows[1, :] = 0.0                                        # all zero: scale 1
    rows[2, :7] = [3.0e4, -1.0, 2.0 ** -20, 7.0, -3.0e4, 0.5, 1e-3]   # scale > 1
    rows[3, :5] = [1e-6, -3e-7, 2e-9, 0.0, 5e-7]            # scale < 1
    rows[4, :] = np.linspace(-2, 2, d, dtype=np.float32)
    rows[5, 0] = 448.0 * 2 ** 5 * (1 + 2.0 ** -7)           # just above a power-of-two boundary
    rows[5, 1:9] = np.float32(448.0 * 2 ** 5) / np.arange(1, 9, dtype=np.float32)
    # a row so small that 2^-k exceeds fp32's range (scale 2^-129): codes
    # 256, -96, 10, 1.5 and a tie at 34 that rounds to 32
    rows[6, :5] = [2.0 ** -121, -1.5 * 2.0 ** -123, 1.25 * 2.0 ** -126, 3 * 2.0 ** -130, 1.0625 * 2.0 ** -124]
    x = bf16_bits(rows)                                     # the values the layer receives
    # one bf16 step above four ties: they round up
    x[0, 41:45] = bf16_bits(np.array([2.0 ** -10, 1 + 1 / 16, 432.0, 3 * 2.0 ** -10], dtype=np.float32)) + 1
    print("[case] fp8 quantize crafted rows", flush=True)
    codes, scale = _check_codes(L, x)
    assert codes[0, 40] == 0x80 and scale[1] == 1.0 and (codes[1] == 0).all()
    assert scale[6] == 2.0 ** -129
    assert (oracle.e4m3_decode(codes[6, :5]) == [256.0, -96.0, 10.0, 1.5, 32.0]).all()


def _ffn_compare(inp, serial):
    wl = inp["workload"]
    L = Layer(inp)
    o = oracle_inputs(inp)
    codes, scale = _check_codes(L, inp["x"])
    x_deq = oracle.e4m3_decode(codes) * scale[:, None]      # exact in bf16 (and fp32)
    l64 = oracle.router_logits(o["x"], o["Wg"], o["bias"])
    idx_o, w_o, _ = oracle.route(l64, wl.k)
    idx_d = torch.from_numpy(idx_o.astype(np.int32)).cuda()
    w_d = torch.from_numpy(w_o.astype(np.float32)).cuda()
    disp = moe.dispatch(L.p, idx_d, L.ws)
    x8 = torch.from_numpy(codes).cuda()
    sc = torch.from_numpy(scale.astype(np.float32)).cuda()
    y8, out8 = moe.ffn_waved_fp8(L.p, x8, sc, L.packed, disp, w_d, L.ws, serial=serial, persistent=not serial)
    torch.cuda.synchronize()
    moe.check_error(L.ws)
    # the bf16 path on the dequantized rows
    xq = x_deq.astype(np.float32) if inp["x"].dtype == np.float32 else bf16_bits(x_deq.astype(np.float32))
    assert (f64(xq) == x_deq).all()
    yb, outb = moe.ffn_waved(L.p, dev(xq), L.packed, disp, w_d, L.ws, serial=serial, persistent=not serial)
    torch.cuda.synchronize()
    moe.check_error(L.ws)
    P = int(disp.offsets[-1].item())
    assert torch.equal(y8[:P], yb[:P]) and torch.equal(out8, outb)
    # and the oracle's layer on the dequantized rows
    w32 = w_d.cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(2)
    toks = np.arange(L.T) if L.T <= 64 else np.sort(rng.choice(L.T, 48, replace=False))
    ref = oracle.forward_tokens(x_deq[toks], idx_o[toks], w32[toks], o["W1"], o["W3"], o["W2"], wl.e_begin,
                                wl.E_local)
    err = rel_err_rows(host_f64(out8)[toks], ref)
    print(f"  out rel err vs oracle on dequantized rows {err:.3g}", flush=True)
    assert err <= OUT_TOL


@pytest.mark.parametrize("name,T", [("tiny", 64), ("decode", 1), ("decode", 8), ("decode", 128), ("mid", 1000)])
@pytest.mark.parametrize("serial", [False, True])
def test_fp8_ffn_equals_bf16_path_on_dequantized_rows(name, T, serial):
    print(f"[case] fp8 ffn {name} T={T} serial={serial}", flush=True)
    _ffn_compare(make_inputs(name, T=T), serial)
