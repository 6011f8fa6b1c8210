"""Thin Python binding of ``libmoe.so`` (include/moe.h).

Argument marshalling only: every step of the layer runs in the library's
HIP kernels.  PyTorch provides device memory (tensor storage) and the
current HIP stream.  The library must be built (``build_lib.build()``); if it
is missing, loading fails loudly -- there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4
MOE_ERR_TIMEOUT = -5
MOE_F32 = 0
MOE_BF16 = 1
MOE_FLAG_SERIAL = 0x1
MOE_FLAG_PERSISTENT = 0x2
MOE_ACT_SWIGLU = 0
MOE_ACT_RELU2 = 1
MOE_WS_BACKWARD = 0x1
MOE_PATH_PERSISTENT = 0
MOE_PATH_PHASES = 1

EXPORTED = (
    "moe_packed_weights_size", "moe_workspace_size", "moe_pack_weights", "moe_route",
    "moe_dispatch", "moe_expert_ffn_waved", "moe_combine", "moe_expert_wgrad",
    "moe_packed_bwd_size", "moe_pack_weights_bwd", "moe_backward", "moe_quantize_fp8",
    "moe_expert_ffn_waved_fp8", "moe_ffn_path", "moe_route_noalloc", "moe_route_dispatch", "moe_probe_mfma",
    "moe_probe_copy", "moe_expert_ffn_waved_save_h", "moe_backward_saved_h", "moe_saved_h_bytes",
    "moe_check_error", "moe_status_string", "moe_version",
)


class Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "T", "d", "I", "E_global", "k", "e_begin", "E_local", "experts_per_wave",
        "x_dtype", "w_dtype", "out_dtype", "activation")]

    def replace(self, **kw) -> "Problem":
        q = Problem()
        for n, _ in self._fields_:
            setattr(q, n, kw.get(n, getattr(self, n)))
        return q

    def as_dict(self) -> dict:
        return {n: getattr(self, n) for n, _ in self._fields_}


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"HIP library not built: {_LIB_PATH} is missing "
                               "(run combine_wave_level_amd.build_lib.build())")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32p, f32p = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
        P = ctypes.POINTER(Problem)
        st = ctypes.c_int
        sig = {
            "moe_packed_weights_size": (ctypes.c_size_t, [P]),
            "moe_workspace_size": (ctypes.c_size_t, [P, ctypes.c_uint32]),
            "moe_ffn_path": (ctypes.c_int32, [P, ctypes.c_int32, ctypes.c_uint32]),
            "moe_pack_weights": (st, [P, vp, vp, vp, vp, vp, vp]),
            "moe_route": (st, [P, vp, vp, f32p, i32p, f32p, f32p, vp, ctypes.c_size_t, vp]),
            "moe_route_noalloc": (st, [P, vp, vp, f32p, i32p, f32p, f32p, vp]),
            "moe_dispatch": (st, [P, i32p, i32p, i32p, i32p, i32p, i32p, vp, ctypes.c_size_t, vp]),
            "moe_route_dispatch": (st, [P, vp, vp, f32p, i32p, f32p, f32p, i32p, i32p, i32p, i32p, i32p, vp,
                                        ctypes.c_size_t, vp]),
            "moe_expert_ffn_waved": (st, [P, vp, vp, i32p, i32p, i32p, f32p, i32p, vp, vp,
                                          ctypes.c_uint32, vp, ctypes.c_size_t, vp]),
            "moe_expert_ffn_waved_save_h": (st, [P, vp, vp, i32p, i32p, i32p, f32p, i32p, vp, vp, f32p,
                                                 ctypes.c_uint32, vp, ctypes.c_size_t, vp]),
            "moe_combine": (st, [P, vp, i32p, f32p, vp, vp]),
            "moe_expert_wgrad": (st, [P, vp, vp, vp, i32p, i32p, i32p, f32p, vp, f32p, f32p, f32p,
                                      vp, ctypes.c_size_t, vp]),
            "moe_packed_bwd_size": (ctypes.c_size_t, [P]),
            "moe_saved_h_bytes": (ctypes.c_size_t, [P]),
            "moe_pack_weights_bwd": (st, [P, vp, vp, vp, vp, vp, vp]),
            "moe_backward": (st, [P, vp, vp, vp, i32p, f32p, i32p, i32p, i32p, vp, vp, f32p, f32p, f32p,
                                  f32p, f32p, f32p, vp, ctypes.c_size_t, vp]),
            "moe_backward_saved_h": (st, [P, vp, vp, vp, i32p, f32p, i32p, i32p, i32p, vp, f32p, vp, f32p, f32p,
                                          f32p, f32p, f32p, f32p, vp, ctypes.c_size_t, vp]),
            "moe_quantize_fp8": (st, [P, vp, vp, f32p, vp]),
            "moe_expert_ffn_waved_fp8": (st, [P, vp, f32p, vp, i32p, i32p, i32p, f32p, i32p, vp, vp,
                                              ctypes.c_uint32, vp, ctypes.c_size_t, vp]),
            "moe_probe_mfma": (st, [f32p, ctypes.c_size_t, ctypes.c_int32, ctypes.POINTER(ctypes.c_double), vp]),
            "moe_probe_copy": (st, [vp, vp, ctypes.c_size_t, vp]),
            "moe_check_error": (st, [vp, vp]),
            "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "moe_version": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().moe_status_string(int(s)).decode()


def _check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoEError(status, where)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def problem(T, d, I, E_global, k, e_begin=0, E_local=None, experts_per_wave=4,
            x_dtype=MOE_BF16, w_dtype=MOE_BF16, out_dtype=MOE_BF16,
            activation=MOE_ACT_SWIGLU) -> Problem:
    E_local = E_global if E_local is None else E_local
    return Problem(T, d, I, E_global, k, e_begin, E_local, experts_per_wave,
                   x_dtype, w_dtype, out_dtype, activation)


def workspace_size(p: Problem, backward: bool = False) -> int:
    """Workspace bytes: the forward entry points' size, or with backward=True
    the size every entry point (moe_expert_wgrad, moe_backward) needs."""
    return int(lib().moe_workspace_size(ctypes.byref(p), MOE_WS_BACKWARD if backward else 0))


def _ffn_flags(serial: bool, persistent: bool) -> int:
    return (MOE_FLAG_SERIAL if serial else 0) | (MOE_FLAG_PERSISTENT if persistent else 0)


def ffn_path(p: Problem, num_cus: int, serial: bool = False, persistent: bool = False) -> int:
    """MOE_PATH_PERSISTENT or MOE_PATH_PHASES: the schedule the expert FFN
    runs on a device with num_cus compute units (serial / persistent: the
    flags MOE_FLAG_SERIAL / MOE_FLAG_PERSISTENT)."""
    r = int(lib().moe_ffn_path(ctypes.byref(p), int(num_cus), _ffn_flags(serial, persistent)))
    if r < 0:
        raise MoEError(r, "moe_ffn_path")
    return r


def packed_weights_size(p: Problem) -> int:
    return int(lib().moe_packed_weights_size(ctypes.byref(p)))


def workspace(p: Problem, device="cuda", backward: bool = False) -> torch.Tensor:
    n = workspace_size(p, backward)
    if n == 0:
        raise MoEError(MOE_ERR_INVALID_ARG, "workspace_size")
    # zero-filled once, so the device error word starts clean
    return torch.zeros(n, dtype=torch.uint8, device=device)


def pack_weights(p: Problem, Wg, W1, W3, W2) -> torch.Tensor:
    n = packed_weights_size(p)
    if n == 0:
        raise MoEError(MOE_ERR_INVALID_ARG, "packed_weights_size")
    packed = torch.empty(n, dtype=torch.uint8, device=W1.device)
    _check(lib().moe_pack_weights(ctypes.byref(p), _p(Wg), _p(W1), _p(W3), _p(W2), _p(packed),
                                  _stream()), "moe_pack_weights")
    return packed


def route(p: Problem, x, packed, ws, bias=None, want_logits=False):
    dev = x.device
    idx = torch.empty((p.T, p.k), dtype=torch.int32, device=dev)
    w = torch.empty((p.T, p.k), dtype=torch.float32, device=dev)
    logits = torch.empty((p.T, p.E_global), dtype=torch.float32, device=dev) if want_logits else None
    _check(lib().moe_route(ctypes.byref(p), _p(x), _p(packed), _p(bias), _p(idx), _p(w), _p(logits),
                           _p(ws), ws.numel(), _stream()), "moe_route")
    return idx, w, logits


ROUTE_NOALLOC_MAX_BYTES = 16 << 20


def route_noalloc(p: Problem, x, packed, bias=None, want_logits=False, out=None):
    """moe_route_noalloc: the router without a workspace (its scratch is the
    library's fixed per-GPU array).  out: optional (idx, w, logits) tensors
    to write into, so that the call itself allocates nothing."""
    dev = x.device
    if out is None:
        idx = torch.empty((p.T, p.k), dtype=torch.int32, device=dev)
        w = torch.empty((p.T, p.k), dtype=torch.float32, device=dev)
        logits = torch.empty((p.T, p.E_global), dtype=torch.float32, device=dev) if want_logits else None
    else:
        idx, w, logits = out
    _check(lib().moe_route_noalloc(ctypes.byref(p), _p(x), _p(packed), _p(bias), _p(idx), _p(w), _p(logits),
                                   _stream()), "moe_route_noalloc")
    return idx, w, logits


@dataclass
class Dispatch:
    counts: torch.Tensor
    offsets: torch.Tensor
    sorted_token: torch.Tensor
    pair_pos: torch.Tensor
    ready_wave: torch.Tensor


def p_max(p: Problem) -> int:
    return p.T * min(p.k, p.E_local)


def dispatch(p: Problem, topk_idx, ws) -> Dispatch:
    dev = topk_idx.device
    d = Dispatch(
        counts=torch.empty(p.E_local, dtype=torch.int32, device=dev),
        offsets=torch.empty(p.E_local + 1, dtype=torch.int32, device=dev),
        sorted_token=torch.empty(max(1, p_max(p)), dtype=torch.int32, device=dev),
        pair_pos=torch.empty((p.T, p.k), dtype=torch.int32, device=dev),
        ready_wave=torch.empty(p.T, dtype=torch.int32, device=dev),
    )
    _check(lib().moe_dispatch(ctypes.byref(p), _p(topk_idx), _p(d.counts), _p(d.offsets),
                              _p(d.sorted_token), _p(d.pair_pos), _p(d.ready_wave), _p(ws),
                              ws.numel(), _stream()), "moe_dispatch")
    return d


def route_dispatch(p: Problem, x, packed, ws, bias=None, want_logits=False):
    """moe_route then moe_dispatch in one call (the same bits; small batches
    select and dispatch in one kernel).  Returns (topk_idx, topk_w, logits,
    Dispatch)."""
    dev = x.device
    idx = torch.empty((p.T, p.k), dtype=torch.int32, device=dev)
    w = torch.empty((p.T, p.k), dtype=torch.float32, device=dev)
    logits = torch.empty((p.T, p.E_global), dtype=torch.float32, device=dev) if want_logits else None
    disp = Dispatch(
        counts=torch.empty(p.E_local, dtype=torch.int32, device=dev),
        offsets=torch.empty(p.E_local + 1, dtype=torch.int32, device=dev),
        sorted_token=torch.empty(max(1, p_max(p)), dtype=torch.int32, device=dev),
        pair_pos=torch.empty((p.T, p.k), dtype=torch.int32, device=dev),
        ready_wave=torch.empty(p.T, dtype=torch.int32, device=dev))
    _check(lib().moe_route_dispatch(
        ctypes.byref(p), _p(x), _p(packed), _p(bias), _p(idx), _p(w), _p(logits), _p(disp.counts),
        _p(disp.offsets), _p(disp.sorted_token), _p(disp.pair_pos), _p(disp.ready_wave), _p(ws), ws.numel(),
        _stream()), "moe_route_dispatch")
    return idx, w, logits, disp


def _out_dtype(p: Problem):
    return torch.bfloat16 if p.out_dtype == MOE_BF16 else torch.float32


def saved_h_shape(p: Problem):
    """Shape (padded rows, gr I) of the fp32 buffer of ffn_waved(save_h=...):
    moe_saved_h_bytes(p) bytes, in the library's block-fragment order (see
    moe_expert_ffn_waved_save_h in include/moe.h)."""
    gr = 2 if p.activation == MOE_ACT_SWIGLU else 1
    n = lib().moe_saved_h_bytes(ctypes.byref(p))
    if n == 0:
        raise MoEError(MOE_ERR_INVALID_ARG, "moe_saved_h_bytes")
    return (n // (4 * gr * p.I), gr * p.I)


def ffn_waved(p: Problem, x, packed, disp: Dispatch, topk_w, ws, fused_combine=True,
              serial=False, y=None, out=None, persistent=False, save_h=None):
    """save_h: an fp32 tensor of saved_h_shape(p) that receives the GEMM1
    pre-activations (moe_expert_ffn_waved_save_h), for backward(saved_h=...)."""
    dev = x.device
    if y is None:
        y = torch.empty((max(1, p_max(p)), p.d), dtype=torch.bfloat16, device=dev)
    if fused_combine and out is None:
        out = torch.empty((p.T, p.d), dtype=_out_dtype(p), device=dev)
    flags = _ffn_flags(serial, persistent)
    args = (ctypes.byref(p), _p(x), _p(packed), _p(disp.offsets), _p(disp.sorted_token),
            _p(disp.pair_pos), _p(topk_w), _p(disp.ready_wave), _p(y), _p(out) if fused_combine else None)
    if save_h is None:
        _check(lib().moe_expert_ffn_waved(*args, flags, _p(ws), ws.numel(), _stream()), "moe_expert_ffn_waved")
    else:
        if tuple(save_h.shape) != saved_h_shape(p) or save_h.dtype != torch.float32:
            raise ValueError(f"save_h must be float32 of shape {saved_h_shape(p)}")
        _check(lib().moe_expert_ffn_waved_save_h(*args, _p(save_h), flags, _p(ws), ws.numel(), _stream()),
               "moe_expert_ffn_waved_save_h")
    return y, (out if fused_combine else None)


def quantize_fp8(p: Problem, x):
    """Per-token e4m3 codes (uint8 [T, d]) and power-of-two scales (fp32 [T]) of x."""
    x8 = torch.empty((p.T, p.d), dtype=torch.uint8, device=x.device)
    scale = torch.empty(p.T, dtype=torch.float32, device=x.device)
    _check(lib().moe_quantize_fp8(ctypes.byref(p), _p(x), _p(x8), _p(scale), _stream()), "moe_quantize_fp8")
    return x8, scale


def ffn_waved_fp8(p: Problem, x8, x_scale, packed, disp: Dispatch, topk_w, ws, fused_combine=True,
                  serial=False, y=None, out=None, persistent=False):
    """moe_expert_ffn_waved with the staging buffer in FP8 (from quantize_fp8)."""
    dev = x8.device
    if y is None:
        y = torch.empty((max(1, p_max(p)), p.d), dtype=torch.bfloat16, device=dev)
    if fused_combine and out is None:
        out = torch.empty((p.T, p.d), dtype=_out_dtype(p), device=dev)
    flags = _ffn_flags(serial, persistent)
    _check(lib().moe_expert_ffn_waved_fp8(
        ctypes.byref(p), _p(x8), _p(x_scale), _p(packed), _p(disp.offsets), _p(disp.sorted_token),
        _p(disp.pair_pos), _p(topk_w), _p(disp.ready_wave), _p(y), _p(out) if fused_combine else None,
        flags, _p(ws), ws.numel(), _stream()), "moe_expert_ffn_waved_fp8")
    return y, (out if fused_combine else None)


def combine(p: Problem, y, pair_pos, topk_w, out=None):
    if out is None:
        out = torch.empty((p.T, p.d), dtype=_out_dtype(p), device=y.device)
    _check(lib().moe_combine(ctypes.byref(p), _p(y), _p(pair_pos), _p(topk_w), _p(out), _stream()),
           "moe_combine")
    return out


def wgrad(p: Problem, x, packed, packed_bwd, disp: Dispatch, topk_w, dout, ws):
    """dW1, dW3, dW2 (dW3 None for the ungated activation)."""
    dev = x.device
    shp13 = (p.E_local, p.d, p.I)
    dW1 = torch.empty(shp13, dtype=torch.float32, device=dev)
    dW3 = torch.empty(shp13, dtype=torch.float32, device=dev) if p.activation == MOE_ACT_SWIGLU else None
    dW2 = torch.empty((p.E_local, p.I, p.d), dtype=torch.float32, device=dev)
    _check(lib().moe_expert_wgrad(
        ctypes.byref(p), _p(x), _p(packed), _p(packed_bwd), _p(disp.offsets), _p(disp.sorted_token),
        _p(disp.pair_pos), _p(topk_w), _p(dout), _p(dW1), _p(dW3), _p(dW2), _p(ws), ws.numel(),
        _stream()), "moe_expert_wgrad")
    return dW1, dW3, dW2


def packed_bwd_size(p: Problem) -> int:
    return int(lib().moe_packed_bwd_size(ctypes.byref(p)))


def pack_weights_bwd(p: Problem, Wg, W1, W3, W2) -> torch.Tensor:
    n = packed_bwd_size(p)
    if n == 0:
        raise MoEError(MOE_ERR_INVALID_ARG, "packed_bwd_size")
    packed = torch.empty(n, dtype=torch.uint8, device=W1.device)
    _check(lib().moe_pack_weights_bwd(ctypes.byref(p), _p(Wg), _p(W1), _p(W3), _p(W2), _p(packed),
                                      _stream()), "moe_pack_weights_bwd")
    return packed


def backward(p: Problem, x, packed, packed_bwd, topk_idx, topk_w, disp: Dispatch, dout, ws,
             want_dtopk_w=True, want_dlogits=False, want_dwg=True, want_dw=False, saved_h=None):
    """Data gradient dx (always) and, on request, dtopk_w, dlogits, dWg and the
    expert weight gradient, in one call.  saved_h: the pre-activations a
    ffn_waved(save_h=...) call kept (moe_backward_saved_h: no recompute)."""
    dev = x.device
    f32 = torch.float32
    dx = torch.empty((p.T, p.d), dtype=x.dtype, device=dev)
    dtw = torch.empty((p.T, p.k), dtype=f32, device=dev) if want_dtopk_w else None
    dlg = torch.empty((p.T, p.E_global), dtype=f32, device=dev) if want_dlogits else None
    dwg = torch.empty((p.d, p.E_global), dtype=f32, device=dev) if want_dwg else None
    dW1 = dW3 = dW2 = None
    if want_dw:
        dW1 = torch.empty((p.E_local, p.d, p.I), dtype=f32, device=dev)
        if p.activation == MOE_ACT_SWIGLU:
            dW3 = torch.empty((p.E_local, p.d, p.I), dtype=f32, device=dev)
        dW2 = torch.empty((p.E_local, p.I, p.d), dtype=f32, device=dev)
    head = (ctypes.byref(p), _p(x), _p(packed), _p(packed_bwd), _p(topk_idx), _p(topk_w), _p(disp.offsets),
            _p(disp.sorted_token), _p(disp.pair_pos), _p(dout))
    tail = (_p(dx), _p(dtw), _p(dlg), _p(dwg), _p(dW1), _p(dW3), _p(dW2), _p(ws), ws.numel(), _stream())
    if saved_h is None:
        _check(lib().moe_backward(*head, *tail), "moe_backward")
    else:
        if tuple(saved_h.shape) != saved_h_shape(p) or saved_h.dtype != torch.float32:
            raise ValueError(f"saved_h must be float32 of shape {saved_h_shape(p)}")
        _check(lib().moe_backward_saved_h(*head, _p(saved_h), *tail), "moe_backward_saved_h")
    return {"dx": dx, "dtopk_w": dtw, "dlogits": dlg, "dWg": dwg, "dW1": dW1, "dW3": dW3, "dW2": dW2}


def probe_mfma(steps: int, out=None):
    """One launch of the library's matrix-core loop on the current stream;
    returns (out, FLOPs of the launch).  Time it with events on that stream."""
    if out is None:
        cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
        out = torch.empty(cus * 512, dtype=torch.float32, device="cuda")
    flops = ctypes.c_double(0.0)
    _check(lib().moe_probe_mfma(_p(out), out.numel() * 4, int(steps), ctypes.byref(flops), _stream()),
           "moe_probe_mfma")
    return out, flops.value


def probe_copy(dst, src) -> None:
    """One launch of the library's plain copy (src -> dst, same byte size)."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise ValueError("dst smaller than src")
    _check(lib().moe_probe_copy(_p(dst), _p(src), n, _stream()), "moe_probe_copy")


def check_error(ws) -> None:
    _check(lib().moe_check_error(_p(ws), _stream()), "moe_check_error")


def forward(p: Problem, x, packed, ws, bias=None, serial=False, want_logits=False, persistent=False,
            save_h=None):
    """route -> dispatch (one call) -> waved expert FFN with fused combine
    (save_h: see ffn_waved)."""
    idx, w, logits, disp = route_dispatch(p, x, packed, ws, bias=bias, want_logits=want_logits)
    y, out = ffn_waved(p, x, packed, disp, w, ws, fused_combine=True, serial=serial, persistent=persistent,
                       save_h=save_h)
    return {"idx": idx, "w": w, "logits": logits, "disp": disp, "y": y, "out": out}
