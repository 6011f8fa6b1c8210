"""The C-ABI library on the CPU: it loads, exports every symbol include/moe.h
declares, sizes buffers, and rejects bad arguments before any HIP call.

No compute entry point is called with arguments that pass validation here:
on a machine without a GPU only the host-side checks run.
"""
import ctypes
import os
import re

import pytest

from combine_wave_level_amd import moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: validation fails first


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    return moe.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert set(names) == set(moe.EXPORTED), names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version(L):
    assert moe.status_string(0) == "ok"
    assert "workspace" in moe.status_string(moe.MOE_ERR_WORKSPACE)
    assert "timed out" in moe.status_string(moe.MOE_ERR_TIMEOUT)
    assert moe.status_string(12345) == "unknown status"
    assert b"gfx950" in L.moe_version()


def _p(**kw):
    base = dict(T=64, d=256, I=128, E_global=8, k=2, e_begin=0, E_local=8, experts_per_wave=4,
                x_dtype=moe.MOE_BF16, w_dtype=moe.MOE_BF16, out_dtype=moe.MOE_BF16, activation=moe.MOE_ACT_SWIGLU)
    base.update(kw)
    return moe.Problem(*[base[n] for n, _ in moe.Problem._fields_])


@pytest.mark.parametrize("kw,ok", [
    ({}, True),
    ({"T": 0}, True),
    ({"d": 96}, False),                        # d % 128
    ({"d": 192}, False),
    ({"I": 100}, False),                       # I % 64
    ({"k": 9}, False),                         # k > E_global
    ({"k": 0}, False),
    ({"E_local": 6}, False),                   # E_local % G
    ({"e_begin": 4, "E_local": 8}, False),     # beyond E_global
    ({"E_global": 512, "E_local": 8}, False),  # router width limit
    ({"x_dtype": 7}, False),
    ({"T": -1}, False),
    ({"activation": moe.MOE_ACT_RELU2}, True),
    ({"activation": 2}, False),
    ({"activation": moe.MOE_ACT_RELU2, "I": 192}, False),   # ungated: I % 128
])
def test_sizes_accept_and_reject(L, kw, ok):
    p = _p(**kw)
    ws = moe.workspace_size(p)
    pk = moe.packed_weights_size(p)
    assert (ws > 0) == ok and (pk > 0) == ok


def test_packed_size_matches_layout(L):
    p = _p(T=10, d=4096, I=1024, E_global=16, E_local=16, k=4)
    epad = 128
    # router + W1|W3 + W2, each expert weight held once
    want = epad * 4096 * 2 + 16 * 2 * 1024 * 4096 * 2 + 16 * 4096 * 1024 * 2
    assert moe.packed_weights_size(p) == want


def _v4share(T=8192):
    return moe.problem(T=T, d=7168, I=2048, E_global=256, k=8, E_local=32, experts_per_wave=4)


def test_forward_workspace_and_pack_exclude_the_backward(L):
    """A forward-only caller of the V3/V4-scale share needs under 1 GB of
    workspace and holds each expert weight once; the backward layout extends
    the forward one (same offsets), so its size is the larger."""
    p = _v4share()
    fwd, bwd = moe.workspace_size(p), moe.workspace_size(p, backward=True)
    assert 0 < fwd < 1 << 30
    assert bwd > fwd
    # the forward regions: dispatch tables, partial router logits, x staging
    # [T, d] bf16, the activations a [P_max, I] bf16 and the kernel counters
    P_max = 8192 * 8
    assert P_max * 2048 * 2 + 8192 * 7168 * 2 < fwd < P_max * 2048 * 2 + 8192 * 7168 * 2 + 64 * 2 ** 20
    router = 256 * 7168 * 2
    experts = 32 * 3 * 7168 * 2048 * 2
    assert moe.packed_weights_size(p) == router + experts
    # the backward buffer: Wg^T, [W1 | W3]^T and W2 (K = d)
    assert L.moe_packed_bwd_size(ctypes.byref(p)) == 256 * 7168 * 2 + experts
    assert L.moe_workspace_size(ctypes.byref(p), 0x80) == 0      # unknown flag


def test_ffn_path_decision(L):
    """The persistent kernel runs only on the whole 8-XCD device and only
    when MOE_FLAG_PERSISTENT asks for it; with no flag, with MOE_FLAG_SERIAL
    and on any other CU count (partition modes, harvested parts) the phase
    kernels run; the two flags together are rejected."""
    p = _p(T=4096, d=4096, I=1024, E_global=16, E_local=16, k=4)
    assert moe.ffn_path(p, 256) == moe.MOE_PATH_PHASES
    assert moe.ffn_path(p, 256, serial=True) == moe.MOE_PATH_PHASES
    assert moe.ffn_path(p, 256, persistent=True) == moe.MOE_PATH_PERSISTENT
    for cus in (32, 64, 128, 224, 240, 304):
        assert moe.ffn_path(p, cus) == moe.MOE_PATH_PHASES, cus
        assert moe.ffn_path(p, cus, persistent=True) == moe.MOE_PATH_PHASES, cus
    shapes = [_p(T=T, d=4096, I=1536, E_global=64, E_local=64, k=6) for T in (4096, 16384)]   # stress
    shapes.append(_p(T=8192, d=7168, I=2048, E_global=256, E_local=32, k=8))                 # V3/V4 share
    shapes += [_p(T=T, d=7168, I=2048, E_global=32, E_local=32, k=8) for T in (1, 8, 32, 128)]  # decode
    for q in shapes:
        assert moe.ffn_path(q, 256) == moe.MOE_PATH_PHASES, q.T
        assert moe.ffn_path(q, 256, persistent=True) == moe.MOE_PATH_PERSISTENT, q.T
    # more m-tiles per XCD than the schedule holds
    big = _p(T=1 << 20, d=4096, I=1024, E_global=16, E_local=16, k=4)
    assert moe.ffn_path(big, 256) == moe.MOE_PATH_PHASES
    assert moe.ffn_path(big, 256, persistent=True) == moe.MOE_PATH_PHASES
    assert L.moe_ffn_path(ctypes.byref(p), 0, 0) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_ffn_path(ctypes.byref(p), 256, 0x80) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_ffn_path(ctypes.byref(p), 256, moe.MOE_FLAG_SERIAL | moe.MOE_FLAG_PERSISTENT) == \
        moe.MOE_ERR_INVALID_ARG
    assert L.moe_ffn_path(ctypes.byref(_p(d=100)), 256, 0) == moe.MOE_ERR_UNSUPPORTED


def test_workspace_grows_with_tokens(L):
    a = moe.workspace_size(_p(T=64))
    b = moe.workspace_size(_p(T=6400))
    assert b > a > 0


def test_route_rejects_before_launch(L):
    p = _p()
    st = L.moe_route(ctypes.byref(p), None, FAKE, None, FAKE, FAKE, None, FAKE, 1 << 30, None)
    assert st == moe.MOE_ERR_INVALID_ARG
    bad = _p(d=100)
    st = L.moe_route(ctypes.byref(bad), FAKE, FAKE, None, FAKE, FAKE, None, FAKE, 1 << 30, None)
    assert st == moe.MOE_ERR_UNSUPPORTED
    st = L.moe_route(ctypes.byref(p), FAKE, FAKE, None, FAKE, FAKE, None, FAKE, 16, None)
    assert st == moe.MOE_ERR_WORKSPACE
    st = L.moe_route(ctypes.byref(p), FAKE, FAKE, None, FAKE, FAKE, None, None, 1 << 30, None)
    assert st == moe.MOE_ERR_WORKSPACE
    st = L.moe_route(ctypes.byref(p), ctypes.c_void_p(0x10004), FAKE, None, FAKE, FAKE, None, FAKE,
                     1 << 30, None)
    assert st == moe.MOE_ERR_INVALID_ARG  # misaligned x
    st = L.moe_route(None, FAKE, FAKE, None, FAKE, FAKE, None, FAKE, 1 << 30, None)
    assert st == moe.MOE_ERR_INVALID_ARG


def test_dispatch_ffn_combine_wgrad_reject_before_launch(L):
    p = _p()
    st = L.moe_dispatch(ctypes.byref(p), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == moe.MOE_ERR_INVALID_ARG
    st = L.moe_dispatch(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, None)
    assert st == moe.MOE_ERR_WORKSPACE
    st = L.moe_expert_ffn_waved(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                0x80, FAKE, 1 << 30, None)
    assert st == moe.MOE_ERR_INVALID_ARG  # unknown flag
    st = L.moe_expert_ffn_waved(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE,
                                0, FAKE, 1 << 30, None)
    assert st == moe.MOE_ERR_INVALID_ARG  # fused combine without pair_pos / weights
    st = L.moe_expert_ffn_waved(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                0, FAKE, 100, None)
    assert st == moe.MOE_ERR_WORKSPACE
    st = L.moe_combine(ctypes.byref(p), None, FAKE, FAKE, FAKE, None)
    assert st == moe.MOE_ERR_INVALID_ARG
    st = L.moe_combine(ctypes.byref(p), FAKE, FAKE, FAKE, ctypes.c_void_p(0x10008), None)
    assert st == moe.MOE_ERR_INVALID_ARG
    st = L.moe_expert_wgrad(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE,
                            FAKE, 1 << 30, None)
    assert st == moe.MOE_ERR_INVALID_ARG
    st = L.moe_expert_wgrad(ctypes.byref(p), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                            FAKE, 1 << 30, None)
    assert st == moe.MOE_ERR_INVALID_ARG                                 # no backward weights
    st = L.moe_expert_wgrad(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                            FAKE, 1, None)
    assert st == moe.MOE_ERR_WORKSPACE
    # the forward-sized workspace is too small for the weight gradient
    fwd = moe.workspace_size(p)
    st = L.moe_expert_wgrad(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                            FAKE, fwd, None)
    assert st == moe.MOE_ERR_WORKSPACE
    st = L.moe_expert_ffn_waved(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                0, FAKE, fwd - 1, None)
    assert st == moe.MOE_ERR_WORKSPACE
    st = L.moe_pack_weights(ctypes.byref(p), None, FAKE, FAKE, FAKE, FAKE, None)
    assert st == moe.MOE_ERR_INVALID_ARG
    assert L.moe_check_error(None, None) == moe.MOE_ERR_INVALID_ARG


def test_backward_rejects_before_launch(L):
    p = _p()
    args = [FAKE] * 9  # x, packed, packed_bwd, idx, w, offsets, sorted_token, pair_pos, dout

    def call(*, a=None, dx=FAKE, dtw=None, dlg=None, dwg=None, dw=(None, None, None), ws=FAKE, nbytes=1 << 30):
        a = args if a is None else a
        return L.moe_backward(ctypes.byref(p), *a, dx, dtw, dlg, dwg, *dw, ws, nbytes, None)

    assert call(dx=None) == moe.MOE_ERR_INVALID_ARG                      # dx required for T > 0
    assert call(a=[FAKE, FAKE, None] + [FAKE] * 6) == moe.MOE_ERR_INVALID_ARG  # no backward weights
    assert call(dw=(FAKE, None, FAKE)) == moe.MOE_ERR_INVALID_ARG          # dW trio incomplete
    assert call(dx=ctypes.c_void_p(0x10008)) == moe.MOE_ERR_INVALID_ARG    # misaligned dx
    assert call(nbytes=64) == moe.MOE_ERR_WORKSPACE
    assert call(nbytes=moe.workspace_size(p)) == moe.MOE_ERR_WORKSPACE      # forward size only
    assert call(ws=None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_pack_weights_bwd(ctypes.byref(p), FAKE, None, FAKE, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_pack_weights_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, None, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_pack_weights_bwd(ctypes.byref(_p(d=96)), FAKE, FAKE, FAKE, FAKE, FAKE, None) == \
        moe.MOE_ERR_UNSUPPORTED
    assert L.moe_packed_bwd_size(ctypes.byref(_p(d=96))) == 0
    # Wg^T (E_global x d bf16) + per local expert [W1 | W3]^T (d x 2I bf16)
    # and W2 (I x d bf16)
    assert L.moe_packed_bwd_size(ctypes.byref(p)) == 8 * 256 * 2 + 8 * 256 * 256 * 2 + 8 * 128 * 256 * 2


def test_saved_pre_activation_entry_points_reject_before_launch(L):
    """moe_expert_ffn_waved_save_h and moe_backward_saved_h need their h
    buffer (16-byte aligned) when T > 0, and otherwise validate as the plain
    entry points do."""
    p = _p()
    ffn = [FAKE] * 9  # x, packed, offsets, sorted_token, pair_pos, topk_w, ready, y, out

    def fwd(h, flags=0, nbytes=1 << 30):
        return L.moe_expert_ffn_waved_save_h(ctypes.byref(p), *ffn, h, flags, FAKE, nbytes, None)

    assert fwd(None) == moe.MOE_ERR_INVALID_ARG
    assert fwd(ctypes.c_void_p(0x10008)) == moe.MOE_ERR_INVALID_ARG       # misaligned h
    assert fwd(FAKE, flags=0x80) == moe.MOE_ERR_INVALID_ARG                # unknown flag
    assert fwd(FAKE, nbytes=100) == moe.MOE_ERR_WORKSPACE
    bwd = [FAKE] * 9  # x, packed, packed_bwd, idx, w, offsets, sorted_token, pair_pos, dout

    def back(h, dx=FAKE, nbytes=1 << 30):
        return L.moe_backward_saved_h(ctypes.byref(p), *bwd, h, dx, None, None, None, None, None, None, FAKE,
                                      nbytes, None)

    assert back(None) == moe.MOE_ERR_INVALID_ARG
    assert back(ctypes.c_void_p(0x10008)) == moe.MOE_ERR_INVALID_ARG
    assert back(FAKE, dx=None) == moe.MOE_ERR_INVALID_ARG                 # dx required for T > 0
    assert back(FAKE, nbytes=moe.workspace_size(p)) == moe.MOE_ERR_WORKSPACE  # forward size only
    # padded row space: P_max + 64 E_local rounded up to 64, gr I columns
    g = moe.problem(T=8, d=256, I=128, E_global=8, k=2)
    assert moe.saved_h_shape(g) == (576, 256)
    assert L.moe_saved_h_bytes(ctypes.byref(g)) == 576 * 256 * 4
    u = moe.problem(T=8, d=256, I=128, E_global=8, k=2, activation=moe.MOE_ACT_RELU2)
    assert moe.saved_h_shape(u) == (576, 128)
    assert L.moe_saved_h_bytes(ctypes.byref(_p(d=96))) == 0


def test_ungated_activation_sizes_and_backward_arguments(L):
    """RELU2 packs W1 alone (no gating projection, W3 may be NULL); its
    backward buffer holds W1 in place of [W1 | W3], and its backward entry
    points take no dW3: a dW3 is rejected before any launch, and SWIGLU still
    requires one."""
    g, u = _p(), _p(activation=moe.MOE_ACT_RELU2)
    router = 128 * 256 * 2                       # Epad x d bf16
    w2 = 8 * 128 * 256 * 2                       # W2^T, E_local x d x I bf16
    assert moe.packed_weights_size(g) == router + 8 * 2 * 128 * 256 * 2 + w2
    assert moe.packed_weights_size(u) == router + 8 * 128 * 256 * 2 + w2
    assert moe.workspace_size(u) > 0
    # Wg^T (8 x 256 bf16), W1 as [d][I] and W2 (K = d), each E_local x d x I bf16
    assert L.moe_packed_bwd_size(ctypes.byref(u)) == 8 * 256 * 2 + 2 * (8 * 256 * 128 * 2)
    assert L.moe_packed_bwd_size(ctypes.byref(g)) == 8 * 256 * 2 + 3 * (8 * 256 * 128 * 2)
    assert L.moe_pack_weights_bwd(ctypes.byref(u), FAKE, None, None, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_pack_weights_bwd(ctypes.byref(g), FAKE, FAKE, None, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    args = [FAKE] * 9
    assert L.moe_backward(ctypes.byref(u), *args, FAKE, None, None, None, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                          None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_backward(ctypes.byref(g), *args, FAKE, None, None, None, FAKE, None, FAKE, FAKE, 1 << 30,
                          None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_expert_wgrad(ctypes.byref(u), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                              FAKE, 1 << 30, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_expert_wgrad(ctypes.byref(g), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                              FAKE, 1 << 30, None) == moe.MOE_ERR_INVALID_ARG
    # W3 is required for SWIGLU only
    assert L.moe_pack_weights(ctypes.byref(g), FAKE, FAKE, None, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG


def test_fp8_dispatch_rejects_before_launch(L):
    p = _p()
    assert L.moe_quantize_fp8(ctypes.byref(p), FAKE, None, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_quantize_fp8(ctypes.byref(p), FAKE, ctypes.c_void_p(0x10008), FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_quantize_fp8(ctypes.byref(_p(d=96)), FAKE, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    f = L.moe_expert_ffn_waved_fp8
    assert f(ctypes.byref(p), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 1 << 30,
             None) == moe.MOE_ERR_INVALID_ARG                         # no scales
    assert f(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0x4, FAKE, 1 << 30,
             None) == moe.MOE_ERR_INVALID_ARG                         # unknown flag
    assert f(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 64,
             None) == moe.MOE_ERR_WORKSPACE


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(moe, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(moe, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        moe.lib()


def test_probes_reject_bad_arguments_before_any_launch(L):
    """The measurement probes validate on the host: null or short output,
    steps out of range, unaligned, ragged or overlapping copies."""
    flops = ctypes.c_double(0.0)
    assert L.moe_probe_mfma(None, 1 << 20, 16, ctypes.byref(flops), None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_probe_mfma(ctypes.c_void_p(256), 1 << 20, 0, ctypes.byref(flops), None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_probe_mfma(ctypes.c_void_p(256), 1 << 20, (1 << 20) + 1, ctypes.byref(flops),
                            None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_probe_mfma(ctypes.c_void_p(256), 1 << 20, 16, None, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_probe_copy(ctypes.c_void_p(4096), ctypes.c_void_p(8192), 100, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_probe_copy(ctypes.c_void_p(4100), ctypes.c_void_p(8192), 64, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_probe_copy(ctypes.c_void_p(4096), ctypes.c_void_p(4096 + 32), 64, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_probe_copy(None, ctypes.c_void_p(8192), 64, None) == moe.MOE_ERR_INVALID_ARG
