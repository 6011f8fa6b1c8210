// moe_api.hip -- the C ABI declared in include/moe.h: argument checks,
// workspace carve-up and launches.  Host-side checks are O(1) and run before
// anything is queued (DeepSeek-V4 launch digest, itsolotime.com, section
// 2.1: per-call host overhead is what a thin generated launcher keeps below
// a microsecond; here the launcher is this hand-written C++).
#include <string.h>

#include "moe_internal.h"
#include "wave_sched.h"

namespace moe {

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// FFN flags: MOE_FLAG_SERIAL or MOE_FLAG_PERSISTENT, not both.
static bool ffn_flags_ok(uint32_t flags) {
  const uint32_t both = MOE_FLAG_SERIAL | MOE_FLAG_PERSISTENT;
  return (flags & ~both) == 0 && (flags & both) != both;
}

static moe_status_t check_problem(const moe_problem_t* p) {
  if (!p) return MOE_ERR_INVALID_ARG;
  if (p->T < 0 || p->d <= 0 || p->I <= 0 || p->E_global <= 0 || p->k <= 0 || p->E_local <= 0 ||
      p->e_begin < 0 || p->experts_per_wave <= 0)
    return MOE_ERR_INVALID_ARG;
  if (p->k > p->E_global || p->e_begin + p->E_local > p->E_global) return MOE_ERR_INVALID_ARG;
  if (p->E_local % p->experts_per_wave != 0) return MOE_ERR_INVALID_ARG;
  const auto dt_ok = [](int32_t t) { return t == MOE_F32 || t == MOE_BF16; };
  if (!dt_ok(p->x_dtype) || !dt_ok(p->w_dtype) || !dt_ok(p->out_dtype)) return MOE_ERR_INVALID_ARG;
  if (p->activation != MOE_ACT_SWIGLU && p->activation != MOE_ACT_RELU2) return MOE_ERR_INVALID_ARG;
  if (p->d % 128 != 0 || p->I % 64 != 0) return MOE_ERR_UNSUPPORTED;
  // an ungated GEMM1 tile spans 128 intermediate indices (a gated one 64)
  if (p->activation == MOE_ACT_RELU2 && p->I % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (p->E_global > 256 || p->k > 64) return MOE_ERR_UNSUPPORTED;
  if (p->T > (1 << 24) || p->d > (1 << 16) || p->I > (1 << 16)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

WsLayout ws_layout(const moe_problem_t& p) {
  WsLayout L{};
  L.nchunks = (p.T + kWave - 1) / kWave;
  L.W = p.E_local / p.experts_per_wave;
  L.ngroups = p.E_local + L.W + 1;
  L.P_max = p.T * (p.k < p.E_local ? p.k : p.E_local);
  L.Ep = static_cast<int>(align_up(static_cast<size_t>(p.E_global), 64));
  L.ctr_region_words = sched_region_words(L.W);
  L.sync_words = sched_counter_words(L.W) + 1;  // + the persistent kernel's exit count (the per-XCD
                                                 // pool counters sit in the last spans of the counters)
  const size_t wg_slots = static_cast<size_t>(L.P_max) / kWgradChunkRows;
  L.wgrad_bytes = wg_slots * 3 * static_cast<size_t>(p.d) * p.I * sizeof(float);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  L.err = take(256);
  L.masks = take(static_cast<size_t>(L.nchunks) * L.ngroups * 8);
  L.bases = take(static_cast<size_t>(L.nchunks) * L.ngroups * 4);
  L.group_off = take(static_cast<size_t>(L.ngroups + 2) * 4);
  L.ready_list = take(static_cast<size_t>(p.T) * 4);
  L.logits = take(static_cast<size_t>(router_splits(p.d, p.E_global, p.x_dtype == MOE_BF16)) * p.T * p.E_global * 4);
  L.xbf = take(static_cast<size_t>(p.T) * p.d * 2);
  L.act = take(static_cast<size_t>(L.P_max) * p.I * 2);
  L.sync = take(L.sync_words * 4);
  L.fwd_total = off;
  const bool xbf = p.x_dtype == MOE_BF16;
  L.bwd_dh = take(static_cast<size_t>(L.P_max) * 2 * p.I * 2);
  L.P_pad = static_cast<int>(align_up(static_cast<size_t>(L.P_max) + 64 * static_cast<size_t>(p.E_local), 64));
  const size_t ppad = static_cast<size_t>(L.P_pad);
  L.bwd_dht = take(ppad * 2 * p.I * 2);
  L.bwd_awt = take(ppad * p.I * 2);
  L.bwd_xst = take(ppad * p.d * 2);
  L.bwd_dst = take(ppad * p.d * 2);
  L.wgrad = take(L.wgrad_bytes);
  L.bwd_g = take(ppad * p.I * 4);
  L.bwd_dwp = take(static_cast<size_t>(L.P_max) * (p.I / 16) * 4);
  L.bwd_dlc = take(static_cast<size_t>(p.T) * p.k * 4);
  L.bwd_dld = take(xbf ? static_cast<size_t>(p.T) * L.Ep * 2 : 0);
  L.bwd_dxr = take(static_cast<size_t>(L.P_max) * p.d * 2);
  L.bwd_dwg = take(xbf ? static_cast<size_t>((p.T + kDwgChunkRows - 1) / kDwgChunkRows) * p.d * L.Ep * 4 : 0);
  L.total = off;
  return L;
}

// bwd: the call uses the backward regions (the whole layout); otherwise the
// forward prefix suffices.
static moe_status_t check_ws(const moe_problem_t* p, const void* ws, size_t ws_bytes, WsLayout* L,
                             bool bwd = false) {
  *L = ws_layout(*p);
  if (!ws || !aligned16(ws) || ws_bytes < (bwd ? L->total : L->fwd_total)) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

static moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_packed_weights_size(const moe_problem_t* p) {
  if (check_problem(p) != MOE_OK) return 0;
  return packed_layout(p->d, p->I, p->E_global, p->E_local, p->x_dtype == MOE_BF16, gate_rows(*p)).total;
}

size_t moe_workspace_size(const moe_problem_t* p, uint32_t flags) {
  if (check_problem(p) != MOE_OK || (flags & ~MOE_WS_BACKWARD)) return 0;
  const WsLayout L = ws_layout(*p);
  return (flags & MOE_WS_BACKWARD) ? L.total : L.fwd_total;
}

int32_t moe_ffn_path(const moe_problem_t* p, int32_t num_cus, uint32_t flags) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (num_cus <= 0 || !ffn_flags_ok(flags)) return MOE_ERR_INVALID_ARG;
  return ffn_uses_persistent(*p, num_cus, flags) ? MOE_PATH_PERSISTENT : MOE_PATH_PHASES;
}

size_t moe_saved_h_bytes(const moe_problem_t* p) {
  if (check_problem(p) != MOE_OK) return 0;
  return static_cast<size_t>(ws_layout(*p).P_pad) * gate_rows(*p) * p->I * 4;
}

size_t moe_packed_bwd_size(const moe_problem_t* p) {
  if (check_problem(p) != MOE_OK) return 0;
  return packed_bwd_layout(*p).total;
}

moe_status_t moe_pack_weights_bwd(const moe_problem_t* p, const void* Wg, const void* W1, const void* W3,
                                  const void* W2, void* packed_bwd, moe_stream_t stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  const bool gated = p->activation == MOE_ACT_SWIGLU;
  if (!Wg || !W1 || (gated && !W3) || !W2 || !packed_bwd) return MOE_ERR_INVALID_ARG;
  if (!aligned16(packed_bwd) || !aligned16(Wg) || !aligned16(W1) || (W3 && !aligned16(W3)) || !aligned16(W2))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_pack_bwd(*p, Wg, W1, W3, W2, packed_bwd, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_pack_weights(const moe_problem_t* p, const void* Wg, const void* W1,
                              const void* W3, const void* W2, void* packed, moe_stream_t stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  const bool need_w3 = p->activation == MOE_ACT_SWIGLU;
  if (!Wg || !W1 || (need_w3 && !W3) || !W2 || !packed) return MOE_ERR_INVALID_ARG;
  if (!aligned16(packed) || !aligned16(Wg) || !aligned16(W1) || (W3 && !aligned16(W3)) || !aligned16(W2))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_pack(*p, Wg, W1, W3, W2, packed, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_route(const moe_problem_t* p, const void* x, const void* packed, const float* bias,
                       int32_t* topk_idx, float* topk_w, float* logits, void* ws, size_t ws_bytes,
                       moe_stream_t stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (p->T > 0 && (!x || !packed || !topk_idx || !topk_w)) return MOE_ERR_INVALID_ARG;
  if ((x && !aligned16(x)) || (packed && !aligned16(packed))) return MOE_ERR_INVALID_ARG;
  WsLayout L;
  if ((st = check_ws(p, ws, ws_bytes, &L)) != MOE_OK) return st;
  float* partial = reinterpret_cast<float*>(static_cast<char*>(ws) + L.logits);
  return hip_status(launch_route(*p, x, packed, bias, topk_idx, topk_w, logits, partial,
                                 static_cast<hipStream_t>(stream)));
}

moe_status_t moe_route_noalloc(const moe_problem_t* p, const void* x, const void* packed, const float* bias,
                               int32_t* topk_idx, float* topk_w, float* logits, moe_stream_t stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (p->T > 0 && (!x || !packed || !topk_idx || !topk_w)) return MOE_ERR_INVALID_ARG;
  if ((x && !aligned16(x)) || (packed && !aligned16(packed))) return MOE_ERR_INVALID_ARG;
  // the partial logits must fit the fixed scratch array
  if (noalloc_route_bytes(*p) > noalloc_scratch_bytes()) return MOE_ERR_UNSUPPORTED;
  if (p->T == 0) return MOE_OK;
  return hip_status(launch_route_noalloc(*p, x, packed, bias, topk_idx, topk_w, logits,
                                         static_cast<hipStream_t>(stream)));
}

moe_status_t moe_dispatch(const moe_problem_t* p, const int32_t* topk_idx, int32_t* expert_counts,
                          int32_t* expert_offsets, int32_t* sorted_token, int32_t* pair_pos,
                          int32_t* token_ready_wave, void* ws, size_t ws_bytes, moe_stream_t stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!expert_counts || !expert_offsets) return MOE_ERR_INVALID_ARG;
  if (p->T > 0 && (!topk_idx || !sorted_token || !pair_pos || !token_ready_wave)) return MOE_ERR_INVALID_ARG;
  WsLayout L;
  if ((st = check_ws(p, ws, ws_bytes, &L)) != MOE_OK) return st;
  return hip_status(launch_dispatch(*p, L, topk_idx, expert_counts, expert_offsets, sorted_token,
                                    pair_pos, token_ready_wave, static_cast<char*>(ws),
                                    static_cast<hipStream_t>(stream)));
}

moe_status_t moe_route_dispatch(const moe_problem_t* p, const void* x, const void* packed, const float* bias,
                                int32_t* topk_idx, float* topk_w, float* logits, int32_t* expert_counts,
                                int32_t* expert_offsets, int32_t* sorted_token, int32_t* pair_pos,
                                int32_t* token_ready_wave, void* ws, size_t ws_bytes, moe_stream_t stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (p->T > 0 && (!x || !packed || !topk_idx || !topk_w)) return MOE_ERR_INVALID_ARG;
  if ((x && !aligned16(x)) || (packed && !aligned16(packed))) return MOE_ERR_INVALID_ARG;
  if (!expert_counts || !expert_offsets) return MOE_ERR_INVALID_ARG;
  if (p->T > 0 && (!sorted_token || !pair_pos || !token_ready_wave)) return MOE_ERR_INVALID_ARG;
  WsLayout L;
  if ((st = check_ws(p, ws, ws_bytes, &L)) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  float* partial = reinterpret_cast<float*>(w + L.logits);
  hipError_t e = launch_route_logits(*p, x, packed, partial, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (route_dispatch_fuses(*p, L))
    return hip_status(launch_dispatch_with_topk(*p, L, partial, bias, topk_idx, topk_w, logits, expert_counts,
                                                expert_offsets, sorted_token, pair_pos, token_ready_wave, w, s));
  if ((e = launch_topk(*p, partial, bias, topk_idx, topk_w, logits, s)) != hipSuccess) return MOE_ERR_HIP;
  return hip_status(launch_dispatch(*p, L, topk_idx, expert_counts, expert_offsets, sorted_token, pair_pos,
                                    token_ready_wave, w, s));
}

namespace {

// moe_expert_ffn_waved, and with hsave != nullptr moe_expert_ffn_waved_save_h.
moe_status_t ffn_waved_call(const moe_problem_t* p, const void* x, const void* packed,
                            const int32_t* expert_offsets, const int32_t* sorted_token, const int32_t* pair_pos,
                            const float* topk_w, const int32_t* token_ready_wave, void* y, void* out,
                            float* hsave, uint32_t flags, void* ws, size_t ws_bytes, moe_stream_t stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!ffn_flags_ok(flags)) return MOE_ERR_INVALID_ARG;
  if (!packed || !expert_offsets) return MOE_ERR_INVALID_ARG;
  if (p->T > 0 && (!x || !sorted_token || !y)) return MOE_ERR_INVALID_ARG;
  if (out && (!pair_pos || !topk_w)) return MOE_ERR_INVALID_ARG;
  if ((x && !aligned16(x)) || !aligned16(packed) || (y && !aligned16(y)) || (out && !aligned16(out)) ||
      (hsave && !aligned16(hsave)))
    return MOE_ERR_INVALID_ARG;
  WsLayout L;
  if ((st = check_ws(p, ws, ws_bytes, &L)) != MOE_OK) return st;
  return hip_status(launch_ffn(*p, L, x, packed, expert_offsets, sorted_token, pair_pos, topk_w,
                               token_ready_wave, y, out, hsave, flags, static_cast<char*>(ws),
                               static_cast<hipStream_t>(stream)));
}

}  // namespace

moe_status_t moe_expert_ffn_waved(const moe_problem_t* p, const void* x, const void* packed,
                                  const int32_t* expert_offsets, const int32_t* sorted_token,
                                  const int32_t* pair_pos, const float* topk_w,
                                  const int32_t* token_ready_wave, void* y, void* out,
                                  uint32_t flags, void* ws, size_t ws_bytes, moe_stream_t stream) {
  return ffn_waved_call(p, x, packed, expert_offsets, sorted_token, pair_pos, topk_w, token_ready_wave, y, out,
                        nullptr, flags, ws, ws_bytes, stream);
}

moe_status_t moe_expert_ffn_waved_save_h(const moe_problem_t* p, const void* x, const void* packed,
                                         const int32_t* expert_offsets, const int32_t* sorted_token,
                                         const int32_t* pair_pos, const float* topk_w,
                                         const int32_t* token_ready_wave, void* y, void* out, float* h,
                                         uint32_t flags, void* ws, size_t ws_bytes, moe_stream_t stream) {
  if (p && p->T > 0 && !h) return MOE_ERR_INVALID_ARG;
  return ffn_waved_call(p, x, packed, expert_offsets, sorted_token, pair_pos, topk_w, token_ready_wave, y, out, h,
                        flags, ws, ws_bytes, stream);
}

moe_status_t moe_quantize_fp8(const moe_problem_t* p, const void* x, uint8_t* x_fp8, float* x_scale,
                              moe_stream_t stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (p->T > 0 && (!x || !x_fp8 || !x_scale)) return MOE_ERR_INVALID_ARG;
  if ((x && !aligned16(x)) || (x_fp8 && !aligned16(x_fp8))) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_quantize_fp8(*p, x, x_fp8, x_scale, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_expert_ffn_waved_fp8(const moe_problem_t* p, const uint8_t* x_fp8, const float* x_scale,
                                      const void* packed, const int32_t* expert_offsets,
                                      const int32_t* sorted_token, const int32_t* pair_pos,
                                      const float* topk_w, const int32_t* token_ready_wave, void* y,
                                      void* out, uint32_t flags, void* ws, size_t ws_bytes,
                                      moe_stream_t stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!ffn_flags_ok(flags)) return MOE_ERR_INVALID_ARG;
  if (!packed || !expert_offsets) return MOE_ERR_INVALID_ARG;
  if (p->T > 0 && (!x_fp8 || !x_scale || !sorted_token || !y)) return MOE_ERR_INVALID_ARG;
  if (out && (!pair_pos || !topk_w)) return MOE_ERR_INVALID_ARG;
  if ((x_fp8 && !aligned16(x_fp8)) || !aligned16(packed) || (y && !aligned16(y)) || (out && !aligned16(out)))
    return MOE_ERR_INVALID_ARG;
  WsLayout L;
  if ((st = check_ws(p, ws, ws_bytes, &L)) != MOE_OK) return st;
  (void)token_ready_wave;
  return hip_status(launch_ffn_fp8(*p, L, x_fp8, x_scale, packed, expert_offsets, sorted_token, pair_pos,
                                   topk_w, y, out, flags, static_cast<char*>(ws),
                                   static_cast<hipStream_t>(stream)));
}

moe_status_t moe_combine(const moe_problem_t* p, const void* y, const int32_t* pair_pos,
                         const float* topk_w, void* out, moe_stream_t stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (p->T > 0 && (!y || !pair_pos || !topk_w || !out)) return MOE_ERR_INVALID_ARG;
  if ((y && !aligned16(y)) || (out && !aligned16(out))) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine(*p, y, pair_pos, topk_w, out, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_expert_wgrad(const moe_problem_t* p, const void* x, const void* packed,
                              const void* packed_bwd, const int32_t* expert_offsets, const int32_t* sorted_token,
                              const int32_t* pair_pos, const float* topk_w, const void* dout,
                              float* dW1, float* dW3, float* dW2, void* ws, size_t ws_bytes,
                              moe_stream_t stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  // dW3 exists for the gated expert only
  const bool gated = p->activation == MOE_ACT_SWIGLU;
  if (!packed || !packed_bwd || !expert_offsets || !dW1 || !dW2 || (gated != (dW3 != nullptr)))
    return MOE_ERR_INVALID_ARG;
  if (p->T > 0 && (!x || !sorted_token || !pair_pos || !topk_w || !dout)) return MOE_ERR_INVALID_ARG;
  if ((x && !aligned16(x)) || (dout && !aligned16(dout)) || !aligned16(packed) || !aligned16(packed_bwd) ||
      !aligned16(dW1) || (dW3 && !aligned16(dW3)) || !aligned16(dW2))
    return MOE_ERR_INVALID_ARG;
  WsLayout L;
  if ((st = check_ws(p, ws, ws_bytes, &L, true)) != MOE_OK) return st;
  BackwardArgs a{};
  a.x = x;
  a.packed = packed;
  a.packed_bwd = packed_bwd;
  a.topk_w = topk_w;
  a.offsets = expert_offsets;
  a.sorted_token = sorted_token;
  a.pair_pos = pair_pos;
  a.dout = dout;
  a.dW1 = dW1;
  a.dW3 = dW3;
  a.dW2 = dW2;
  return hip_status(launch_backward(*p, L, a, static_cast<char*>(ws), static_cast<hipStream_t>(stream)));
}

namespace {

// moe_backward, and with hsaved != nullptr moe_backward_saved_h.
moe_status_t backward_call(const moe_problem_t* p, const void* x, const void* packed,
                           const void* packed_bwd, const int32_t* topk_idx, const float* topk_w,
                           const int32_t* expert_offsets, const int32_t* sorted_token,
                           const int32_t* pair_pos, const void* dout, void* dx, float* dtopk_w,
                           float* dlogits, float* dWg, float* dW1, float* dW3, float* dW2, const float* hsaved,
                           void* ws, size_t ws_bytes, moe_stream_t stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!packed || !packed_bwd || !expert_offsets) return MOE_ERR_INVALID_ARG;
  if (p->T > 0 && (!x || !topk_idx || !topk_w || !sorted_token || !pair_pos || !dout || !dx))
    return MOE_ERR_INVALID_ARG;
  // the weight gradient: dW1, dW2 (and dW3 for the gated expert; none for
  // the ungated one), all or nothing
  const bool gated = p->activation == MOE_ACT_SWIGLU;
  const bool any_w = dW1 || dW3 || dW2;
  const bool all_w = dW1 && dW2 && (gated ? dW3 != nullptr : dW3 == nullptr);
  if (any_w && !all_w) return MOE_ERR_INVALID_ARG;
  if ((x && !aligned16(x)) || !aligned16(packed) || !aligned16(packed_bwd) || (dout && !aligned16(dout)) ||
      (dx && !aligned16(dx)) || (dW1 && !aligned16(dW1)) || (dW3 && !aligned16(dW3)) ||
      (dW2 && !aligned16(dW2)) || (hsaved && !aligned16(hsaved)))
    return MOE_ERR_INVALID_ARG;
  WsLayout L;
  if ((st = check_ws(p, ws, ws_bytes, &L, true)) != MOE_OK) return st;
  BackwardArgs a{};
  a.x = x;
  a.packed = packed;
  a.packed_bwd = packed_bwd;
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  a.offsets = expert_offsets;
  a.sorted_token = sorted_token;
  a.pair_pos = pair_pos;
  a.dout = dout;
  a.dx = p->T > 0 ? dx : nullptr;
  a.dtopk_w = dtopk_w;
  a.dlogits = dlogits;
  a.dWg = dWg;
  a.dW1 = dW1;
  a.dW3 = dW3;
  a.dW2 = dW2;
  a.hsaved = hsaved;
  return hip_status(launch_backward(*p, L, a, static_cast<char*>(ws), static_cast<hipStream_t>(stream)));
}

}  // namespace

moe_status_t moe_backward(const moe_problem_t* p, const void* x, const void* packed,
                          const void* packed_bwd, const int32_t* topk_idx, const float* topk_w,
                          const int32_t* expert_offsets, const int32_t* sorted_token,
                          const int32_t* pair_pos, const void* dout, void* dx, float* dtopk_w,
                          float* dlogits, float* dWg, float* dW1, float* dW3, float* dW2, void* ws,
                          size_t ws_bytes, moe_stream_t stream) {
  return backward_call(p, x, packed, packed_bwd, topk_idx, topk_w, expert_offsets, sorted_token, pair_pos, dout,
                       dx, dtopk_w, dlogits, dWg, dW1, dW3, dW2, nullptr, ws, ws_bytes, stream);
}

moe_status_t moe_backward_saved_h(const moe_problem_t* p, const void* x, const void* packed,
                                  const void* packed_bwd, const int32_t* topk_idx, const float* topk_w,
                                  const int32_t* expert_offsets, const int32_t* sorted_token,
                                  const int32_t* pair_pos, const void* dout, const float* h, void* dx,
                                  float* dtopk_w, float* dlogits, float* dWg, float* dW1, float* dW3,
                                  float* dW2, void* ws, size_t ws_bytes, moe_stream_t stream) {
  if (p && p->T > 0 && !h) return MOE_ERR_INVALID_ARG;
  return backward_call(p, x, packed, packed_bwd, topk_idx, topk_w, expert_offsets, sorted_token, pair_pos, dout,
                       dx, dtopk_w, dlogits, dWg, dW1, dW3, dW2, h, ws, ws_bytes, stream);
}

moe_status_t moe_check_error(void* ws, moe_stream_t stream) {
  if (!ws) return MOE_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t word = 0;
  if (hipMemcpyAsync(&word, ws, sizeof(word), hipMemcpyDeviceToHost, s) != hipSuccess) return MOE_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return MOE_ERR_HIP;
  if (word != 0) {
    const int32_t zero = 0;
    if (hipMemcpyAsync(ws, &zero, sizeof(zero), hipMemcpyHostToDevice, s) != hipSuccess) return MOE_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return MOE_ERR_HIP;
    return static_cast<moe_status_t>(word);
  }
  return MOE_OK;
}

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or option";
    case MOE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_TIMEOUT: return "device-side wait timed out";
  }
  return "unknown status";
}

const char* moe_version(void) { return "moe-mi355x 0.1 (gfx950)"; }

}  // extern "C"
