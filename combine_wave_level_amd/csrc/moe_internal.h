// moe_internal.h -- host-side plumbing shared by the library's translation
// units: the workspace layout and the kernel launchers.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"
#include "moe_common.h"

namespace moe {

// Workspace carve-up.  Every region is 256-byte aligned.
//   err        int32 device error word (bounded waits write MOE_ERR_TIMEOUT)
//   masks      uint64 [nchunks][ngroups]: per 64-token chunk, one bit per
//              token for each local expert it picked (groups 0..E_local-1)
//              and for its ready wave (groups E_local .. E_local+W: slot 0 =
//              no local pick, slot w+1 = ready after wave w)
//   bases      int32 [nchunks][ngroups]: exclusive scan of the chunk counts
//              over chunks, per group
//   group_off  int32 [ngroups + 1]: start of each group in its sorted order
//              (experts: pair rows; ready slots: positions in ready_list)
//   ready_list int32 [T]: tokens ordered by ready wave, ascending token id
//              inside a wave
//   logits     fp32 [splits][T][E_global] partial router logits (K split)
//   xbf        bf16 [T][d]: x rounded for the FFN (fp32 x), or the
//              dequantized FP8 rows (FP8 dispatch on the large shapes)
//   act        bf16 [P_max][I]: a = silu(h1) * h3, sorted-row order
//   sync       int32 counters of the persistent expert-wave kernel
//   bwd_dh     bf16 [P_max][2I]: dH1 | dH3 per routed row (backward)
//   The weight gradient's operands, transposed so that the reduction index
//   (the routed rows) is contiguous; column k of these [.][P_pad] matrices
//   is a routed row, each expert's rows starting at a multiple of 64
//   (seg_e = sum over e' < e of its row count rounded up to 64), the
//   columns past an expert's rows zero:
//   bwd_dht    bf16 [2I][P_pad] (dH1 | dH3)^T, MFMA fragment layout
//   bwd_awt    bf16 [I][P_pad]  (w * a)^T, rows
//   bwd_xst    bf16 [d][P_pad]  x^T of the routed rows, rows
//   bwd_dst    bf16 [d][P_pad]  dout^T of the routed rows, fragment layout
//   wgrad      fp32 isolated partial buffers of the weight gradient
//   bwd_g      fp32 [P_pad][I]: dout W2^T per routed row, block-fragment
//              layout over the padded row space (ffn_parts.h)
//   bwd_dwp    fp32 [P_max][I / 16]: partial sums of the combine-weight
//              gradient of each routed row, one per 16 intermediate indices
//   bwd_dlc    fp32 [T][k]: gradient of the picked logits
//   bwd_dld    bf16 [T][Ep]: dense logits gradient (bf16 x only)
//   bwd_dxr    bf16 [P_max][d]: data gradient of each routed row
//   bwd_dwg    fp32 [ceil(T / kDwgChunkRows)][d][Ep]: isolated partials of
//              dWg (bf16 x only)
//   The forward regions (err .. sync) come first: fwd_total bytes hold them,
//   and a workspace of that size serves every forward entry point; the
//   backward regions follow (total).
struct WsLayout {
  size_t err, masks, bases, group_off, ready_list, logits, xbf, act, sync, bwd_dh, bwd_dht, bwd_awt,
      bwd_xst, bwd_dst, wgrad, bwd_g, bwd_dwp, bwd_dlc, bwd_dld, bwd_dxr, bwd_dwg, fwd_total, total;
  int nchunks, W, ngroups, P_max;
  int P_pad;             // columns of the transposed weight-gradient operands
  int Ep;                // E_global rounded up to 64 (columns of the dense logits gradient)
  int ctr_region_words;  // per-XCD counter region of the persistent kernel
  size_t sync_words, wgrad_bytes;
};

WsLayout ws_layout(const moe_problem_t& p);

// Packed W13 rows per intermediate index: 2 (W1 and W3) for SwiGLU, 1 (W1)
// for the ungated activation.
inline int gate_rows(const moe_problem_t& p) { return p.activation == MOE_ACT_SWIGLU ? 2 : 1; }

// Rows of the weight-gradient split along the routed rows of one expert:
// each chunk of this many rows reduces into its own partial slot.
constexpr int kWgradChunkRows = 2048;
// Tokens per isolated partial of the router-weight gradient dWg.
constexpr int kDwgChunkRows = 1024;

// Backward weight buffer (moe_pack_weights_bwd):
//   wgt  : Wg^T as [E_global][d] row-major in the dtype of x (router rows
//          for the router's share of dx);
//   w13t : per local expert, [W1 | W3]^T as [d][2I] in fragment layout
//          (K = 2I: the W1 columns, then the W3 columns), the weights of
//          dx = dH1 W1^T + dH3 W3^T;
//   w2b  : per local expert, W2 as [I][d] in fragment layout (K = d), the
//          operand of dA = dy W2^T.
struct PackedBwdLayout {
  size_t wgt, w13t, w2b, total;
};

inline PackedBwdLayout packed_bwd_layout(const moe_problem_t& p) {
  PackedBwdLayout L;
  size_t off = 0;
  L.wgt = off;
  off += align_up(static_cast<size_t>(p.E_global) * p.d * (p.x_dtype == MOE_BF16 ? 2 : 4), 256);
  L.w13t = off;
  off += align_up(static_cast<size_t>(p.E_local) * p.d * (p.activation == MOE_ACT_SWIGLU ? 2 : 1) * p.I * 2, 256);
  L.w2b = off;
  off += align_up(static_cast<size_t>(p.E_local) * p.d * p.I * 2, 256);
  L.total = off;
  return L;
}

// Arguments of one backward call (pointers as passed to moe_backward;
// dx == nullptr: weight gradient only; dW1 == nullptr: no weight gradient).
struct BackwardArgs {
  const void* x;
  const void* packed;
  const void* packed_bwd;
  const int32_t* topk_idx;
  const float* topk_w;
  const int32_t* offsets;
  const int32_t* sorted_token;
  const int32_t* pair_pos;
  const void* dout;
  void* dx;
  float* dtopk_w;
  float* dlogits;
  float* dWg;
  float* dW1;
  float* dW3;
  float* dW2;
  // the forward's GEMM1 pre-activations [P][gr I] fp32 (packed column
  // order) or nullptr: recompute them
  const float* hsaved;
};

// ------------------------------------------------------------ launchers
// Each returns hipSuccess or the launch error.  Shapes are validated by the
// caller (moe_api.hip) before these run.

hipError_t launch_pack(const moe_problem_t& p, const void* Wg, const void* W1, const void* W3,
                       const void* W2, void* packed, hipStream_t s);
hipError_t launch_pack_bwd(const moe_problem_t& p, const void* Wg, const void* W1, const void* W3,
                           const void* W2, void* packed_bwd, hipStream_t s);

hipError_t launch_route(const moe_problem_t& p, const void* x, const void* packed,
                        const float* bias, int32_t* topk_idx, float* topk_w, float* logits,
                        float* partial, hipStream_t s);
// Fixed number of ranges the router's reduction over d is cut into (bf16 x;
// depends on the layer only: d and E_global).
int router_splits(int d, int E_global, bool x_bf16);

// moe_route_noalloc: bytes of scratch a problem's router needs, the fixed
// scratch size, and the launch on the fixed device array.
size_t noalloc_route_bytes(const moe_problem_t& p);
size_t noalloc_scratch_bytes();
hipError_t launch_route_noalloc(const moe_problem_t& p, const void* x, const void* packed, const float* bias,
                                int32_t* topk_idx, float* topk_w, float* logits, hipStream_t s);

hipError_t launch_dispatch(const moe_problem_t& p, const WsLayout& L, const int32_t* topk_idx,
                           int32_t* counts, int32_t* offsets, int32_t* sorted_token,
                           int32_t* pair_pos, int32_t* ready_wave, char* ws, hipStream_t s);

// moe_route_dispatch: the router's logits kernel, then (small batches) the
// top-k and the dispatch in one workgroup, or the top-k kernel and the
// dispatch kernels.  kFusedTopkMaxTokens bounds the one-workgroup top-k to
// one round of its 16 wavefronts (one token each): measured at decode, one
// round saves a launch (T = 1: 25.9 -> 21.7 us for the two steps), two
// rounds cost more than the launch (T = 32: 26 -> 30.6 us).
constexpr int kFusedTopkMaxTokens = 16;
bool route_dispatch_fuses(const moe_problem_t& p, const WsLayout& L);
hipError_t launch_route_logits(const moe_problem_t& p, const void* x, const void* packed, float* partial,
                               hipStream_t s);
hipError_t launch_topk(const moe_problem_t& p, const float* partial, const float* bias, int32_t* topk_idx,
                       float* topk_w, float* logits, hipStream_t s);
hipError_t launch_dispatch_with_topk(const moe_problem_t& p, const WsLayout& L, const float* partial,
                                     const float* bias, int32_t* topk_idx, float* topk_w, float* logits,
                                     int32_t* counts, int32_t* offsets, int32_t* sorted_token,
                                     int32_t* pair_pos, int32_t* ready_wave, char* ws, hipStream_t s);

// Whether moe_expert_ffn_waved runs the persistent expert-wave kernel
// (true) or the phase-by-phase kernels (false) on a device with `cus`
// compute units, for flags as passed.  The persistent kernel deals its
// tickets to kXcds per-XCD streams and a workgroup serves the stream of the
// XCD it runs on, so it needs the whole gfx950 device (kXcds XCDs of
// kCusPerXcd CUs; a partitioned or harvested device leaves streams without
// workgroups) and a schedule that fits its tables.
bool ffn_uses_persistent(const moe_problem_t& p, int cus, uint32_t flags);

hipError_t launch_ffn(const moe_problem_t& p, const WsLayout& L, const void* x, const void* packed,
                      const int32_t* offsets, const int32_t* sorted_token, const int32_t* pair_pos,
                      const float* topk_w, const int32_t* ready_wave, void* y, void* out, float* hsave,
                      uint32_t flags, char* ws, hipStream_t s);

// Returns the bf16 token-order staging copy of x used by the expert GEMMs:
// x itself when it is bf16, else a rounded copy written to the workspace.
hipError_t stage_x_bf16(const moe_problem_t& p, const WsLayout& L, const void* x, char* ws,
                        hipStream_t s, const uint16_t** xb);

// Zero-fills n 32-bit words with a kernel (no memset node, so callers may
// capture the stream into a graph).
hipError_t fill_zero(void* p, size_t n, hipStream_t s);

// FP8 dispatch: per-token e4m3 codes and power-of-two scales of x, and the
// expert FFN on them (same schedule and GEMM2, GEMM1 pulling the codes).
hipError_t launch_quantize_fp8(const moe_problem_t& p, const void* x, uint8_t* x8, float* xscale, hipStream_t s);
// The dequantized bf16 rows of the FP8 staging buffer (T x d).
hipError_t launch_dequant_fp8(const moe_problem_t& p, const uint8_t* x8, const float* xscale, uint16_t* xb,
                              hipStream_t s);
hipError_t launch_ffn_fp8(const moe_problem_t& p, const WsLayout& L, const uint8_t* x8, const float* xscale,
                          const void* packed, const int32_t* offsets, const int32_t* sorted_token,
                          const int32_t* pair_pos, const float* topk_w, void* y, void* out, uint32_t flags,
                          char* ws, hipStream_t s);

hipError_t launch_combine(const moe_problem_t& p, const void* y, const int32_t* pair_pos,
                          const float* topk_w, void* out, hipStream_t s);

hipError_t launch_backward(const moe_problem_t& p, const WsLayout& L, const BackwardArgs& a, char* ws,
                           hipStream_t s);

}  // namespace moe
