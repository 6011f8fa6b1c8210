/*
 * moe.h -- C ABI of one GPU's share of a fine-grained expert-parallel MoE
 * layer, for AMD Instinct MI355X (gfx950).
 *
 * The layer, as the DeepSeek-V4 report describes it (DeepSeek-V4 launch
 * digest, itsolotime.com, Thai translation of the report's infrastructure
 * chapter, section 1.1; 10100.com commentary, section on fine-grained
 * compute/communication overlap of the EP all-to-all): route each token to
 * its top-k experts, dispatch the tokens to their experts, run each expert's
 * FFN (Linear, SwiGLU, Linear), and combine the expert outputs back into
 * token order weighted by the router.  Experts are processed in waves of a
 * few experts (digest section 1.2); inside one persistent kernel the current
 * wave's GEMMs overlap the dispatch pulls of the next wave and the combine of
 * finished tokens, or the same tiles run as grid-wide phases, which measured
 * faster on one GPU and are the default (see moe_ffn_path).  Results
 * are batch invariant and deterministic (digest
 * section 3; 10100.com section on batch-invariant and deterministic
 * operators): a token's output bits do not depend on the batch it sits in,
 * and repeated runs give identical bits, including the weight gradient.
 *
 * Conventions for every entry point
 *   - All pointers are device pointers unless stated otherwise; tensors are
 *     dense, row-major, and 16-byte aligned.  The caller owns every buffer;
 *     the library never allocates device memory.
 *   - Calls are asynchronous on `stream` (0 = the null stream).  Host-side
 *     argument checks run first and return an error before anything is
 *     launched; a failed launch returns MOE_ERR_HIP.
 *   - bf16 means IEEE-754 binary32 truncated to its upper 16 bits; every
 *     rounding to bf16 in the library is round-to-nearest-even.
 *   - "Local" experts are the global ids [e_begin, e_begin + E_local).
 *     P (the number of routed pairs that land on local experts) is known
 *     only on the device; buffers indexed by pair row are sized for the
 *     upper bound P_max = T * min(k, E_local).
 *   - No function keeps state between calls; calls on different streams
 *     with disjoint buffers may run concurrently.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* moe_stream_t; /* a hipStream_t */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, bad shape, misaligned buffer  */
  MOE_ERR_UNSUPPORTED = -2, /* valid but outside what the kernels handle   */
  MOE_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required  */
  MOE_ERR_HIP = -4,         /* a HIP runtime call or launch failed         */
  MOE_ERR_TIMEOUT = -5      /* a device-side bounded wait expired          */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

/* Expert activation.  SWIGLU: a = silu(x W1) * (x W3) (the layer of the
 * workloads).  RELU2: the cheap element-wise activation the DeepSeek-V4
 * launch digest (section 1.4, activation-function bullet) recommends instead
 * of SwiGLU, with no exponential, no division and no gating projection; the
 * pages do not name the function, the reading here is squared ReLU,
 * a = max(x W1, 0)^2, and W3 is not used.  The backward entry points take
 * both: with RELU2 there is no W3 and no dW3 (its pointers are NULL) and
 * dH1 = dA * 2 max(h1, 0) (the derivative of max(h, 0)^2, 0 at h = 0). */
typedef enum { MOE_ACT_SWIGLU = 0, MOE_ACT_RELU2 = 1 } moe_activation_t;

/* Shape of one layer share.  Limits checked by every call:
 *   T >= 0; d, I > 0 with d % 128 == 0 and I % 64 == 0 (MOE_ERR_UNSUPPORTED
 *   otherwise); 1 <= k <= E_global; E_global <= 256 and k <= 64
 *   (MOE_ERR_UNSUPPORTED beyond); E_local >= 1; 0 <= e_begin,
 *   e_begin + E_local <= E_global;
 *   1 <= experts_per_wave, E_local % experts_per_wave == 0;
 *   x_dtype in {F32, BF16}; out_dtype in {F32, BF16};
 *   activation in {SWIGLU, RELU2}; RELU2 needs I % 128 == 0
 *   (MOE_ERR_UNSUPPORTED otherwise). */
typedef struct {
  int32_t T;                /* tokens in the batch                         */
  int32_t d;                /* hidden size                                 */
  int32_t I;                /* expert intermediate size                    */
  int32_t E_global;         /* router width (experts over all GPUs)        */
  int32_t k;                /* experts per token                           */
  int32_t e_begin;          /* first local expert id                       */
  int32_t E_local;          /* local experts                               */
  int32_t experts_per_wave; /* G: experts per wave                         */
  int32_t x_dtype;          /* moe_dtype_t of x and the router weights     */
  int32_t w_dtype;          /* moe_dtype_t of the unpacked expert weights  */
  int32_t out_dtype;        /* moe_dtype_t of the layer output             */
  int32_t activation;       /* moe_activation_t of the experts             */
} moe_problem_t;

/* Flags for moe_expert_ffn_waved (at most one of the two).  With neither,
 * the library picks the schedule (moe_ffn_path). */
#define MOE_FLAG_SERIAL 0x1u /* run gather+GEMM1, GEMM2, combine as separate
                                grid-wide phases (the library's default;
                                same bits, no overlap)                       */
#define MOE_FLAG_PERSISTENT 0x2u /* run the persistent expert-wave kernel
                                whenever it fits (same bits)                 */

/* ------------------------------------------------------------ sizing */

/* Bytes of the packed weight buffer moe_pack_weights writes. 0 on bad shape. */
size_t moe_packed_weights_size(const moe_problem_t* p);

/* Flags for moe_workspace_size. */
#define MOE_WS_BACKWARD 0x1u /* size for the backward entry points too     */

/* Bytes of workspace for problem p.  flags = 0: what the forward entry
 * points need (moe_route, moe_dispatch, moe_expert_ffn_waved,
 * moe_expert_ffn_waved_fp8); MOE_WS_BACKWARD: what every entry point needs,
 * moe_expert_wgrad and moe_backward included.  The forward regions sit at
 * the same offsets in both layouts, so one workspace of the larger size
 * serves every entry point (not concurrently).  A forward entry point never
 * touches bytes past the forward size.  0 on a bad shape or unknown flag. */
size_t moe_workspace_size(const moe_problem_t* p, uint32_t flags);

/* Which schedule moe_expert_ffn_waved (and _fp8) runs for problem p with
 * these flags on a device of num_cus compute units:
 *   MOE_PATH_PERSISTENT: the persistent expert-wave kernel.  It hands out
 *     tiles from one ticket stream per XCD and a workgroup serves the stream
 *     of the XCD it runs on, so it needs the whole MI355X (8 XCDs of 32 CUs,
 *     num_cus == 256; a partitioned or harvested device would leave streams
 *     without workgroups) and at most 512 m-tiles per XCD;
 *   MOE_PATH_PHASES: gather + GEMM1, GEMM2 and combine as grid-wide phases
 *     (MOE_FLAG_SERIAL, or when the persistent kernel does not fit).
 * With neither flag the library runs the phases: on MI355X they measured
 * 1 to 16% faster than the persistent kernel on the mid and stress layers,
 * the V3/V4-scale share and decode at T = 1, 32 and 128 (at T = 8 the
 * persistent kernel measured up to 2% faster).  MOE_FLAG_PERSISTENT takes
 * the persistent kernel whenever it fits.  Both schedules give the same
 * bits.  The library calls this with the current device's CU count.
 * Returns a moe_status_t (< 0) on a bad argument. */
#define MOE_PATH_PERSISTENT 0
#define MOE_PATH_PHASES 1
int32_t moe_ffn_path(const moe_problem_t* p, int32_t num_cus, uint32_t flags);

/* ------------------------------------------------------------ weights */

/* One-time re-layout of the weights into the library's MFMA fragment
 * layout (not part of the per-batch path; weights are parameters).
 *   Wg [d, E_global] in x_dtype (router), W1, W3 [E_local, d, I] and
 *   W2 [E_local, I, d] in w_dtype, all row-major in math layout
 *   (h1 = x W1, h3 = x W3, y = a W2); W3 may be NULL for RELU2.
 *   packed: moe_packed_weights_size(p) bytes, written entirely.
 * Expert weights are rounded to bf16 (RNE) when w_dtype is F32. */
moe_status_t moe_pack_weights(const moe_problem_t* p, const void* Wg, const void* W1,
                              const void* W3, const void* W2, void* packed,
                              moe_stream_t stream);

/* Bytes of the backward weight buffer moe_pack_weights_bwd writes. 0 on a
 * bad shape. */
size_t moe_packed_bwd_size(const moe_problem_t* p);

/* One-time re-layout of the weights the gradients read (weights are
 * parameters; forward-only callers never need this buffer): Wg^T in the
 * dtype of x, and per local expert [W1 | W3]^T (W1^T alone for RELU2) and
 * W2 (K = d) in the MFMA fragment layout.
 *   Wg [d, E_global] in x_dtype; W1, W3 [E_local, d, I] and W2 [E_local, I,
 *   d] in w_dtype (rounded to bf16 when F32); W3 may be NULL for RELU2.
 *   packed_bwd: moe_packed_bwd_size(p) bytes, written entirely. */
moe_status_t moe_pack_weights_bwd(const moe_problem_t* p, const void* Wg, const void* W1,
                                  const void* W3, const void* W2, void* packed_bwd,
                                  moe_stream_t stream);

/* ------------------------------------------------------------ the path */

/* Router (workload definition of the layer: softmax over all E_global
 * experts, top-k, weights renormalised over the k picks; named as the "MoE
 * Routing" kernel of TileKernels in digest section 1.3).
 *   x [T, d] in x_dtype; bias [E_global] fp32 or NULL (added to the logits).
 *   Out: topk_idx [T, k] int32 global expert ids in rank order (descending
 *   score, ties to the lower id); topk_w [T, k] fp32; logits [T, E_global]
 *   fp32 when non-NULL (the router scores the selection was made on).
 * Logits accumulate in fp32 in a fixed order that depends on the layer only
 * (for bf16 x the reduction over d is cut into up to 8 equal ranges, 2 when
 * E_global > 64, each summed in ascending index order, and the ranges are
 * added in ascending order; then the bias); selection is made on the fp32 logits; weights are
 * exp(l_j - l_max) / sum over the picks, i.e. softmax followed by
 * renormalisation.  ws holds the partial logits (moe_workspace_size). */
moe_status_t moe_route(const moe_problem_t* p, const void* x, const void* packed,
                       const float* bias, int32_t* topk_idx, float* topk_w, float* logits,
                       void* ws, size_t ws_bytes, moe_stream_t stream);

/* moe_route for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same kernels and the same results bit for bit, with the router's scratch
 * (its partial logits, splits x T x E_global fp32, splits as described for
 * moe_route; the fp32 router: T x E_global fp32) in a fixed device array of
 * MOE_ROUTE_NOALLOC_MAX_BYTES that the library holds on every GPU it runs on
 * until the process ends, instead of a caller workspace.  The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine); the caller
 * still passes inputs and outputs as for moe_route.  A problem whose scratch
 * exceeds the array returns MOE_ERR_UNSUPPORTED before any launch.  Every
 * call on a GPU uses that GPU's one array: calls that overlap on one GPU
 * (different streams, threads or processes' graphs) race.  The first call
 * on each device looks up the array's device address (thread safe). */
#define MOE_ROUTE_NOALLOC_MAX_BYTES (16u << 20)
moe_status_t moe_route_noalloc(const moe_problem_t* p, const void* x, const void* packed,
                               const float* bias, int32_t* topk_idx, float* topk_w, float* logits,
                               moe_stream_t stream);

/* Dispatch metadata: a deterministic counting sort of the routed pairs by
 * local expert (10100.com, deterministic operators: pre-sorting instead of
 * unordered atomics).  Inside an expert, pairs are in ascending token order.
 *   topk_idx [T, k] int32 (from moe_route or any caller).
 *   Out: expert_counts [E_local], expert_offsets [E_local + 1] (exclusive
 *   scan), sorted_token [P_max] (row -> token; rows >= P unwritten),
 *   pair_pos [T, k] (pair -> row, -1 for non-local experts),
 *   token_ready_wave [T] (last wave, (e - e_begin) / G, holding one of the
 *   token's local experts; -1 if none).  All int32.
 * Also fills the workspace's scheduling tables used by
 * moe_expert_ffn_waved, so call it with the same workspace first. */
moe_status_t moe_dispatch(const moe_problem_t* p, const int32_t* topk_idx,
                          int32_t* expert_counts, int32_t* expert_offsets,
                          int32_t* sorted_token, int32_t* pair_pos, int32_t* token_ready_wave,
                          void* ws, size_t ws_bytes, moe_stream_t stream);

/* moe_route followed by moe_dispatch in one call, with the same outputs
 * bit for bit (both definitions above).  For small batches (T <= 16: one
 * token per wavefront of the dispatch's one workgroup) the top-k selection
 * runs inside the dispatch's workgroup, so the two steps take two kernel
 * launches (logits; top-k and dispatch) instead of three: the launches
 * dominate a decode step's router and dispatch.  Arguments: those
 * of moe_route, then those of moe_dispatch (topk_idx written, then read). */
moe_status_t moe_route_dispatch(const moe_problem_t* p, const void* x, const void* packed, const float* bias,
                                int32_t* topk_idx, float* topk_w, float* logits, int32_t* expert_counts,
                                int32_t* expert_offsets, int32_t* sorted_token, int32_t* pair_pos,
                                int32_t* token_ready_wave, void* ws, size_t ws_bytes, moe_stream_t stream);

/* Expert FFN in expert waves (digest sections 1.1, 1.2, 1.4: per pair
 * h1 = x W1, h3 = x W3, a = silu(h1) * h3, y = a W2).
 *   x [T, d] in x_dtype: the staging buffer the dispatch pulls gather from.
 *   packed: from moe_pack_weights.  expert_offsets, sorted_token, pair_pos,
 *   token_ready_wave: from moe_dispatch (same workspace).  topk_w [T, k].
 *   Out: y [P_max, d] bf16 expert outputs in sorted-row order; out [T, d] in
 *   out_dtype when non-NULL: the combine (on the phase schedule its own
 *   grid-wide pass, fused into the persistent kernel; the same bits; tokens
 *   with no local pick get zeros).
 * Each GEMM accumulates in fp32 over K in one fixed ascending order with one
 * MFMA shape, never split; a is rounded to bf16 before the second GEMM and y
 * is rounded to bf16.  flags: 0 (the library's schedule, see
 * moe_ffn_path), MOE_FLAG_SERIAL or MOE_FLAG_PERSISTENT; any other value is
 * MOE_ERR_INVALID_ARG.
 * After one moe_dispatch the call may be repeated on the same workspace any
 * number of times: moe_dispatch zeroes the persistent kernel's tickets and
 * counters, and every launch zeroes them again as it ends.  Calls that
 * overlap on one workspace race. */
moe_status_t moe_expert_ffn_waved(const moe_problem_t* p, const void* x, const void* packed,
                                  const int32_t* expert_offsets, const int32_t* sorted_token,
                                  const int32_t* pair_pos, const float* topk_w,
                                  const int32_t* token_ready_wave, void* y, void* out,
                                  uint32_t flags, void* ws, size_t ws_bytes,
                                  moe_stream_t stream);

/* moe_expert_ffn_waved that also keeps the first GEMM's pre-activations for
 * the backward: activation saving in place of recomputation (the launch
 * digest, itsolotime.com, names flexible activation checkpointing among the
 * training framework's features, section 5.4, without details; which tensor
 * to keep is this library's choice).  Outputs y and out are bit-identical
 * to moe_expert_ffn_waved's.
 *   h: moe_saved_h_bytes(p) bytes, caller-owned, 16-byte aligned, required
 *   when T > 0.  It receives the fp32 accumulators of every routed row:
 *   columns in packed order (gr = 2 for SWIGLU: columns 32 q .. 32 q + 15
 *   hold h1 = x W1 for intermediate indices 16 q .. 16 q + 15, columns
 *   32 q + 16 .. 32 q + 31 hold h3 = x W3 for the same indices; gr = 1 for
 *   RELU2: column i holds h1 for index i); rows in a padded row space where
 *   routed row r of local expert e (sorted-row order) is row s = seg[e] + r
 *   - expert_offsets[e], seg[e] = the sum over local experts e' < e of their
 *   row counts each rounded up to 64; element (s, c) at float offset
 *   ((s / 16) * (gr I / 16) + c / 16) * 256 + ((s % 16) + 16 ((c % 16) / 4))
 *   * 4 + c % 4 (16 x 16 blocks in the MFMA accumulator order).  Other
 *   bytes are not written.  Pass h, the same routing and the same
 *   workspace's dispatch to moe_backward_saved_h.
 * Errors as moe_expert_ffn_waved, plus MOE_ERR_INVALID_ARG for a NULL or
 * misaligned h. */
/* Bytes of the h buffer of moe_expert_ffn_waved_save_h / moe_backward_saved_h:
 * P_pad * gr * I * 4 with P_pad = P_max + 64 E_local rounded up to 64 (0
 * for an invalid problem). */
size_t moe_saved_h_bytes(const moe_problem_t* p);

moe_status_t moe_expert_ffn_waved_save_h(const moe_problem_t* p, const void* x, const void* packed,
                                         const int32_t* expert_offsets, const int32_t* sorted_token,
                                         const int32_t* pair_pos, const float* topk_w,
                                         const int32_t* token_ready_wave, void* y, void* out, float* h,
                                         uint32_t flags, void* ws, size_t ws_bytes, moe_stream_t stream);

/* FP8 dispatch (digest section 1.4, compute/communication bullet: tokens go
 * to the experts in FP8, results come back in BF16).  Per token t:
 * scale[t] = 2^k, k the smallest integer with max_i |x[t, i]| <= 448 * 2^k
 * (1 for an all-zero row), and x_fp8[t, i] = the OCP E4M3 code nearest to
 * x[t, i] / scale[t] (ties to even; a negative value that rounds to zero
 * gives -0).  The scale granularity and the format details are not on the
 * pages; an e4m3 value times a power of two is exact in bf16.
 *   x [T, d] in x_dtype.  Out: x_fp8 [T, d] bytes, x_scale [T] fp32. */
moe_status_t moe_quantize_fp8(const moe_problem_t* p, const void* x, uint8_t* x_fp8, float* x_scale,
                              moe_stream_t stream);

/* moe_expert_ffn_waved with the token-order staging buffer in FP8: the
 * GEMM1 tiles pull the e4m3 rows (d bytes per routed pair instead of 2d)
 * and convert them to bf16 times the token's scale in registers; results are
 * bit-identical to moe_expert_ffn_waved run on the dequantized rows
 * (x_fp8 * x_scale, exact in bf16).  Arguments as for moe_expert_ffn_waved,
 * with x replaced by x_fp8 [T, d] and x_scale [T] from moe_quantize_fp8. */
moe_status_t moe_expert_ffn_waved_fp8(const moe_problem_t* p, const uint8_t* x_fp8, const float* x_scale,
                                      const void* packed, const int32_t* expert_offsets,
                                      const int32_t* sorted_token, const int32_t* pair_pos,
                                      const float* topk_w, const int32_t* token_ready_wave, void* y,
                                      void* out, uint32_t flags, void* ws, size_t ws_bytes,
                                      moe_stream_t stream);

/* Combine (digest section 1.1; 10100.com deterministic operators): for each
 * token, out[t] = sum over ranks j = 0..k-1 with pair_pos[t, j] >= 0 of
 * topk_w[t, j] * y[pair_pos[t, j]], accumulated in fp32 with fused
 * multiply-adds in ascending j, rounded once to out_dtype.  No atomics.
 *   y [P_max, d] bf16; pair_pos [T, k]; topk_w [T, k]; out [T, d]. */
moe_status_t moe_combine(const moe_problem_t* p, const void* y, const int32_t* pair_pos,
                         const float* topk_w, void* out, moe_stream_t stream);

/* Deterministic weight gradient of L = <dout, out> (10100.com deterministic
 * operators; digest section 3: isolated per-block buffers reduced in a fixed
 * order, no float atomics).  With dy = topk_w[t, j] * dout[t] per routed row:
 *   dW2_e = a^T dy,  dW1_e = x^T dH1,  dW3_e = x^T dH3,
 *   dA = dy W2_e^T,  dH3 = dA * silu(h1),
 *   dH1 = dA * h3 * s * (1 + h1 (1 - s)),  s = sigmoid(h1),
 * with h1, h3 recomputed exactly as the forward computes them; RELU2:
 *   dH1 = (2 dA) * max(h1, 0), a = max(h1, 0)^2, no dW3.
 *   packed, packed_bwd: from moe_pack_weights and moe_pack_weights_bwd.
 *   dout [T, d] bf16.  Out (fp32, math layout): dW1, dW3 [E_local, d, I]
 *   (dW3 NULL for RELU2, required for SWIGLU), dW2 [E_local, I, d], every
 *   element written.  ws: the MOE_WS_BACKWARD size. */
moe_status_t moe_expert_wgrad(const moe_problem_t* p, const void* x, const void* packed,
                              const void* packed_bwd, const int32_t* expert_offsets,
                              const int32_t* sorted_token,
                              const int32_t* pair_pos, const float* topk_w, const void* dout,
                              float* dW1, float* dW3, float* dW2, void* ws, size_t ws_bytes,
                              moe_stream_t stream);

/* Backward of the layer share: data gradient, router gradients and
 * (optionally) the expert weight gradient of L = <dout, out>, with the
 * routing held fixed (the top-k choice is piecewise constant in the logits).
 * Deterministic and batch invariant (10100.com deterministic operators;
 * digest section 3): no float atomics; every per-token result depends on
 * the token's own rows only; reductions over tokens use fixed chunks summed
 * in ascending order.  With dy = topk_w[t, j] * dout[t] per routed row and
 * h1, h3 recomputed exactly as the forward computes them:
 *   dA = dy W2^T, dH3 = dA * silu(h1), dH1 = dA * h3 * s * (1 + h1 (1 - s))
 *     (RELU2: dH1 = (2 dA) * max(h1, 0), no dH3),
 *   dtopk_w[t, j] = <dout[t], y> = <dout[t] W2^T, silu(h1) * h3> for a local
 *     pick (summed from fixed partials over 32 intermediate indices), 0 for a
 *     pick whose expert is not local;
 *   dl[t, j] = topk_w[t, j] * (dtopk_w[t, j] - sum_m topk_w[t, m] dtopk_w[t, m])
 *     (renormalised softmax over the picks), 0 off the picks;
 *   dx[t] = sum_j [local] (dH1 W1^T + dH3 W3^T) of the pick's row (each row
 *     rounded to bf16, summed in fp32 in ascending j) + sum_j dl[t, j]
 *     Wg[:, idx[t, j]] (fp32 fused multiply-adds, ascending j), rounded once
 *     to x_dtype;
 *   dWg = x^T dl (bf16 x: dl rounded to bf16, MFMA products over chunks of
 *     1024 tokens, chunk partials summed in ascending order; fp32 x: fp32
 *     fused multiply-adds in ascending token order).
 * On an expert-parallel share these are this GPU's additive shares of the
 * layer's gradients (out is this GPU's partial sum).
 *   x, packed, topk_idx, topk_w, expert_offsets, sorted_token, pair_pos: as
 *   in the forward (same workspace after moe_dispatch, of the
 *   MOE_WS_BACKWARD size); packed_bwd from moe_pack_weights_bwd; dout [T, d]
 *   bf16.
 *   Out: dx [T, d] in x_dtype (required when T > 0); dtopk_w [T, k] fp32,
 *   dlogits [T, E_global] fp32 (dense, zeros off the picks), dWg
 *   [d, E_global] fp32: each optional (NULL = not computed); dW1, dW3 [E_local,
 *   d, I] and dW2 [E_local, I, d] fp32: all three or none (RELU2: dW1 and
 *   dW2 or neither, dW3 NULL), the same bits as moe_expert_wgrad. */
moe_status_t moe_backward(const moe_problem_t* p, const void* x, const void* packed,
                          const void* packed_bwd, const int32_t* topk_idx, const float* topk_w,
                          const int32_t* expert_offsets, const int32_t* sorted_token,
                          const int32_t* pair_pos, const void* dout, void* dx, float* dtopk_w,
                          float* dlogits, float* dWg, float* dW1, float* dW3, float* dW2, void* ws,
                          size_t ws_bytes, moe_stream_t stream);

/* moe_backward with h1, h3 read from h (written by moe_expert_ffn_waved_save_h
 * on the same x, weights and dispatch) instead of recomputed: the first
 * GEMM, half of the backward's matrix products before the weight gradient,
 * is skipped.  The stored values are the accumulators the recomputation
 * produces, so every output is bit-identical to moe_backward's.  Arguments
 * as moe_backward, plus h (moe_saved_h_bytes(p) bytes, 16-byte aligned,
 * required when T > 0; only the routed rows are read). */
moe_status_t moe_backward_saved_h(const moe_problem_t* p, const void* x, const void* packed,
                                  const void* packed_bwd, const int32_t* topk_idx, const float* topk_w,
                                  const int32_t* expert_offsets, const int32_t* sorted_token,
                                  const int32_t* pair_pos, const void* dout, const float* h, void* dx,
                                  float* dtopk_w, float* dlogits, float* dWg, float* dW1, float* dW3,
                                  float* dW2, void* ws, size_t ws_bytes, moe_stream_t stream);

/* Synchronises `stream`, then reads the device error word of the workspace
 * (set by a bounded wait of moe_expert_ffn_waved that expired) and clears
 * it.  moe_dispatch clears the word when a layer call starts; a workspace
 * must be zero-filled once when allocated.  Returns MOE_OK, MOE_ERR_TIMEOUT
 * or MOE_ERR_HIP. */
moe_status_t moe_check_error(void* ws, moe_stream_t stream);

/* Static English text of a status code. */
const char* moe_status_string(moe_status_t s);

/* Library build identification (static string). */
const char* moe_version(void);

/* ------------------------------------------------------------ measurement probes
 * Not part of the layer: they measure, on the running device, the two
 * denominators the layer's kernels are compared against (the matrix-core
 * rate and the HBM copy rate), next to the published peaks. */

/* One launch of a matrix-core loop: every wavefront (8 per workgroup, one
 * workgroup per CU) runs `steps` rounds of 16 independent
 * v_mfma_f32_16x16x32_bf16 on register operands.  out: device, at least
 * num_cus * 512 floats (one sum per thread keeps the work alive).  *flops
 * receives the launch's FLOP count (num_cus * 8 * steps * 16 * 16384).
 * steps in [1, 2^20]; MOE_ERR_INVALID_ARG otherwise or when out is too small. */
moe_status_t moe_probe_mfma(float* out, size_t out_bytes, int32_t steps, double* flops, moe_stream_t stream);

/* One launch of a plain device-to-device copy of `bytes` (a multiple of 16;
 * src and dst 16-byte aligned and not overlapping): 2 * bytes of HBM traffic. */
moe_status_t moe_probe_copy(void* dst, const void* src, size_t bytes, moe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
