// route.hip -- router: logits, top-k, renormalised weights.
//
// The layer definition fixes the router as softmax over all experts, top-k,
// and renormalisation of the k weights (the pages name it only as the "MoE
// Routing" kernel of TileKernels: DeepSeek-V4 launch digest, itsolotime.com,
// section 1.3).  Softmax followed by renormalisation over the picks equals
// exp(l_j - l_max) / sum_{picks} exp(l_j' - l_max), and softmax is monotone,
// so the kernel selects on the fp32 logits and exponentiates only the k
// picks.
//
// Batch invariance (digest section 3): a token's logits come from its own
// row only (the fixed-K-order MFMA tile for bf16 x, a fixed ascending fma
// chain for fp32 x), and one wavefront does the token's selection in a
// fixed reduction order.
#include "gemm_tile.h"
#include "moe_internal.h"
#include "route_topk.h"

namespace moe {
namespace {

// ---------------------------------------------------------------- logits, bf16 x

// Partial logits of K range [s * ks, (s + 1) * ks), s = blockIdx.y: the
// reduction over d is cut into a fixed number of ranges that depends on the
// layer only (router_splits: d and the number of experts), so every token
// sees the same summation order at any batch size; topk_kernel adds the
// ranges in ascending s.
template <class C>
__global__ __launch_bounds__(256) void router_logits_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg, float* __restrict__ partial,
    int T, int d, int E, int ks) {
  extern __shared__ __align__(16) uint16_t lds[];
  const int nblk_e = (E + C::BW - 1) / C::BW;
  const int et = blockIdx.x % nblk_e, tt = blockIdx.x / nblk_e;
  const int split = blockIdx.y;
  const int t0 = tt * C::BT;
  TokRows<C> trow;
#pragma unroll
  for (int i = 0; i < C::LT; ++i) {
    const int t = min(t0 + trow_index<C>(i), T - 1);
    trow.p[i] = x + static_cast<size_t>(t) * d + static_cast<size_t>(split) * ks;
  }
  TileAcc<C> acc;
  tile_mma<C>(wg + frag_offset(et * C::BW / 16, split * (ks / 32), d / 32), d / 32, ks / C::BK, trow, lds, acc);
  float* out = partial + static_cast<size_t>(split) * T * E;
  const int lane = lane_id();
  const int wr = tile_wr<C>(), wt = tile_wt<C>();
#pragma unroll
  for (int a = 0; a < C::AW; ++a) {
    const int e0 = et * C::BW + (wr * C::AW + a) * 16 + 4 * (lane / 16);
#pragma unroll
    for (int b = 0; b < C::AT; ++b) {
      const int t = t0 + (wt * C::AT + b) * 16 + (lane & 15);
      if (t >= T) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = e0 + r;
        if (e < E) out[static_cast<size_t>(t) * E + e] = acc.v[a][b][r];
      }
    }
  }
}

// ---------------------------------------------------------------- logits, fp32 x

// One thread per (token, expert); sum over the hidden index in ascending
// order with explicit fused multiply-adds.
__global__ __launch_bounds__(256) void router_logits_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ wg, float* __restrict__ logits, int T, int d,
    int E, int Epad) {
  const size_t id = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (id >= static_cast<size_t>(T) * E) return;
  const int t = static_cast<int>(id / E), e = static_cast<int>(id % E);
  const float* xr = x + static_cast<size_t>(t) * d;
  float acc = 0.f;
  for (int i = 0; i < d; ++i) acc = fmaf(xr[i], wg[static_cast<size_t>(i) * Epad + e], acc);
  logits[id] = acc;
}

// ---------------------------------------------------------------- top-k

// One wavefront per token (topk_token in route_topk.h).
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ partial, int splits,
                                                   const float* __restrict__ bias, int T, int E,
                                                   int k, int32_t* __restrict__ topk_idx,
                                                   float* __restrict__ topk_w, float* __restrict__ logits) {
  const int t = blockIdx.x * 4 + wave_id();
  if (t >= T) return;
  topk_token(partial, splits, bias, T, E, k, t, topk_idx, topk_w, logits);
}

template <class C>
hipError_t launch_logits_mfma(const moe_problem_t& p, const void* x, const uint16_t* wg,
                              float* partial, int splits, hipStream_t s) {
  const int nblk_e = (p.E_global + C::BW - 1) / C::BW;
  const int nblk_t = (p.T + C::BT - 1) / C::BT;
  router_logits_mfma_kernel<C><<<dim3(nblk_e * nblk_t, splits), 256, C::LDS_BYTES, s>>>(
      static_cast<const uint16_t*>(x), wg, partial, p.T, p.d, p.E_global, p.d / splits);
  return hipGetLastError();
}

}  // namespace

int router_splits(int d, int E_global, bool x_bf16) {
  if (!x_bf16) return 1;
  // wide routers (many experts) already have work for the whole chip, and
  // their partial logits would cost more traffic than the split saves
  for (int sp = E_global > 64 ? 2 : 8; sp > 1; sp >>= 1)
    if ((d / 64) % sp == 0) return sp;
  return 1;
}

hipError_t launch_route_logits(const moe_problem_t& p, const void* x, const void* packed, float* partial,
                               hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  const bool xbf = p.x_dtype == MOE_BF16;
  const PackedLayout L = packed_layout(p.d, p.I, p.E_global, p.E_local, xbf, gate_rows(p));
  const char* base = static_cast<const char*>(packed);
  const int splits = router_splits(p.d, p.E_global, xbf);
  if (xbf) {
    // token tiles of 32 or 64 rows and the K split give the logits product
    // hundreds of workgroups at the mid and V3/V4 sizes and keep a decode
    // step's reduction short
    const uint16_t* wg = reinterpret_cast<const uint16_t*>(base + L.router);
    if (p.E_global <= 32) return launch_logits_mfma<TileCfg<32, 32, 2, 2, 64, 4>>(p, x, wg, partial, splits, s);
    if (p.E_global <= 64) return launch_logits_mfma<TileCfg<64, 32, 2, 2, 64, 4>>(p, x, wg, partial, splits, s);
    return launch_logits_mfma<TileCfg<128, 128, 2, 2, 64, 3>>(p, x, wg, partial, splits, s);
  }
  const size_t n = static_cast<size_t>(p.T) * p.E_global;
  router_logits_f32_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(
      static_cast<const float*>(x), reinterpret_cast<const float*>(base + L.router), partial, p.T, p.d,
      p.E_global, L.Epad);
  return hipGetLastError();
}

hipError_t launch_topk(const moe_problem_t& p, const float* partial, const float* bias, int32_t* topk_idx,
                       float* topk_w, float* logits, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  const int splits = router_splits(p.d, p.E_global, p.x_dtype == MOE_BF16);
  topk_kernel<<<(p.T + 3) / 4, 256, 0, s>>>(partial, splits, bias, p.T, p.E_global, p.k, topk_idx, topk_w,
                                            logits);
  return hipGetLastError();
}

hipError_t launch_route(const moe_problem_t& p, const void* x, const void* packed,
                        const float* bias, int32_t* topk_idx, float* topk_w, float* logits,
                        float* partial, hipStream_t s) {
  hipError_t e = launch_route_logits(p, x, packed, partial, s);
  if (e != hipSuccess) return e;
  return launch_topk(p, partial, bias, topk_idx, topk_w, logits, s);
}

}  // namespace moe
