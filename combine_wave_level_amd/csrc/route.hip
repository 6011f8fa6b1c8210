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

namespace moe {
namespace {

// ---------------------------------------------------------------- logits, bf16 x

template <class C>
__global__ __launch_bounds__(256) void router_logits_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg, const float* __restrict__ bias,
    float* __restrict__ logits, int T, int d, int E) {
  extern __shared__ __align__(16) uint16_t lds[];
  const int nblk_e = (E + C::BW - 1) / C::BW;
  const int et = blockIdx.x % nblk_e, tt = blockIdx.x / nblk_e;
  const int t0 = tt * C::BT;
  TokRows<C> trow;
#pragma unroll
  for (int i = 0; i < C::LT; ++i) {
    const int t = min(t0 + trow_index<C>(i), T - 1);
    trow.p[i] = x + static_cast<size_t>(t) * d;
  }
  TileAcc<C> acc;
  tile_mma<C>(wg + frag_offset(et * C::BW / 16, 0, d / 32), d / 32, d / C::BK, trow, lds, acc);
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
        if (e < E) logits[static_cast<size_t>(t) * E + e] = bias ? acc.v[a][b][r] + bias[e] : acc.v[a][b][r];
      }
    }
  }
}

// ---------------------------------------------------------------- logits, fp32 x

// One thread per (token, expert); sum over the hidden index in ascending
// order with explicit fused multiply-adds.
__global__ __launch_bounds__(256) void router_logits_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ wg, const float* __restrict__ bias,
    float* __restrict__ logits, int T, int d, int E, int Epad) {
  const size_t id = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (id >= static_cast<size_t>(T) * E) return;
  const int t = static_cast<int>(id / E), e = static_cast<int>(id % E);
  const float* xr = x + static_cast<size_t>(t) * d;
  float acc = 0.f;
  for (int i = 0; i < d; ++i) acc = fmaf(xr[i], wg[static_cast<size_t>(i) * Epad + e], acc);
  logits[id] = bias ? acc + bias[e] : acc;
}

// ---------------------------------------------------------------- top-k

// Order used by the selection: higher score first, lower expert id on ties.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// One wavefront per token; lane l holds experts l, l+64, l+128, l+192.
// k rounds of a butterfly arg-max; round j's winner is recorded by lane j.
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E,
                                                   int k, int32_t* __restrict__ topk_idx,
                                                   float* __restrict__ topk_w) {
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + wave_id();
  if (t >= T) return;
  float v[4];
  bool live[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    live[q] = e < E;
    v[q] = live[q] ? logits[static_cast<size_t>(t) * E + e] : 0.f;
  }
  float my_v = 0.f;
  int my_i = -1;
  for (int j = 0; j < k; ++j) {
    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (live[q] && better(v[q], lane + 64 * q, bv, bi)) {
        bv = v[q];
        bi = lane + 64 * q;
      }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const float ov = __shfl_xor(bv, m, kWave);
      const int oi = __shfl_xor(bi, m, kWave);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    // every lane now holds the same winner (the order is a total order)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (lane + 64 * q == bi) live[q] = false;
    if (lane == j) {
      my_v = bv;
      my_i = bi;
    }
  }
  const float vmax = __shfl(my_v, 0, kWave);
  const float ex = (lane < k) ? expf(my_v - vmax) : 0.f;
  float sum = 0.f;
  for (int j = 0; j < k; ++j) sum += __shfl(ex, j, kWave);  // ascending rank order
  if (lane < k) {
    topk_idx[static_cast<size_t>(t) * k + lane] = my_i;
    topk_w[static_cast<size_t>(t) * k + lane] = ex / sum;
  }
}

template <class C>
hipError_t launch_logits_mfma(const moe_problem_t& p, const void* x, const uint16_t* wg,
                              const float* bias, float* logits, hipStream_t s) {
  const int nblk_e = (p.E_global + C::BW - 1) / C::BW;
  const int nblk_t = (p.T + C::BT - 1) / C::BT;
  router_logits_mfma_kernel<C><<<nblk_e * nblk_t, 256, C::LDS_BYTES, s>>>(
      static_cast<const uint16_t*>(x), wg, bias, logits, p.T, p.d, p.E_global);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const moe_problem_t& p, const void* x, const void* packed,
                        const float* bias, int32_t* topk_idx, float* topk_w, float* logits,
                        hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  const bool xbf = p.x_dtype == MOE_BF16;
  const PackedLayout L = packed_layout(p.d, p.I, p.E_global, p.E_local, xbf);
  const char* base = static_cast<const char*>(packed);
  hipError_t e;
  if (xbf) {
    const uint16_t* wg = reinterpret_cast<const uint16_t*>(base + L.router);
    if (p.E_global <= 32)
      e = launch_logits_mfma<TileCfg<32, 128, 1, 4, 64, 3>>(p, x, wg, bias, logits, s);
    else if (p.E_global <= 64)
      e = launch_logits_mfma<TileCfg<64, 128, 2, 2, 64, 3>>(p, x, wg, bias, logits, s);
    else
      e = launch_logits_mfma<TileCfg<128, 128, 2, 2, 64, 3>>(p, x, wg, bias, logits, s);
  } else {
    const size_t n = static_cast<size_t>(p.T) * p.E_global;
    router_logits_f32_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(
        static_cast<const float*>(x), reinterpret_cast<const float*>(base + L.router), bias, logits,
        p.T, p.d, p.E_global, L.Epad);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  topk_kernel<<<(p.T + 3) / 4, 256, 0, s>>>(logits, p.T, p.E_global, p.k, topk_idx, topk_w);
  return hipGetLastError();
}

}  // namespace moe
