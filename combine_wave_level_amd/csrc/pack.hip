// pack.hip -- one-time re-layout of router and expert weights into the
// MFMA fragment layout described in moe_common.h.  Not on the per-batch
// path: weights are parameters and are packed once.
#include "moe_internal.h"

namespace moe {
namespace {

// Reads element (k, n) of a math-layout source S[K][N] (row stride ld).
template <bool SRC_BF16>
__device__ __forceinline__ uint16_t src_bf16(const void* src, size_t k, size_t n, size_t ld) {
  if constexpr (SRC_BF16) {
    return static_cast<const uint16_t*>(src)[k * ld + n];
  } else {
    return f32_to_bf16(static_cast<const float*>(src)[k * ld + n]);
  }
}

// Writes M = S^T ([N][K], N rows) in fragment layout.  One thread produces
// one 16-byte slot: row n, k-group (8 k values).  Consecutive threads take
// consecutive n, so each of the 8 strided source reads is coalesced.
// mode 0: plain transpose of S (N = n_src columns; rows >= n_src are zero).
// mode 1: W1/W3 interleave: packed row block 2b <- W1 columns 16b.., block
//         2b+1 <- W3 columns 16b.. (S = W1, S2 = W3, each [K][N/2]).
// mode 2: no transpose: the source already is M[N][K] (row stride K); the
//         8 values of a slot are one contiguous 16-byte read.
// mode 3: no transpose, K concatenated: k < K/2 from S, k >= K/2 from S2,
//         each [N][K/2] (row stride K/2).
template <bool SRC_BF16, int MODE>
__global__ void pack_frag_kernel(const void* __restrict__ S, const void* __restrict__ S2,
                                 uint16_t* __restrict__ dst, int K, int N, int n_src,
                                 size_t src_mat_stride, size_t dst_mat_stride) {
  const int mat = blockIdx.y;
  const size_t n = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int KG = K / 8;  // k-groups
  // grid.x covers N * KG slots with n fastest inside a k-group
  const size_t slot = n;
  if (slot >= static_cast<size_t>(N) * KG) return;
  const int row = static_cast<int>(slot % N);
  const int kg = static_cast<int>(slot / N);
  const char* base = static_cast<const char*>(S) + mat * src_mat_stride * (SRC_BF16 ? 2 : 4);
  const char* base2 = S2 ? static_cast<const char*>(S2) + mat * src_mat_stride * (SRC_BF16 ? 2 : 4)
                         : nullptr;
  uint16_t v[8];
  if (MODE == 2) {
    for (int e = 0; e < 8; ++e) v[e] = src_bf16<SRC_BF16>(base, row, static_cast<size_t>(kg) * 8 + e, K);
  } else if (MODE == 3) {
    const size_t half = static_cast<size_t>(K / 2), k0 = static_cast<size_t>(kg) * 8;
    const void* src = k0 < half ? base : base2;
    const size_t kk = k0 < half ? k0 : k0 - half;
    for (int e = 0; e < 8; ++e) v[e] = src_bf16<SRC_BF16>(src, row, kk + e, half);
  } else if (MODE == 0) {
    for (int e = 0; e < 8; ++e)
      v[e] = row < n_src ? src_bf16<SRC_BF16>(base, static_cast<size_t>(kg) * 8 + e, row, n_src) : 0;
  } else {
    const int blk = row / 16, within = row % 16;
    const int col = (blk / 2) * 16 + within;
    const void* src = (blk & 1) ? base2 : base;
    for (int e = 0; e < 8; ++e) v[e] = src_bf16<SRC_BF16>(src, static_cast<size_t>(kg) * 8 + e, col, n_src);
  }
  const int nb = row / 16, r = row % 16, kb = kg / 4, g = kg % 4;
  uint16_t* out = dst + mat * dst_mat_stride + frag_offset(nb, kb, K / 32) + (g * 16 + r) * 8;
  u32x4 pk;
  pk.x = v[0] | (static_cast<uint32_t>(v[1]) << 16);
  pk.y = v[2] | (static_cast<uint32_t>(v[3]) << 16);
  pk.z = v[4] | (static_cast<uint32_t>(v[5]) << 16);
  pk.w = v[6] | (static_cast<uint32_t>(v[7]) << 16);
  st16(out, pk);
}

// fp32 router weights stay in math layout [d][E_global]; rows padded to Epad
// columns with zeros.
__global__ void pack_router_f32_kernel(const float* __restrict__ Wg, float* __restrict__ dst, int d,
                                       int E, int Epad) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<size_t>(d) * Epad) return;
  const int row = static_cast<int>(i / Epad), col = static_cast<int>(i % Epad);
  dst[i] = col < E ? Wg[static_cast<size_t>(row) * E + col] : 0.f;
}

// Wg [d][E] -> Wg^T [E][d], element type kept (uint16 bf16 bits or fp32).
template <class T>
__global__ void transpose_kernel(const T* __restrict__ src, T* __restrict__ dst, int d, int E) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<size_t>(d) * E) return;
  const size_t e = i / d, row = i % d;
  dst[i] = src[row * E + e];
}

}  // namespace

hipError_t launch_pack_bwd(const moe_problem_t& p, const void* Wg, const void* W1, const void* W3,
                           const void* W2, void* packed_bwd, hipStream_t s) {
  const PackedBwdLayout L = packed_bwd_layout(p);
  char* base = static_cast<char*>(packed_bwd);
  const int threads = 256;
  const size_t n = static_cast<size_t>(p.d) * p.E_global;
  const unsigned blocks = static_cast<unsigned>((n + threads - 1) / threads);
  if (p.x_dtype == MOE_BF16)
    transpose_kernel<uint16_t><<<blocks, threads, 0, s>>>(static_cast<const uint16_t*>(Wg),
                                                          reinterpret_cast<uint16_t*>(base + L.wgt), p.d, p.E_global);
  else
    transpose_kernel<float><<<blocks, threads, 0, s>>>(static_cast<const float*>(Wg),
                                                       reinterpret_cast<float*>(base + L.wgt), p.d, p.E_global);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t src_stride = static_cast<size_t>(p.d) * p.I;
  uint16_t* dst = reinterpret_cast<uint16_t*>(base + L.w13t);
  if (p.activation == MOE_ACT_SWIGLU) {
    // [W1 | W3]^T: [d][2I] per expert, K = 2I
    const size_t slots = static_cast<size_t>(p.d) * (2 * p.I / 8);
    dim3 grid(static_cast<unsigned>((slots + threads - 1) / threads), p.E_local);
    const size_t dst_stride = static_cast<size_t>(p.d) * 2 * p.I;
    if (p.w_dtype == MOE_BF16)
      pack_frag_kernel<true, 3><<<grid, threads, 0, s>>>(W1, W3, dst, 2 * p.I, p.d, p.I, src_stride, dst_stride);
    else
      pack_frag_kernel<false, 3><<<grid, threads, 0, s>>>(W1, W3, dst, 2 * p.I, p.d, p.I, src_stride, dst_stride);
  } else {
    // ungated: W1 itself is [d][I] = the dx product's weights with K = I
    const size_t slots = static_cast<size_t>(p.d) * (p.I / 8);
    dim3 grid(static_cast<unsigned>((slots + threads - 1) / threads), p.E_local);
    if (p.w_dtype == MOE_BF16)
      pack_frag_kernel<true, 2><<<grid, threads, 0, s>>>(W1, nullptr, dst, p.I, p.d, p.I, src_stride, src_stride);
    else
      pack_frag_kernel<false, 2><<<grid, threads, 0, s>>>(W1, nullptr, dst, p.I, p.d, p.I, src_stride, src_stride);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // W2 as [I][d] (K = d) for dA = dy W2^T
  {
    const size_t slots2 = static_cast<size_t>(p.I) * (p.d / 8);
    dim3 grid2(static_cast<unsigned>((slots2 + threads - 1) / threads), p.E_local);
    const size_t stride = static_cast<size_t>(p.d) * p.I;
    uint16_t* dst2 = reinterpret_cast<uint16_t*>(base + L.w2b);
    if (p.w_dtype == MOE_BF16)
      pack_frag_kernel<true, 2><<<grid2, threads, 0, s>>>(W2, nullptr, dst2, p.d, p.I, p.I, stride, stride);
    else
      pack_frag_kernel<false, 2><<<grid2, threads, 0, s>>>(W2, nullptr, dst2, p.d, p.I, p.I, stride, stride);
  }
  return hipGetLastError();
}

hipError_t launch_pack(const moe_problem_t& p, const void* Wg, const void* W1, const void* W3,
                       const void* W2, void* packed, hipStream_t s) {
  const bool xbf = p.x_dtype == MOE_BF16;
  const bool wbf = p.w_dtype == MOE_BF16;
  const PackedLayout L = packed_layout(p.d, p.I, p.E_global, p.E_local, xbf, gate_rows(p));
  char* base = static_cast<char*>(packed);
  const int threads = 256;
  // router
  if (xbf) {
    const size_t slots = static_cast<size_t>(L.Epad) * (p.d / 8);
    dim3 grid(static_cast<unsigned>((slots + threads - 1) / threads), 1);
    pack_frag_kernel<true, 0><<<grid, threads, 0, s>>>(Wg, nullptr,
        reinterpret_cast<uint16_t*>(base + L.router), p.d, L.Epad, p.E_global, 0, 0);
  } else {
    const size_t n = static_cast<size_t>(p.d) * L.Epad;
    pack_router_f32_kernel<<<static_cast<unsigned>((n + threads - 1) / threads), threads, 0, s>>>(
        static_cast<const float*>(Wg), reinterpret_cast<float*>(base + L.router), p.d, p.E_global,
        L.Epad);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.E_local == 0) return hipSuccess;
  if (p.activation != MOE_ACT_SWIGLU) {
    // ungated: W1^T as [I][d] per expert, K = d
    const size_t slots = static_cast<size_t>(p.I) * (p.d / 8);
    dim3 grid(static_cast<unsigned>((slots + threads - 1) / threads), p.E_local);
    const size_t stride = static_cast<size_t>(p.d) * p.I;
    uint16_t* dst = reinterpret_cast<uint16_t*>(base + L.w13);
    if (wbf)
      pack_frag_kernel<true, 0><<<grid, threads, 0, s>>>(W1, nullptr, dst, p.d, p.I, p.I, stride, stride);
    else
      pack_frag_kernel<false, 0><<<grid, threads, 0, s>>>(W1, nullptr, dst, p.d, p.I, p.I, stride, stride);
  } else {
    // W13: [2I][d] per expert, K = d
    const size_t slots = static_cast<size_t>(2 * p.I) * (p.d / 8);
    dim3 grid(static_cast<unsigned>((slots + threads - 1) / threads), p.E_local);
    const size_t src_stride = static_cast<size_t>(p.d) * p.I;
    const size_t dst_stride = static_cast<size_t>(2 * p.I) * p.d;
    uint16_t* dst = reinterpret_cast<uint16_t*>(base + L.w13);
    if (wbf)
      pack_frag_kernel<true, 1><<<grid, threads, 0, s>>>(W1, W3, dst, p.d, 2 * p.I, p.I, src_stride, dst_stride);
    else
      pack_frag_kernel<false, 1><<<grid, threads, 0, s>>>(W1, W3, dst, p.d, 2 * p.I, p.I, src_stride, dst_stride);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // W2^T: [d][I] per expert, K = I
  {
    const size_t slots = static_cast<size_t>(p.d) * (p.I / 8);
    dim3 grid(static_cast<unsigned>((slots + threads - 1) / threads), p.E_local);
    const size_t stride = static_cast<size_t>(p.d) * p.I;
    uint16_t* dst = reinterpret_cast<uint16_t*>(base + L.w2);
    if (wbf)
      pack_frag_kernel<true, 0><<<grid, threads, 0, s>>>(W2, nullptr, dst, p.I, p.d, p.d, stride, stride);
    else
      pack_frag_kernel<false, 0><<<grid, threads, 0, s>>>(W2, nullptr, dst, p.I, p.d, p.d, stride, stride);
  }
  return hipGetLastError();
}

}  // namespace moe
