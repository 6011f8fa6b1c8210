// gemm_tile.h -- the one bf16 MFMA tile product used by the router logits
// and both expert GEMMs.
//
// A tile computes D[n][t] = sum_k Wt[n][k] * X[t][k] for BW weight rows n
// (output features) and BT token rows t, fp32 accumulation, K walked in
// 64-wide steps in ascending order, each step as two ascending 32-wide MFMA
// k-slices.  Weights are the MFMA A operand (read from the packed fragment
// layout), tokens the B operand (gathered rows, staged in LDS in the same
// fragment layout).  Whatever BW, BT or wave arrangement a caller picks,
// every output element sees the same instruction sequence over K, so its
// bits depend only on its own weight row and token row: the batch invariance
// the DeepSeek-V4 kernel library asks for (launch digest, itsolotime.com,
// section 3; 10100.com commentary, batch-invariant operators: no split-K
// whose shape follows the batch size).
#pragma once

#include "moe_common.h"

namespace moe {

template <int BW_, int BT_, int WR_, int WT_>
struct TileCfg {
  static constexpr int BW = BW_, BT = BT_, WR = WR_, WT = WT_;
  static_assert(WR * WT == 4, "4 wavefronts per workgroup");
  static_assert(BW % (16 * WR) == 0 && BT % (16 * WT) == 0, "wave tile must hold whole MFMA blocks");
  static constexpr int NFW = BW / 16 * 2;  // weight fragments per 64-wide K step
  static constexpr int NFT = BT / 16 * 2;  // token fragments per K step
  static constexpr int AW = BW / WR / 16;  // MFMA row blocks per wave
  static constexpr int AT = BT / WT / 16;  // MFMA column blocks per wave
  static constexpr int LW = (NFW + 3) / 4; // weight fragments each wave loads
  static constexpr int LT = (NFT + 3) / 4; // token fragments each wave loads
  static constexpr int STAGE = (NFW + NFT) * 512;        // bf16 elements per LDS stage
  static constexpr size_t LDS_BYTES = 2 * STAGE * 2;     // double buffered
};

// Accumulators of one wave: acc[a][b] is the 16x16 block of weight row block
// (wr * AW + a) and token block (wt * AT + b) of the tile.
template <class C>
struct TileAcc {
  f32x4 v[C::AW][C::AT];
};

// Computes one tile.
//   wtile : packed weights, fragment (first row block of the tile, kb = 0)
//   KB    : fragments along K of that matrix (K / 32)
//   nk    : number of 64-wide K steps (K / 64)
//   trow  : for each token fragment this thread loads (f = wave + 4 i), a
//           pointer to element k = 0 of its token row (already gathered
//           and clamped to a valid row by the caller)
//   lds   : C::LDS_BYTES of shared memory
// All 256 threads of the workgroup must call it.  Ends with a barrier so the
// caller may reuse lds right away.
template <class C>
__device__ __forceinline__ void tile_mma(const uint16_t* __restrict__ wtile, int KB, int nk,
                                         const uint16_t* const (&trow)[C::LT], uint16_t* lds,
                                         TileAcc<C>& acc) {
  const int lane = lane_id(), wave = wave_id();
  const int wr = wave / C::WT, wt = wave % C::WT;
  const int g = lane / 16;
#pragma unroll
  for (int a = 0; a < C::AW; ++a)
#pragma unroll
    for (int b = 0; b < C::AT; ++b) acc.v[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 wreg[C::LW], treg[C::LT];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < C::LW; ++i) {
      const int f = wave + 4 * i;
      if (f < C::NFW) {
        const int nb = f >> 1, kc = f & 1;
        wreg[i] = ld16(wtile + frag_offset(nb, 2 * kt + kc, KB) + lane * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < C::LT; ++i) {
      const int f = wave + 4 * i;
      if (f < C::NFT) {
        const int kc = f & 1;
        treg[i] = ld16(trow[i] + kt * 64 + kc * 32 + g * 8);
      }
    }
  };
  auto lstore = [&](int buf) {
    uint16_t* st = lds + buf * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::LW; ++i) {
      const int f = wave + 4 * i;
      if (f < C::NFW) st16(st + f * 512 + lane * 8, wreg[i]);
    }
#pragma unroll
    for (int i = 0; i < C::LT; ++i) {
      const int f = wave + 4 * i;
      if (f < C::NFT) st16(st + (C::NFW + f) * 512 + lane * 8, treg[i]);
    }
  };

  gload(0);
  lstore(0);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    __syncthreads();  // stage cur written; stage cur^1 no longer read
    if (kt + 1 < nk) gload(kt + 1);
    const uint16_t* st = lds + cur * C::STAGE;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 af[C::AW], bfr[C::AT];
#pragma unroll
      for (int a = 0; a < C::AW; ++a) af[a] = ld16(st + ((wr * C::AW + a) * 2 + ks) * 512 + lane * 8);
#pragma unroll
      for (int b = 0; b < C::AT; ++b)
        bfr[b] = ld16(st + (C::NFW + (wt * C::AT + b) * 2 + ks) * 512 + lane * 8);
#pragma unroll
      for (int a = 0; a < C::AW; ++a)
#pragma unroll
        for (int b = 0; b < C::AT; ++b) acc.v[a][b] = mfma16x16x32(af[a], bfr[b], acc.v[a][b]);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
  }
  __syncthreads();
}

// Row index (0..BT-1) inside the tile of the token fragment a thread loads.
template <class C>
__device__ __forceinline__ int trow_index(int i) {
  const int f = wave_id() + 4 * i;
  return (f >> 1) * 16 + (lane_id() & 15);
}

}  // namespace moe
