// gemm_tile.h -- the one bf16 MFMA tile product used by the router logits
// and both expert GEMMs.
//
// A tile computes D[n][t] = sum_k Wt[n][k] * X[t][k] for BW weight rows n
// (output features) and BT token rows t, fp32 accumulation, K walked in
// BK-wide steps in ascending order, each step as ascending 32-wide MFMA
// k-slices.  Weights are the MFMA A operand (read from the packed fragment
// layout), tokens the B operand (gathered rows).  Whatever BW, BT, BK or wave
// arrangement a caller picks, every output element sees the same instruction
// sequence over K, so its bits depend only on its own weight row and token
// row: the batch invariance the DeepSeek-V4 kernel library asks for (launch
// digest, itsolotime.com, section 3; 10100.com commentary, batch-invariant
// operators: no split-K whose shape follows the batch size).
//
// Data movement (gfx950): both operands go global -> LDS with 16-byte
// direct-to-LDS loads (global_load_lds_dwordx4).  One such load of a
// wavefront writes 1 KiB of LDS linearly by lane, which is exactly one MFMA
// fragment in the fragment layout, for the packed weights and for gathered
// token rows alike; MFMA operands are then read back with conflict-free
// 16-byte LDS reads.  NST stages are in flight; completion is tracked with
// explicit vmcnt waits and raw barriers (a full __syncthreads would drain
// the prefetch of later stages at every step).
#pragma once

#include "moe_common.h"

namespace moe {

template <int BW_, int BT_, int WR_, int WT_, int BK_, int NST_>
struct TileCfg {
  static constexpr int BW = BW_, BT = BT_, WR = WR_, WT = WT_, BK = BK_, NST = NST_;
  static_assert(WR * WT == 4, "4 wavefronts per workgroup");
  static_assert(NST >= 2 && NST <= 4, "2 to 4 LDS stages");
  static_assert(BK % 32 == 0 && BK >= 32, "K step is whole MFMA k-slices");
  static_assert(BW % (16 * WR) == 0 && BT % (16 * WT) == 0, "wave tile must hold whole MFMA blocks");
  static constexpr int KS = BK / 32;            // MFMA k-slices per K step
  static constexpr int NFW = BW / 16 * KS;      // weight fragments per K step
  static constexpr int NFT = BT / 16 * KS;      // token fragments per K step
  static_assert(NFW % 4 == 0 && NFT % 4 == 0, "fragments split evenly over the 4 wavefronts");
  static constexpr int LW = NFW / 4;            // weight fragments each wave loads per step
  static constexpr int LT = NFT / 4;            // token fragments each wave loads per step
  static constexpr int AW = BW / WR / 16;       // MFMA row blocks per wave
  static constexpr int AT = BT / WT / 16;       // MFMA column blocks per wave
  static constexpr int STAGE = (NFW + NFT) * 512;  // bf16 elements per LDS stage
  static constexpr size_t LDS_BYTES = static_cast<size_t>(NST) * STAGE * 2;
  static_assert(LW + LT <= 63 / (NST > 1 ? NST - 1 : 1), "vmcnt budget");
};

// Accumulators of one wave: v[a][b] is the 16x16 block of weight row block
// (wr * AW + a) and token block (wt * AT + b) of the tile.
template <class C>
struct TileAcc {
  f32x4 v[C::AW][C::AT];
};

// Per-lane row pointers of the token fragments a wave loads (see tile_mma).
template <class C>
struct TokRows {
  const uint16_t* p[C::LT];
};

// Token fragment i of this wave (i < C::LT) covers token block tb and k-slice
// kc of the step; its rows in the tile are tb * 16 + (lane % 16).
template <class C>
__device__ __forceinline__ int tok_frag_block(int i) { return (4 * i + wave_id()) / C::KS; }
template <class C>
__device__ __forceinline__ int tok_frag_slice(int i) { return (4 * i + wave_id()) % C::KS; }

// Row index (0..BT-1) inside the tile of the token fragment i this lane loads.
template <class C>
__device__ __forceinline__ int trow_index(int i) {
  return tok_frag_block<C>(i) * 16 + (lane_id() & 15);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Issues this wave's direct-to-LDS loads of K step kt into stage kt % NST.
template <class C>
__device__ __forceinline__ void tile_issue(const uint16_t* __restrict__ wtile, int KB,
                                           const TokRows<C>& trow, uint16_t* lds, int kt) {
  const int lane = lane_id(), wave = wave_id();
  uint16_t* st = lds + (kt % C::NST) * C::STAGE;
#pragma unroll
  for (int i = 0; i < C::LW; ++i) {
    const int f = 4 * i + wave;  // weight fragment of the step
    const int nb = f / C::KS, kc = f % C::KS;
    __builtin_amdgcn_global_load_lds(wtile + frag_offset(nb, kt * C::KS + kc, KB) + lane * 8,
                                     st + f * 512, 16, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < C::LT; ++i) {
    const int f = 4 * i + wave;  // token fragment of the step
    const int kc = f % C::KS;
    __builtin_amdgcn_global_load_lds(trow.p[i] + kt * C::BK + kc * 32 + (lane >> 4) * 8,
                                     st + (C::NFW + f) * 512, 16, 0, 0);
  }
}

// Computes one tile.
//   wtile : packed weights, fragment (first row block of the tile, kb = 0)
//   KB    : fragments along K of that matrix (K / 32)
//   nk    : number of BK-wide K steps (K / BK); must be wave-uniform
//   trow  : for each token fragment this wave loads (i < C::LT), a pointer to
//           element k = 0 of this lane's token row (gathered and clamped to a
//           valid row by the caller)
//   lds   : C::LDS_BYTES of shared memory
// All 256 threads must call it.  On entry no direct-to-LDS load of this
// workgroup may be in flight; on exit none is, and a barrier has passed, so
// the caller may reuse lds right away.
template <class C>
__device__ __forceinline__ void tile_mma(const uint16_t* __restrict__ wtile, int KB, int nk,
                                         const TokRows<C>& trow, uint16_t* lds,
                                         TileAcc<C>& acc) {
  const int lane = lane_id(), wave = wave_id();
  const int wr = wave / C::WT, wt = wave % C::WT;
#pragma unroll
  for (int a = 0; a < C::AW; ++a)
#pragma unroll
    for (int b = 0; b < C::AT; ++b) acc.v[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // prologue: NST-1 steps in flight
#pragma unroll
  for (int s = 0; s < C::NST - 1; ++s)
    if (s < nk) tile_issue<C>(wtile, KB, trow, lds, s);

  for (int kt = 0; kt < nk; ++kt) {
    // this wave's loads of step kt are done once at most the later in-flight
    // steps remain outstanding
    const int later = min(C::NST - 2, nk - 1 - kt);
    if (later <= 0) {
      wait_vmcnt<0>();
    } else if constexpr (C::NST >= 3) {
      if (later == 1) wait_vmcnt<(C::LW + C::LT)>();
      else wait_vmcnt<(C::NST - 2) * (C::LW + C::LT)>();
    }
    __builtin_amdgcn_s_barrier();  // every wave's step-kt data is in LDS; stage (kt-1) is free
    if (kt + C::NST - 1 < nk) tile_issue<C>(wtile, KB, trow, lds, kt + C::NST - 1);
    const uint16_t* st = lds + (kt % C::NST) * C::STAGE;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 af[C::AW], bfr[C::AT];
#pragma unroll
      for (int a = 0; a < C::AW; ++a) af[a] = ld16(st + ((wr * C::AW + a) * C::KS + ks) * 512 + lane * 8);
#pragma unroll
      for (int b = 0; b < C::AT; ++b)
        bfr[b] = ld16(st + (C::NFW + (wt * C::AT + b) * C::KS + ks) * 512 + lane * 8);
#pragma unroll
      for (int a = 0; a < C::AW; ++a)
#pragma unroll
        for (int b = 0; b < C::AT; ++b) acc.v[a][b] = mfma16x16x32(af[a], bfr[b], acc.v[a][b]);
    }
  }
  // all LDS reads of this tile done before anyone refills the stages
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
}

}  // namespace moe
