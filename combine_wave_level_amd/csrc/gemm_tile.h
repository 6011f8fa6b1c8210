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
//
// Gathered token rows are the costly operand: a load instruction whose
// lanes read 64 bytes from each of 16 rows costs the vector-memory path
// about 2.7 times as long per byte as one that reads whole 128-byte lines
// (measured on gfx950 with the data in L2: ~15 against ~42 B per clock per
// CU).  Tiles with TL set therefore fetch each token row as whole 128-byte
// lines, 64 k per row, covering two 32-wide K steps per load (see TileCfg).
#pragma once

#include "moe_common.h"

namespace moe {

template <int BW_, int BT_, int WR_, int WT_, int BK_, int NST_, bool SKIPB_ = false, bool FP8T_ = false,
          bool TCOH_ = false, bool WNT_ = false, bool TL_ = false>
struct TileCfg {
  static constexpr int BW = BW_, BT = BT_, WR = WR_, WT = WT_, BK = BK_, NST = NST_;
  // SKIPB: skip the MFMA work of every 16-row token block past the valid
  // rows (for tall token tiles that are mostly empty, as in small batches);
  // otherwise only a wave whose token rows are all invalid skips its work.
  static constexpr bool SKIPB = SKIPB_;
  // FP8T: the token rows are OCP e4m3 bytes with one scale per row (FP8
  // dispatch).  They go to LDS as bytes, 1 KiB = 16 rows x 64 k per wave
  // load, and each lane converts its 8 bytes to bf16 (times the row's scale)
  // right before the MFMA; K is still walked in the same ascending 32-wide
  // slices, so the products equal those of the bf16 rows of the dequantized
  // values, bit for bit.
  static constexpr bool FP8T = FP8T_;
  static_assert(!FP8T || BK % 64 == 0, "fp8 token fragments hold 64 k");
  // TCOH: the token rows are read with device-coherent loads (rows another
  // XCD wrote during the same kernel and wrote back from its L2).
  static constexpr bool TCOH = TCOH_;
  // WNT: the weight fragments are loaded with the non-temporal hint, for
  // shapes that stream each weight tile once (small batches: an expert's
  // weights serve one or two m-tiles).  Measured at decode T = 1: the FFN
  // 0.149 -> 0.138 ms; on the compute-bound shapes, whose weight tiles are
  // reused by several m-tiles through the L2, the hint cost up to 6%.
  static constexpr bool WNT = WNT_;
  // TL: token rows as whole 128-byte lines.  One wavefront load covers 8
  // rows x 64 k (8 lanes per row, 16 bytes each), i.e. the token operand of
  // two consecutive K steps; the token tile of such a double step (BT x 64
  // bf16) sits in one of two LDS slots after the NST weight stages.  Inside
  // a 1 KiB load block, row r's 16-byte chunk c (k = 8c .. 8c+7) is stored
  // at position c ^ (r % 8), which keeps the MFMA operand reads of 16 rows
  // free of LDS bank conflicts (measured on gfx950 with the conflict counter:
  // none for this swizzle, a quarter of the LDS cycles when the block's
  // parity is also XORed in, half with no swizzle).  Only the data movement differs:
  // the MFMA sequence over K, and so every result bit, is that of the same
  // tile without TL.
  static constexpr bool TL = TL_;
  static_assert(!TL || (BK == 32 && NST_ == 4 && !FP8T_ && BT_ % 8 == 0),
                "TL: 32-wide K steps, 4 weight stages, bf16 tokens");
  static constexpr int NW = WR * WT;            // wavefronts per workgroup
  static constexpr int NTHREADS = 64 * NW;
  static_assert(NW == 4 || NW == 8, "4 or 8 wavefronts per workgroup");
  static_assert(NST >= 2 && NST <= 8, "2 to 8 LDS stages");
  static_assert(BK % 32 == 0 && BK >= 32, "K step is whole MFMA k-slices");
  static_assert(BW % (16 * WR) == 0 && BT % (16 * WT) == 0, "wave tile must hold whole MFMA blocks");
  static constexpr int KS = BK / 32;            // MFMA k-slices per K step
  static constexpr int TKS = FP8T ? KS / 2 : KS;  // token fragments per 16-row block per K step
  static constexpr int NFW = BW / 16 * KS;      // weight fragments per K step
  static constexpr int NFT = BT / 16 * TKS;     // token fragments per K step
  static constexpr int NFT2 = BT / 8;           // TL: token loads (8 rows each) per double step
  static_assert(NFW % NW == 0 && (TL ? NFT2 % NW == 0 : NFT % NW == 0),
                "fragments split evenly over the wavefronts");
  static constexpr int LW = NFW / NW;           // weight fragments each wave loads per step
  // token loads each wave issues per step (TL: per double step)
  static constexpr int LT = TL ? NFT2 / NW : NFT / NW;
  static constexpr int AW = BW / WR / 16;       // MFMA row blocks per wave
  static constexpr int AT = BT / WT / 16;       // MFMA column blocks per wave
  // bf16 elements per LDS stage (TL: the weight fragments only)
  static constexpr int STAGE = (NFW + (TL ? 0 : NFT)) * 512;
  static constexpr int TSTAGE = TL ? BT * 64 : 0;  // TL: bf16 elements per token slot
  static constexpr size_t LDS_BYTES = (static_cast<size_t>(NST) * STAGE + 2 * TSTAGE) * 2;
  static_assert(TL ? 2 * LW + LT <= 63 : (NST - 1) * (LW + LT) <= 63,
                "vmcnt budget: NST-1 steps of loads in flight");
  // Register double-buffering of the MFMA operands (4 wavefronts, one per
  // SIMD).  With 8 wavefronts two share a SIMD and hide each other's LDS
  // latency; their register budget (256 per lane) has no room for a second
  // operand set.
  static constexpr bool DBUF = (NW == 4);
  static_assert(!TL || !DBUF, "TL: 8 wavefronts");
};

// Wave w of the workgroup computes weight row blocks wr * AW .. + AW - 1 and
// token blocks wt * AT .. + AT - 1 of the tile, wr = w % WR, wt = w / WR.
// With 8 wavefronts, waves w and w + 4 (which usually share a SIMD) hold the
// same weight rows and different tokens, so a partly filled token tile
// leaves each SIMD with the same amount of work.
template <class C>
__device__ __forceinline__ int tile_wr() { return wave_id() % C::WR; }
template <class C>
__device__ __forceinline__ int tile_wt() { return wave_id() / C::WR; }

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
__device__ __forceinline__ int tok_frag_block(int i) { return (C::NW * i + wave_id()) / C::TKS; }
template <class C>
__device__ __forceinline__ int tok_frag_slice(int i) { return (C::NW * i + wave_id()) % C::TKS; }

// Scales of this lane's token rows (FP8T only): s[b] for token block
// wt * AT + b.
template <class C>
struct TokScale {
  float s[C::FP8T ? C::AT : 1];
};

// Row index (0..BT-1) inside the tile of the token fragment i this lane loads
// (TL: of load block NW i + wave, 8 rows, 8 lanes per row).
template <class C>
__device__ __forceinline__ int trow_index(int i) {
  if constexpr (C::TL) return (C::NW * i + wave_id()) * 8 + (lane_id() >> 3);
  return tok_frag_block<C>(i) * 16 + (lane_id() & 15);
}

// s_waitcnt lgkmcnt(0) as the builtin, so that the compiler's own wait
// insertion knows LDS reads issued before it are complete; the empty asm
// keeps memory operations from moving across it.
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt(63) expcnt(7) lgkmcnt(0)
  asm volatile("" ::: "memory");
}

// Workgroup barrier without the waits of __syncthreads (which would drain
// the loads of later stages); the empty asm statements keep the compiler
// from moving memory operations across it.
__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// The same tile with device-coherent token-row loads.
template <class C>
using TokCoherent = TileCfg<C::BW, C::BT, C::WR, C::WT, C::BK, C::NST, C::SKIPB, C::FP8T, true, C::WNT, C::TL>;

// Issues this wave's direct-to-LDS loads of the weight fragments of K step kt
// into stage kt % NST.
template <class C>
__device__ __forceinline__ void tile_issue_w(const uint16_t* __restrict__ wtile, int KB, uint16_t* lds, int kt) {
  const int lane = lane_id(), wave = wave_id();
  uint16_t* st = lds + (kt % C::NST) * C::STAGE;
#pragma unroll
  for (int i = 0; i < C::LW; ++i) {
    const int f = C::NW * i + wave;  // weight fragment of the step
    const int nb = f / C::KS, kc = f % C::KS;
    if constexpr (C::WNT)
      lds_dma16_nt(wtile + frag_offset(nb, kt * C::KS + kc, KB) + lane * 8, st + f * 512);
    else
      lds_dma16(wtile + frag_offset(nb, kt * C::KS + kc, KB) + lane * 8, st + f * 512);
  }
}

// TL: the token lines of double step j (k = 64 j .. 64 j + 63) into token
// slot j % 2.  Load block b = NW i + wave holds rows 8b .. 8b+7; lane l
// takes row 8b + l/8 and the chunk that belongs at position l % 8, i.e.
// chunk (l % 8) ^ (l / 8).
template <class C>
__device__ __forceinline__ void tile_issue_tl(const TokRows<C>& trow, uint16_t* lds, int j) {
  const int lane = lane_id(), wave = wave_id();
  uint16_t* ts = lds + C::NST * C::STAGE + (j & 1) * C::TSTAGE;
#pragma unroll
  for (int i = 0; i < C::LT; ++i) {
    const int b = C::NW * i + wave;
    const int chunk = (lane & 7) ^ (lane >> 3);
    if constexpr (C::TCOH)
      lds_dma16_coherent(trow.p[i] + j * 64 + chunk * 8, ts + b * 512);
    else
      lds_dma16(trow.p[i] + j * 64 + chunk * 8, ts + b * 512);
  }
}

// Issues this wave's direct-to-LDS loads of K step kt into stage kt % NST.
template <class C>
__device__ __forceinline__ void tile_issue(const uint16_t* __restrict__ wtile, int KB,
                                           const TokRows<C>& trow, uint16_t* lds, int kt) {
  static_assert(!C::TL, "TL tiles issue weights and token lines separately");
  const int lane = lane_id(), wave = wave_id();
  uint16_t* st = lds + (kt % C::NST) * C::STAGE;
  tile_issue_w<C>(wtile, KB, lds, kt);
#pragma unroll
  for (int i = 0; i < C::LT; ++i) {
    const int f = C::NW * i + wave;  // token fragment of the step
    const int kc = f % C::TKS;
    if constexpr (C::FP8T) {
      // row bytes kt * BK + 64 kc .. + 63: lane l takes 16 of them
      const char* row = reinterpret_cast<const char*>(trow.p[i]);
      lds_dma16(row + kt * C::BK + kc * 64 + (lane >> 4) * 16, st + (C::NFW + f) * 512);
    } else if constexpr (C::TCOH) {
      lds_dma16_coherent(trow.p[i] + kt * C::BK + kc * 32 + (lane >> 4) * 8, st + (C::NFW + f) * 512);
    } else {
      lds_dma16(trow.p[i] + kt * C::BK + kc * 32 + (lane >> 4) * 8, st + (C::NFW + f) * 512);
    }
  }
}

// The MFMA operand of k-slice ks (0 .. KS-1 of a K step) of token block tb
// from an fp8 fragment in LDS: lane l needs row l % 16, k = 32 ks + 8 (l / 16)
// .. + 7, i.e. 8 bytes of the 1 KiB fragment that holds 64 k of the block
// (slot = 16 (k / 16) + row, 16 bytes each), converted to bf16 times scale.
template <class C>
__device__ __forceinline__ u32x4 fp8_token_frag(const uint16_t* st, int tb, int ks, float scale) {
  const int lane = lane_id();
  const int frag = tb * C::TKS + ks / 2, kin = (ks % 2) * 32 + 8 * (lane >> 4);
  const char* base = reinterpret_cast<const char*>(st + (C::NFW + frag) * 512);
  const u32x2 raw = *reinterpret_cast<const u32x2*>(base + ((kin / 16) * 16 + (lane & 15)) * 16 + (kin % 16));
  return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x, scale, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x, scale, true)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.y, scale, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.y, scale, true))};
}

// MFMA operands of one 32-wide k-slice for one wave.
template <class C>
struct TileFrags {
  u32x4 a[C::AW];
  u32x4 b[C::AT];
};

// ACT = false: none of this wave's token rows is valid; the wave then neither
// reads operands nor multiplies (its accumulators stay unused) but still
// takes part in the loads and barriers.
// nbv (C::SKIPB only, wave-uniform): token blocks of this wave that hold
// valid rows; blocks b >= nbv are neither read nor multiplied.
template <class C, bool ACT>
__device__ __forceinline__ void tile_read_frags(const uint16_t* st, int ks, TileFrags<C>& f, int nbv,
                                                const TokScale<C>& tsc) {
  if constexpr (!ACT) return;
  const int lane = lane_id();
  const int wr = tile_wr<C>(), wt = tile_wt<C>();
#pragma unroll
  for (int a = 0; a < C::AW; ++a) f.a[a] = ld16(st + ((wr * C::AW + a) * C::KS + ks) * 512 + lane * 8);
#pragma unroll
  for (int b = 0; b < C::AT; ++b)
    if (!C::SKIPB || b < nbv) {
      if constexpr (C::FP8T)
        f.b[b] = fp8_token_frag<C>(st, wt * C::AT + b, ks, tsc.s[b]);
      else
        f.b[b] = ld16(st + (C::NFW + (wt * C::AT + b) * C::KS + ks) * 512 + lane * 8);
    }
}

// TL: the operands of K step kt: weights from stage kt % NST, tokens from
// slot (kt / 2) % 2, k-slice kt % 2 of the slot's 64 k.
template <class C, bool ACT>
__device__ __forceinline__ void tile_read_frags_tl(const uint16_t* lds, int kt, TileFrags<C>& f, int nbv) {
  if constexpr (!ACT) return;
  const int lane = lane_id();
  const int wr = tile_wr<C>(), wt = tile_wt<C>();
  const uint16_t* st = lds + (kt % C::NST) * C::STAGE;
  const uint16_t* ts = lds + C::NST * C::STAGE + ((kt >> 1) & 1) * C::TSTAGE;
#pragma unroll
  for (int a = 0; a < C::AW; ++a) f.a[a] = ld16(st + (wr * C::AW + a) * 512 + lane * 8);
  // lane l: row 16 tb + l % 16 (block 2 tb + (l / 8) % 2, row l % 8 of it),
  // chunk 4 (kt % 2) + l / 16
  const int hb = (lane >> 3) & 1, rr = lane & 7;
  const int pos = (4 * (kt & 1) + (lane >> 4)) ^ rr;
  const uint16_t* tl = ts + hb * 512 + rr * 64 + pos * 8;
#pragma unroll
  for (int b = 0; b < C::AT; ++b)
    if (!C::SKIPB || b < nbv) f.b[b] = ld16(tl + (wt * C::AT + b) * 1024);
}

template <class C, bool ACT>
__device__ __forceinline__ void tile_mfma(const TileFrags<C>& f, TileAcc<C>& acc, int nbv) {
  if constexpr (!ACT) return;
#pragma unroll
  for (int b = 0; b < C::AT; ++b)
    if (!C::SKIPB || b < nbv) {
#pragma unroll
      for (int a = 0; a < C::AW; ++a) acc.v[a][b] = mfma16x16x32(f.a[a], f.b[b], acc.v[a][b]);
    }
}

// vmcnt wait that leaves `later` K steps of this wave's loads outstanding
// (0 <= later <= NST - 2; wave-uniform).
template <class C, int N>
__device__ __forceinline__ void wait_steps_left_from(int later) {
  if constexpr (N <= C::NST - 2) {
    if (later == N) wait_vmcnt<N * (C::LW + C::LT)>();
    else wait_steps_left_from<C, N + 1>(later);
  }
}
template <class C>
__device__ __forceinline__ void wait_steps_left(int later) {
  if (later <= 0) wait_vmcnt<0>();
  else wait_steps_left_from<C, 1>(later);
}

// One K step kt of the main loop.  On entry the operands of the step's first
// k-slice are in (or on their way to) the register set of parity PAR.  Each
// k-slice first starts the LDS reads of the next slice into the other set,
// then runs its MFMAs, so LDS latency hides behind the matrix core.  At the
// last slice the wave waits for step kt + 1, the workgroup passes a barrier
// (after which stage kt is fully consumed), step kt + NST is issued into that
// stage, and the next step's first slice is read.
template <class C, int PAR, bool ACT>
__device__ __forceinline__ void tile_step(const uint16_t* __restrict__ wtile, int KB, int nk, int kt,
                                          const TokRows<C>& trow, uint16_t* lds, TileFrags<C>& f0,
                                          TileFrags<C>& f1, TileAcc<C>& acc, int nbv, const TokScale<C>& tsc) {
  const uint16_t* st = lds + (kt % C::NST) * C::STAGE;
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    TileFrags<C>& cur = ((PAR + ks) & 1) ? f1 : f0;
    TileFrags<C>& nxt = ((PAR + ks) & 1) ? f0 : f1;
    // this slice's operands (read one slice earlier) have arrived; waiting
    // here, before the next reads go out, keeps the compiler from waiting
    // on those as well
    wait_lgkm0();
    if (ks + 1 < C::KS) {
      tile_read_frags<C, ACT>(st, ks + 1, nxt, nbv, tsc);
    } else if (kt + 1 < nk) {
      wait_steps_left<C>(min(C::NST - 2, nk - 2 - kt));
      raw_barrier();
      if (kt + C::NST < nk) tile_issue<C>(wtile, KB, trow, lds, kt + C::NST);
      tile_read_frags<C, ACT>(lds + ((kt + 1) % C::NST) * C::STAGE, 0, nxt, nbv, tsc);
    }
    __builtin_amdgcn_sched_barrier(0);
    tile_mfma<C, ACT>(cur, acc, nbv);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// TL: after iteration i's issues, wait for the loads of step i+1 (see
// tile_mma_run).
template <class C>
__device__ __forceinline__ void tl_wait_next(int i, int nk) {
  if (i + 1 >= nk) return;
  if (i & 1) {
    if (i + 3 < nk) wait_vmcnt<C::LW>(); else wait_vmcnt<0>();
  } else {
    if (i + 2 < nk) wait_vmcnt<2 * C::LW + C::LT>(); else wait_vmcnt<0>();
  }
}

template <class C, bool ACT>
__device__ __forceinline__ void tile_mma_run(const uint16_t* __restrict__ wtile, int KB, int nk,
                                             const TokRows<C>& trow, uint16_t* lds, TileAcc<C>& acc,
                                             int nbv, const TokScale<C>& tsc) {

  if constexpr (C::TL) {
    // Weights NST-1 = 3 steps ahead, token lines one double step ahead.  In
    // issue order: T(0), W(0), W(1), W(2), then iteration i issues W(i+3)
    // and, for even i, T(i/2+1).  After iteration i's issues, the loads
    // issued after the last one step i+1 needs are: even i (needs T(i/2),
    // issued with W(i+1) at iteration i-2): W(i+2), W(i+3), T(i/2+1); odd i
    // (needs T((i+1)/2), issued at iteration i-1): W(i+3) -- each only where
    // it exists.  K = 64 * (nk/2).
    //
    // Ping-pong: every wavefront runs the same loop body -- read step i's
    // operands, barrier, multiply step i, barrier -- but waves 4-7 pass one
    // extra barrier before the loop and waves 0-3 one after it, so the two
    // wavefronts of a SIMD (w and w + 4) run one phase apart: while one
    // multiplies, the other reads from LDS, and the matrix core no longer
    // waits out every step's read latency.  Both barriers of iteration i are
    // preceded by the wait for step i+1's loads (a wave reaches barrier
    // 2i+2, the one before step i+1's first read, through one of them) and
    // the first by lgkmcnt(0) (no stage is refilled before its last reader
    // has its data).  Measured against the same loop without the offset:
    // 4-8% faster tiles in a dense benchmark, same bits.
    const bool late = uniform(wave_id()) >= C::NW / 2;
    TileFrags<C> f;
    tile_issue_tl<C>(trow, lds, 0);
#pragma unroll
    for (int s = 0; s < C::NST - 1; ++s)
      if (s < nk) tile_issue_w<C>(wtile, KB, lds, s);
    if (nk > 2) wait_vmcnt<2 * C::LW>(); else wait_vmcnt<C::LW>();
    raw_barrier();
    if (late) raw_barrier();
    for (int i = 0; i < nk; ++i) {
      if (i + 3 < nk) tile_issue_w<C>(wtile, KB, lds, i + 3);
      if (!(i & 1) && i + 2 < nk) tile_issue_tl<C>(trow, lds, i / 2 + 1);
      tile_read_frags_tl<C, ACT>(lds, i, f, nbv);
      tl_wait_next<C>(i, nk);
      wait_lgkm0();
      raw_barrier();
      __builtin_amdgcn_sched_barrier(0);
      tile_mfma<C, ACT>(f, acc, nbv);
      __builtin_amdgcn_sched_barrier(0);
      tl_wait_next<C>(i, nk);
      raw_barrier();
    }
    if (!late) raw_barrier();
    wait_vmcnt<0>();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    raw_barrier();
  } else if constexpr (!C::DBUF) {
    // single operand set: steps 0 .. NST-2 in flight; step kt waits for its
    // own loads, passes a barrier (stage kt-1 is then free), issues step
    // kt + NST - 1 into that stage and computes from LDS
#pragma unroll
    for (int s = 0; s < C::NST - 1; ++s)
      if (s < nk) tile_issue<C>(wtile, KB, trow, lds, s);
    for (int kt = 0; kt < nk; ++kt) {
      wait_steps_left<C>(min(C::NST - 2, nk - 1 - kt));
      raw_barrier();
      if (kt + C::NST - 1 < nk) tile_issue<C>(wtile, KB, trow, lds, kt + C::NST - 1);
      const uint16_t* st = lds + (kt % C::NST) * C::STAGE;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        TileFrags<C> f;
        tile_read_frags<C, ACT>(st, ks, f, nbv, tsc);
        tile_mfma<C, ACT>(f, acc, nbv);
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    raw_barrier();
  } else {
    // prologue: steps 0 .. NST-2 in flight, wait for step 0, then issue step
    // NST-1 (at most NST-1 steps of loads are ever outstanding)
#pragma unroll
    for (int s = 0; s < C::NST - 1; ++s)
      if (s < nk) tile_issue<C>(wtile, KB, trow, lds, s);
    wait_steps_left<C>(min(C::NST - 2, nk - 1));
    if (C::NST - 1 < nk) tile_issue<C>(wtile, KB, trow, lds, C::NST - 1);
    raw_barrier();
    TileFrags<C> f0, f1;
    tile_read_frags<C, ACT>(lds, 0, f0, nbv, tsc);

    constexpr int P1 = C::KS & 1;  // register-set parity of the step after an even step
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      tile_step<C, 0, ACT>(wtile, KB, nk, kt, trow, lds, f0, f1, acc, nbv, tsc);
      tile_step<C, P1, ACT>(wtile, KB, nk, kt + 1, trow, lds, f0, f1, acc, nbv, tsc);
    }
    if (kt < nk) tile_step<C, 0, ACT>(wtile, KB, nk, kt, trow, lds, f0, f1, acc, nbv, tsc);
    // all LDS reads of this tile done before anyone refills the stages
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    raw_barrier();
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
//   tvalid: rows 0 .. tvalid-1 of the token tile are valid (wave-uniform);
//           MFMA work on token rows past them is skipped (whole waves, or
//           whole 16-row blocks with C::SKIPB), and the accumulators of
//           skipped rows hold no meaningful values
//   tsc   : C::FP8T only: the scales of this lane's token rows (trow then
//           points at rows of e4m3 bytes)
// All C::NTHREADS threads must call it.  On entry no direct-to-LDS load of this
// workgroup may be in flight; on exit none is, and a barrier has passed, so
// the caller may reuse lds right away.
template <class C>
__device__ __forceinline__ void tile_mma(const uint16_t* __restrict__ wtile, int KB, int nk,
                                         const TokRows<C>& trow, uint16_t* lds,
                                         TileAcc<C>& acc, int tvalid = C::BT, const TokScale<C>* tsc = nullptr) {
  TokScale<C> sc{};
  if constexpr (C::FP8T) sc = *tsc;
#pragma unroll
  for (int a = 0; a < C::AW; ++a)
#pragma unroll
    for (int b = 0; b < C::AT; ++b) acc.v[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  // both paths pass the same barriers in the same order
  const int first = uniform(tile_wt<C>() * C::AT * 16);
  const int nbv = C::SKIPB ? min(C::AT, (tvalid - first + 15) / 16) : C::AT;
  if (first < tvalid)
    tile_mma_run<C, true>(wtile, KB, nk, trow, lds, acc, nbv, sc);
  else
    tile_mma_run<C, false>(wtile, KB, nk, trow, lds, acc, nbv, sc);
}

}  // namespace moe
