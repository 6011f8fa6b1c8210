// ffn_parts.h -- the pieces of the expert FFN shared by the phase-by-phase
// kernels and the persistent expert-wave kernel: tile decoding, the GEMM1
// (gather + gate/up + SwiGLU) tile, the GEMM2 (down) tile, and the combine of
// one token.  Both schedules call exactly these functions, so they produce
// the same bits.
//
// Layer per token-expert pair (DeepSeek-V4 launch digest, itsolotime.com,
// section 1.4, compute/communication bullet: gating, up and down
// projections): h1 = x W1, h3 = x W3, a = silu(h1) * h3, y = a W2.
#pragma once

#include "gemm_tile.h"
#include "wave_sched.h"

namespace moe {

// Tile shapes of the expert GEMMs (BW output features x BT pair rows).  The
// shape only decides which workgroup computes which outputs; every shape
// runs the same per-element instruction sequence over K.
//   large : many rows per expert (MFMA bound): 256 x 256 tiles, 8 wavefronts
//           of 128 x 64, two per SIMD, token rows fetched as whole 128-byte
//           lines (TL; measured on MI355X against the 64-byte pieces of the
//           plain tile: FFN 1-2% faster on the mid and stress layers, 5% on
//           the V3/V4-scale share, where the layer streams from HBM)
//   mid   : any shape the boundary accepts (d % 128 == 0, I % 64 == 0), also
//           with TL
//   small : a handful of rows per expert (weight streaming, HBM bound):
//           token tiles of 32 or 64 rows (empty 16-row blocks skipped) and
//           6 to 7 LDS stages, so that each workgroup keeps 80 to 96 KiB of
//           weights in flight, loaded with the non-temporal hint
// GEMM1 and GEMM2 of one shape use the same workgroup size (NT threads).
struct FfnLarge {
  using G1 = TileCfg<256, 256, 2, 4, 32, 4, false, false, false, false, true>;
  using G2 = TileCfg<256, 256, 2, 4, 32, 4, false, false, false, false, true>;
  static constexpr int NT = 512;
  static constexpr bool WHOLE_EXPERTS = true;  // deal experts whole to XCDs
};
struct FfnMid {
  using G1 = TileCfg<128, 256, 2, 4, 32, 4, false, false, false, false, true>;
  using G2 = TileCfg<128, 256, 2, 4, 32, 4, false, false, false, false, true>;
  static constexpr int NT = 512;
  static constexpr bool WHOLE_EXPERTS = true;
};
struct FfnSmall {
  using G1 = TileCfg<128, 32, 4, 1, 64, 7, true, false, false, true>;
  using G2 = TileCfg<128, 32, 4, 1, 64, 7, true, false, false, true>;
  static constexpr int NT = 256;
  static constexpr bool WHOLE_EXPERTS = false;  // deal single m-tiles: balance
};
struct FfnSmall64 {
  using G1 = TileCfg<128, 64, 4, 1, 64, 6, true, false, false, true>;
  using G2 = TileCfg<128, 64, 4, 1, 64, 6, true, false, false, true>;
  static constexpr int NT = 256;
  static constexpr bool WHOLE_EXPERTS = false;
};

// FP8 dispatch on the weight-streaming shapes: the GEMM1 token operand in
// e4m3 (the GEMM2 tiles are unchanged).  An fp8 token fragment holds 64 k,
// so the GEMM1 K step is 64 (128 for the 32-row tile, whose two token blocks
// must give each of its four wavefronts one load per step).  (The large
// shapes dequantize the rows first and run the bf16 tiles.)
struct FfnSmallF8 {
  using G1 = TileCfg<128, 32, 4, 1, 128, 4, true, true, false, true>;
  using G2 = FfnSmall::G2;
  static constexpr int NT = 256;
  static constexpr bool WHOLE_EXPERTS = false;
};
struct FfnSmall64F8 {
  using G1 = TileCfg<128, 64, 4, 1, 64, 6, true, true, false, true>;
  using G2 = FfnSmall64::G2;
  static constexpr int NT = 256;
  static constexpr bool WHOLE_EXPERTS = false;
};

template <class F>
constexpr size_t ffn_lds_bytes() {
  static_assert(F::G1::NTHREADS == F::NT && F::G2::NTHREADS == F::NT, "one workgroup size per shape");
  static_assert(F::G1::BT == F::G2::BT, "GEMM1 and GEMM2 share the m-tiles");
  return F::G1::LDS_BYTES > F::G2::LDS_BYTES ? F::G1::LDS_BYTES : F::G2::LDS_BYTES;
}
constexpr int kMaxLocalExperts = 256;

// Per-workgroup table: m-tile prefix over local experts (rows split into
// BT-row tiles).  mt_pre[e] = first m-tile of expert e, mt_pre[E_local] =
// total.  Built from expert_offsets by thread 0.
__device__ __forceinline__ void build_mtile_prefix(const int32_t* __restrict__ offsets, int E_local,
                                                   int BT, int32_t* mt_pre) {
  if (threadIdx.x == 0) {
    int run = 0;
    for (int e = 0; e < E_local; ++e) {
      mt_pre[e] = run;
      run += (offsets[e + 1] - offsets[e] + BT - 1) / BT;
    }
    mt_pre[E_local] = run;
  }
}

// seg[e] = first row of expert e in the padded row space of the saved
// pre-activations and the backward's per-row buffers: the routed rows of the
// experts before it, each rounded up to 64 (so that every m-tile starts on
// a 16-row block).  seg[E_local] = total.  Built by thread 0.
__device__ __forceinline__ void build_seg_prefix(const int32_t* __restrict__ offsets, int E_local, int32_t* seg) {
  if (threadIdx.x == 0) {
    int run = 0;
    for (int e = 0; e < E_local; ++e) {
      seg[e] = run;
      run += (offsets[e + 1] - offsets[e] + 63) & ~63;
    }
    seg[E_local] = run;
  }
}

// Block-fragment layout of an fp32 matrix [rows][16 ncb] (rows in the padded
// row space): the 16 x 16 block (rb, cb) is 256 contiguous floats, lane l
// of a wavefront holding row 16 rb + l % 16, columns 16 cb + 4 (l / 16) ..
// + 3 -- the MFMA accumulator layout of one block, so a wavefront stores or
// loads a block as one contiguous 1 KiB.  Float offset of lane l's 4 values:
__host__ __device__ __forceinline__ size_t blockfrag_offset(size_t rb, int cb, int ncb, int lane) {
  return ((rb * static_cast<size_t>(ncb) + static_cast<size_t>(cb)) * 64 + static_cast<size_t>(lane)) * 4;
}

// Expert owning global m-tile mt (binary search in mt_pre[lo..hi]).
__device__ __forceinline__ int expert_of_mtile(const int32_t* mt_pre, int lo, int hi, int mt) {
  // invariant: mt_pre[lo] <= mt < mt_pre[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (mt_pre[mid] <= mt) lo = mid; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ float silu_mul(float h1, float h3) {
  // silu(h1) * h3 with silu(h) = h / (1 + exp(-h)); IEEE division
  return (h1 / (1.0f + expf(-h1))) * h3;
}

// The ungated activation: max(h, 0)^2 (no exponential, no division).
__device__ __forceinline__ float relu_sq(float h) {
  const float r = fmaxf(h, 0.0f);
  return r * r;
}

// Output staging through LDS.  A tile's BT x COLS bf16 results are written
// to LDS as [row][16-byte chunk] with the chunk index XOR-swizzled by the
// row (the 8-byte writes of a lane group's 16 rows then hit distinct banks),
// and leave LDS as whole rows, 16 contiguous bytes per lane: every global
// store instruction writes full 128-byte lines instead of 32-byte pieces of
// 16 rows.
template <int COLS>
struct OutStage {
  static constexpr int CH = COLS / 8;  // 16-byte chunks per row
  static_assert((CH & (CH - 1)) == 0 && CH >= 4 && CH <= 64, "chunks per row: a power of 2, 4..64");
  static constexpr int RPI = 64 / CH;  // rows one wavefront instruction covers
  __device__ static int slot(int t, int c) { return t * CH + (c ^ (t % CH)); }
};

// Puts 4 values (row t, columns n .. n+3 of the tile, n % 4 == 0) into the stage.
template <int COLS>
__device__ __forceinline__ void out_put(uint16_t* lds, int t, int n, const u32x2& v) {
  *reinterpret_cast<u32x2*>(lds + OutStage<COLS>::slot(t, n / 8) * 8 + ((n / 4) & 1) * 4) = v;
}

// Rows 0 .. count-1 of the stage to dst + t * ld.  Brackets itself with
// barriers: the stage is complete before it is read and fully read before
// the caller reuses LDS.
template <int COLS, int NW>
__device__ __forceinline__ void out_flush(const uint16_t* lds, uint16_t* __restrict__ dst, size_t ld,
                                          int count) {
  using O = OutStage<COLS>;
  __syncthreads();
  const int lane = lane_id(), c = lane % O::CH;
  for (int r0 = wave_id() * O::RPI; r0 < count; r0 += NW * O::RPI) {
    const int t = r0 + lane / O::CH;
    if (t < count) st16(dst + static_cast<size_t>(t) * ld + c * 8, ld16(lds + O::slot(t, c) * 8));
  }
  __syncthreads();
}

// GEMM1 tile: rows [row0, row0 + BT) of expert e's segment (count rows
// valid), BW packed rows of W13 starting at row block nt * BW / 16, i.e.
// intermediate indices [nt * BW/2, nt * BW/2 + BW/2) (gated = false: W13
// holds W1 only and the tile covers indices [nt * BW, nt * BW + BW)).  The operand rows are
// pulled straight from the token-order staging buffer xb by sorted_token:
// the dispatch pull lands in LDS.
// FP8T tiles: xb is the e4m3 staging buffer (d bytes per token) and xscale
// the tokens' scales.
// hsave (optional, wave-uniform): the tile's fp32 accumulators h of its
// valid rows are also stored to hsave, block-fragment layout over packed
// columns (16 columns of W1, then the same 16 intermediate indices of W3,
// ... when gated; W1's columns in order when not), the tile's rows from row
// hrow0 (a multiple of 16) of the padded row space, for a backward that
// reads the pre-activations instead of recomputing them.
template <class C, bool GATED = true>
__device__ __forceinline__ void gemm1_tile(const uint16_t* __restrict__ xb,
                                           const uint16_t* __restrict__ w13e,
                                           const int32_t* __restrict__ sorted_token,
                                           uint16_t* __restrict__ act, int row0, int count, int nt,
                                           int d, int I, uint16_t* lds,
                                           const float* __restrict__ xscale = nullptr,
                                           float* __restrict__ hsave = nullptr, int hrow0 = 0) {
  static_assert(!GATED || C::AW % 2 == 0, "gate/up row blocks pair up inside a wave");
  constexpr int COLS = C::BW / 2;
  static_assert(static_cast<size_t>(C::BT) * COLS * 2 <= C::LDS_BYTES, "output stage fits the tile's LDS");
  const int lane = lane_id();
  const int wr = tile_wr<C>(), wt = tile_wt<C>();
  TokRows<C> trow;
#pragma unroll
  for (int i = 0; i < C::LT; ++i) {
    const int r = min(trow_index<C>(i), count - 1);
    const size_t tok = static_cast<size_t>(sorted_token[row0 + r]);
    if constexpr (C::FP8T)
      trow.p[i] = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(xb) + tok * d);
    else
      trow.p[i] = xb + tok * d;
  }
  TokScale<C> tsc;
  if constexpr (C::FP8T) {
#pragma unroll
    for (int b = 0; b < C::AT; ++b)
      tsc.s[b] = xscale[sorted_token[row0 + min((wt * C::AT + b) * 16 + (lane & 15), count - 1)]];
  }
  TileAcc<C> acc;
  tile_mma<C>(w13e + frag_offset(nt * (C::BW / 16), 0, d / 32), d / 32, d / C::BK, trow, lds, acc, count, &tsc);
  if (hsave != nullptr) {
    const int ncb = (GATED ? 2 : 1) * I / 16;
#pragma unroll
    for (int b = 0; b < C::AT; ++b) {
      if ((wt * C::AT + b) * 16 >= count) continue;  // wave-uniform: rows past the valid ones
      if ((wt * C::AT + b) * 16 + (lane & 15) >= count) continue;
      const size_t rb = static_cast<size_t>(hrow0 / 16 + wt * C::AT + b);
#pragma unroll
      for (int a = 0; a < C::AW; ++a) {
        const int cb = nt * (C::BW / 16) + wr * C::AW + a;
        *reinterpret_cast<f32x4*>(hsave + blockfrag_offset(rb, cb, ncb, lane)) = acc.v[a][b];
      }
    }
  }
  if constexpr (!GATED) {
    // ungated: every row block is W1; a = max(h, 0)^2 for BW intermediate
    // indices per tile
    static_assert(static_cast<size_t>(C::BT) * C::BW * 2 <= C::LDS_BYTES, "output stage fits the tile's LDS");
#pragma unroll
    for (int b = 0; b < C::AT; ++b) {
      if ((wt * C::AT + b) * 16 >= count) continue;  // wave-uniform: rows past the valid ones
      const int t = (wt * C::AT + b) * 16 + (lane & 15);
#pragma unroll
      for (int a = 0; a < C::AW; ++a) {
        const int n = (wr * C::AW + a) * 16 + 4 * (lane / 16);
        const f32x4 h = acc.v[a][b];
        u32x2 pk;
        pk.x = pack_bf16x2(relu_sq(h[0]), relu_sq(h[1]));
        pk.y = pack_bf16x2(relu_sq(h[2]), relu_sq(h[3]));
        out_put<C::BW>(lds, t, n, pk);
      }
    }
    out_flush<C::BW, C::NW>(lds, act + static_cast<size_t>(row0) * I + nt * C::BW, I, count);
  } else {
#pragma unroll
  for (int b = 0; b < C::AT; ++b) {
    if ((wt * C::AT + b) * 16 >= count) continue;  // wave-uniform: rows past the valid ones
    const int t = (wt * C::AT + b) * 16 + (lane & 15);
#pragma unroll
    for (int a = 0; a < C::AW; a += 2) {
      // row blocks wr * AW + a (W1) and + 1 (W3): intermediate block (wr * AW + a) / 2 of the tile
      const int n = ((wr * C::AW + a) / 2) * 16 + 4 * (lane / 16);
      const f32x4 h1 = acc.v[a][b], h3 = acc.v[a + 1][b];
      u32x2 pk;
      pk.x = pack_bf16x2(silu_mul(h1[0], h3[0]), silu_mul(h1[1], h3[1]));
      pk.y = pack_bf16x2(silu_mul(h1[2], h3[2]), silu_mul(h1[3], h3[3]));
      out_put<COLS>(lds, t, n, pk);
    }
  }
  out_flush<COLS, C::NW>(lds, act + static_cast<size_t>(row0) * I + nt * COLS, I, count);
  }
}

// GEMM2 tile: y[row0 .. row0 + count) x features [nt * BW, nt * BW + BW).
template <class C>
__device__ __forceinline__ void gemm2_tile(const uint16_t* __restrict__ act,
                                           const uint16_t* __restrict__ w2e, uint16_t* __restrict__ y,
                                           int row0, int count, int nt, int d, int I, uint16_t* lds) {
  constexpr int COLS = C::BW;
  static_assert(static_cast<size_t>(C::BT) * COLS * 2 <= C::LDS_BYTES, "output stage fits the tile's LDS");
  TokRows<C> trow;
#pragma unroll
  for (int i = 0; i < C::LT; ++i) {
    const int r = min(trow_index<C>(i), count - 1);
    trow.p[i] = act + static_cast<size_t>(row0 + r) * I;
  }
  TileAcc<C> acc;
  tile_mma<C>(w2e + frag_offset(nt * (C::BW / 16), 0, I / 32), I / 32, I / C::BK, trow, lds, acc, count);
  const int lane = lane_id();
  const int wr = tile_wr<C>(), wt = tile_wt<C>();
#pragma unroll
  for (int b = 0; b < C::AT; ++b) {
    if ((wt * C::AT + b) * 16 >= count) continue;  // wave-uniform: rows past the valid ones
    const int t = (wt * C::AT + b) * 16 + (lane & 15);
#pragma unroll
    for (int a = 0; a < C::AW; ++a) {
      const int n = (wr * C::AW + a) * 16 + 4 * (lane / 16);
      const f32x4 v = acc.v[a][b];
      u32x2 pk;
      pk.x = pack_bf16x2(v[0], v[1]);
      pk.y = pack_bf16x2(v[2], v[3]);
      out_put<COLS>(lds, t, n, pk);
    }
  }
  out_flush<COLS, C::NW>(lds, y + static_cast<size_t>(row0) * d + nt * COLS, d, count);
}

// 16 bytes of row r of y at element offset c8.  COHERENT: a device-coherent
// (sc1) load, for y rows another XCD wrote during the same kernel.
template <bool COHERENT>
__device__ __forceinline__ u32x4 load_y16(const uint16_t* __restrict__ y, int r, int d, int c8) {
  const uint16_t* row = y + static_cast<size_t>(r) * d;
  if constexpr (COHERENT) {
    // buffer resource over the row: base, stride 0, d * 2 bytes, raw 32-bit format
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(row), 0, d * 2, 0x00020000);
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, c8 * 2, 0, 16));
  } else {
    return ld16(row + c8);
  }
}

// Column split of the combine.  For a small batch the tokens alone give too
// few tasks to spread the combine's reads over the chip, so each token's d
// columns are split into `parts` ranges handled independently (each range
// at least 64 16-byte chunks, one per lane).  The split never changes a
// result bit: every output element is still one accumulation over j.
__host__ __device__ inline int combine_parts(int T, int d) {
  const int max_parts = d / 512 > 1 ? d / 512 : 1;
  const int tok_tasks = (T + 7) / 8;
  const int want = tok_tasks > 0 ? (512 + tok_tasks - 1) / tok_tasks : 1;
  return want < 1 ? 1 : (want > max_parts ? max_parts : want);
}
// 16-byte column chunks [cb, ce) of part `part` of `parts`.
__host__ __device__ inline void combine_cols(int d, int parts, int part, int& cb, int& ce) {
  const int u = d / 8;
  cb = static_cast<int>(static_cast<long long>(u) * part / parts);
  ce = static_cast<int>(static_cast<long long>(u) * (part + 1) / parts);
}

// Combine of token t, 16-byte column chunks [cb, ce), by one wavefront:
// out[t] = sum_j w[t, j] * y[pair_pos[t, j]] over local picks, fp32 fused
// multiply-adds in ascending j, one rounding.  Each lane takes
// kCombineChunks chunks at a time and the picks kCombineGroup at a time; all
// of a group's loads are issued before its first multiply-add, so a lane
// keeps up to kCombineChunks * kCombineGroup row reads in flight and a
// token of d = 4096 with four picks takes two round trips to memory (the
// accumulation order of every element stays ascending j).
constexpr int kCombineGroup = 4;
constexpr int kCombineChunks = 4;

template <bool OUT_BF16>
__device__ __forceinline__ void combine_store(void* __restrict__ out, int t, int d, int c, const float (&acc)[8]) {
  if constexpr (OUT_BF16) {
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(acc[2 * e], acc[2 * e + 1]);
    st16(static_cast<uint16_t*>(out) + static_cast<size_t>(t) * d + c * 8, o);
  } else {
    float* o = static_cast<float*>(out) + static_cast<size_t>(t) * d + c * 8;
    *reinterpret_cast<f32x4*>(o) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4*>(o + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
  }
}

__device__ __forceinline__ void combine_fma(float w, const u32x4& v, float (&acc)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc[2 * e] = fmaf(w, __uint_as_float(v[e] << 16), acc[2 * e]);
    acc[2 * e + 1] = fmaf(w, __uint_as_float(v[e] & 0xffff0000u), acc[2 * e + 1]);
  }
}

template <bool OUT_BF16, bool COHERENT>
__device__ __forceinline__ void combine_token(int t, const uint16_t* __restrict__ y,
                                              const int32_t* __restrict__ pair_pos,
                                              const float* __restrict__ topk_w, int k, int d, int cb,
                                              int ce, void* __restrict__ out) {
  const int lane = lane_id();
  const int32_t* pp = pair_pos + static_cast<size_t>(t) * k;
  const float* pw = topk_w + static_cast<size_t>(t) * k;
  for (int c0 = cb; c0 < ce; c0 += kCombineChunks * kWave) {
    int c[kCombineChunks];
    bool h[kCombineChunks];
    float acc[kCombineChunks][8];
#pragma unroll
    for (int q = 0; q < kCombineChunks; ++q) {
      c[q] = c0 + q * kWave + lane;
      h[q] = c[q] < ce;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[q][e] = 0.f;
    }
    for (int j0 = 0; j0 < k; j0 += kCombineGroup) {
      int r[kCombineGroup];
      u32x4 v[kCombineGroup][kCombineChunks];
#pragma unroll
      for (int g = 0; g < kCombineGroup; ++g) {
        r[g] = uniform(j0 + g < k ? pp[j0 + g] : -1);
        if (r[g] >= 0) {
#pragma unroll
          for (int q = 0; q < kCombineChunks; ++q)
            if (h[q]) v[g][q] = load_y16<COHERENT>(y, r[g], d, c[q] * 8);
        }
      }
#pragma unroll
      for (int g = 0; g < kCombineGroup; ++g) {
        if (r[g] < 0) continue;
        const float w = pw[j0 + g];
#pragma unroll
        for (int q = 0; q < kCombineChunks; ++q) combine_fma(w, v[g][q], acc[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < kCombineChunks; ++q)
      if (h[q]) combine_store<OUT_BF16>(out, t, d, c[q], acc[q]);
  }
}

}  // namespace moe
