// backward.hip -- deterministic backward of the layer share: the weight
// gradient of the experts (dW1, dW3, dW2), the data gradient dx, and the
// router's gradients (of the combine weights, of the logits, of Wg).
//
// 10100.com commentary (batch-invariant and deterministic operators) and
// the DeepSeek-V4 launch digest (itsolotime.com, section 3): gradients must
// be bitwise identical across repeated backward passes, so there are no
// unordered float atomics: work is pre-sorted, each unit writes an isolated
// buffer, and a final reduction sums the buffers in a fixed order.
//
// L = <dout, out>, out[t] = sum_j w[t, j] y[pair_pos[t, j]] over local picks,
// routing held fixed.  Per local expert e with routed rows r (token t_r,
// router weight w_r):
//   stage 1 (per row tile x 64 intermediate indices)
//     h1, h3   = x_r W1, x_r W3   (the forward's GEMM1 tile, same bits)
//     g        = dout_t W2^T      (fp32),   dA = w_r g
//     s        = sigmoid(h1),     silu = h1 s,   a = silu h3
//     dH3      = dA silu,         dH1 = dA h3 s (1 + h1 (1 - s))
//     aw       = w_r a
//     -> dH1 | dH3 (one [P][2I] row) and aw rounded to bf16, sorted-row
//        order; the combine-weight gradient dw_r = <dout_t, y_r> = <g, a>
//        as fixed partial sums over 32 intermediate indices each
//   gate (one wavefront per token)
//     dw_j  = partials of the pick's row summed in ascending order (0 for a
//             pick whose expert is not local),
//     dl_j  = w_j (dw_j - sum_m w_m dw_m): the renormalised softmax over
//             the picks, differentiated (the top-k choice itself is
//             piecewise constant)
//   dX (per row tile x output tile): dx_r = [dH1 | dH3] [W1 | W3]^T, K = 2I
//     ascending, the forward GEMM2's tile with W13^T as the weights
//   scatter (per token): dx[t] = sum_j dx_{pair_pos[t, j]} (fp32, ascending
//     j) + sum_j dl_j Wg[:, idx_j] (fused multiply-adds, ascending j), one
//     rounding to the dtype of x
//   dWg = x^T dl: fixed chunks of kDwgChunkRows tokens, each an isolated
//     partial, summed in ascending chunk order
//   weight gradient (per output tile, per fixed chunk of kWgradChunkRows
//   rows)
//     dW1_e += x^T dH1,  dW3_e += x^T dH3,  dW2_e += aw^T dout
//     the K (= row) index is walked in ascending order inside a chunk; the
//     first chunk of an expert writes dW directly, chunk c >= 1 writes its
//     own partial slot; then dW_e += partial slots in ascending chunk order.
// Every per-token result (dx, dw, dl) depends on the token's own rows only,
// so it is batch invariant as the forward is.
#include <mutex>
#include <vector>

#include "ffn_parts.h"
#include "moe_internal.h"

namespace moe {
namespace {

// The tiles of the recompute: the forward's GEMM1 tiles, 256 weight rows
// (128 intermediate indices) when 2I allows, else 128 (the mid tile); 256
// routed rows, 8 wavefronts.  The shape does not change the bits.
using BwdCfg = FfnMid::G1;
using BwdCfgL = FfnLarge::G1;

// LDS row strides (bf16 elements) of the transposing stages: rows of 256 and
// 64 values plus 8, so that 16-byte reads stay aligned and the 2-byte
// transposed writes of one instruction spread over the banks.
constexpr int kStageRow = BwdCfg::BT + 8;
static_assert(BwdCfgL::BT == BwdCfg::BT, "one stage row length");
constexpr int kGatherRow = 72;

// The recompute's epilogue stages (dH1 | dH3)^T and (w a)^T of the tile in
// LDS for the transposed weight-gradient operands: in one pass when the
// three fit, else (the 256-wide tile) dH first and w a in a second pass.
// SAVED: the accumulators come from the forward's saved pre-activations (no
// product, so no operand stages in LDS).
template <class C, bool GATED = true, bool SAVED = false>
struct BwdDh {
  static constexpr int NI = GATED ? C::BW / 2 : C::BW;  // intermediate indices per tile
  static constexpr int NH = GATED ? 2 * NI : NI;        // staged dH rows: (dH1 | dH3) or dH1
  static constexpr size_t DH_BYTES = static_cast<size_t>(NH) * kStageRow * 2;
  static constexpr size_t AW_BYTES = static_cast<size_t>(NI) * kStageRow * 2;
  static constexpr bool ONE_PASS = DH_BYTES + AW_BYTES <= 160 * 1024 - 8 * 1024;
  static constexpr size_t STAGE = ONE_PASS ? DH_BYTES + AW_BYTES : DH_BYTES;
  static constexpr size_t LDS = (SAVED || STAGE > C::LDS_BYTES) ? STAGE : C::LDS_BYTES;
  static_assert(LDS <= 160 * 1024 - 8 * 1024, "recompute LDS (with the static tables) fits a CU");
};

// ---------------------------------------------------------------- stage 1

// g = dout W2^T per routed row, fp32, block-fragment layout [P_pad][I] over
// the padded row space (seg): BW intermediate indices x BT routed rows per
// tile, K = d in ascending order (256 wide when I % 256 == 0, BwdCfg when
// I % 128 == 0, else the 64-wide BwdCfgG; the shape does not change the
// bits).
using BwdCfgG = TileCfg<64, 256, 1, 8, 64, 3>;

template <class C>
__global__ __launch_bounds__(C::NTHREADS) void bwd_g_kernel(
    const uint16_t* __restrict__ dout, const uint16_t* __restrict__ w2b,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_token, int E_local, int d,
    int I, float* __restrict__ g) {
  extern __shared__ __align__(16) uint16_t lds[];
  __shared__ int32_t mt_pre[kMaxLocalExperts + 1];
  __shared__ int32_t seg[kMaxLocalExperts + 1];
  __shared__ int32_t xcd_order;
  build_mtile_prefix(offsets, E_local, C::BT, mt_pre);
  build_seg_prefix(offsets, E_local, seg);
  if (threadIdx.x == 0) xcd_order = phase_xcd_order(mt_pre, E_local);
  __syncthreads();
  const int NT = I / C::BW;
  const bool xo = uniform(xcd_order) != 0;
  const PhaseTiles pt = phase_tiles(uniform(mt_pre[E_local] * NT), xo, static_cast<int>(blockIdx.x),
                                    static_cast<int>(gridDim.x));
  const int lane = lane_id(), wr = tile_wr<C>(), wt = tile_wt<C>();
  for (int tile = pt.begin + pt.first; tile < pt.end; tile += pt.stride) {
    int e, mt, nt;
    phase_tile(mt_pre, E_local, NT, tile, xo, e, mt, nt);
    e = uniform(e);
    mt = uniform(mt);
    nt = uniform(nt);
    const int row0 = uniform(offsets[e] + (mt - mt_pre[e]) * C::BT);
    const int count = uniform(min(C::BT, offsets[e + 1] - row0));
    TokRows<C> trow;
#pragma unroll
    for (int i = 0; i < C::LT; ++i) {
      const int r = min(trow_index<C>(i), count - 1);
      trow.p[i] = dout + static_cast<size_t>(sorted_token[row0 + r]) * d;
    }
    TileAcc<C> acc;
    tile_mma<C>(w2b + static_cast<size_t>(e) * I * d + frag_offset(nt * (C::BW / 16), 0, d / 32), d / 32,
                d / C::BK, trow, lds, acc, count);
    const int hrow0 = uniform(seg[e] + (mt - mt_pre[e]) * C::BT);
#pragma unroll
    for (int b = 0; b < C::AT; ++b) {
      const int t = (wt * C::AT + b) * 16 + (lane & 15);
      if (t >= count) continue;
      const size_t rb = static_cast<size_t>(hrow0 / 16 + wt * C::AT + b);
#pragma unroll
      for (int a = 0; a < C::AW; ++a) {
        const int cb = nt * (C::BW / 16) + wr * C::AW + a;
        *reinterpret_cast<f32x4*>(g + blockfrag_offset(rb, cb, I / 16, lane)) = acc.v[a][b];
      }
    }
  }
}

// h1, h3 recomputed with the forward's GEMM1 arithmetic, or read from the
// forward's saved accumulators hsaved [P][GR I] (the same bits; BW packed rows =
// BW/2 intermediate indices x BT routed rows per tile, K = d ascending; the
// tile shape never changes the bits), then per element
//   dA = w g, s = sigmoid(h1), silu = h1 s, a = silu h3,
//   dH3 = dA silu, dH1 = dA h3 s (1 + h1 (1 - s)), aw = w a,
// and the combine-weight gradient's partial sum_i g_i a_i over each block
// of 16 intermediate indices (in-lane over 4 consecutive indices, then over
// the block's 4 lane groups): dwp [P_max][I / 16] (null: skipped).
// Outputs: dH rows [P][2I] (dH1 | dH3) for the dx product and, when dht is
// not null, (dH1 | dH3)^T fragments and (w a)^T rows for the weight
// gradient, transposed through an LDS stage.
template <class C, bool GATED, bool SAVED>
__global__ __launch_bounds__(C::NTHREADS) void bwd_dh_kernel(
    const uint16_t* __restrict__ xb, const uint16_t* __restrict__ w13, const float* __restrict__ g,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_token,
    const int32_t* __restrict__ pair_pos, const float* __restrict__ topk_w, int E_local, int d, int I,
    int k, int P_pad, uint16_t* __restrict__ dh, uint16_t* __restrict__ dht, uint16_t* __restrict__ awt,
    float* __restrict__ dwp, const float* __restrict__ hsaved) {
  using D = BwdDh<C, GATED, SAVED>;
  static_assert(!GATED || C::AW % 2 == 0, "gate/up row blocks pair up inside a wave");
  constexpr int GR = GATED ? 2 : 1;  // packed W13 rows per intermediate index
  extern __shared__ __align__(16) uint16_t lds[];
  __shared__ int32_t mt_pre[kMaxLocalExperts + 1];
  __shared__ int32_t seg[kMaxLocalExperts + 1];
  __shared__ float wrow[C::BT];
  __shared__ int32_t xcd_order;
  build_mtile_prefix(offsets, E_local, C::BT, mt_pre);
  build_seg_prefix(offsets, E_local, seg);
  if (threadIdx.x == 0) xcd_order = phase_xcd_order(mt_pre, E_local);
  __syncthreads();
  constexpr int NI = D::NI;
  uint16_t* sdh = lds;  // [NH][kStageRow]: (dH1 | dH3)^T (or dH1^T) of the tile
  // [NI][kStageRow]: (w a)^T, after sdh, or over it in the second pass
  uint16_t* saw = D::ONE_PASS ? lds + D::NH * kStageRow : lds;
  const bool trans = dht != nullptr;
  const int NT = GR * I / C::BW, NQ = I / 16;
  const bool xo = uniform(xcd_order) != 0;
  const PhaseTiles pt = phase_tiles(uniform(mt_pre[E_local] * NT), xo, static_cast<int>(blockIdx.x),
                                    static_cast<int>(gridDim.x));
  const int lane = lane_id(), wr = tile_wr<C>(), wt = tile_wt<C>();
  for (int tile = pt.begin + pt.first; tile < pt.end; tile += pt.stride) {
    int e, mt, nt;
    phase_tile(mt_pre, E_local, NT, tile, xo, e, mt, nt);
    e = uniform(e);
    mt = uniform(mt);
    nt = uniform(nt);
    const int row0 = uniform(offsets[e] + (mt - mt_pre[e]) * C::BT);
    const int count = uniform(min(C::BT, offsets[e + 1] - row0));
    // router weight of each row of the tile (0 past the valid rows)
    for (int r = threadIdx.x; r < C::BT; r += C::NTHREADS) {
      const int row = row0 + min(r, count - 1), t = sorted_token[row];
      float w = 0.f;
      for (int j = 0; j < k; ++j) {
        const bool hit = pair_pos[static_cast<size_t>(t) * k + j] == row;
        w = hit ? topk_w[static_cast<size_t>(t) * k + j] : w;
      }
      wrow[r] = r < count ? w : 0.f;
    }
    // first row of the tile in the padded row space of g and hsaved
    const int hrow0 = uniform(seg[e] + (mt - mt_pre[e]) * C::BT);
    TileAcc<C> acc;
    if constexpr (SAVED) {
      // the forward's accumulators, laid out as this product leaves them:
      // a row past count holds row count-1's values (its operand row is
      // clamped to that row) in a wavefront with a valid row, and zeros in
      // a wavefront with none (tile_mma skips it)
#pragma unroll
      for (int a = 0; a < C::AW; ++a)
#pragma unroll
        for (int b = 0; b < C::AT; ++b) acc.v[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (wt * C::AT * 16 < count) {
        const int ncb = GR * I / 16;
#pragma unroll
        for (int b = 0; b < C::AT; ++b) {
          const int hr = hrow0 + min((wt * C::AT + b) * 16 + (lane & 15), count - 1);
          const int hl = (hr & 15) + 16 * (lane / 16);  // lane of that row in its block
#pragma unroll
          for (int a = 0; a < C::AW; ++a) {
            const int cb = nt * (C::BW / 16) + wr * C::AW + a;
            acc.v[a][b] = *reinterpret_cast<const f32x4*>(hsaved + blockfrag_offset(hr / 16, cb, ncb, hl));
          }
        }
      }
      __syncthreads();  // the wrow writes before the reads below
    } else {
      TokRows<C> trow;
#pragma unroll
      for (int i = 0; i < C::LT; ++i) {
        const int r = min(trow_index<C>(i), count - 1);
        trow.p[i] = xb + static_cast<size_t>(sorted_token[row0 + r]) * d;
      }
      // barriers inside order the wrow writes before the reads below
      tile_mma<C>(w13 + static_cast<size_t>(e) * GR * I * d + frag_offset(nt * (C::BW / 16), 0, d / 32), d / 32,
                  d / C::BK, trow, lds, acc, count);
    }
    // second-pass staging keeps the tile's w a values as bf16 pairs (not the
    // accumulators) across the read-out of the first stage (gated; the
    // ungated epilogue recomputes w a from the accumulators instead)
    uint32_t vaw[(D::ONE_PASS || !GATED) ? 1 : C::AT][(D::ONE_PASS || !GATED) ? 1 : C::AW / 2][2];

    // wave (wr, wt): row blocks a (W1) and a + 1 (W3) of intermediate block
    // (wr * AW + a) / 2; lane l holds indices 4 (l / 16) + 0..3 of the block
    // for tile row (wt * AT + b) * 16 + l % 16.  Rows past count compute
    // zeros (w = 0): the padding of the transposed operands.
    if constexpr (!GATED) {
      // ungated: row block a is intermediate block wr * AW + a; per element
      // r = max(h, 0), a = r^2, dA = w g, dH = (2 dA) r, aw = w a
#pragma unroll
      for (int b = 0; b < C::AT; ++b) {
        const int t = (wt * C::AT + b) * 16 + (lane & 15);
        const bool valid = t < count;
        const float w = wrow[t];
#pragma unroll
        for (int a = 0; a < C::AW; ++a) {
          const int il = (wr * C::AW + a) * 16 + 4 * (lane / 16);
          const int i0 = nt * NI + il;
          const f32x4 g4 = valid ? *reinterpret_cast<const f32x4*>(
                                       g + blockfrag_offset((hrow0 + t) / 16, i0 / 16, I / 16, lane))
                                 : f32x4{0.f, 0.f, 0.f, 0.f};
          float v1[4], va[4];
          float part = 0.f;  // <g, a> over the lane's 4 indices
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float rl = fmaxf(acc.v[a][b][r], 0.0f);
            const float act = rl * rl;
            const float dA = w * g4[r];
            v1[r] = (dA * 2.0f) * rl;
            va[r] = w * act;
            part = fmaf(g4[r], act, part);
          }
          part += __shfl_xor(part, 16, kWave);
          part += __shfl_xor(part, 32, kWave);
          if (dwp && valid && lane < 16) dwp[static_cast<size_t>(row0 + t) * NQ + i0 / 16] = part;
          if (valid) {
            const size_t o = static_cast<size_t>(row0 + t) * I + i0;
            *reinterpret_cast<u32x2*>(dh + o) = u32x2{pack_bf16x2(v1[0], v1[1]), pack_bf16x2(v1[2], v1[3])};
          }
          if (trans) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              sdh[(il + r) * kStageRow + t] = f32_to_bf16(v1[r]);
              if constexpr (D::ONE_PASS) saw[(il + r) * kStageRow + t] = f32_to_bf16(va[r]);
            }
          }
        }
      }
    } else {
#pragma unroll
    for (int b = 0; b < C::AT; ++b) {
      const int t = (wt * C::AT + b) * 16 + (lane & 15);
      const bool valid = t < count;
      const float w = wrow[t];
#pragma unroll
      for (int a = 0; a < C::AW; a += 2) {
        const int il = ((wr * C::AW + a) / 2) * 16 + 4 * (lane / 16);
        const int i0 = nt * NI + il;
        const f32x4 g4 = valid ? *reinterpret_cast<const f32x4*>(
                                     g + blockfrag_offset((hrow0 + t) / 16, i0 / 16, I / 16, lane))
                               : f32x4{0.f, 0.f, 0.f, 0.f};
        float v1[4], v3[4], va[4];
        float part = 0.f;  // <g, a> over the lane's 4 indices
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float h1 = acc.v[a][b][r], h3 = acc.v[a + 1][b][r];
          const float dA = w * g4[r];
          const float s = 1.0f / (1.0f + expf(-h1));
          const float silu = h1 * s;
          const float act = silu * h3;
          v3[r] = dA * silu;
          v1[r] = ((dA * h3) * s) * (1.0f + h1 * (1.0f - s));
          va[r] = w * act;
          part = fmaf(g4[r], act, part);
        }
        // the block's four lane groups: a fixed butterfly (every lane ends
        // with the same, commutatively equal sum)
        part += __shfl_xor(part, 16, kWave);
        part += __shfl_xor(part, 32, kWave);
        if (dwp && valid && lane < 16) dwp[static_cast<size_t>(row0 + t) * NQ + i0 / 16] = part;
        if (valid) {
          const size_t o = static_cast<size_t>(row0 + t) * 2 * I + i0;
          *reinterpret_cast<u32x2*>(dh + o) = u32x2{pack_bf16x2(v1[0], v1[1]), pack_bf16x2(v1[2], v1[3])};
          *reinterpret_cast<u32x2*>(dh + o + I) = u32x2{pack_bf16x2(v3[0], v3[1]), pack_bf16x2(v3[2], v3[3])};
        }
        if (trans) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            sdh[(il + r) * kStageRow + t] = f32_to_bf16(v1[r]);
            sdh[(NI + il + r) * kStageRow + t] = f32_to_bf16(v3[r]);
            if constexpr (D::ONE_PASS) saw[(il + r) * kStageRow + t] = f32_to_bf16(va[r]);
          }
        }
        if constexpr (!D::ONE_PASS) {
#pragma unroll
          for (int r = 0; r < 2; ++r)
            vaw[b][a / 2][r] = static_cast<uint32_t>(f32_to_bf16(va[2 * r])) |
                               (static_cast<uint32_t>(f32_to_bf16(va[2 * r + 1])) << 16);
        }
      }
    }
    }
    if (trans) {
      // the tile's rows are columns k0 .. k0 + BT - 1 of the transposed
      // operands; columns up to the expert's rows rounded to 64 are written
      __syncthreads();
      const int k0 = hrow0;
      const int rows_pad = (count + 63) & ~63;
      const int KB = P_pad / 32;
      // (dH1 | dH3)^T (or dH1^T) fragments: NH / 16 row blocks x rows_pad / 32 k blocks
      constexpr int NB = D::NH / 16;
      for (int q = threadIdx.x; q < NB * (rows_pad / 32) * 64; q += C::NTHREADS) {
        const int frag = q / 64, slot = q % 64;
        const int nl = (frag % NB) * 16 + slot % 16, kl = (frag / NB) * 32 + (slot / 16) * 8;
        const int n = nl < NI ? nt * NI + nl : I + nt * NI + (nl - NI);  // nl < NI always when ungated
        st16(dht + frag_offset(n / 16, (k0 + kl) / 32, KB) + ((kl % 32) / 8 * 16 + n % 16) * 8,
             ld16(sdh + nl * kStageRow + kl));
      }
      if constexpr (!D::ONE_PASS) {
        // second pass: the w a values (kept as bf16 pairs when gated,
        // recomputed from the accumulators when ungated), staged over the
        // read-out sdh
        __syncthreads();
#pragma unroll
        for (int b = 0; b < C::AT; ++b) {
          const int t = (wt * C::AT + b) * 16 + (lane & 15);
          if constexpr (GATED) {
#pragma unroll
            for (int a = 0; a < C::AW; a += 2) {
              const int il = ((wr * C::AW + a) / 2) * 16 + 4 * (lane / 16);
#pragma unroll
              for (int r = 0; r < 4; ++r)
                saw[(il + r) * kStageRow + t] = static_cast<uint16_t>(vaw[b][a / 2][r / 2] >> (16 * (r % 2)));
            }
          } else {
            const float w = wrow[t];
#pragma unroll
            for (int a = 0; a < C::AW; ++a) {
              const int il = (wr * C::AW + a) * 16 + 4 * (lane / 16);
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float rl = fmaxf(acc.v[a][b][r], 0.0f);
                saw[(il + r) * kStageRow + t] = f32_to_bf16(w * (rl * rl));
              }
            }
          }
        }
        __syncthreads();
      }
      // (w a)^T rows: NI indices x rows_pad / 8 chunks of 8 columns
      const int ng = rows_pad / 8;
      for (int q = threadIdx.x; q < NI * ng; q += C::NTHREADS) {
        const int il = q / ng, gq = q % ng;
        st16(awt + static_cast<size_t>(nt * NI + il) * P_pad + k0 + gq * 8, ld16(saw + il * kStageRow + gq * 8));
      }
    }
    __syncthreads();  // wrow and the stage reused by the next tile
  }
}

// ---------------------------------------------------------------- transposed x, dout

// x and dout of the routed rows, transposed: xst [d][P_pad] (rows) and dst
// [d][P_pad] (fragment layout), column k = routed row (expert segments
// padded to 64 with zeros).  blockIdx.x: 64-column block, blockIdx.y:
// 64-feature block; blocks past the last segment exit.
__global__ __launch_bounds__(256) void bwd_gather_t_kernel(
    const uint16_t* __restrict__ xb, const uint16_t* __restrict__ dout,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_token, int E_local,
    int d, int P_pad, uint16_t* __restrict__ xst, uint16_t* __restrict__ dst) {
  __shared__ int32_t seg[kMaxLocalExperts + 1];
  __shared__ __align__(16) uint16_t sx[64 * kGatherRow];
  __shared__ __align__(16) uint16_t sd[64 * kGatherRow];
  build_seg_prefix(offsets, E_local, seg);
  __syncthreads();
  const int k0 = blockIdx.x * 64;
  if (k0 >= seg[E_local]) return;
  const int e = expert_of_mtile(seg, 0, E_local, k0);
  const int r0 = offsets[e] + (k0 - seg[e]), rend = offsets[e + 1];
  const int f0 = blockIdx.y * 64;
  for (int q = threadIdx.x; q < 512; q += 256) {
    const int r = q / 8, c = q % 8;
    u32x4 vx = u32x4{0u, 0u, 0u, 0u}, vd = u32x4{0u, 0u, 0u, 0u};
    if (r0 + r < rend) {
      const size_t t = static_cast<size_t>(sorted_token[r0 + r]);
      vx = ld16(xb + t * d + f0 + c * 8);
      vd = ld16(dout + t * d + f0 + c * 8);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sh = (j & 1) * 16;
      sx[(c * 8 + j) * kGatherRow + r] = static_cast<uint16_t>(vx[j / 2] >> sh);
      sd[(c * 8 + j) * kGatherRow + r] = static_cast<uint16_t>(vd[j / 2] >> sh);
    }
  }
  __syncthreads();
  const int KB = P_pad / 32;
  for (int q = threadIdx.x; q < 512; q += 256) {
    const int f = q / 8, g = q % 8;
    st16(xst + static_cast<size_t>(f0 + f) * P_pad + k0 + g * 8, ld16(sx + f * kGatherRow + g * 8));
    const int frag = q / 64, slot = q % 64;
    const int fl = (frag % 4) * 16 + slot % 16, kl = (frag / 4) * 32 + (slot / 16) * 8;
    st16(dst + frag_offset((f0 + fl) / 16, (k0 + kl) / 32, KB) + ((kl % 32) / 8 * 16 + (f0 + fl) % 16) * 8,
         ld16(sd + fl * kGatherRow + kl));
  }
}

// ---------------------------------------------------------------- gate

// One wavefront per token; lane j < k handles pick j.  dtopk_w, dlogits and
// dld may be null.  dlc [T][k] receives the picked logits' gradients; dld
// [T][Ep] the dense logits gradient in bf16 (the dWg product's operand).
__global__ __launch_bounds__(256) void bwd_gate_kernel(
    const float* __restrict__ dwp, int NQ, const int32_t* __restrict__ pair_pos,
    const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_w, int T, int k, int E, int Ep,
    float* __restrict__ dtopk_w, float* __restrict__ dlc, float* __restrict__ dlogits,
    uint16_t* __restrict__ dld) {
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + wave_id();
  if (t >= T) return;
  float w = 0.f, dw = 0.f;
  int e = -1;
  if (lane < k) {
    const size_t o = static_cast<size_t>(t) * k + lane;
    w = topk_w[o];
    e = topk_idx[o];
    const int r = pair_pos[o];
    if (r >= 0) {
      const float* q = dwp + static_cast<size_t>(r) * NQ;
      for (int i = 0; i < NQ; ++i) dw += q[i];
    }
  }
  float s = 0.f;
  for (int j = 0; j < k; ++j) s = fmaf(__shfl(w, j, kWave), __shfl(dw, j, kWave), s);
  const float dl = w * (dw - s);
  if (lane < k) {
    const size_t o = static_cast<size_t>(t) * k + lane;
    if (dtopk_w) dtopk_w[o] = dw;
    dlc[o] = dl;
  }
  if (dlogits || dld) {
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int ej = __shfl(e, j, kWave);
      const float gj = __shfl(dl, j, kWave);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (lane + 64 * q == ej) v[q] = gj;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int col = lane + 64 * q;
      if (dlogits && col < E) dlogits[static_cast<size_t>(t) * E + col] = v[q];
      if (dld && col < Ep) dld[static_cast<size_t>(t) * Ep + col] = f32_to_bf16(v[q]);
    }
  }
}

// ---------------------------------------------------------------- dX

// dx rows of one row tile x BW output features: the GEMM2 tile of the
// forward with A = [dH1 | dH3] (K = 2I) and the W13^T fragments.
template <class F>
__global__ __launch_bounds__(F::NT) void bwd_dx_gemm_kernel(
    const uint16_t* __restrict__ dh, const uint16_t* __restrict__ w13t,
    const int32_t* __restrict__ offsets, uint16_t* __restrict__ dxr, int E_local, int d, int K2) {
  using C = typename F::G2;
  extern __shared__ __align__(16) uint16_t lds[];
  __shared__ int32_t mt_pre[kMaxLocalExperts + 1];
  __shared__ int32_t xcd_order;
  build_mtile_prefix(offsets, E_local, C::BT, mt_pre);
  if (threadIdx.x == 0) xcd_order = phase_xcd_order(mt_pre, E_local);
  __syncthreads();
  const int NT = d / C::BW;
  const bool xo = uniform(xcd_order) != 0;
  const PhaseTiles pt = phase_tiles(uniform(mt_pre[E_local] * NT), xo, static_cast<int>(blockIdx.x),
                                    static_cast<int>(gridDim.x));
  for (int tile = pt.begin + pt.first; tile < pt.end; tile += pt.stride) {
    int e, mt, nt;
    phase_tile(mt_pre, E_local, NT, tile, xo, e, mt, nt);
    e = uniform(e);
    mt = uniform(mt);
    nt = uniform(nt);
    const int row0 = uniform(offsets[e] + (mt - mt_pre[e]) * C::BT);
    const int count = uniform(min(C::BT, offsets[e + 1] - row0));
    gemm2_tile<C>(dh, w13t + static_cast<size_t>(e) * d * K2, dxr, row0, count, nt, d, K2, lds);
  }
}

// 8 consecutive elements of row e of Wg^T (bf16 or fp32) as floats.
template <bool XBF>
__device__ __forceinline__ void load_wgt8(const void* __restrict__ wgt, int e, int d, int c, float (&v)[8]) {
  if constexpr (XBF) {
    const u32x4 q = ld16(static_cast<const uint16_t*>(wgt) + static_cast<size_t>(e) * d + c * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(q[i] << 16);
      v[2 * i + 1] = __uint_as_float(q[i] & 0xffff0000u);
    }
  } else {
    const float* p = static_cast<const float*>(wgt) + static_cast<size_t>(e) * d + c * 8;
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  }
}

// One wavefront per (token, column part), 16-byte column chunks of dx:
//   dx[t] = sum_j dxr[pair_pos[t, j]] (fp32 adds, ascending j, local picks)
//         + sum_j dl[t, j] Wg[:, idx[t, j]] (fused multiply-adds, ascending j)
// rounded once to the dtype of x.  As in the forward combine, a lane takes
// kCombineChunks chunks at a time and issues a group's row reads before
// adding them: up to kCombineChunks * kCombineGroup reads in flight.
template <bool XBF>
__global__ __launch_bounds__(256) void bwd_dx_scatter_kernel(
    const uint16_t* __restrict__ dxr, const int32_t* __restrict__ pair_pos,
    const int32_t* __restrict__ topk_idx, const float* __restrict__ dlc, const void* __restrict__ wgt,
    int T, int k, int d, int E, int parts, void* __restrict__ dx) {
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + wave_id();
  if (t >= T) return;
  int cb, ce;
  combine_cols(d, parts, blockIdx.y, cb, ce);
  const int32_t* pp = pair_pos + static_cast<size_t>(t) * k;
  const int32_t* pi = topk_idx + static_cast<size_t>(t) * k;
  const float* pg = dlc + static_cast<size_t>(t) * k;
  for (int c0 = cb; c0 < ce; c0 += kCombineChunks * kWave) {
    int c[kCombineChunks];
    bool h[kCombineChunks];
    float acc[kCombineChunks][8];
#pragma unroll
    for (int u = 0; u < kCombineChunks; ++u) {
      c[u] = c0 + u * kWave + lane;
      h[u] = c[u] < ce;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[u][i] = 0.f;
    }
    for (int j0 = 0; j0 < k; j0 += kCombineGroup) {
      int r[kCombineGroup];
      u32x4 v[kCombineGroup][kCombineChunks];
#pragma unroll
      for (int q = 0; q < kCombineGroup; ++q) {
        r[q] = uniform(j0 + q < k ? pp[j0 + q] : -1);
        if (r[q] >= 0) {
#pragma unroll
          for (int u = 0; u < kCombineChunks; ++u)
            if (h[u]) v[q][u] = ld16(dxr + static_cast<size_t>(r[q]) * d + c[u] * 8);
        }
      }
#pragma unroll
      for (int q = 0; q < kCombineGroup; ++q) {
        if (r[q] < 0) continue;
#pragma unroll
        for (int u = 0; u < kCombineChunks; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[u][2 * i] = acc[u][2 * i] + __uint_as_float(v[q][u][i] << 16);
            acc[u][2 * i + 1] = acc[u][2 * i + 1] + __uint_as_float(v[q][u][i] & 0xffff0000u);
          }
      }
    }
    for (int j = 0; j < k; ++j) {
      const int e = uniform(pi[j]);
      if (e < 0 || e >= E) continue;  // not a router id: no router row to read
      const float g = pg[j];
#pragma unroll
      for (int u = 0; u < kCombineChunks; ++u) {
        if (!h[u]) continue;
        float wv[8];
        load_wgt8<XBF>(wgt, e, d, c[u], wv);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[u][i] = fmaf(g, wv[i], acc[u][i]);
      }
    }
#pragma unroll
    for (int u = 0; u < kCombineChunks; ++u) {
      if (!h[u]) continue;
      if constexpr (XBF) {
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[u][2 * i], acc[u][2 * i + 1]);
        st16(static_cast<uint16_t*>(dx) + static_cast<size_t>(t) * d + c[u] * 8, o);
      } else {
        float* o = static_cast<float*>(dx) + static_cast<size_t>(t) * d + c[u] * 8;
        *reinterpret_cast<f32x4*>(o) = f32x4{acc[u][0], acc[u][1], acc[u][2], acc[u][3]};
        *reinterpret_cast<f32x4*>(o + 4) = f32x4{acc[u][4], acc[u][5], acc[u][6], acc[u][7]};
      }
    }
  }
}

// ---------------------------------------------------------------- products over rows

// 8x8 bf16 transpose: in[j] holds row j (8 values along u); returns, for
// each u, the 8 values along rows packed in 4 words (row pairs).
__device__ __forceinline__ void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const uint32_t sel = (u & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int q = 0; q < 4; ++q) out[u][q] = __builtin_amdgcn_perm(in[2 * q + 1][u >> 1], in[2 * q][u >> 1], sel);
  }
}

// D[u][v] = sum_r P[r][u] * Q[r][v] over rows r of one chunk, written to
// out[v * Udim + u] (fp32).  P and Q rows are either direct (row index r)
// or gathered through sorted_token.
__device__ __forceinline__ void wgrad_tile(const uint16_t* __restrict__ P, bool p_gather, int p_ld, int Udim,
                           const uint16_t* __restrict__ Q, bool q_gather, int q_ld, int Vdim,
                           const int32_t* __restrict__ sorted_token, int rbeg, int rend, int ut,
                           int vt, float* __restrict__ out, uint16_t* lds) {
  using C = TileCfg<128, 128, 2, 2, 64, 2>;
  const int lane = lane_id(), wave = wave_id();
  const int wr = wave / C::WT, wt = wave % C::WT;
  // thread's 8x8 block: operand (P for tid < 128), row group rg, u group ug
  const int tid = threadIdx.x;
  const bool isP = tid < 128;
  const int rg = (tid & 127) / 16, ug = tid & 15;
  const uint16_t* M = isP ? P : Q;
  const bool gather = isP ? p_gather : q_gather;
  const int ld = isP ? p_ld : q_ld;
  const int dim = isP ? Udim : Vdim;
  const int col0 = (isP ? ut : vt) * 128 + ug * 8;
  const bool col_ok = col0 < dim;  // dims are multiples of 64, so 8-groups are whole
  f32x4 acc[C::AW][C::AT];
#pragma unroll
  for (int a = 0; a < C::AW; ++a)
#pragma unroll
    for (int b = 0; b < C::AT; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 raw[8];
  auto gload = [&](int kbase) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = kbase + rg * 8 + j;
      if (r < rend && col_ok) {
        const size_t row = gather ? static_cast<size_t>(sorted_token[r]) : static_cast<size_t>(r);
        raw[j] = ld16(M + row * ld + col0);
      } else {
        raw[j] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto lstore = [&](int buf) {
    u32x4 tr[8];
    transpose8x8(raw, tr);
    uint16_t* st = lds + buf * C::STAGE + (isP ? 0 : C::NFW * 512);
    const int ks = rg / 4, slot_hi = (rg % 4) * 16;
#pragma unroll
    for (int uu = 0; uu < 8; ++uu) {
      const int u = ug * 8 + uu;  // 0..127 inside the tile
      st16(st + ((u / 16) * 2 + ks) * 512 + (slot_hi + (u % 16)) * 8, tr[uu]);
    }
  };
  const int nk = uniform((rend - rbeg + 63) / 64);
  if (nk > 0) {
    gload(rbeg);
    lstore(0);
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    __syncthreads();
    if (kt + 1 < nk) gload(rbeg + (kt + 1) * 64);
    const uint16_t* st = lds + cur * C::STAGE;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 af[C::AW], bfr[C::AT];
#pragma unroll
      for (int a = 0; a < C::AW; ++a) af[a] = ld16(st + ((wr * C::AW + a) * 2 + ks) * 512 + lane * 8);
#pragma unroll
      for (int b = 0; b < C::AT; ++b) bfr[b] = ld16(st + (C::NFW + (wt * C::AT + b) * 2 + ks) * 512 + lane * 8);
#pragma unroll
      for (int a = 0; a < C::AW; ++a)
#pragma unroll
        for (int b = 0; b < C::AT; ++b) acc[a][b] = mfma16x16x32(af[a], bfr[b], acc[a][b]);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
  }
  __syncthreads();
#pragma unroll
  for (int a = 0; a < C::AW; ++a) {
    const int u = ut * 128 + (wr * C::AW + a) * 16 + 4 * (lane / 16);
    if (u >= Udim) continue;
#pragma unroll
    for (int b = 0; b < C::AT; ++b) {
      const int v = vt * 128 + (wt * C::AT + b) * 16 + (lane & 15);
      if (v >= Vdim) continue;
      *reinterpret_cast<f32x4*>(out + static_cast<size_t>(v) * Udim + u) = acc[a][b];
    }
  }
}


// ---------------------------------------------------------------- dWg

// bf16 x: part[c][i][e] = sum over tokens of chunk c of x[t][i] dld[t][e].
__global__ __launch_bounds__(256) void bwd_dwg_kernel(const uint16_t* __restrict__ dld,
                                                      const uint16_t* __restrict__ xb, int T, int d,
                                                      int Ep, float* __restrict__ part) {
  extern __shared__ __align__(16) uint16_t lds[];
  const int tU = (Ep + 127) / 128, tV = d / 128;
  const int tpc = tU * tV;
  const int total = tpc * ((T + kDwgChunkRows - 1) / kDwgChunkRows);
  for (int task = blockIdx.x; task < total; task += gridDim.x) {
    const int c = task / tpc, rel = task % tpc;
    const int ut = rel % tU, vt = rel / tU;
    const int rbeg = c * kDwgChunkRows, rend = min(T, rbeg + kDwgChunkRows);
    wgrad_tile(dld, false, Ep, Ep, xb, false, d, d, nullptr, rbeg, rend, ut, vt,
               part + static_cast<size_t>(c) * d * Ep, lds);
  }
}

// dWg[i][e] = sum of the chunk partials in ascending chunk order.
__global__ __launch_bounds__(256) void bwd_dwg_reduce_kernel(const float* __restrict__ part, int nch,
                                                             int d, int E, int Ep, float* __restrict__ dWg) {
  const size_t id = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (id >= static_cast<size_t>(d) * E) return;
  const size_t i = id / E, e = id % E;
  const size_t mat = static_cast<size_t>(d) * Ep;
  float acc = part[i * Ep + e];
  for (int c = 1; c < nch; ++c) acc += part[c * mat + i * Ep + e];
  dWg[id] = acc;
}

// fp32 x (the router then runs on fp32 values): dWg[i][e] = sum over tokens
// in ascending order, picks in ascending j, of x[t][i] dl[t, j] where
// idx[t, j] = e; one thread per element, fused multiply-adds.
__global__ __launch_bounds__(256) void bwd_dwg_f32_kernel(const float* __restrict__ x,
                                                          const int32_t* __restrict__ topk_idx,
                                                          const float* __restrict__ dlc, int T, int k,
                                                          int d, int E, float* __restrict__ dWg) {
  const size_t id = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (id >= static_cast<size_t>(d) * E) return;
  const int i = static_cast<int>(id / E), e = static_cast<int>(id % E);
  float acc = 0.f;
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j)
      if (topk_idx[static_cast<size_t>(t) * k + j] == e)
        acc = fmaf(x[static_cast<size_t>(t) * d + i], dlc[static_cast<size_t>(t) * k + j], acc);
  dWg[id] = acc;
}

// ---------------------------------------------------------------- weight gradient

__device__ __forceinline__ int n_chunks(int rows) {
  return rows <= kWgradChunkRows ? 1 : (rows + kWgradChunkRows - 1) / kWgradChunkRows;
}

// dW1 | dW3 and dW2 of one (expert, row chunk) per task, with the tile
// product of the forward: D[n][t] = sum over the chunk's routed rows k of
// A[n][k] B[t][k], K walked in ascending order.
//   dW1 | dW3: A = (dH1 | dH3)^T fragments (n over 2I), B = x^T rows (t over d),
//              D[n][t] = dW1[t][n] (n < I) or dW3[t][n - I];
//   dW2:       A = dout^T fragments (n over d), B = (w * a)^T rows (t over I),
//              D[n][t] = dW2[t][n].
// Chunk c of expert e covers its routed rows c * kWgradChunkRows .. (padded
// to 64 with zero columns); chunk 0 writes dW, chunk c >= 1 its own partial
// slot.  An expert without rows has one empty chunk: its dW is written zero.
template <class C>
__global__ __launch_bounds__(C::NTHREADS) void bwd_wgrad_kernel(
    const uint16_t* __restrict__ dht, const uint16_t* __restrict__ awt,
    const uint16_t* __restrict__ xst, const uint16_t* __restrict__ dst,
    const int32_t* __restrict__ offsets, int E_local, int d, int I, int gr, int P_pad,
    float* __restrict__ dW1, float* __restrict__ dW3, float* __restrict__ dW2,
    float* __restrict__ partial) {
  extern __shared__ __align__(16) uint16_t lds[];
  __shared__ int32_t task_pre[kMaxLocalExperts + 1];
  __shared__ int32_t slot_pre[kMaxLocalExperts + 1];
  __shared__ int32_t seg[kMaxLocalExperts + 1];
  // gr = 2: the (dH1 | dH3)^T rows give dW1 (n < I) and dW3; gr = 1: dW1 only
  const int n13 = gr * I / C::BW, t13 = (d + C::BT - 1) / C::BT;
  const int n2 = d / C::BW, t2 = (I + C::BT - 1) / C::BT;
  const int per_chunk = n13 * t13 + n2 * t2;
  build_seg_prefix(offsets, E_local, seg);
  if (threadIdx.x == 0) {
    int run = 0, srun = 0;
    for (int e = 0; e < E_local; ++e) {
      const int nc = n_chunks(offsets[e + 1] - offsets[e]);
      task_pre[e] = run;
      slot_pre[e] = srun;
      run += nc * per_chunk;
      srun += nc - 1;
    }
    task_pre[E_local] = run;
    slot_pre[E_local] = srun;
  }
  __syncthreads();
  const size_t mat = static_cast<size_t>(d) * I;
  const int KB = P_pad / 32;
  const int lane = lane_id();
  const int wr = tile_wr<C>(), wt = tile_wt<C>();
  const int total = uniform(task_pre[E_local]);
  for (int task = blockIdx.x; task < total; task += gridDim.x) {
    const int e = uniform(expert_of_mtile(task_pre, 0, E_local, task));
    int rel = task - uniform(task_pre[e]);
    const int c = rel / per_chunk;
    rel %= per_chunk;
    const bool m13 = rel < n13 * t13;
    if (!m13) rel -= n13 * t13;
    const int nt = m13 ? rel % n13 : rel % n2, tt = m13 ? rel / n13 : rel / n2;
    const int padded = uniform((offsets[e + 1] - offsets[e] + 63) & ~63);
    const int kbeg = uniform(seg[e] + c * kWgradChunkRows);
    const int kend = uniform(seg[e] + min(padded, (c + 1) * kWgradChunkRows));
    const int nk = uniform((kend - kbeg) / C::BK);
    const int Tdim = m13 ? d : I;
    const uint16_t* A = (m13 ? dht : dst) + frag_offset(nt * (C::BW / 16), kbeg / 32, KB);
    const uint16_t* Bm = m13 ? xst : awt;
    TokRows<C> trow;
#pragma unroll
    for (int i = 0; i < C::LT; ++i) {
      const int t = min(tt * C::BT + trow_index<C>(i), Tdim - 1);
      trow.p[i] = Bm + static_cast<size_t>(t) * P_pad + kbeg;
    }
    TileAcc<C> acc;
    tile_mma<C>(A, KB, nk, trow, lds, acc, min(C::BT, Tdim - tt * C::BT));
    float* base[3];
    if (c == 0) {
      base[0] = dW1 + e * mat;
      base[1] = dW3 ? dW3 + e * mat : nullptr;  // no dW3 when ungated (never written then)
      base[2] = dW2 + e * mat;
    } else {
      float* slot = partial + static_cast<size_t>(uniform(slot_pre[e]) + c - 1) * 3 * mat;
      base[0] = slot;
      base[1] = slot + mat;
      base[2] = slot + 2 * mat;
    }
#pragma unroll
    for (int aa = 0; aa < C::AW; ++aa) {
      const int n = nt * C::BW + (wr * C::AW + aa) * 16 + 4 * (lane / 16);
#pragma unroll
      for (int b = 0; b < C::AT; ++b) {
        const int t = tt * C::BT + (wt * C::AT + b) * 16 + (lane & 15);
        if (t >= Tdim) continue;
        float* o = m13 ? (n < I ? base[0] + static_cast<size_t>(t) * I + n : base[1] + static_cast<size_t>(t) * I + (n - I))
                       : base[2] + static_cast<size_t>(t) * d + n;
        *reinterpret_cast<f32x4*>(o) = acc.v[aa][b];
      }
    }
  }
}

// dW_e += partial slots of chunks 1 .. n-1 in ascending order (dW3 only
// when gr = 2).
__global__ __launch_bounds__(256) void wgrad_reduce_kernel(const int32_t* __restrict__ offsets,
                                                           int E_local, size_t mat, int gr,
                                                           float* __restrict__ dW1,
                                                           float* __restrict__ dW3,
                                                           float* __restrict__ dW2,
                                                           const float* __restrict__ partial) {
  int slot = 0;
  for (int e = 0; e < E_local; ++e) {
    const int nc = n_chunks(offsets[e + 1] - offsets[e]);
    if (nc > 1) {
      for (size_t i = (static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4; i < 3 * mat;
           i += static_cast<size_t>(gridDim.x) * blockDim.x * 4) {
        const int m = static_cast<int>(i / mat);
        if (m == 1 && gr == 1) continue;
        const size_t o = i % mat;
        float* dst = (m == 0 ? dW1 : m == 1 ? dW3 : dW2) + e * mat + o;
        f32x4 acc = *reinterpret_cast<const f32x4*>(dst);
        for (int c = 1; c < nc; ++c) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(partial + (static_cast<size_t>(slot + c - 1) * 3 + m) * mat + o);
          acc = f32x4{acc[0] + v[0], acc[1] + v[1], acc[2] + v[2], acc[3] + v[3]};
        }
        *reinterpret_cast<f32x4*>(dst) = acc;
      }
    }
    slot += nc - 1;
  }
}


// Tile shape of the dX product (rows per expert decide, as in the forward).
enum class DxShape { Small, Small64, Large, Mid };

DxShape pick_dx_shape(const moe_problem_t& p) {
  const double rows = static_cast<double>(p.T) * p.k / p.E_global;
  if (rows < 96.0) return p.T <= FfnSmall::G2::BT ? DxShape::Small : DxShape::Small64;
  if (p.d % FfnLarge::G2::BW == 0) return DxShape::Large;
  return DxShape::Mid;
}

template <class F>
hipError_t launch_dx_gemm(const moe_problem_t& p, const uint16_t* dh, const uint16_t* w13t,
                          const int32_t* offsets, uint16_t* dxr, int cus, hipStream_t s) {
  int per_cu = 0;
  hipError_t e;
  constexpr size_t lds = F::G2::LDS_BYTES;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, bwd_dx_gemm_kernel<F>, F::NT, lds)) != hipSuccess)
    return e;
  bwd_dx_gemm_kernel<F><<<max(1, per_cu) * cus, F::NT, lds, s>>>(dh, w13t, offsets, dxr, p.E_local, p.d,
                                                                 gate_rows(p) * p.I);
  return hipGetLastError();
}

template <class C>
hipError_t launch_g(const moe_problem_t& p, const BackwardArgs& a, const uint16_t* w2b, float* g, int cus,
                    hipStream_t s) {
  int per_cu = 0;
  hipError_t e;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, bwd_g_kernel<C>, C::NTHREADS, C::LDS_BYTES)) !=
      hipSuccess)
    return e;
  bwd_g_kernel<C><<<max(1, per_cu) * cus, C::NTHREADS, C::LDS_BYTES, s>>>(
      static_cast<const uint16_t*>(a.dout), w2b, a.offsets, a.sorted_token, p.E_local, p.d, p.I, g);
  return hipGetLastError();
}

template <class C>
hipError_t launch_wgrad(const moe_problem_t& p, const WsLayout& L, const uint16_t* dht, const uint16_t* awt,
                        const uint16_t* xst, const uint16_t* dst, const BackwardArgs& a, float* partial, int cus,
                        hipStream_t s) {
  int per_cu = 0;
  hipError_t e;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, bwd_wgrad_kernel<C>, C::NTHREADS,
                                                        C::LDS_BYTES)) != hipSuccess)
    return e;
  bwd_wgrad_kernel<C><<<max(1, per_cu) * cus, C::NTHREADS, C::LDS_BYTES, s>>>(
      dht, awt, xst, dst, a.offsets, p.E_local, p.d, p.I, gate_rows(p), L.P_pad, a.dW1, a.dW3, a.dW2, partial);
  return hipGetLastError();
}

// The recompute with the gradient epilogue on tile C.
template <class C, bool GATED, bool SAVED>
hipError_t launch_dh_kind(const moe_problem_t& p, const WsLayout& L, const BackwardArgs& a, const uint16_t* xb,
                          const uint16_t* w13, const float* g, uint16_t* dh, uint16_t* dht, uint16_t* awt,
                          float* dwp, int cus, hipStream_t s) {
  constexpr size_t lds = BwdDh<C, GATED, SAVED>::LDS;
  int per_cu = 0;
  hipError_t e;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, bwd_dh_kernel<C, GATED, SAVED>, C::NTHREADS,
                                                        lds)) != hipSuccess)
    return e;
  bwd_dh_kernel<C, GATED, SAVED><<<max(1, per_cu) * cus, C::NTHREADS, lds, s>>>(
      xb, w13, g, a.offsets, a.sorted_token, a.pair_pos, a.topk_w, p.E_local, p.d, p.I, p.k, L.P_pad, dh, dht, awt,
      dwp, a.hsaved);
  return hipGetLastError();
}

template <class C, bool GATED>
hipError_t launch_dh_act(const moe_problem_t& p, const WsLayout& L, const BackwardArgs& a, const uint16_t* xb,
                         const uint16_t* w13, const float* g, uint16_t* dh, uint16_t* dht, uint16_t* awt,
                         float* dwp, int cus, hipStream_t s) {
  if (a.hsaved) return launch_dh_kind<C, GATED, true>(p, L, a, xb, w13, g, dh, dht, awt, dwp, cus, s);
  return launch_dh_kind<C, GATED, false>(p, L, a, xb, w13, g, dh, dht, awt, dwp, cus, s);
}

template <class C>
hipError_t launch_dh(const moe_problem_t& p, const WsLayout& L, const BackwardArgs& a, const uint16_t* xb,
                     const uint16_t* w13, const float* g, uint16_t* dh, uint16_t* dht, uint16_t* awt, float* dwp,
                     int cus, hipStream_t s) {
  if (gate_rows(p) == 2) return launch_dh_act<C, true>(p, L, a, xb, w13, g, dh, dht, awt, dwp, cus, s);
  return launch_dh_act<C, false>(p, L, a, xb, w13, g, dh, dht, awt, dwp, cus, s);
}

// The weight gradient's branch (the transposed x and dout rows, then the
// weight-gradient tiles and their reduction) shares no buffer with the data
// gradient's branch (gate, dx rows, scatter, dWg) and runs on a second stream
// of the device, forked from and joined back into the caller's stream with
// events: the CUs one branch leaves idle at the tail of a kernel, or while
// an HBM-bound kernel runs, take the other branch's tiles.  Every kernel
// computes what it computed in order; only their overlap changes, never a
// bit.  The stream is created once per device (default priority, not
// blocking on the null stream) and kept; the events belong to one call.
hipError_t side_stream(hipStream_t* out) {
  static std::mutex mu;
  static std::vector<hipStream_t> streams;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if (static_cast<size_t>(dev) >= streams.size()) streams.resize(dev + 1, nullptr);
  if (!streams[dev] && (e = hipStreamCreateWithFlags(&streams[dev], hipStreamNonBlocking)) != hipSuccess) {
    streams[dev] = nullptr;
    return e;
  }
  *out = streams[dev];
  return hipSuccess;
}

struct ForkEvents {
  hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
  hipError_t create() {
    for (auto& e : ev) {
      const hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableTiming);
      if (r != hipSuccess) return r;
    }
    return hipSuccess;
  }
  // destroying an event whose waits are enqueued is allowed: its resources
  // are released once it completes
  ~ForkEvents() {
    for (auto e : ev)
      if (e) (void)hipEventDestroy(e);
  }
};

// s2 continues after everything enqueued on s so far.
hipError_t fork_to(hipStream_t s, hipStream_t s2, hipEvent_t ev) {
  hipError_t e = hipEventRecord(ev, s);
  return e != hipSuccess ? e : hipStreamWaitEvent(s2, ev, 0);
}

}  // namespace

hipError_t launch_backward(const moe_problem_t& p, const WsLayout& L, const BackwardArgs& a, char* ws,
                           hipStream_t s) {
  const PackedLayout PL = packed_layout(p.d, p.I, p.E_global, p.E_local, p.x_dtype == MOE_BF16, gate_rows(p));
  const char* pk = static_cast<const char*>(a.packed);
  const uint16_t* w13 = reinterpret_cast<const uint16_t*>(pk + PL.w13);
  const PackedBwdLayout BL = packed_bwd_layout(p);
  const char* pb = static_cast<const char*>(a.packed_bwd);
  const uint16_t* w2b = reinterpret_cast<const uint16_t*>(pb + BL.w2b);
  const bool want_dw = a.dW1 != nullptr;
  const bool want_data = a.dx != nullptr;
  const bool xbf = p.x_dtype == MOE_BF16;
  uint16_t* dh = reinterpret_cast<uint16_t*>(ws + L.bwd_dh);
  uint16_t* dht = want_dw ? reinterpret_cast<uint16_t*>(ws + L.bwd_dht) : nullptr;
  uint16_t* awt = reinterpret_cast<uint16_t*>(ws + L.bwd_awt);
  uint16_t* xst = reinterpret_cast<uint16_t*>(ws + L.bwd_xst);
  uint16_t* dst = reinterpret_cast<uint16_t*>(ws + L.bwd_dst);
  float* dwp = want_data ? reinterpret_cast<float*>(ws + L.bwd_dwp) : nullptr;
  float* dlc = reinterpret_cast<float*>(ws + L.bwd_dlc);
  uint16_t* dld = (want_data && a.dWg && xbf) ? reinterpret_cast<uint16_t*>(ws + L.bwd_dld) : nullptr;
  uint16_t* dxr = reinterpret_cast<uint16_t*>(ws + L.bwd_dxr);
  float* partial = reinterpret_cast<float*>(ws + L.wgrad);
  const uint16_t* xb = nullptr;
  hipError_t e;
  int dev = 0, cus = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  // the same bf16 staging copy of x that the forward GEMM1 reads
  if ((e = stage_x_bf16(p, L, a.x, ws, s, &xb)) != hipSuccess) return e;
  const size_t words = static_cast<size_t>(p.E_local) * p.d * p.I;
  if (p.T == 0) {
    // no rows: every gradient is zero (dx, dtopk_w and dlogits are empty)
    if (want_dw) {
      if ((e = fill_zero(a.dW1, words, s)) != hipSuccess) return e;
      if (a.dW3 && (e = fill_zero(a.dW3, words, s)) != hipSuccess) return e;
      if ((e = fill_zero(a.dW2, words, s)) != hipSuccess) return e;
    }
    if (a.dWg) return fill_zero(a.dWg, static_cast<size_t>(p.d) * p.E_global, s);
    return hipSuccess;
  }
  // the weight-gradient branch on s2: the transposes now (they need only x
  // and dout), the tiles once the recompute below has run
  hipStream_t s2 = s;
  ForkEvents fk;
  if (want_dw) {
    if ((e = side_stream(&s2)) != hipSuccess) return e;
    if ((e = fk.create()) != hipSuccess) return e;
    if ((e = fork_to(s, s2, fk.ev[0])) != hipSuccess) return e;
    bwd_gather_t_kernel<<<dim3(L.P_pad / 64, p.d / 64), 256, 0, s2>>>(
        xb, static_cast<const uint16_t*>(a.dout), a.offsets, a.sorted_token, p.E_local, p.d, L.P_pad, xst, dst);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // joins s2 back into s (also after a failed launch, so that no work of
  // this call is left behind on s2)
  auto finish = [&](hipError_t r) {
    if (want_dw) {
      const hipError_t j = fork_to(s2, s, fk.ev[2]);
      if (r == hipSuccess) r = j;
    }
    return r;
  };
  float* g = reinterpret_cast<float*>(ws + L.bwd_g);
  if (p.I % FfnLarge::G1::BW == 0)
    e = launch_g<FfnLarge::G1>(p, a, w2b, g, cus, s);
  else if (p.I % BwdCfg::BW == 0)
    e = launch_g<BwdCfg>(p, a, w2b, g, cus, s);
  else
    e = launch_g<BwdCfgG>(p, a, w2b, g, cus, s);
  if (e != hipSuccess) return finish(e);
  const int gr = gate_rows(p);
  // from saved pre-activations the kernel only streams memory: the 128-wide
  // tiles (twice as many, half the work each) leave a shorter last round
  if (!a.hsaved && (gr * p.I) % BwdCfgL::BW == 0)
    e = launch_dh<BwdCfgL>(p, L, a, xb, w13, g, dh, dht, awt, dwp, cus, s);
  else
    e = launch_dh<BwdCfg>(p, L, a, xb, w13, g, dh, dht, awt, dwp, cus, s);
  if (e != hipSuccess) return finish(e);
  if (want_dw) {
    if ((e = fork_to(s, s2, fk.ev[1])) != hipSuccess) return finish(e);
    if ((gr * p.I) % FfnLarge::G1::BW == 0 && p.d % FfnLarge::G1::BW == 0)
      e = launch_wgrad<FfnLarge::G1>(p, L, dht, awt, xst, dst, a, partial, cus, s2);
    else
      e = launch_wgrad<FfnMid::G1>(p, L, dht, awt, xst, dst, a, partial, cus, s2);
    if (e != hipSuccess) return finish(e);
    wgrad_reduce_kernel<<<cus * 4, 256, 0, s2>>>(a.offsets, p.E_local, static_cast<size_t>(p.d) * p.I,
                                                 gate_rows(p), a.dW1, a.dW3, a.dW2, partial);
    if ((e = hipGetLastError()) != hipSuccess) return finish(e);
  }
  if (want_data) {
    const uint16_t* w13t = reinterpret_cast<const uint16_t*>(pb + BL.w13t);
    const void* wgt = pb + BL.wgt;
    bwd_gate_kernel<<<(p.T + 3) / 4, 256, 0, s>>>(dwp, p.I / 16, a.pair_pos, a.topk_idx, a.topk_w, p.T, p.k,
                                                  p.E_global, L.Ep, a.dtopk_w, dlc, a.dlogits, dld);
    if ((e = hipGetLastError()) != hipSuccess) return finish(e);
    // dWg needs only x and the gate's dl: with a weight gradient it goes to
    // s2 behind the weight-gradient tiles, next to the dx rows and scatter
    hipStream_t sg = s;
    if (a.dWg && want_dw) {
      if ((e = fork_to(s, s2, fk.ev[3])) != hipSuccess) return finish(e);
      sg = s2;
    }
    switch (pick_dx_shape(p)) {
      case DxShape::Small: e = launch_dx_gemm<FfnSmall>(p, dh, w13t, a.offsets, dxr, cus, s); break;
      case DxShape::Small64: e = launch_dx_gemm<FfnSmall64>(p, dh, w13t, a.offsets, dxr, cus, s); break;
      case DxShape::Large: e = launch_dx_gemm<FfnLarge>(p, dh, w13t, a.offsets, dxr, cus, s); break;
      default: e = launch_dx_gemm<FfnMid>(p, dh, w13t, a.offsets, dxr, cus, s); break;
    }
    if (e != hipSuccess) return finish(e);
    const int parts = combine_parts(p.T, p.d);
    const dim3 grid((p.T + 3) / 4, parts);
    if (xbf)
      bwd_dx_scatter_kernel<true><<<grid, 256, 0, s>>>(dxr, a.pair_pos, a.topk_idx, dlc, wgt, p.T, p.k, p.d,
                                                       p.E_global, parts, a.dx);
    else
      bwd_dx_scatter_kernel<false><<<grid, 256, 0, s>>>(dxr, a.pair_pos, a.topk_idx, dlc, wgt, p.T, p.k, p.d,
                                                        p.E_global, parts, a.dx);
    if ((e = hipGetLastError()) != hipSuccess) return finish(e);
    if (a.dWg) {
      const size_t n = static_cast<size_t>(p.d) * p.E_global;
      const unsigned blocks = static_cast<unsigned>((n + 255) / 256);
      if (xbf) {
        using C = TileCfg<128, 128, 2, 2, 64, 2>;
        float* part = reinterpret_cast<float*>(ws + L.bwd_dwg);
        bwd_dwg_kernel<<<cus * 2, 256, C::LDS_BYTES, sg>>>(dld, xb, p.T, p.d, L.Ep, part);
        if ((e = hipGetLastError()) != hipSuccess) return finish(e);
        bwd_dwg_reduce_kernel<<<blocks, 256, 0, sg>>>(part, (p.T + kDwgChunkRows - 1) / kDwgChunkRows, p.d,
                                                      p.E_global, L.Ep, a.dWg);
      } else {
        bwd_dwg_f32_kernel<<<blocks, 256, 0, sg>>>(static_cast<const float*>(a.x), a.topk_idx, dlc, p.T, p.k,
                                                   p.d, p.E_global, a.dWg);
      }
      if ((e = hipGetLastError()) != hipSuccess) return finish(e);
    }
  }
  return finish(hipSuccess);
}

}  // namespace moe
