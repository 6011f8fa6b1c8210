// wgrad.hip -- deterministic weight gradient of the expert FFN.
//
// 10100.com commentary (batch-invariant and deterministic operators) and
// the DeepSeek-V4 launch digest (itsolotime.com, section 3): gradients must
// be bitwise identical across repeated backward passes, so there are no
// unordered float atomics: work is pre-sorted, each unit writes an isolated
// buffer, and a final reduction sums the buffers in a fixed order.
//
// Per local expert e with routed rows r (token t_r, router weight w_r):
//   stage 1 (per row tile x 64 intermediate indices)
//     h1, h3   = x_r W1, x_r W3   (the forward's GEMM1 tile, same bits)
//     g        = dout_t W2^T      (fp32),   dA = w_r g
//     s        = sigmoid(h1),     silu = h1 s
//     dH3      = dA silu,         dH1 = dA h3 s (1 + h1 (1 - s))
//     aw       = w_r silu h3
//     -> dH1, dH3, aw rounded to bf16, sorted-row order
//   stage 2 (per output tile, per fixed chunk of kWgradChunkRows rows)
//     dW1_e += x^T dH1,  dW3_e += x^T dH3,  dW2_e += aw^T dout
//     the K (= row) index is walked in ascending order inside a chunk; the
//     first chunk of an expert writes dW directly, chunk c >= 1 writes its
//     own partial slot;
//   stage 3: dW_e += partial slots in ascending chunk order.
#include "ffn_parts.h"
#include "moe_internal.h"

namespace moe {
namespace {

using DhCfg13 = TileCfg<128, 128, 2, 2, 64, 3>;  // 128 packed rows = 64 (h1, h3) pairs
using DhCfgG = TileCfg<64, 128, 2, 2, 64, 3>;    // 64 rows of W2 (as [I][d])
static_assert(DhCfg13::BT == DhCfgG::BT, "same row tile");

__global__ __launch_bounds__(256) void wgrad_dh_kernel(
    const uint16_t* __restrict__ xb, const uint16_t* __restrict__ dout,
    const uint16_t* __restrict__ w13, const uint16_t* __restrict__ w2b,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_token,
    const int32_t* __restrict__ pair_pos, const float* __restrict__ topk_w, int E_local, int d,
    int I, int k, uint16_t* __restrict__ dH1, uint16_t* __restrict__ dH3, uint16_t* __restrict__ aw) {
  extern __shared__ __align__(16) uint16_t lds[];
  __shared__ int32_t mt_pre[kMaxLocalExperts + 1];
  __shared__ float wrow[128];
  build_mtile_prefix(offsets, E_local, DhCfg13::BT, mt_pre);
  __syncthreads();
  const int NT = I / 64;
  const int total = uniform(mt_pre[E_local] * NT);
  const int lane = lane_id();
  static_assert(DhCfg13::WR == 2 && DhCfg13::WT == 2 && DhCfgG::WR == 2 && DhCfgG::WT == 2, "epilogue below");
  const int wr = tile_wr<DhCfg13>(), wt = tile_wt<DhCfg13>();
  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const int mt = tile / NT, nt = tile % NT;
    const int e = uniform(expert_of_mtile(mt_pre, 0, E_local, mt));
    const int row0 = uniform(offsets[e] + (mt - mt_pre[e]) * 128);
    const int count = uniform(min(128, offsets[e + 1] - row0));
    {
      // router weight of each row of the tile (threads 128..255 duplicate
      // threads 0..127 and store the same value: no divergent branch here)
      const int r = threadIdx.x & 127;
      const int row = row0 + min(r, count - 1), t = sorted_token[row];
      float w = 0.f;
      for (int j = 0; j < k; ++j) {
        const bool hit = pair_pos[static_cast<size_t>(t) * k + j] == row;
        w = hit ? topk_w[static_cast<size_t>(t) * k + j] : w;
      }
      wrow[r] = r < count ? w : 0.f;
    }
    // h1, h3: exactly the forward GEMM1 tile
    TokRows<DhCfg13> trx;
    TokRows<DhCfgG> trd;
#pragma unroll
    for (int i = 0; i < DhCfg13::LT; ++i) {
      const int r = min(trow_index<DhCfg13>(i), count - 1);
      trx.p[i] = xb + static_cast<size_t>(sorted_token[row0 + r]) * d;
    }
#pragma unroll
    for (int i = 0; i < DhCfgG::LT; ++i) {
      const int r = min(trow_index<DhCfgG>(i), count - 1);
      trd.p[i] = dout + static_cast<size_t>(sorted_token[row0 + r]) * d;
    }
    TileAcc<DhCfg13> acc13;
    tile_mma<DhCfg13>(w13 + static_cast<size_t>(e) * 2 * I * d + frag_offset(nt * 8, 0, d / 32), d / 32,
                      d / DhCfg13::BK, trx, lds, acc13);
    TileAcc<DhCfgG> accg;
    tile_mma<DhCfgG>(w2b + static_cast<size_t>(e) * I * d + frag_offset(nt * 4, 0, d / 32), d / 32,
                     d / DhCfgG::BK, trd, lds, accg);
    // wave (wr, wt): acc13 row blocks 4wr..4wr+3 = (h1, h3) pairs of
    // intermediate blocks 2wr, 2wr+1 of this tile; accg row blocks 2wr, 2wr+1.
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int i0 = nt * 64 + (wr * 2 + a) * 16 + 4 * (lane / 16);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int tr = (wt * 4 + b) * 16 + (lane & 15);
        if (tr >= count) continue;
        const float w = wrow[tr];
        float v1[4], v3[4], va[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float h1 = acc13.v[2 * a][b][r], h3 = acc13.v[2 * a + 1][b][r];
          const float dA = w * accg.v[a][b][r];
          const float s = 1.0f / (1.0f + expf(-h1));
          const float silu = h1 * s;
          v3[r] = dA * silu;
          v1[r] = ((dA * h3) * s) * (1.0f + h1 * (1.0f - s));
          va[r] = w * (silu * h3);
        }
        const size_t o = static_cast<size_t>(row0 + tr) * I + i0;
        *reinterpret_cast<u32x2*>(dH1 + o) = u32x2{pack_bf16x2(v1[0], v1[1]), pack_bf16x2(v1[2], v1[3])};
        *reinterpret_cast<u32x2*>(dH3 + o) = u32x2{pack_bf16x2(v3[0], v3[1]), pack_bf16x2(v3[2], v3[3])};
        *reinterpret_cast<u32x2*>(aw + o) = u32x2{pack_bf16x2(va[0], va[1]), pack_bf16x2(va[2], va[3])};
      }
    }
    __syncthreads();  // wrow reused by the next tile
  }
}

// ---------------------------------------------------------------- stage 2

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

__device__ __forceinline__ int n_chunks(int rows) {
  return rows <= kWgradChunkRows ? 1 : (rows + kWgradChunkRows - 1) / kWgradChunkRows;
}

__global__ __launch_bounds__(256) void wgrad_w_kernel(
    const uint16_t* __restrict__ xb, const uint16_t* __restrict__ dout,
    const uint16_t* __restrict__ dH1, const uint16_t* __restrict__ dH3,
    const uint16_t* __restrict__ aw, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_token, int E_local, int d, int I, float* __restrict__ dW1,
    float* __restrict__ dW3, float* __restrict__ dW2, float* __restrict__ partial) {
  extern __shared__ __align__(16) uint16_t lds[];
  __shared__ int32_t task_pre[kMaxLocalExperts + 1];
  __shared__ int32_t slot_pre[kMaxLocalExperts + 1];
  const int tI = (I + 127) / 128, tD = (d + 127) / 128;
  const int tpm = tI * tD;  // tiles per matrix (dW1/dW3: u = i, v = f; dW2: u = n, v = i)
  if (threadIdx.x == 0) {
    int run = 0, srun = 0;
    for (int e = 0; e < E_local; ++e) {
      const int nc = n_chunks(offsets[e + 1] - offsets[e]);
      task_pre[e] = run;
      slot_pre[e] = srun;
      run += nc * 3 * tpm;
      srun += nc - 1;
    }
    task_pre[E_local] = run;
    slot_pre[E_local] = srun;
  }
  __syncthreads();
  const size_t mat = static_cast<size_t>(d) * I;
  const int total = uniform(task_pre[E_local]);
  for (int task = blockIdx.x; task < total; task += gridDim.x) {
    const int e = uniform(expert_of_mtile(task_pre, 0, E_local, task));
    int rel = task - uniform(task_pre[e]);
    const int c = rel / (3 * tpm);
    rel %= 3 * tpm;
    const int m = rel / tpm, t = rel % tpm;
    const int r0 = uniform(offsets[e]), rows = uniform(offsets[e + 1]) - r0;
    const int rbeg = r0 + c * kWgradChunkRows;
    const int rend = r0 + min(rows, (c + 1) * kWgradChunkRows);
    float* base;
    if (c == 0) {
      base = (m == 0 ? dW1 : m == 1 ? dW3 : dW2) + e * mat;
    } else {
      base = partial + (static_cast<size_t>(uniform(slot_pre[e]) + c - 1) * 3 + m) * mat;
    }
    if (m < 2) {
      const int ut = t % tI, vt = t / tI;
      wgrad_tile(m == 0 ? dH1 : dH3, false, I, I, xb, true, d, d, sorted_token, rbeg, rend, ut, vt,
                 base, lds);
    } else {
      const int ut = t % tD, vt = t / tD;
      wgrad_tile(dout, true, d, d, aw, false, I, I, sorted_token, rbeg, rend, ut, vt, base, lds);
    }
  }
}

// dW_e += partial slots of chunks 1 .. n-1 in ascending order.
__global__ __launch_bounds__(256) void wgrad_reduce_kernel(const int32_t* __restrict__ offsets,
                                                           int E_local, size_t mat,
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

}  // namespace

hipError_t launch_wgrad(const moe_problem_t& p, const WsLayout& L, const void* x, const void* packed,
                        const int32_t* offsets, const int32_t* sorted_token,
                        const int32_t* pair_pos, const float* topk_w, const void* dout,
                        float* dW1, float* dW3, float* dW2, char* ws, hipStream_t s) {
  const PackedLayout PL = packed_layout(p.d, p.I, p.E_global, p.E_local, p.x_dtype == MOE_BF16);
  const char* pk = static_cast<const char*>(packed);
  const uint16_t* w13 = reinterpret_cast<const uint16_t*>(pk + PL.w13);
  const uint16_t* w2b = reinterpret_cast<const uint16_t*>(pk + PL.w2b);
  const size_t PI = static_cast<size_t>(L.P_max) * p.I;
  uint16_t* dH1 = reinterpret_cast<uint16_t*>(ws + L.wgrad);
  uint16_t* dH3 = dH1 + PI;
  uint16_t* aw = dH3 + PI;
  float* partial = reinterpret_cast<float*>(ws + L.wgrad + align_up(PI * 2 * 3, 256));
  const uint16_t* xb = nullptr;
  hipError_t e;
  int dev = 0, cus = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  // the same bf16 staging copy of x that the forward GEMM1 reads
  if ((e = stage_x_bf16(p, L, x, ws, s, &xb)) != hipSuccess) return e;
  if (p.T == 0) {
    // no rows: every gradient is zero
    const size_t words = static_cast<size_t>(p.E_local) * p.d * p.I;
    if ((e = fill_zero(dW1, words, s)) != hipSuccess) return e;
    if ((e = fill_zero(dW3, words, s)) != hipSuccess) return e;
    return fill_zero(dW2, words, s);
  }
  const size_t lds13 = DhCfg13::LDS_BYTES > DhCfgG::LDS_BYTES ? DhCfg13::LDS_BYTES : DhCfgG::LDS_BYTES;
  wgrad_dh_kernel<<<cus * 2, 256, lds13, s>>>(xb, static_cast<const uint16_t*>(dout), w13, w2b, offsets,
                                              sorted_token, pair_pos, topk_w, p.E_local, p.d, p.I, p.k,
                                              dH1, dH3, aw);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  using C = TileCfg<128, 128, 2, 2, 64, 2>;
  wgrad_w_kernel<<<cus * 2, 256, C::LDS_BYTES, s>>>(xb, static_cast<const uint16_t*>(dout), dH1, dH3, aw,
                                                    offsets, sorted_token, p.E_local, p.d, p.I, dW1, dW3,
                                                    dW2, partial);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  wgrad_reduce_kernel<<<cus * 4, 256, 0, s>>>(offsets, p.E_local, static_cast<size_t>(p.d) * p.I, dW1,
                                              dW3, dW2, partial);
  return hipGetLastError();
}

}  // namespace moe
