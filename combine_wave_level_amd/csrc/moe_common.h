// moe_common.h -- device-side building blocks shared by the MoE kernels
// (gfx950 / CDNA4 only).
//
// Numeric policy (DeepSeek-V4 launch digest, itsolotime.com, section 2.3:
// precision first, no fast-math, explicit rounding): every file is compiled
// with -ffp-contract=off and without fast-math, so each float operation is
// the one written; fused multiply-adds are written explicitly with fmaf;
// float -> bf16 is round-to-nearest-even; exp is the device library expf.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ------------------------------------------------------------------ bf16

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even (gfx950's v_cvt_pk_bf16_f32, which the
// compiler emits for a float -> bf16 conversion); NaN stays a quiet NaN.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return static_cast<uint16_t>(pack_bf16x2(f, 0.0f) & 0xffffu);
}

// ------------------------------------------------------------------ MFMA
//
// One instruction shape for every product in the library:
// v_mfma_f32_16x16x32_bf16, D[16x16] += A[16x32] * B[32x16] in fp32.
// Operand fragments: lane l holds 8 consecutive k (group g = l / 16,
// k = 8g .. 8g+7) of row (A) or column (B) l % 16.  Result: lane l holds
// D[4 * (l / 16) + r][l % 16] for r = 0..3.  Keeping this single shape and
// an ascending K order everywhere is what makes each output element's bits
// independent of the tile it is computed in, hence of the batch.

__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ------------------------------------------------------------------ layout
//
// Fragment layout of a bf16 matrix M[N][K] (N rows, K the reduction index):
// fragment (nb, kb) covers rows 16nb .. 16nb+15 and k 32kb .. 32kb+31, is
// 1 KiB long, and stores M[16nb + (s % 16)][32kb + 8(s / 16) + 0..7] at
// 16-byte slot s (0..63): exactly lane s's MFMA operand.  Fragments of one
// row block are consecutive along K.  In elements:
__host__ __device__ __forceinline__ size_t frag_offset(int nb, int kb, int KB) {
  return (static_cast<size_t>(nb) * KB + kb) * 512;
}

// Packed weight buffer (written once by moe_pack_weights):
//   router   : Wg^T as [Epad][d], Epad = E_global rounded up to 128 rows, in
//              fragment layout when x is bf16; plain row-major fp32 when x
//              is fp32 (the router then runs on the vector ALUs).
//   W13      : per local expert, [2I][d] fragment layout; row block 2b holds
//              W1 columns 16b .. 16b+15 and row block 2b+1 the W3 columns
//              with the same indices, so gate and up values of one
//              intermediate index meet in the same lane (ungated
//              activation: W1^T only, [I][d]).
//   W2       : per local expert, W2^T as [d][I] in fragment layout.
// (The copies of the weights that only the gradients read live in the
// backward buffer, moe_pack_weights_bwd, so a forward-only caller holds each
// expert weight once.)
struct PackedLayout {
  size_t router, w13, w2, total;
  int Epad;
};

__host__ __device__ inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// gate_rows: 2 when W13 holds W1 and W3 (SwiGLU), 1 when it holds W1 only
// (an ungated activation).
__host__ __device__ inline PackedLayout packed_layout(int d, int I, int E_global, int E_local,
                                                      int x_is_bf16, int gate_rows = 2) {
  PackedLayout L;
  L.Epad = static_cast<int>(align_up(static_cast<size_t>(E_global), 128));
  size_t off = 0;
  L.router = off;
  off += align_up(static_cast<size_t>(L.Epad) * d * (x_is_bf16 ? 2 : 4), 256);
  L.w13 = off;
  off += align_up(static_cast<size_t>(E_local) * gate_rows * I * d * 2, 256);
  L.w2 = off;
  off += align_up(static_cast<size_t>(E_local) * d * I * 2, 256);
  L.total = off;
  return L;
}

// ------------------------------------------------------------------ misc

// Marks a value as the same in every lane (it must be: e.g. read from LDS
// after a barrier).  Loops and branches that contain barriers must be
// steered by such values only: if the compiler sees a divergent condition
// it may restructure the loop per lane, and lanes of one wavefront then
// execute different iterations between barriers.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// 16-byte direct-to-LDS load (global_load_lds_dwordx4): lane l copies 16
// bytes at g into LDS at (wave's base) + 16 l.  Kept out of templates so that
// the builtin is checked once, in device compilation only.
__device__ __forceinline__ void lds_dma16(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
}
// The same load with the non-temporal hint (cache policy nt): data read
// once, which the caches should not keep in preference to reused lines.
__device__ __forceinline__ void lds_dma16_nt(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 2);
}
// The same load at device scope (cache policy sc1): coherent with stores
// that another XCD wrote back from its L2.
__device__ __forceinline__ void lds_dma16_coherent(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 16);
}
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

}  // namespace moe
