// quant.hip -- FP8 dispatch: the per-token e4m3 copy of the token rows that
// the expert GEMMs pull.
//
// DeepSeek-V4 launch digest (itsolotime.com), section 1.4 (compute/
// communication bullet): the dispatch sends each token to its experts in
// FP8 and the combine returns BF16.  The pages fix neither the FP8 format
// details nor the scale granularity; here: OCP E4M3 (largest magnitude 448,
// subnormals, no infinities) and one power-of-two scale per token, the
// smallest 2^k with max_i |x[t, i]| <= 448 * 2^k.  An e4m3 value times a
// power of two is exactly representable in bf16, so the experts see the
// dequantized rows without a further rounding.  The router keeps the
// unquantized x.
#include "moe_internal.h"

namespace moe {
namespace {

// 8 consecutive values of row t as floats (bf16 or fp32 x).
template <bool XBF>
__device__ __forceinline__ void load8(const void* __restrict__ x, size_t t, int d, int c, float (&v)[8]) {
  if constexpr (XBF) {
    const u32x4 q = ld16(static_cast<const uint16_t*>(x) + t * d + c * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(q[i] << 16);
      v[2 * i + 1] = __uint_as_float(q[i] & 0xffff0000u);
    }
  } else {
    const float* p = static_cast<const float*>(x) + t * d + c * 8;
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  }
}

// Four values to four e4m3 bytes (round to nearest even), v[0] in the low byte.
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false));
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, d, static_cast<int>(lo), true));
}

// One wavefront per token: the row's largest magnitude (an exact maximum),
// its scale, then the codes of x / scale (an exact power-of-two division).
template <bool XBF>
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const void* __restrict__ x, int T, int d,
                                                           uint8_t* __restrict__ x8, float* __restrict__ xscale) {
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + wave_id();
  if (t >= T) return;
  const int nchunk = d / 8;
  float amax = 0.f;
  for (int c = lane; c < nchunk; c += kWave) {
    float v[8];
    load8<XBF>(x, static_cast<size_t>(t), d, c, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
  }
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, kWave));
  // amax = f 2^e with f in [0.5, 1) and 448 = 0.875 * 2^9: amax <= 448 * 2^k
  // holds first at k = e - 9 when f <= 0.875, else at k = e - 8
  int e = 0;
  const float f = frexpf(amax, &e);
  const int k = amax > 0.f ? e - 9 + (f > 0.875f ? 1 : 0) : 0;
  // x / 2^k as two exact power-of-two products: 2^-k alone overflows fp32
  // for rows whose largest magnitude is below about 2^-119 (k <= -128), and
  // each factor here stays within fp32's normal range; a value the first
  // product takes below fp32's normal range is far below half the smallest
  // e4m3 step after the second, so its code (+-0) is the exact one
  const float s1 = ldexpf(1.0f, (-k) / 2), s2 = ldexpf(1.0f, -k - (-k) / 2);
  for (int c = lane; c < nchunk; c += kWave) {
    float v[8];
    load8<XBF>(x, static_cast<size_t>(t), d, c, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (v[j] * s1) * s2;
    const u32x2 o{pack_fp8x4(v[0], v[1], v[2], v[3]), pack_fp8x4(v[4], v[5], v[6], v[7])};
    *reinterpret_cast<u32x2*>(x8 + static_cast<size_t>(t) * d + c * 8) = o;
  }
  if (lane == 0) xscale[t] = ldexpf(1.0f, k);
}

// The dequantized rows as bf16: 8 codes per thread, each pair through the
// same scaled conversion the fp8 GEMM tiles apply in registers (an e4m3
// value times a power of two is exact in bf16).
__global__ __launch_bounds__(256) void dequant_fp8_kernel(const uint8_t* __restrict__ x8,
                                                          const float* __restrict__ xscale, int d, size_t n8,
                                                          uint16_t* __restrict__ xb) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n8) return;
  const size_t t = i * 8 / d;
  const float sc = xscale[t];
  const u32x2 raw = *reinterpret_cast<const u32x2*>(x8 + i * 8);
  const u32x4 o{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x, sc, false)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x, sc, true)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.y, sc, false)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.y, sc, true))};
  st16(xb + i * 8, o);
}

}  // namespace

hipError_t launch_dequant_fp8(const moe_problem_t& p, const uint8_t* x8, const float* xscale, uint16_t* xb,
                              hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  const size_t n8 = static_cast<size_t>(p.T) * p.d / 8;
  dequant_fp8_kernel<<<static_cast<unsigned>((n8 + 255) / 256), 256, 0, s>>>(x8, xscale, p.d, n8, xb);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8(const moe_problem_t& p, const void* x, uint8_t* x8, float* xscale, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  const unsigned blocks = static_cast<unsigned>((p.T + 3) / 4);
  if (p.x_dtype == MOE_BF16)
    quantize_fp8_kernel<true><<<blocks, 256, 0, s>>>(x, p.T, p.d, x8, xscale);
  else
    quantize_fp8_kernel<false><<<blocks, 256, 0, s>>>(x, p.T, p.d, x8, xscale);
  return hipGetLastError();
}

}  // namespace moe
