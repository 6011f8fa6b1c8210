// probe.hip -- measurement probes for the roofline denominators: a
// matrix-core loop and a plain copy, launched through the C ABI so that the
// measured rates come from the same device, clocks and launch path as the
// layer's kernels.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kProbeThreads = 512;  // 8 wavefronts, two per SIMD
constexpr int kProbeAcc = 16;       // independent accumulators per wavefront

__global__ __launch_bounds__(kProbeThreads) void probe_mfma_kernel(float* __restrict__ out, int steps) {
  f32x4 acc[kProbeAcc];
#pragma unroll
  for (int i = 0; i < kProbeAcc; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // operands from the thread index, so that nothing folds at compile time
  const uint32_t t = threadIdx.x;
  const u32x4 a{0x3c003c00u ^ (t & 7u), 0x3c003c00u, 0x3b803b80u, 0x3b803b80u ^ (t & 3u)};
  const u32x4 b{0x3a003a00u, 0x3a003a00u ^ (t & 1u), 0x39803980u, 0x39803980u};
  for (int s = 0; s < steps; ++s) {
#pragma unroll
    for (int i = 0; i < kProbeAcc; ++i) acc[i] = mfma16x16x32(a, b, acc[i]);
  }
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < kProbeAcc; ++i) sum += (acc[i][0] + acc[i][1]) + (acc[i][2] + acc[i][3]);
  out[static_cast<size_t>(blockIdx.x) * kProbeThreads + threadIdx.x] = sum;
}

// One 16-byte word per thread per round, four workgroups of 256 per CU:
// the fastest of the simple copies measured on MI355X (5.7 TB/s of read +
// written bytes for 1 GiB; unrolled rounds and more workgroups measured
// 4.1-5.3 TB/s).
__global__ __launch_bounds__(256) void probe_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                         size_t n) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    dst[i] = src[i];
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

moe_status_t moe_probe_mfma(float* out, size_t out_bytes, int32_t steps, double* flops, moe_stream_t stream) {
  if (!out || !flops || steps < 1 || steps > (1 << 20)) return MOE_ERR_INVALID_ARG;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return MOE_ERR_HIP;
  if (out_bytes < static_cast<size_t>(cus) * kProbeThreads * sizeof(float)) return MOE_ERR_INVALID_ARG;
  *flops = static_cast<double>(cus) * (kProbeThreads / 64) * steps * kProbeAcc * (2.0 * 16 * 16 * 32);
  probe_mfma_kernel<<<cus, kProbeThreads, 0, static_cast<hipStream_t>(stream)>>>(out, steps);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status_t moe_probe_copy(void* dst, const void* src, size_t bytes, moe_stream_t stream) {
  if (!dst || !src || bytes % 16 != 0) return MOE_ERR_INVALID_ARG;
  const uintptr_t d = reinterpret_cast<uintptr_t>(dst), s = reinterpret_cast<uintptr_t>(src);
  if ((d | s) & 15u) return MOE_ERR_INVALID_ARG;
  if (d < s + bytes && s < d + bytes) return MOE_ERR_INVALID_ARG;  // overlap
  if (bytes == 0) return MOE_OK;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return MOE_ERR_HIP;
  probe_copy_kernel<<<cus * 4, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
