// ffn.hip -- the expert FFN of the layer share, scheduled in expert waves.
//
// DeepSeek-V4 launch digest (itsolotime.com), section 1.2: experts are split
// into waves of a few experts; once all tokens of a wave have arrived its
// compute starts, and in steady state the current wave's compute, the
// dispatch of the next wave's tokens and the return of finished experts'
// results run at the same time.  10100.com commentary (fine-grained overlap
// section): the three-stage pipeline lives in one mega-kernel, pull-based.
//
// On one MI355X the "communication" phases are HBM traffic:
//   dispatch pull : GEMM1's operand loader gathers x rows by sorted_token
//                   from the token-order staging buffer straight into LDS;
//   combine       : tokens whose last local expert has finished are summed
//                   back into token order while later waves still compute.
// The persistent kernel claims tasks from one ticket counter in a static
// order; block b of that order holds GEMM1 tiles of wave b, GEMM2 tiles of
// wave b-1 and combine tasks of the tokens that became ready after wave b-2,
// so every wait is on work ticketed one block earlier.  A task only ever
// waits on tasks with smaller tickets, which are held by running
// workgroups, so the schedule cannot deadlock whatever the grid size.
// Tickets decide which workgroup runs a tile, never the arithmetic: the
// result bits equal those of the phase-by-phase kernels (MOE_FLAG_SERIAL).
#include "ffn_parts.h"
#include "moe_internal.h"
#include "wave_sched.h"

namespace moe {
namespace {

// ---------------------------------------------------------------- staging

__global__ void f32_to_bf16_kernel(const float* __restrict__ x, uint16_t* __restrict__ xb, size_t n) {
  const size_t i = (static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  const f32x4 v = *reinterpret_cast<const f32x4*>(x + i);
  u32x2 pk;
  pk.x = pack_bf16x2(v[0], v[1]);
  pk.y = pack_bf16x2(v[2], v[3]);
  *reinterpret_cast<u32x2*>(xb + i) = pk;
}

__global__ void fill_zero_kernel(int32_t* __restrict__ p, size_t n) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// ---------------------------------------------------------------- phase kernels

__global__ __launch_bounds__(256) void gemm1_phase_kernel(
    const uint16_t* __restrict__ xb, const uint16_t* __restrict__ w13,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_token,
    uint16_t* __restrict__ act, int E_local, int d, int I) {
  extern __shared__ __align__(16) uint16_t lds[];
  __shared__ int32_t mt_pre[kMaxLocalExperts + 1];
  build_mtile_prefix(offsets, E_local, G1Cfg::BT, mt_pre);
  __syncthreads();
  const int NT = 2 * I / G1Cfg::BW;
  const int total = uniform(mt_pre[E_local] * NT);
  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const int mt = tile / NT, nt = tile % NT;
    const int e = uniform(expert_of_mtile(mt_pre, 0, E_local, mt));
    const int row0 = uniform(offsets[e] + (mt - mt_pre[e]) * G1Cfg::BT);
    const int count = uniform(min(G1Cfg::BT, offsets[e + 1] - row0));
    gemm1_tile(xb, w13 + static_cast<size_t>(e) * 2 * I * d, sorted_token, act, row0, count, nt, d, I, lds);
  }
}

__global__ __launch_bounds__(256) void gemm2_phase_kernel(
    const uint16_t* __restrict__ act, const uint16_t* __restrict__ w2,
    const int32_t* __restrict__ offsets, uint16_t* __restrict__ y, int E_local, int d, int I) {
  extern __shared__ __align__(16) uint16_t lds[];
  __shared__ int32_t mt_pre[kMaxLocalExperts + 1];
  build_mtile_prefix(offsets, E_local, G2Cfg::BT, mt_pre);
  __syncthreads();
  const int NT = d / G2Cfg::BW;
  const int total = uniform(mt_pre[E_local] * NT);
  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const int mt = tile / NT, nt = tile % NT;
    const int e = uniform(expert_of_mtile(mt_pre, 0, E_local, mt));
    const int row0 = uniform(offsets[e] + (mt - mt_pre[e]) * G2Cfg::BT);
    const int count = uniform(min(G2Cfg::BT, offsets[e + 1] - row0));
    gemm2_tile(act, w2 + static_cast<size_t>(e) * d * I, y, row0, count, nt, d, I, lds);
  }
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y,
                                                      const int32_t* __restrict__ pair_pos,
                                                      const float* __restrict__ topk_w, int T,
                                                      int k, int d, void* __restrict__ out) {
  const int t = blockIdx.x * 4 + wave_id();
  if (t < T) combine_token<OUT_BF16>(t, y, pair_pos, topk_w, k, d, out);
}

// ---------------------------------------------------------------- persistent

// Upper bound of any single wait of the persistent kernel.
constexpr long long kWaitTimeoutSeconds = 2;

struct WaveArgs {
  const uint16_t* xb;
  const uint16_t* w13;
  const uint16_t* w2;
  const int32_t* offsets;
  const int32_t* sorted_token;
  const int32_t* pair_pos;
  const float* topk_w;
  const int32_t* ready_list;
  const int32_t* ready_off;  // [W + 2]: start of ready slot s (s = 0: no local pick)
  uint16_t* act;
  uint16_t* y;
  void* out;                 // nullptr: no fused combine
  int32_t* sync;             // counters, layout in wave_sched.h
  int32_t* err;
  int E_local, G, W, d, I, k;
  long long timeout_ticks;   // bound of each wait, in wall-clock ticks
};

// The three primitives below are the only cross-workgroup operations of
// the persistent kernel.  They are called by all threads, inside the task
// loop that also contains the tiles' barriers, so none of them contains a
// lane-divergent branch: "one thread does X" is written as a wave-uniform
// branch on wave 0 with the lane selection folded into the operand.  (A
// lane-divergent if around the counter atomics lets the compiler move that
// block onto the loop's back edge and run the other lanes' next iteration,
// barriers included, before lane 0's atomics.)

__device__ __forceinline__ int wave_uniform() { return uniform(static_cast<int>(threadIdx.x) / kWave); }

// Claims the next ticket for the workgroup.
__device__ __forceinline__ int claim_ticket(int32_t* ticket, int32_t* s_ticket) {
  if (wave_uniform() == 0) {
    // one increment per workgroup: lane 0 adds 1, the other lanes add 0
    const int v = __hip_atomic_fetch_add(ticket, lane_id() == 0 ? 1 : 0, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    // lane 0's pre-op value; every lane stores the same value
    *s_ticket = __shfl(v, 0, kWave);
  }
  __syncthreads();
  const int tk = uniform(*s_ticket);
  __syncthreads();
  return tk;
}

// Bounded wait until *p >= target.  Wave 0 polls with relaxed loads,
// sleeping between polls: no cache maintenance inside the loop (an acquire
// per poll would invalidate the L2's non-local lines on every iteration and
// starve the producers).  The wait is bounded by wall-clock ticks; on
// expiry MOE_ERR_TIMEOUT is recorded and the wait ends (results are then
// invalid, but the kernel still drains).  After the barrier every wave
// performs one agent-scope acquire.
__device__ __forceinline__ void wait_geq(const int32_t* p, int target, long long timeout_ticks,
                                         int32_t* err) {
  if (wave_uniform() == 0) {
    if (uniform(__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) < target) {
      const long long t0 = wall_clock64();
      while (uniform(__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) < target) {
        if (wall_clock64() - t0 > timeout_ticks) {
          __hip_atomic_store(err, static_cast<int32_t>(MOE_ERR_TIMEOUT), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(8);
      }
    }
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Publish this workgroup's finished global stores, then count them: every
// wave releases its own stores at agent scope, the barrier orders those
// releases before the increment.
__device__ __forceinline__ void signal_add(int32_t* p) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (wave_uniform() == 0)
    __hip_atomic_fetch_add(p, lane_id() == 0 ? 1 : 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void ffn_waved_kernel(WaveArgs A) {
  extern __shared__ __align__(16) uint16_t lds[];
  __shared__ WaveSchedule S;
  __shared__ int32_t s_ticket;
  static_assert(G1Cfg::BT == G2Cfg::BT, "GEMM1 and GEMM2 share the m-tiles");
  if (threadIdx.x == 0)
    sched_build(S, A.offsets, A.ready_off, A.E_local, A.G, G1Cfg::BT, 2 * A.I / G1Cfg::BW,
                A.d / G2Cfg::BW, A.out != nullptr);
  __syncthreads();
  const int total = uniform(S.total);
  const int NT1 = uniform(S.NT1);
  int32_t* ticket = A.sync;

  // Every value that steers this loop is made wave-uniform explicitly (the
  // ticket and the decoded task come from LDS), so all waves run the same
  // iterations between barriers.
  for (int tk = claim_ticket(ticket, &s_ticket); tk < total; tk = claim_ticket(ticket, &s_ticket)) {
    Task t = sched_decode(S, tk);
    t.kind = uniform(t.kind);
    t.wave = uniform(t.wave);
    t.mt = uniform(t.mt);
    t.expert = uniform(t.expert);
    t.nt = uniform(t.nt);
    t.slot = uniform(t.slot);
    t.chunk = uniform(t.chunk);
    if (t.kind == kTaskGemm1) {
      // GEMM1 + SwiGLU tile of wave t.wave (its A rows pulled from the staging x)
      const int row0 = uniform(A.offsets[t.expert] + (t.mt - S.mt_pre[t.expert]) * G1Cfg::BT);
      const int count = uniform(min(G1Cfg::BT, A.offsets[t.expert + 1] - row0));
      gemm1_tile(A.xb, A.w13 + static_cast<size_t>(t.expert) * 2 * A.I * A.d, A.sorted_token, A.act,
                 row0, count, t.nt, A.d, A.I, lds);
      signal_add(A.sync + sched_g1done_index(S, t.mt));
    } else if (t.kind == kTaskGemm2) {
      // GEMM2 tile, once every GEMM1 tile of its m-tile is done
      const int row0 = uniform(A.offsets[t.expert] + (t.mt - S.mt_pre[t.expert]) * G2Cfg::BT);
      const int count = uniform(min(G2Cfg::BT, A.offsets[t.expert + 1] - row0));
      wait_geq(A.sync + sched_g1done_index(S, t.mt), NT1, A.timeout_ticks, A.err);
      gemm2_tile(A.act, A.w2 + static_cast<size_t>(t.expert) * A.d * A.I, A.y, row0, count, t.nt,
                 A.d, A.I, lds);
      signal_add(A.sync + sched_g2done_index(S, t.wave));
    } else {
      // combine of tokens whose last local wave is t.slot - 1
      for (int w = 0; w <= t.slot - 1; ++w)
        wait_geq(A.sync + sched_g2done_index(S, w), uniform(S.n_g2[w]), A.timeout_ticks, A.err);
      const int base = uniform(A.ready_off[t.slot] + t.chunk * kCombineTokens);
      const int end = uniform(min(base + kCombineTokens, A.ready_off[t.slot + 1]));
      for (int i = base + wave_uniform(); i < end; i += 4)
        combine_token<OUT_BF16>(A.ready_list[i], A.y, A.pair_pos, A.topk_w, A.k, A.d, A.out);
      __syncthreads();
    }
  }
}

}  // namespace

hipError_t launch_ffn(const moe_problem_t& p, const WsLayout& L, const void* x, const void* packed,
                      const int32_t* offsets, const int32_t* sorted_token, const int32_t* pair_pos,
                      const float* topk_w, const int32_t* ready_wave, void* y, void* out,
                      uint32_t flags, char* ws, hipStream_t s) {
  (void)ready_wave;
  const PackedLayout PL = packed_layout(p.d, p.I, p.E_global, p.E_local, p.x_dtype == MOE_BF16);
  const char* pk = static_cast<const char*>(packed);
  const uint16_t* w13 = reinterpret_cast<const uint16_t*>(pk + PL.w13);
  const uint16_t* w2 = reinterpret_cast<const uint16_t*>(pk + PL.w2);
  uint16_t* act = reinterpret_cast<uint16_t*>(ws + L.act);
  const bool out_bf16 = p.out_dtype == MOE_BF16;
  const uint16_t* xb = nullptr;
  hipError_t e;
  if ((e = stage_x_bf16(p, L, x, ws, s, &xb)) != hipSuccess) return e;
  int dev = 0, cus = 0, per_cu = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;

  if (flags & MOE_FLAG_SERIAL) {
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, gemm1_phase_kernel, 256, kFfnLds)) != hipSuccess)
      return e;
    const int grid = max(1, per_cu) * cus;
    gemm1_phase_kernel<<<grid, 256, kFfnLds, s>>>(xb, w13, offsets, sorted_token, act, p.E_local, p.d, p.I);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    gemm2_phase_kernel<<<grid, 256, kFfnLds, s>>>(act, w2, offsets, static_cast<uint16_t*>(y), p.E_local, p.d, p.I);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (out && p.T > 0) {
      if (out_bf16)
        combine_kernel<true><<<(p.T + 3) / 4, 256, 0, s>>>(static_cast<const uint16_t*>(y), pair_pos, topk_w, p.T, p.k, p.d, out);
      else
        combine_kernel<false><<<(p.T + 3) / 4, 256, 0, s>>>(static_cast<const uint16_t*>(y), pair_pos, topk_w, p.T, p.k, p.d, out);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
  }

  int32_t* sync = reinterpret_cast<int32_t*>(ws + L.sync);
  if ((e = fill_zero(sync, L.sync_words, s)) != hipSuccess) return e;
  WaveArgs A;
  A.xb = xb;
  A.w13 = w13;
  A.w2 = w2;
  A.offsets = offsets;
  A.sorted_token = sorted_token;
  A.pair_pos = pair_pos;
  A.topk_w = topk_w;
  A.ready_list = reinterpret_cast<const int32_t*>(ws + L.ready_list);
  A.ready_off = reinterpret_cast<const int32_t*>(ws + L.group_off) + p.E_local + 1;
  A.act = act;
  A.y = static_cast<uint16_t*>(y);
  A.out = out;
  A.sync = sync;
  A.err = reinterpret_cast<int32_t*>(ws + L.err);
  A.E_local = p.E_local;
  A.G = p.experts_per_wave;
  A.W = L.W;
  A.d = p.d;
  A.I = p.I;
  A.k = p.k;
  int wall_khz = 0;
  if ((e = hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, dev)) != hipSuccess) return e;
  A.timeout_ticks = static_cast<long long>(max(wall_khz, 1)) * 1000ll * kWaitTimeoutSeconds;
  auto kern = out_bf16 ? ffn_waved_kernel<true> : ffn_waved_kernel<false>;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, kFfnLds)) != hipSuccess) return e;
  const int grid = max(1, per_cu) * cus;
  kern<<<grid, 256, kFfnLds, s>>>(A);
  return hipGetLastError();
}

hipError_t fill_zero(void* p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  fill_zero_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(static_cast<int32_t*>(p), n);
  return hipGetLastError();
}

hipError_t stage_x_bf16(const moe_problem_t& p, const WsLayout& L, const void* x, char* ws,
                        hipStream_t s, const uint16_t** xb) {
  *xb = static_cast<const uint16_t*>(x);
  if (p.x_dtype != MOE_F32 || p.T == 0) return hipSuccess;
  const size_t n = static_cast<size_t>(p.T) * p.d;
  f32_to_bf16_kernel<<<static_cast<unsigned>((n / 4 + 255) / 256), 256, 0, s>>>(
      static_cast<const float*>(x), reinterpret_cast<uint16_t*>(ws + L.xbf), n);
  *xb = reinterpret_cast<const uint16_t*>(ws + L.xbf);
  return hipGetLastError();
}

hipError_t launch_combine(const moe_problem_t& p, const void* y, const int32_t* pair_pos,
                          const float* topk_w, void* out, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  if (p.out_dtype == MOE_BF16)
    combine_kernel<true><<<(p.T + 3) / 4, 256, 0, s>>>(static_cast<const uint16_t*>(y), pair_pos, topk_w, p.T, p.k, p.d, out);
  else
    combine_kernel<false><<<(p.T + 3) / 4, 256, 0, s>>>(static_cast<const uint16_t*>(y), pair_pos, topk_w, p.T, p.k, p.d, out);
  return hipGetLastError();
}

}  // namespace moe
