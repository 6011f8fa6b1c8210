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
//   combine       : tokens whose last local wave has finished are summed
//                   back into token order while later waves still compute.
// The persistent kernel claims tasks from per-XCD ticket streams in the
// static order of wave_sched.h.  Tickets decide which workgroup runs a tile,
// never the arithmetic: the result bits equal those of the phase-by-phase
// kernels (MOE_FLAG_SERIAL).
//
// Coherence on an 8-XCD device (each XCD has its own L2):
//   GEMM1 -> GEMM2 of one m-tile stay on one XCD.  The producer waits for
//   its stores to reach the L2 (vmcnt) and bumps a counter; the consumer
//   polls it and drops its CU's L1 copies.  No L2 write-back or invalidate.
//   Spread schedules (small batches whose m-tiles do not divide evenly over
//   the XCDs) split every m-tile's tiles over all XCDs: there the XCD's last
//   GEMM1 tile of the m-tile writes the L2 back and publishes device-wide,
//   and GEMM2 reads the activations with device-coherent loads.
//   GEMM2 -> combine crosses XCDs.  The last GEMM2 tile of a wave on an XCD
//   writes that L2 back once (agent-scope release) and adds the XCD's tile
//   count to a device-wide counter; combine tasks wait for the device-wide
//   counters and read y with device-coherent (sc1) loads.
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

// GATED: W13 holds W1 and W3 (SwiGLU); else W1 only (squared ReLU).
template <class F, bool GATED>
__global__ __launch_bounds__(F::NT) void gemm1_phase_kernel(
    const uint16_t* __restrict__ xb, const uint16_t* __restrict__ w13,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_token,
    uint16_t* __restrict__ act, int E_local, int d, int I, const float* __restrict__ xscale,
    float* __restrict__ hsave) {
  constexpr int gr = GATED ? 2 : 1;  // packed W13 rows per intermediate index
  using C = typename F::G1;
  extern __shared__ __align__(16) uint16_t lds[];
  __shared__ int32_t mt_pre[kMaxLocalExperts + 1];
  __shared__ int32_t seg[kMaxLocalExperts + 1];
  __shared__ int32_t xcd_order;
  build_mtile_prefix(offsets, E_local, C::BT, mt_pre);
  if (threadIdx.x == 0) xcd_order = F::WHOLE_EXPERTS && phase_xcd_order(mt_pre, E_local);
  if (hsave != nullptr) build_seg_prefix(offsets, E_local, seg);
  __syncthreads();
  const int NT = gr * I / C::BW;
  const bool xo = uniform(xcd_order) != 0;
  const PhaseTiles r = phase_tiles(uniform(mt_pre[E_local] * NT), xo, static_cast<int>(blockIdx.x),
                                   static_cast<int>(gridDim.x));
  for (int g = r.begin + r.first; g < r.end; g += r.stride) {
    int e, mt, nt;
    phase_tile(mt_pre, E_local, NT, g, xo, e, mt, nt);
    e = uniform(e);
    mt = uniform(mt);
    nt = uniform(nt);
    const int row0 = uniform(offsets[e] + (mt - mt_pre[e]) * C::BT);
    const int count = uniform(min(C::BT, offsets[e + 1] - row0));
    const int hrow0 = hsave != nullptr ? uniform(seg[e] + (mt - mt_pre[e]) * C::BT) : 0;
    gemm1_tile<C, GATED>(xb, w13 + static_cast<size_t>(e) * gr * I * d, sorted_token, act, row0, count, nt, d,
                         I, lds, xscale, hsave, hrow0);
  }
}

template <class F>
__global__ __launch_bounds__(F::NT) void gemm2_phase_kernel(
    const uint16_t* __restrict__ act, const uint16_t* __restrict__ w2,
    const int32_t* __restrict__ offsets, uint16_t* __restrict__ y, int E_local, int d, int I) {
  using C = typename F::G2;
  extern __shared__ __align__(16) uint16_t lds[];
  __shared__ int32_t mt_pre[kMaxLocalExperts + 1];
  __shared__ int32_t xcd_order;
  build_mtile_prefix(offsets, E_local, C::BT, mt_pre);
  if (threadIdx.x == 0) xcd_order = F::WHOLE_EXPERTS && phase_xcd_order(mt_pre, E_local);
  __syncthreads();
  const int NT = d / C::BW;
  const bool xo = uniform(xcd_order) != 0;
  const PhaseTiles r = phase_tiles(uniform(mt_pre[E_local] * NT), xo, static_cast<int>(blockIdx.x),
                                   static_cast<int>(gridDim.x));
  for (int g = r.begin + r.first; g < r.end; g += r.stride) {
    int e, mt, nt;
    phase_tile(mt_pre, E_local, NT, g, xo, e, mt, nt);
    e = uniform(e);
    mt = uniform(mt);
    nt = uniform(nt);
    const int row0 = uniform(offsets[e] + (mt - mt_pre[e]) * C::BT);
    const int count = uniform(min(C::BT, offsets[e + 1] - row0));
    gemm2_tile<C>(act, w2 + static_cast<size_t>(e) * d * I, y, row0, count, nt, d, I, lds);
  }
}

// One wavefront per (token, column part); blockIdx.y = part.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y,
                                                      const int32_t* __restrict__ pair_pos,
                                                      const float* __restrict__ topk_w, int T,
                                                      int k, int d, int parts, void* __restrict__ out) {
  const int t = blockIdx.x * 4 + wave_id();
  int cb, ce;
  combine_cols(d, parts, blockIdx.y, cb, ce);
  if (t < T) combine_token<OUT_BF16, false>(t, y, pair_pos, topk_w, k, d, cb, ce, out);
}

// ---------------------------------------------------------------- persistent

// Upper bound of any single wait of the persistent kernel.
constexpr long long kWaitTimeoutSeconds = 2;

struct WaveArgs {
  const uint16_t* xb;        // token-order staging buffer (bf16, or e4m3 bytes for FP8 dispatch)
  const float* xscale;       // FP8 dispatch: per-token scales (else unused)
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
  int32_t* ctr;              // counters, layout in wave_sched.h, then the exit count
  int32_t* err;
  int ctr_words;             // counter words including the exit count (the last one)
  int E_local, G, W, d, I, k;
  int region_words;
  int cb_parts;              // column parts of a combine task
  long long timeout_ticks;   // bound of each wait, in wall-clock ticks
};

// The primitives below are the only cross-workgroup operations of the
// persistent kernel.  They are called by all threads, inside the task loop
// that also contains the tiles' barriers, so none of them contains a
// lane-divergent branch: "one thread does X" is written as a wave-uniform
// branch on wave 0 with the lane selection folded into the operand.  (A
// lane-divergent if around the counter atomics lets the compiler move that
// block onto the loop's back edge and run the other lanes' next iteration,
// barriers included, before lane 0's atomics.)

__device__ __forceinline__ int wave_uniform() { return uniform(static_cast<int>(threadIdx.x) / kWave); }

__device__ __forceinline__ int xcc_id() {
  // HW_REG_XCC_ID (hardware register 20), bits [3:0]
  return static_cast<int>(__builtin_amdgcn_s_getreg(20 | (0 << 6) | ((4 - 1) << 11))) & (kXcds - 1);
}

// Adds v (taken from lane 0) to *p; returns the old value to the whole wave.
__device__ __forceinline__ int wave0_atomic_add(int32_t* p, int v) {
  const int r = __hip_atomic_fetch_add(p, lane_id() == 0 ? v : 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return uniform(__shfl(r, 0, kWave));
}

// Ticket claims are split in two so that the atomic's round trip overlaps
// a task: wave 0 issues the claim of the next ticket when a task starts
// (claim_issue; lane 0 adds 1, every lane gets its own return value) and
// the workgroup reads it when the task ends (claim_finish).  A workgroup
// thus holds one claimed ticket while it works on the previous one; since
// every task waits only on smaller tickets, the smallest unfinished ticket
// is always being worked on and every wait still ends.
__device__ __forceinline__ int claim_issue(int32_t* ticket) {
  return __hip_atomic_fetch_add(ticket, lane_id() == 0 ? 1 : 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int claim_finish(int r, int32_t* s_ticket) {
  if (wave_uniform() == 0) *s_ticket = uniform(__shfl(r, 0, kWave));
  __syncthreads();
  const int tk = uniform(*s_ticket);
  __syncthreads();
  return tk;
}

// Bounded poll by wave 0 until *p >= target.  Relaxed loads only: no cache
// maintenance inside the loop.  On expiry MOE_ERR_TIMEOUT is recorded and
// the wait ends (results are then invalid, but the kernel still drains).
__device__ __forceinline__ void poll_geq(const int32_t* p, int target, long long timeout_ticks,
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
        __builtin_amdgcn_s_sleep(4);
      }
    }
  }
}

// XCD-local producer side: every wave's stores have reached the (shared)
// L2 before the counter moves.
__device__ __forceinline__ void local_signal(int32_t* p) {
  wait_vmcnt<0>();
  __syncthreads();
  if (wave_uniform() == 0) wave0_atomic_add(p, 1);
}

// Spread schedules: the hand-off of an m-tile crosses XCDs.  Every tile's
// stores reach the L2 before the XCD's counter moves; the XCD's last tile of
// the m-tile writes the L2 back (agent-scope release) and adds the XCD's
// tiles to the device-wide counter.
__device__ __forceinline__ void spread_signal(int32_t* local, int32_t* all, int mine) {
  wait_vmcnt<0>();
  __syncthreads();
  if (wave_uniform() == 0) {
    const int done = wave0_atomic_add(local, 1) + 1;
    if (done == mine) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      wave0_atomic_add(all, mine);
    }
  }
}

// XCD-local consumer side: bounded poll of the counter (device-scope loads,
// which skip the CU's L1; a workgroup-scope load may keep returning the L1
// line it first read), then drop this CU's L1 lines so the following loads
// come from the L2 the producer wrote.
__device__ __forceinline__ void local_wait(const int32_t* p, int target, long long timeout_ticks,
                                           int32_t* err) {
  poll_geq(p, target, timeout_ticks, err);
  __syncthreads();
  asm volatile("buffer_inv sc0" ::: "memory");
}

template <class F, bool OUT_BF16, bool GATED>
__device__ __forceinline__ void ffn_waved_run(const WaveArgs& A) {
  using C1 = typename F::G1;
  using C2 = typename F::G2;
  static_assert(C1::BT == C2::BT, "GEMM1 and GEMM2 share the m-tiles");
  extern __shared__ __align__(16) uint16_t lds[];
  __shared__ WaveSchedule S;
  __shared__ int32_t s_off[kMaxLocalExperts + 1];    // expert row offsets
  __shared__ int32_t s_ready[kSchedMaxWaves + 2];     // ready-slot starts in the ready list
  __shared__ int32_t s_ticket;
  __shared__ int32_t s_wdone;  // waves 0 .. s_wdone - 1 seen finished on every XCD
  const int xcd = uniform(xcc_id());
  int32_t* ticket = A.ctr + sched_ticket_index(xcd);
  // the first ticket is claimed now: the atomic's round trip overlaps the
  // schedule build (which waits on no other workgroup)
  int claim = 0;
  if (wave_uniform() == 0) claim = claim_issue(ticket);
  // The schedule (the steps of sched_build, spread over the workgroup).
  // The dispatch tables go to LDS first, in parallel; the m-tile prefix,
  // the single-m-tile dealing, the combine placement and the prefix sums
  // run on many threads (one thread takes tens of microseconds over them:
  // a wave issues a dependent scalar instruction every few cycles at best).
  for (int e = threadIdx.x; e <= A.E_local; e += F::NT) s_off[e] = A.offsets[e];
  for (int w = threadIdx.x; w <= A.W + 1; w += F::NT) s_ready[w] = A.ready_off[w];
  for (int i = threadIdx.x; i <= kSchedMaxLocal + kSchedMaxLag; i += F::NT) S.cb_pos[i] = 0;
  for (int e = threadIdx.x; e < A.E_local; e += F::NT) S.mt_pre[e + 1] = sched_mtiles(A.offsets, e, C1::BT);
  if (threadIdx.x == 0) {
    // GEMM2 lag: kSchedMaxLag m-tiles, i.e. an XCD runs the GEMM1 tiles of
    // (nearly) all its m-tiles before their GEMM2 tiles.  Interleaving the two
    // closer puts both operand sets (x and W1/W3, act and W2) through the
    // XCD's L2 at once; measured on the mid layer the short lags (2 to 4
    // m-tiles) cost 20% against 8 and more.
    sched_init(S, A.E_local, A.G, (GATED ? 2 : 1) * A.I / C1::BW, A.d / C2::BW, xcd, kSchedMaxLag);
    S.mt_pre[0] = 0;
    S.cb_pre[0] = 0;
    s_wdone = 0;
  }
  __syncthreads();
  if (wave_uniform() == 0) sched_scan_wave(S.mt_pre, A.E_local + 1);
  __syncthreads();
  if (F::WHOLE_EXPERTS) {
    if (threadIdx.x == 0) sched_deal_whole(S, A.E_local);
  } else {
    sched_deal_single(S, A.E_local, threadIdx.x, F::NT);
  }
  __syncthreads();
  if (uniform(S.err) == 0) {
    sched_groups(S, threadIdx.x, F::NT);
    sched_place(S, s_ready, A.out != nullptr ? A.cb_parts : 0, threadIdx.x, F::NT,
                [](int32_t* p, int v) { atomicAdd(p, v); });
    __syncthreads();
    // the two prefix sums on two wavefronts
    if (wave_uniform() == 0) sched_scan_wave(S.cb_pos, S.n_local + S.lag + 1);
    if (wave_uniform() == 1) sched_scan_wave(S.cb_pre, S.W + 2);
    __syncthreads();
    const int npos = uniform(S.n_local + S.lag);
    for (int i = threadIdx.x; i <= npos; i += F::NT) S.pos[i] = sched_pos_of(S, i);
    if (threadIdx.x == 0) S.total = sched_pos_of(S, npos);
  }
  __syncthreads();
  if (uniform(S.err) != 0) {
    // more m-tiles on this XCD than the schedule holds (the host bounds this)
    if (wave_uniform() == 0 && lane_id() == 0)
      __hip_atomic_store(A.err, static_cast<int32_t>(MOE_ERR_UNSUPPORTED), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const int total = uniform(S.total);
  const int NT1 = uniform(S.NT1);
  const int spread = F::WHOLE_EXPERTS ? 0 : uniform(S.spread);
  const int rw = A.region_words;

  // Every value that steers this loop is made wave-uniform explicitly (the
  // ticket and the decoded task come from LDS), so all waves run the same
  // iterations between barriers.
  for (int tk = claim_finish(claim, &s_ticket); tk < total; tk = claim_finish(claim, &s_ticket)) {
    if (wave_uniform() == 0) claim = claim_issue(ticket);
    Task t = sched_decode(S, tk);
    t.kind = uniform(t.kind);
    t.wave = uniform(t.wave);
    t.loc = uniform(t.loc);
    t.mt = uniform(t.mt);
    t.expert = uniform(t.expert);
    t.nt = uniform(t.nt);
    t.slot = uniform(t.slot);
    t.chunk = uniform(t.chunk);
    if (t.kind == kTaskGemm1) {
      // GEMM1 + SwiGLU tile (its operand rows pulled from the staging x)
      const int row0 = uniform(s_off[t.expert] + (t.mt - S.mt_pre[t.expert]) * C1::BT);
      const int count = uniform(min(C1::BT, s_off[t.expert + 1] - row0));
      gemm1_tile<C1, GATED>(A.xb, A.w13 + static_cast<size_t>(t.expert) * (GATED ? 2 : 1) * A.I * A.d,
                            A.sorted_token, A.act, row0, count, t.nt, A.d, A.I, lds, A.xscale);
      if (spread)
        spread_signal(A.ctr + sched_g1done_index(S, rw, t.loc), A.ctr + sched_g1all_index(S, rw, t.loc), NT1);
      else
        local_signal(A.ctr + sched_g1done_index(S, rw, t.loc));
    } else if (t.kind == kTaskGemm2) {
      // GEMM2 tile, once every GEMM1 tile of its m-tile is done (same XCD)
      const int row0 = uniform(s_off[t.expert] + (t.mt - S.mt_pre[t.expert]) * C2::BT);
      const int count = uniform(min(C2::BT, s_off[t.expert + 1] - row0));
      if constexpr (!F::WHOLE_EXPERTS) {
        if (spread) {
          // every XCD's GEMM1 tiles of the m-tile; the activations are read
          // with device-coherent loads
          local_wait(A.ctr + sched_g1all_index(S, rw, t.loc), uniform(S.NT1_all), A.timeout_ticks, A.err);
          gemm2_tile<TokCoherent<C2>>(A.act, A.w2 + static_cast<size_t>(t.expert) * A.d * A.I, A.y, row0, count,
                                      t.nt, A.d, A.I, lds);
        }
      }
      if (!spread) {
        local_wait(A.ctr + sched_g1done_index(S, rw, t.loc), NT1, A.timeout_ticks, A.err);
        gemm2_tile<C2>(A.act, A.w2 + static_cast<size_t>(t.expert) * A.d * A.I, A.y, row0, count,
                       t.nt, A.d, A.I, lds);
      }
      wait_vmcnt<0>();
      __syncthreads();
      if (wave_uniform() == 0) {
        const int mine = uniform(sched_g2_of_wave(S, t.wave));
        const int done = wave0_atomic_add(A.ctr + sched_g2local_index(S, rw, t.wave), 1) + 1;
        if (done == mine) {
          // last GEMM2 tile of this wave on this XCD: write the L2 back once,
          // then publish the XCD's tiles device-wide
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
          wave0_atomic_add(A.ctr + sched_g2all_index(S, rw, t.wave), mine);
        }
      }
    } else {
      // combine of tokens whose last local wave is t.slot - 1; waves this
      // workgroup already saw finished are not polled again
      for (int w = uniform(s_wdone); w <= t.slot - 1; ++w)
        poll_geq(A.ctr + sched_g2all_index(S, rw, w), uniform(sched_g2_all(S, w)), A.timeout_ticks, A.err);
      __syncthreads();
      if (threadIdx.x == 0 && t.slot > s_wdone) s_wdone = t.slot;
      const int parts = A.cb_parts;
      const int base = uniform(s_ready[t.slot] + (t.chunk / parts) * kCombineTokens);
      const int end = uniform(min(base + kCombineTokens, s_ready[t.slot + 1]));
      int cb, ce;
      combine_cols(A.d, parts, t.chunk % parts, cb, ce);
      for (int i = base + wave_uniform(); i < end; i += F::NT / kWave)
        combine_token<OUT_BF16, true>(A.ready_list[i], A.y, A.pair_pos, A.topk_w, A.k, A.d, cb, ce, A.out);
      __syncthreads();
    }
  }
  if (A.out == nullptr) return;
  // The last ready slot (tokens whose last local wave is the last one) from
  // this XCD's pool (chunks xcd, xcd + 8, ...): claim a chunk, and if there
  // was one, wait once for every wave on every XCD, then take chunks until
  // none is left (a workgroup that finds the pool empty leaves without
  // polling).  The pool's claims are split like the stream's (issue at chunk
  // start, read at chunk end).
  const int b0 = uniform(s_ready[A.W]);
  const int ntok = uniform(s_ready[A.W + 1]) - b0;
  const int pparts = sched_pool_parts(A.cb_parts);
  const int mine = sched_pool_share(sched_pool_chunks(ntok, pparts), xcd);
  if (mine == 0) return;
  int32_t* pool = A.ctr + sched_pool_index(A.W, xcd);
  int pc = 0;
  if (wave_uniform() == 0) pc = claim_issue(pool);
  int j = claim_finish(pc, &s_ticket);
  if (j >= mine) return;
  for (int w = uniform(s_wdone); w < A.W; ++w)
    poll_geq(A.ctr + sched_g2all_index(S, rw, w), uniform(sched_g2_all(S, w)), A.timeout_ticks, A.err);
  __syncthreads();
  for (; j < mine; j = claim_finish(pc, &s_ticket)) {
    if (wave_uniform() == 0) pc = claim_issue(pool);
    const int c = xcd + kXcds * j;
    const int base = b0 + (c / pparts) * kCombineTokens;
    const int end = min(base + kCombineTokens, b0 + ntok);
    int cb, ce;
    combine_cols(A.d, pparts, c % pparts, cb, ce);
    for (int i = base + wave_uniform(); i < end; i += F::NT / kWave)
      combine_token<OUT_BF16, true>(A.ready_list[i], A.y, A.pair_pos, A.topk_w, A.k, A.d, cb, ce, A.out);
    __syncthreads();
  }
}

// The kernel: the task loop, then the exit count.  The last workgroup to
// leave clears every counter (the exit count included), so the next launch
// on this workspace starts from zero without a fill of its own.  Every
// workgroup waits for its own memory operations (its counter atomics
// included) to complete before it is counted, so no counter is touched after
// the clear.  That wait is all the exit needs: the data stores of the
// workgroup (outputs) are published by the end of the kernel, and an
// agent-scope release here would write the XCD's whole L2 back once per
// workgroup while other workgroups still combine (measured on the mid layer:
// the pool's last chunks ran three times slower and the kernel 35 us longer).
template <class F, bool OUT_BF16, bool GATED>
__global__ __launch_bounds__(F::NT) void ffn_waved_kernel(WaveArgs A) {
  __shared__ int32_t s_last;
  ffn_waved_run<F, OUT_BF16, GATED>(A);
  wait_vmcnt<0>();
  __syncthreads();
  if (wave_uniform() == 0) {
    const int prev = wave0_atomic_add(A.ctr + A.ctr_words - 1, 1);
    if (lane_id() == 0) s_last = prev == static_cast<int>(gridDim.x) - 1;
  }
  __syncthreads();
  if (s_last) {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    for (int i = threadIdx.x; i < A.ctr_words; i += F::NT)
      __hip_atomic_store(A.ctr + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Tile shape of the expert GEMMs.  The shape never changes result bits.
//   small batches (mean routed rows per expert under 96, assuming uniform
//   routing): token tiles of 32 rows for T <= 32 (all rows of an expert: a
//   token picks an expert at most once), else 64;
//   otherwise 256 x 256 tiles when the widths allow, else the mid shape.
enum class FfnShape { Small, Small64, Large, Mid };

template <class F>
bool ffn_shape_fits(const moe_problem_t& p) {
  return p.d % F::G1::BK == 0 && p.I % F::G2::BK == 0 && (gate_rows(p) * p.I) % F::G1::BW == 0 &&
         p.d % F::G2::BW == 0;
}

FfnShape pick_ffn_shape(const moe_problem_t& p) {
  const double rows = static_cast<double>(p.T) * p.k / p.E_global;
  if (rows < 96.0) {
    if (p.T <= FfnSmall::G1::BT && ffn_shape_fits<FfnSmall>(p)) return FfnShape::Small;
    if (ffn_shape_fits<FfnSmall64>(p)) return FfnShape::Small64;
  }
  if (ffn_shape_fits<FfnLarge>(p)) return FfnShape::Large;
  return FfnShape::Mid;
}

// m-tile rows of the shape a problem runs (GEMM1 and GEMM2 share them).
int ffn_mtile_rows(const moe_problem_t& p) {
  switch (pick_ffn_shape(p)) {
    case FfnShape::Small: return FfnSmall::G1::BT;
    case FfnShape::Small64: return FfnSmall64::G1::BT;
    case FfnShape::Large: return FfnLarge::G1::BT;
    default: return FfnMid::G1::BT;
  }
}

template <class F>
hipError_t launch_ffn_cfg(const moe_problem_t& p, const WsLayout& L, const uint16_t* xb, const float* xscale,
                          const uint16_t* w13, const uint16_t* w2, const int32_t* offsets,
                          const int32_t* sorted_token, const int32_t* pair_pos, const float* topk_w,
                          void* y, void* out, float* hsave, uint32_t flags, char* ws, hipStream_t s) {
  hipError_t e;
  int dev = 0, cus = 0, per_cu = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  const bool out_bf16 = p.out_dtype == MOE_BF16;
  uint16_t* act = reinterpret_cast<uint16_t*>(ws + L.act);
  // saving the pre-activations runs the phase kernels: the persistent
  // kernel's register budget has no room for the stores (same bits)
  if (hsave != nullptr || !ffn_uses_persistent(p, cus, flags)) {
    constexpr size_t l1 = F::G1::LDS_BYTES, l2 = F::G2::LDS_BYTES;
    auto g1 = gate_rows(p) == 2 ? gemm1_phase_kernel<F, true> : gemm1_phase_kernel<F, false>;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, g1, F::NT, l1)) != hipSuccess) return e;
    g1<<<max(1, per_cu) * cus, F::NT, l1, s>>>(xb, w13, offsets, sorted_token, act, p.E_local, p.d, p.I, xscale,
                                               hsave);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, gemm2_phase_kernel<F>, F::NT, l2)) != hipSuccess)
      return e;
    gemm2_phase_kernel<F><<<max(1, per_cu) * cus, F::NT, l2, s>>>(act, w2, offsets, static_cast<uint16_t*>(y),
                                                                 p.E_local, p.d, p.I);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (out && p.T > 0) return launch_combine(p, y, pair_pos, topk_w, out, s);
    return hipSuccess;
  }
  // the counters are zero: moe_dispatch clears them and every launch of the
  // kernel clears them again as it ends
  int32_t* ctr = reinterpret_cast<int32_t*>(ws + L.sync);
  WaveArgs A;
  A.xb = xb;
  A.xscale = xscale;
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
  A.ctr = ctr;
  A.err = reinterpret_cast<int32_t*>(ws + L.err);
  A.E_local = p.E_local;
  A.G = p.experts_per_wave;
  A.W = L.W;
  A.d = p.d;
  A.I = p.I;
  A.k = p.k;
  A.region_words = L.ctr_region_words;
  A.ctr_words = static_cast<int>(L.sync_words);
  A.cb_parts = combine_parts(p.T, p.d);
  int wall_khz = 0;
  if ((e = hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, dev)) != hipSuccess) return e;
  A.timeout_ticks = static_cast<long long>(max(wall_khz, 1)) * 1000ll * kWaitTimeoutSeconds;
  const bool gated = gate_rows(p) == 2;
  auto kern = out_bf16 ? (gated ? ffn_waved_kernel<F, true, true> : ffn_waved_kernel<F, true, false>)
                       : (gated ? ffn_waved_kernel<F, false, true> : ffn_waved_kernel<F, false, false>);
  constexpr size_t lds = ffn_lds_bytes<F>();
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, F::NT, lds)) != hipSuccess) return e;
  kern<<<max(1, per_cu) * cus, F::NT, lds, s>>>(A);
  return hipGetLastError();
}

}  // namespace

// The schedule the library picks when the caller does not force one: the
// phase kernels.  Both give the same bits.  The persistent kernel hides the
// combine of finished waves under later waves' GEMMs and has no phase
// boundaries, but it deals the work to the XCDs in whole m-tiles (whole
// experts for the large tile shapes) from per-XCD ticket streams and keeps
// an m-tile's GEMM1 -> GEMM2 hand-off inside one XCD; the phase kernels
// spread every phase's tiles over all 256 CUs, in the XCD-affine order
// where experts average two m-tiles or more.  Measured on MI355X (one box,
// FFN with the fused combine), phases against the persistent kernel:
//   mid layer, T=4096, 16 experts, top-4: 0.471 to 0.478 against 0.498 ms;
//   stress layer, T=4096, 64 experts, top-6, one hot expert: 1.198 to
//     1.202 against 1.215 to 1.231 ms;
//   V3/V4-scale share, T=8192, 32 of 256 experts, top-8: 1.078 against
//     1.156 to 1.163 ms;
//   stress layer, T=16384: 3.42 against 3.95 to 3.97 ms;
//   decode, T = 1, 32, 128 (small tile shapes): the persistent kernel 7 to
//     12% slower.
// So the persistent kernel runs only when MOE_FLAG_PERSISTENT asks for it.
bool ffn_uses_persistent(const moe_problem_t& p, int cus, uint32_t flags) {
  if (flags & MOE_FLAG_SERIAL) return false;
  // every per-XCD ticket stream needs workgroups: the whole device
  if (cus != kXcds * kCusPerXcd) return false;
  // the schedule holds at most kSchedMaxLocal m-tiles per XCD; larger
  // problems run the phase-by-phase path (same kernels, same bits)
  const int W = p.E_local / p.experts_per_wave;
  const long long P_max = static_cast<long long>(p.T) * (p.k < p.E_local ? p.k : p.E_local);
  const long long mt_bound = P_max / ffn_mtile_rows(p) + p.E_local + 1;
  if (mt_bound / kXcds + W + 1 > kSchedMaxLocal) return false;
  return (flags & MOE_FLAG_PERSISTENT) != 0;
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

hipError_t launch_ffn(const moe_problem_t& p, const WsLayout& L, const void* x, const void* packed,
                      const int32_t* offsets, const int32_t* sorted_token, const int32_t* pair_pos,
                      const float* topk_w, const int32_t* ready_wave, void* y, void* out, float* hsave,
                      uint32_t flags, char* ws, hipStream_t s) {
  (void)ready_wave;
  const PackedLayout PL = packed_layout(p.d, p.I, p.E_global, p.E_local, p.x_dtype == MOE_BF16, gate_rows(p));
  const char* pk = static_cast<const char*>(packed);
  const uint16_t* w13 = reinterpret_cast<const uint16_t*>(pk + PL.w13);
  const uint16_t* w2 = reinterpret_cast<const uint16_t*>(pk + PL.w2);
  const uint16_t* xb = nullptr;
  hipError_t e;
  if ((e = stage_x_bf16(p, L, x, ws, s, &xb)) != hipSuccess) return e;
  switch (pick_ffn_shape(p)) {
    case FfnShape::Small:
      return launch_ffn_cfg<FfnSmall>(p, L, xb, nullptr, w13, w2, offsets, sorted_token, pair_pos, topk_w, y,
                                      out, hsave, flags, ws, s);
    case FfnShape::Small64:
      return launch_ffn_cfg<FfnSmall64>(p, L, xb, nullptr, w13, w2, offsets, sorted_token, pair_pos, topk_w, y,
                                         out, hsave, flags, ws, s);
    case FfnShape::Large:
      return launch_ffn_cfg<FfnLarge>(p, L, xb, nullptr, w13, w2, offsets, sorted_token, pair_pos, topk_w, y,
                                      out, hsave, flags, ws, s);
    default:
      return launch_ffn_cfg<FfnMid>(p, L, xb, nullptr, w13, w2, offsets, sorted_token, pair_pos, topk_w, y,
                                    out, hsave, flags, ws, s);
  }
}

hipError_t launch_ffn_fp8(const moe_problem_t& p, const WsLayout& L, const uint8_t* x8, const float* xscale,
                          const void* packed, const int32_t* offsets, const int32_t* sorted_token,
                          const int32_t* pair_pos, const float* topk_w, void* y, void* out, uint32_t flags,
                          char* ws, hipStream_t s) {
  const PackedLayout PL = packed_layout(p.d, p.I, p.E_global, p.E_local, p.x_dtype == MOE_BF16, gate_rows(p));
  const char* pk = static_cast<const char*>(packed);
  const uint16_t* w13 = reinterpret_cast<const uint16_t*>(pk + PL.w13);
  const uint16_t* w2 = reinterpret_cast<const uint16_t*>(pk + PL.w2);
  // the fp8 tiles take the bytes through the bf16 tiles' row pointers
  const uint16_t* xb = reinterpret_cast<const uint16_t*>(x8);
  const FfnShape shape = pick_ffn_shape(p);
  if (shape == FfnShape::Small)
    return launch_ffn_cfg<FfnSmallF8>(p, L, xb, xscale, w13, w2, offsets, sorted_token, pair_pos, topk_w, y, out,
                                      nullptr, flags, ws, s);
  if (shape == FfnShape::Small64)
    return launch_ffn_cfg<FfnSmall64F8>(p, L, xb, xscale, w13, w2, offsets, sorted_token, pair_pos, topk_w, y,
                                        out, nullptr, flags, ws, s);
  // Large and mid batches are compute-bound: the rows are dequantized once
  // on arrival (T x d bytes read, 2 T x d written, exact in bf16) and the
  // bf16 tiles run on them; the conversions inside the GEMM1 tile would
  // cost the 256 x 256 tile its register budget.
  uint16_t* xs = reinterpret_cast<uint16_t*>(ws + L.xbf);
  hipError_t e = launch_dequant_fp8(p, x8, xscale, xs, s);
  if (e != hipSuccess) return e;
  if (shape == FfnShape::Large)
    return launch_ffn_cfg<FfnLarge>(p, L, xs, nullptr, w13, w2, offsets, sorted_token, pair_pos, topk_w, y, out,
                                    nullptr, flags, ws, s);
  return launch_ffn_cfg<FfnMid>(p, L, xs, nullptr, w13, w2, offsets, sorted_token, pair_pos, topk_w, y, out,
                                nullptr, flags, ws, s);
}

hipError_t launch_combine(const moe_problem_t& p, const void* y, const int32_t* pair_pos,
                          const float* topk_w, void* out, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  const int parts = combine_parts(p.T, p.d);
  const dim3 grid((p.T + 3) / 4, parts);
  if (p.out_dtype == MOE_BF16)
    combine_kernel<true><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(y), pair_pos, topk_w, p.T, p.k, p.d,
                                              parts, out);
  else
    combine_kernel<false><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(y), pair_pos, topk_w, p.T, p.k, p.d,
                                               parts, out);
  return hipGetLastError();
}

}  // namespace moe
