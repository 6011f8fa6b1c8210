// wave_sched.h -- the static task order of the persistent expert-wave kernel,
// as host+device functions so that the schedule can be checked on the CPU.
//
// DeepSeek-V4 launch digest (itsolotime.com), section 1.2: in steady state
// the compute of the current wave, the dispatch of the next wave's tokens
// and the return of finished experts' results run at the same time.  The
// order below realises that: block b of the ticket sequence holds
//   GEMM1 tiles of wave b          (their operand loads are the pulls),
//   GEMM2 tiles of wave b-1,
//   combine tasks of ready slot b-1 (tokens whose last local wave is b-2;
//                                    slot 0 = tokens with no local pick),
// for b = 0 .. W+1.  A GEMM2 tile waits for the GEMM1 tiles of its m-tile
// (ticketed one block earlier); a combine task waits for all GEMM2 tiles of
// waves <= its slot - 1 (ticketed at least one block earlier).  Every wait
// is on smaller tickets, so the order is deadlock free for any grid.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kSchedMaxExperts = 256;
constexpr int kSchedMaxWaves = 256;
constexpr int kCombineTokens = 16;  // tokens per combine task

struct WaveSchedule {
  int W, G, NT1, NT2, total;
  int32_t mt_pre[kSchedMaxExperts + 1];  // first m-tile of each local expert
  int32_t blk_start[kSchedMaxWaves + 3]; // first ticket of block b, b = 0 .. W+2
  int32_t n_g1[kSchedMaxWaves + 1];
  int32_t n_g2[kSchedMaxWaves + 1];
  int32_t n_cb[kSchedMaxWaves + 2];
};

enum TaskKind { kTaskGemm1 = 0, kTaskGemm2 = 1, kTaskCombine = 2 };

struct Task {
  int kind;
  int wave;      // GEMM1 / GEMM2: expert wave of the tile
  int mt;        // global m-tile index (GEMM1 / GEMM2)
  int expert;    // local expert (GEMM1 / GEMM2)
  int nt;        // output-feature tile (GEMM1 / GEMM2)
  int slot;      // combine: ready slot
  int chunk;     // combine: chunk of kCombineTokens tokens inside the slot
};

// Binary search: the expert whose m-tile range holds mt, with
// mt_pre[lo] <= mt < mt_pre[hi].
__host__ __device__ inline int sched_expert_of(const int32_t* mt_pre, int lo, int hi, int mt) {
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (mt_pre[mid] <= mt) lo = mid; else hi = mid;
  }
  return lo;
}

// Builds the schedule from the dispatch tables.  offsets [E_local + 1] =
// first pair row of each local expert; ready_off [W + 2] = first position of
// each ready slot in the ready list.  BT = rows per m-tile.  NT1 / NT2 =
// output tiles of GEMM1 / GEMM2 per m-tile.  with_combine = 0 drops the
// combine tasks (no fused combine).
__host__ __device__ inline void sched_build(WaveSchedule& S, const int32_t* offsets,
                                            const int32_t* ready_off, int E_local, int G, int BT,
                                            int NT1, int NT2, int with_combine) {
  S.W = E_local / G;
  S.G = G;
  S.NT1 = NT1;
  S.NT2 = NT2;
  int run = 0;
  for (int e = 0; e < E_local; ++e) {
    S.mt_pre[e] = run;
    run += (offsets[e + 1] - offsets[e] + BT - 1) / BT;
  }
  S.mt_pre[E_local] = run;
  for (int w = 0; w < S.W; ++w) {
    const int mts = S.mt_pre[(w + 1) * G] - S.mt_pre[w * G];
    S.n_g1[w] = mts * NT1;
    S.n_g2[w] = mts * NT2;
  }
  for (int s = 0; s <= S.W; ++s)
    S.n_cb[s] = with_combine ? (ready_off[s + 1] - ready_off[s] + kCombineTokens - 1) / kCombineTokens : 0;
  run = 0;
  for (int b = 0; b <= S.W + 1; ++b) {
    S.blk_start[b] = run;
    if (b < S.W) run += S.n_g1[b];
    if (b >= 1 && b <= S.W) run += S.n_g2[b - 1];
    if (b >= 1) run += S.n_cb[b - 1];
  }
  S.blk_start[S.W + 2] = run;
  S.total = run;
}

// Decodes ticket tk (0 <= tk < S.total).
__host__ __device__ inline Task sched_decode(const WaveSchedule& S, int tk) {
  int b = 0;
  while (S.blk_start[b + 1] <= tk) ++b;
  int rel = tk - S.blk_start[b];
  Task t{};
  const int g1n = (b < S.W) ? S.n_g1[b] : 0;
  const int g2n = (b >= 1 && b <= S.W) ? S.n_g2[b - 1] : 0;
  if (rel < g1n) {
    t.kind = kTaskGemm1;
    t.wave = b;
    t.mt = S.mt_pre[b * S.G] + rel / S.NT1;
    t.nt = rel % S.NT1;
    t.expert = sched_expert_of(S.mt_pre, b * S.G, (b + 1) * S.G, t.mt);
    return t;
  }
  rel -= g1n;
  if (rel < g2n) {
    t.kind = kTaskGemm2;
    t.wave = b - 1;
    t.mt = S.mt_pre[(b - 1) * S.G] + rel / S.NT2;
    t.nt = rel % S.NT2;
    t.expert = sched_expert_of(S.mt_pre, (b - 1) * S.G, b * S.G, t.mt);
    return t;
  }
  rel -= g2n;
  t.kind = kTaskCombine;
  t.slot = b - 1;
  t.chunk = rel;
  return t;
}

// Counter layout of the persistent kernel: [0] ticket, [1 .. W] GEMM2 tiles
// finished per wave, [1 + W ..] GEMM1 tiles finished per m-tile.
__host__ __device__ inline int sched_g2done_index(const WaveSchedule&, int w) { return 1 + w; }
__host__ __device__ inline int sched_g1done_index(const WaveSchedule& S, int mt) { return 1 + S.W + mt; }

}  // namespace moe
