// wave_sched.h -- the static task order of the persistent expert-wave kernel,
// as host+device functions so that the schedule can be checked on the CPU.
//
// DeepSeek-V4 launch digest (itsolotime.com), section 1.2: in steady state
// the compute of the current wave, the dispatch of the next wave's tokens
// and the return of finished experts' results run at the same time.
//
// MI355X has 8 XCDs, each with its own L2.  The m-tiles (BT-row slices of
// each expert's sorted rows) of every expert wave are split into 8
// contiguous ranges, one per XCD (when a wave's m-tiles do not divide by 8,
// the extra ones go to the XCDs after those that took the previous wave's
// extras, so the XCDs stay within one m-tile of each other), and every
// workgroup takes tasks only from its own XCD's ticket stream.  GEMM1 ->
// GEMM2 dependencies therefore never leave an XCD's L2; only the combine,
// which reads y rows of every XCD, crosses XCDs.
//
// Inside one XCD's stream, block b of the ticket sequence holds
//   GEMM1 tiles of the XCD's m-tiles in wave b (their operand loads are the
//                                              dispatch pulls),
//   GEMM2 tiles of the XCD's m-tiles in wave b-1,
//   the XCD's share of the combine chunks of ready slot b-1 (tokens whose
//   last local wave is b-2; slot 0 = tokens with no local pick),
// for b = 0 .. W+1.  A GEMM2 tile waits for its m-tile's GEMM1 tiles (same
// stream, smaller tickets).  A combine task waits until every XCD finished
// the GEMM2 tiles of waves <= its slot - 1; those tiles sit in blocks <=
// slot of every stream and wait only on smaller tickets of their own
// stream, so by induction over the waves every wait ends, for any grid.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kXcds = 8;                // XCDs of an MI355X
constexpr int kSchedMaxExperts = 256;
constexpr int kSchedMaxWaves = 256;
constexpr int kCombineTokens = 8;       // tokens per combine task
constexpr int kCtrPad = 64;             // int32 words (256 B) between counters of different XCDs

struct WaveSchedule {
  int W, G, NT1, NT2, total, xcd, n_local;
  int32_t mt_pre[kSchedMaxExperts + 1];  // first m-tile of each local expert
  int32_t blk_start[kSchedMaxWaves + 3]; // first ticket of block b, b = 0 .. W+2
  int32_t mlo[kSchedMaxWaves];           // first m-tile of this XCD in wave w
  int32_t loc_pre[kSchedMaxWaves];       // this XCD's m-tiles in waves < w
  int32_t n_g1[kSchedMaxWaves];          // this XCD's GEMM1 tiles of wave w
  int32_t n_g2[kSchedMaxWaves];          // this XCD's GEMM2 tiles of wave w
  int32_t g2_all[kSchedMaxWaves];        // GEMM2 tiles of wave w over all XCDs
  int32_t n_cb[kSchedMaxWaves + 1];      // this XCD's combine chunks of slot s
};

enum TaskKind { kTaskGemm1 = 0, kTaskGemm2 = 1, kTaskCombine = 2 };

struct Task {
  int kind;
  int wave;      // GEMM1 / GEMM2: expert wave of the tile
  int mt;        // global m-tile index (GEMM1 / GEMM2)
  int expert;    // local expert (GEMM1 / GEMM2)
  int nt;        // output-feature tile (GEMM1 / GEMM2)
  int slot;      // combine: ready slot
  int chunk;     // combine: global chunk inside the slot: token chunk (of
                 // kCombineTokens) chunk / cb_parts, column part chunk % cb_parts
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

// Share of XCD x when n m-tiles of one wave are split over the XCDs and the
// n % kXcds extra m-tiles go to XCDs rot, rot + 1, ... (mod kXcds).
__host__ __device__ inline int sched_xcd_share(int n, int rot, int x) {
  return n / kXcds + (((x - rot + kXcds) % kXcds) < (n % kXcds) ? 1 : 0);
}

// Builds XCD xcd's schedule from the dispatch tables.  offsets [E_local + 1]
// = first pair row of each local expert; ready_off [W + 2] = first position
// of each ready slot in the ready list.  BT = rows per m-tile.  NT1 / NT2 =
// output tiles of GEMM1 / GEMM2 per m-tile.  cb_parts = column parts per
// combine chunk of kCombineTokens tokens (0: no combine tasks, no fused
// combine).
__host__ __device__ inline void sched_build(WaveSchedule& S, const int32_t* offsets,
                                            const int32_t* ready_off, int E_local, int G, int BT,
                                            int NT1, int NT2, int cb_parts, int xcd) {
  S.W = E_local / G;
  S.G = G;
  S.NT1 = NT1;
  S.NT2 = NT2;
  S.xcd = xcd;
  int run = 0;
  for (int e = 0; e < E_local; ++e) {
    S.mt_pre[e] = run;
    run += (offsets[e + 1] - offsets[e] + BT - 1) / BT;
  }
  S.mt_pre[E_local] = run;
  int rot = 0, loc = 0;
  for (int w = 0; w < S.W; ++w) {
    const int a = S.mt_pre[w * G], n = S.mt_pre[(w + 1) * G] - a;
    int lo = a;
    for (int y = 0; y < xcd; ++y) lo += sched_xcd_share(n, rot, y);
    const int cnt = sched_xcd_share(n, rot, xcd);
    S.mlo[w] = lo;
    S.loc_pre[w] = loc;
    loc += cnt;
    S.n_g1[w] = cnt * NT1;
    S.n_g2[w] = cnt * NT2;
    S.g2_all[w] = n * NT2;
    rot = (rot + n % kXcds) % kXcds;
  }
  S.n_local = loc;
  for (int s = 0; s <= S.W; ++s) {
    const int chunks = cb_parts * ((ready_off[s + 1] - ready_off[s] + kCombineTokens - 1) / kCombineTokens);
    S.n_cb[s] = chunks > xcd ? (chunks - xcd + kXcds - 1) / kXcds : 0;
  }
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

// Decodes ticket tk (0 <= tk < S.total) of this XCD's stream.
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
    t.mt = S.mlo[b] + rel / S.NT1;
    t.nt = rel % S.NT1;
    t.expert = sched_expert_of(S.mt_pre, b * S.G, (b + 1) * S.G, t.mt);
    return t;
  }
  rel -= g1n;
  if (rel < g2n) {
    t.kind = kTaskGemm2;
    t.wave = b - 1;
    t.mt = S.mlo[b - 1] + rel / S.NT2;
    t.nt = rel % S.NT2;
    t.expert = sched_expert_of(S.mt_pre, (b - 1) * S.G, b * S.G, t.mt);
    return t;
  }
  rel -= g2n;
  t.kind = kTaskCombine;
  t.slot = b - 1;
  t.chunk = S.xcd + kXcds * rel;
  return t;
}

// Counter layout (int32 words) of the persistent kernel.  Counters touched
// by different XCDs never share a 256-byte span:
//   [x * kCtrPad]                   ticket of XCD x
//   region(x) = kXcds * kCtrPad + x * region_words:
//     region(x) + w                 GEMM2 tiles of wave w finished on XCD x
//     region(x) + W + j             GEMM1 tiles finished of XCD x's j-th m-tile
//                                   (j = loc_pre[w] + mt - mlo[w])
//   kXcds * (kCtrPad + region_words) + w   GEMM2 tiles of wave w finished, all XCDs
// region_words >= W + (m-tiles of one XCD), rounded up to kCtrPad; one XCD
// holds at most max_mtiles / kXcds + W m-tiles (one extra per wave at most).
__host__ __device__ inline int sched_region_words(int W, int max_mtiles) {
  const int per_xcd = max_mtiles / kXcds + W + 1;
  return ((W + per_xcd + kCtrPad - 1) / kCtrPad) * kCtrPad;
}
__host__ __device__ inline size_t sched_counter_words(int W, int max_mtiles) {
  return static_cast<size_t>(kXcds) * (kCtrPad + sched_region_words(W, max_mtiles)) + W + kCtrPad;
}
__host__ __device__ inline int sched_ticket_index(int xcd) { return xcd * kCtrPad; }
__host__ __device__ inline int sched_g2local_index(const WaveSchedule& S, int rw, int w) {
  return kXcds * kCtrPad + S.xcd * rw + w;
}
__host__ __device__ inline int sched_g1done_index(const WaveSchedule& S, int rw, int w, int mt) {
  return kXcds * kCtrPad + S.xcd * rw + S.W + S.loc_pre[w] + (mt - S.mlo[w]);
}
__host__ __device__ inline int sched_g2all_index(const WaveSchedule& S, int rw, int w) {
  return kXcds * (kCtrPad + rw) + w;
}

}  // namespace moe
