// wave_sched.h -- the static task order of the persistent expert-wave kernel,
// as host+device functions so that the schedule can be checked on the CPU.
//
// DeepSeek-V4 launch digest (itsolotime.com), section 1.2: in steady state
// the compute of the current wave, the dispatch of the next wave's tokens
// and the return of finished experts' results run at the same time.
//
// MI355X has 8 XCDs, each with its own L2.  The m-tiles (BT-row slices of
// each expert's sorted rows) are dealt to the XCDs in expert (= wave) order,
// each deal to the XCD with the least m-tiles so far (lowest id on ties).
// For compute-bound shapes an expert is dealt whole, so its weights are read
// by one XCD only (an expert with more m-tiles than an eighth of all, a hot
// expert, is dealt in chunks of at most that many); for weight-streaming
// shapes, where every m-tile streams its expert's weights anyway, m-tiles
// are dealt one by one, which balances the XCDs to within one m-tile.  Every workgroup takes tasks only from its own XCD's
// ticket stream, so GEMM1 -> GEMM2 dependencies never leave an XCD's L2;
// only the combine, which reads y rows of every XCD, crosses XCDs.
//
// Inside one XCD's stream the XCD's m-tiles are taken in wave order,
// m_0 .. m_{n-1}, and the tickets run through positions i = 0 .. n+L-1:
//   the GEMM1 tiles of m_i (i < n; their operand loads are the dispatch
//   pulls),
//   the GEMM2 tiles of m_{i-L} (i >= L),
//   the XCD's share of the combine chunks of every ready slot s whose
//   position is i (tokens whose last local wave is s-1; slot 0 = tokens with
//   no local pick): the position of the GEMM2 tiles of the XCD's last m-tile
//   of a wave <= s + 1.
// GEMM2 of an m-tile thus trails its GEMM1 by L m-tiles (the kernel uses a
// long lag: an XCD's GEMM1 tiles mostly run before its GEMM2 tiles, which
// keeps the two operand sets from sharing the XCD's L2 at the same time).  A GEMM2 tile waits for its m-tile's
// GEMM1 tiles (same stream, smaller tickets).  A combine task waits until
// every XCD finished the GEMM2 tiles of waves <= its slot - 1; in every
// stream those tiles sit at smaller tickets than that stream's combine
// tasks of the slot and wait only on smaller tickets of their own stream,
// so every wait ends, for any grid.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kXcds = 8;                // XCDs of an MI355X
constexpr int kSchedMaxExperts = 256;
constexpr int kSchedMaxWaves = 256;
constexpr int kSchedMaxLocal = 512;     // m-tiles of one XCD
constexpr int kSchedMaxLag = 64;       // GEMM2 lag, in m-tiles
constexpr int kCombineTokens = 8;       // tokens per combine task
constexpr int kCtrPad = 64;             // int32 words (256 B) between counters of different XCDs

struct WaveSchedule {
  int W, G, NT1, NT2, total, xcd, n_local, lag, err;
  int32_t mt_pre[kSchedMaxExperts + 1];  // first m-tile of each local expert
  int32_t loc_mt[kSchedMaxLocal];        // global m-tile of this XCD's j-th m-tile (ascending)
  int32_t loc_pre[kSchedMaxWaves + 1];   // this XCD's m-tiles in waves < w (loc_pre[W] = n_local)
  int32_t cb_pre[kSchedMaxWaves + 2];    // this XCD's combine tasks of slots < s
  int32_t pos[kSchedMaxLocal + kSchedMaxLag + 1];     // first ticket of position i, i = 0 .. n+L
  int32_t cb_pos[kSchedMaxLocal + kSchedMaxLag + 1];  // this XCD's combine tasks at positions < i
};

enum TaskKind { kTaskGemm1 = 0, kTaskGemm2 = 1, kTaskCombine = 2 };

struct Task {
  int kind;
  int wave;      // GEMM1 / GEMM2: expert wave of the tile
  int loc;       // GEMM1 / GEMM2: index of the m-tile among this XCD's m-tiles
  int mt;        // global m-tile index (GEMM1 / GEMM2)
  int expert;    // local expert (GEMM1 / GEMM2)
  int nt;        // output-feature tile (GEMM1 / GEMM2)
  int slot;      // combine: ready slot
  int chunk;     // combine: global chunk inside the slot: token chunk (of
                 // kCombineTokens) chunk / cb_parts, column part chunk % cb_parts
};

// Largest i in [lo, hi) with a[i] <= v, given a[lo] <= v (a nondecreasing).
__host__ __device__ inline int sched_last_leq(const int32_t* a, int lo, int hi, int v) {
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] <= v) lo = mid; else hi = mid;
  }
  return lo;
}

// The expert whose m-tile range holds mt, with mt_pre[lo] <= mt < mt_pre[hi].
__host__ __device__ inline int sched_expert_of(const int32_t* mt_pre, int lo, int hi, int mt) {
  return sched_last_leq(mt_pre, lo, hi, mt);
}

// Builds XCD xcd's schedule from the dispatch tables.  offsets [E_local + 1]
// = first pair row of each local expert; ready_off [W + 2] = first position
// of each ready slot in the ready list.  BT = rows per m-tile.  NT1 / NT2 =
// output tiles of GEMM1 / GEMM2 per m-tile.  cb_parts = column parts per
// combine chunk of kCombineTokens tokens (0: no combine tasks, no fused
// combine).  lag = L (1 .. kSchedMaxLag).  whole_experts: deal experts whole
// (else single m-tiles).  S.err = 1 if the XCD holds more than
// kSchedMaxLocal m-tiles (the schedule is then empty).
__host__ __device__ inline void sched_build(WaveSchedule& S, const int32_t* offsets,
                                            const int32_t* ready_off, int E_local, int G, int BT,
                                            int NT1, int NT2, int cb_parts, int xcd, int lag,
                                            bool whole_experts) {
  S.W = E_local / G;
  S.lag = lag < 1 ? 1 : (lag > kSchedMaxLag ? kSchedMaxLag : lag);
  S.G = G;
  S.NT1 = NT1;
  S.NT2 = NT2;
  S.xcd = xcd;
  S.err = 0;
  int run = 0;
  for (int e = 0; e < E_local; ++e) {
    S.mt_pre[e] = run;
    run += (offsets[e + 1] - offsets[e] + BT - 1) / BT;
  }
  S.mt_pre[E_local] = run;
  // deal the m-tiles to the least-loaded XCD (lowest id on ties): whole
  // experts (above the share in chunks of the share) or single m-tiles
  const int share = (run + kXcds - 1) / kXcds;
  int load[kXcds];
  for (int y = 0; y < kXcds; ++y) load[y] = 0;
  int loc = 0, w_next = 0;
  for (int e = 0; e < E_local; ++e) {
    while (w_next <= e / G && w_next < S.W) S.loc_pre[w_next++] = loc;
    int first = S.mt_pre[e];
    int n = S.mt_pre[e + 1] - first;
    while (n > 0) {
      int x = 0;
      for (int y = 1; y < kXcds; ++y) x = load[y] < load[x] ? y : x;
      const int take = whole_experts ? (n > share ? share : n) : 1;
      load[x] += take;
      if (x == xcd) {
        for (int q = 0; q < take; ++q) {
          if (loc < kSchedMaxLocal) S.loc_mt[loc] = first + q;
          ++loc;
        }
      }
      first += take;
      n -= take;
    }
  }
  while (w_next <= S.W) S.loc_pre[w_next++] = loc;
  S.n_local = loc;
  if (loc > kSchedMaxLocal) {
    S.err = 1;
    S.n_local = 0;
    S.total = 0;
    return;
  }
  // combine tasks of this XCD per slot, and the position of each slot
  const int L = S.lag, npos = loc + L;  // positions 0 .. npos - 1
  int cb = 0;
  for (int i = 0; i <= npos; ++i) S.cb_pos[i] = 0;
  for (int s = 0; s <= S.W; ++s) {
    S.cb_pre[s] = cb;
    const int chunks = cb_parts * ((ready_off[s + 1] - ready_off[s] + kCombineTokens - 1) / kCombineTokens);
    const int mine = chunks > xcd ? (chunks - xcd + kXcds - 1) / kXcds : 0;
    cb += mine;
    // position of the GEMM2 tiles of the last m-tile of a wave <= s + 1
    // (slot s needs waves <= s - 1 of every XCD: two waves of slack for
    // XCDs that run behind this one)
    const int last = S.loc_pre[s + 2 < S.W ? s + 2 : S.W] - 1;
    const int at = last >= 0 ? last + L : 0;
    S.cb_pos[at + 1] += mine;  // counted from position at + 1 on
  }
  S.cb_pre[S.W + 1] = cb;
  // cb_pos[i] = combine tasks at positions < i (prefix of the per-position counts)
  for (int i = 1; i <= npos; ++i) S.cb_pos[i] += S.cb_pos[i - 1];
  run = 0;
  for (int i = 0; i < npos; ++i) {
    S.pos[i] = run;
    if (i < loc) run += NT1;
    if (i >= L) run += NT2;
    run += S.cb_pos[i + 1] - S.cb_pos[i];
  }
  S.pos[npos] = run;
  S.total = run;
}

// GEMM2 tiles of wave w on this XCD.
__host__ __device__ inline int sched_g2_of_wave(const WaveSchedule& S, int w) {
  return (S.loc_pre[w + 1] - S.loc_pre[w]) * S.NT2;
}
// GEMM2 tiles of wave w over all XCDs.
__host__ __device__ inline int sched_g2_all(const WaveSchedule& S, int w) {
  return (S.mt_pre[(w + 1) * S.G] - S.mt_pre[w * S.G]) * S.NT2;
}

// Fills the m-tile fields of t for this XCD's m-tile j.
__host__ __device__ inline void sched_local_mtile(const WaveSchedule& S, int j, Task& t) {
  // wave w with loc_pre[w] <= j < loc_pre[w + 1] (waves without local m-tiles skipped)
  int w = sched_last_leq(S.loc_pre, 0, S.W, j);
  while (S.loc_pre[w + 1] <= j) ++w;
  t.wave = w;
  t.loc = j;
  t.mt = S.loc_mt[j];
  t.expert = sched_expert_of(S.mt_pre, w * S.G, (w + 1) * S.G, t.mt);
}

// Decodes ticket tk (0 <= tk < S.total) of this XCD's stream.
__host__ __device__ inline Task sched_decode(const WaveSchedule& S, int tk) {
  const int n = S.n_local, L = S.lag;
  const int i = sched_last_leq(S.pos, 0, n + L, tk);
  int o = tk - S.pos[i];
  Task t{};
  if (i < n) {
    if (o < S.NT1) {
      t.kind = kTaskGemm1;
      t.nt = o;
      sched_local_mtile(S, i, t);
      return t;
    }
    o -= S.NT1;
  }
  if (i >= L) {
    if (o < S.NT2) {
      t.kind = kTaskGemm2;
      t.nt = o;
      sched_local_mtile(S, i - L, t);
      return t;
    }
    o -= S.NT2;
  }
  t.kind = kTaskCombine;
  const int idx = S.cb_pos[i] + o;
  // slot s with cb_pre[s] <= idx < cb_pre[s + 1] (slots without tasks skipped)
  int sl = sched_last_leq(S.cb_pre, 0, S.W + 1, idx);
  while (S.cb_pre[sl + 1] <= idx) ++sl;
  t.slot = sl;
  t.chunk = S.xcd + kXcds * (idx - S.cb_pre[sl]);
  return t;
}

// Counter layout (int32 words) of the persistent kernel.  Counters touched
// by different XCDs never share a 256-byte span:
//   [x * kCtrPad]                   ticket of XCD x
//   region(x) = kXcds * kCtrPad + x * region_words:
//     region(x) + w                 GEMM2 tiles of wave w finished on XCD x
//     region(x) + W + j             GEMM1 tiles finished of XCD x's m-tile j
//   kXcds * (kCtrPad + region_words) + w   GEMM2 tiles of wave w finished, all XCDs
// region_words >= W + kSchedMaxLocal, rounded up to kCtrPad.
__host__ __device__ inline int sched_region_words(int W) {
  return ((W + kSchedMaxLocal + kCtrPad - 1) / kCtrPad) * kCtrPad;
}
__host__ __device__ inline size_t sched_counter_words(int W) {
  return static_cast<size_t>(kXcds) * (kCtrPad + sched_region_words(W)) + W + kCtrPad;
}
__host__ __device__ inline int sched_ticket_index(int xcd) { return xcd * kCtrPad; }
__host__ __device__ inline int sched_g2local_index(const WaveSchedule& S, int rw, int w) {
  return kXcds * kCtrPad + S.xcd * rw + w;
}
__host__ __device__ inline int sched_g1done_index(const WaveSchedule& S, int rw, int loc) {
  return kXcds * kCtrPad + S.xcd * rw + S.W + loc;
}
__host__ __device__ inline int sched_g2all_index(const WaveSchedule& S, int rw, int w) {
  return kXcds * (kCtrPad + rw) + w;
}

}  // namespace moe
