// wave_sched.h -- the static task order of the persistent expert-wave kernel,
// as host+device functions so that the schedule can be checked on the CPU.
//
// DeepSeek-V4 launch digest (itsolotime.com), section 1.2: in steady state
// the compute of the current wave, the dispatch of the next wave's tokens
// and the return of finished experts' results run at the same time.
//
// MI355X has 8 XCDs, each with its own L2.  Every XCD gets the same number
// of m-tiles (BT-row slices of each expert's sorted rows), to within one: XCD
// x may take at most cap_x = floor(n / 8) (+ 1 for the first n % 8 XCDs).
// The m-tiles are dealt in expert (= wave) order, each deal to the XCD with
// the most room left (lowest id on ties).  For compute-bound shapes a deal
// is as much of the expert as fits that room, so an expert is split only
// when the roomiest XCD fills up and its weights are mostly read by one XCD;
// for weight-streaming shapes, where every m-tile streams its expert's
// weights anyway, m-tiles are dealt one by one, which also spreads every
// wave over the XCDs.  Every workgroup takes tasks only from its own XCD's
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
  int32_t need[kSchedMaxWaves + 1];      // work units by which every XCD ends waves < s (see sched_build)
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
// sched_build = sched_build_tables (dealing, combine placement; leaves in
// cb_pos[i + 1] the combine tasks placed at position i) + sched_build_positions
// (prefix sums into cb_pos and the first ticket of every position).  The
// kernel runs the tables on one thread and the positions on a wavefront
// (sched_scan_cb_pos_wave, then sched_pos_of per position); the prefix sums
// are exact integer sums, so both give the same schedule.  cb_pos_zeroed:
// cb_pos[0 .. kSchedMaxLocal + kSchedMaxLag] already holds zeros.
__host__ __device__ inline void sched_build_tables(WaveSchedule& S, const int32_t* offsets,
                                                   const int32_t* ready_off, int E_local, int G, int BT,
                                                   int NT1, int NT2, int cb_parts, int xcd, int lag,
                                                   bool whole_experts, bool cb_pos_zeroed) {
  S.W = E_local / G;
  const int W = S.W;  // loop bounds in registers (stores into S may alias its fields)
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
  // deal the m-tiles to the XCD with the most room (lowest id on ties): as
  // much of the expert as fits, or single m-tiles; the rooms sum to the
  // m-tiles still to deal, so every deal finds room
  int room[kXcds], cap[kXcds], cnt[kXcds];
  for (int y = 0; y < kXcds; ++y) {
    cap[y] = room[y] = run / kXcds + (y < run % kXcds ? 1 : 0);
    cnt[y] = 0;
  }
  // Work model for placing the combine (an m-tile's GEMM1 tiles cost 2
  // units: K = d over 2I features; its GEMM2 tiles 1 unit: K = I over d
  // features): XCD y's stream ends the GEMM2 tiles of its first c m-tiles
  // after 2 min(c + L, cap_y) + c units.  need[s] = the largest such time
  // over the XCDs for the m-tiles of waves < s.
  const int L = S.lag;
  S.need[0] = 0;
  int loc = 0, w_next = 0;
  int w_e = 0, in_wave = 0;  // wave of expert e and its rank in the wave (no integer division)
  for (int e = 0; e < E_local; ++e) {
    while (w_next <= w_e && w_next < W) S.loc_pre[w_next++] = loc;
    int first = S.mt_pre[e];
    int n = S.mt_pre[e + 1] - first;
    while (n > 0) {
      int x = 0;
      for (int y = 1; y < kXcds; ++y) x = room[y] > room[x] ? y : x;
      const int take = whole_experts ? (n < room[x] ? n : room[x]) : 1;
      room[x] -= take;
      cnt[x] += take;
      if (x == xcd) {
        for (int q = 0; q < take; ++q) {
          if (loc < kSchedMaxLocal) S.loc_mt[loc] = first + q;
          ++loc;
        }
      }
      first += take;
      n -= take;
    }
    if (++in_wave == G) {
      int t = 0;
      for (int y = 0; y < kXcds; ++y) {
        const int ty = cnt[y] > 0 ? 2 * (cnt[y] + L < cap[y] ? cnt[y] + L : cap[y]) + cnt[y] : 0;
        t = ty > t ? ty : t;
      }
      S.need[++w_e] = t;
      in_wave = 0;
    }
  }
  while (w_next <= W) S.loc_pre[w_next++] = loc;
  S.n_local = loc;
  if (loc > kSchedMaxLocal) {
    S.err = 1;
    S.n_local = 0;
    S.total = 0;
    return;
  }
  // combine tasks of this XCD per slot, and the position of each slot
  const int npos = loc + L;  // positions 0 .. npos - 1
  int cb = 0;
  if (!cb_pos_zeroed)
    for (int i = 0; i <= npos; ++i) S.cb_pos[i] = 0;
  int p_time = 0;  // first position whose work reaches need[s] (need grows with s)
  for (int s = 0; s <= W; ++s) {
    S.cb_pre[s] = cb;
    const int chunks = cb_parts * ((ready_off[s + 1] - ready_off[s] + kCombineTokens - 1) / kCombineTokens);
    const int mine = chunks > xcd ? (chunks - xcd + kXcds - 1) / kXcds : 0;
    cb += mine;
    // position of the GEMM2 tiles of the last m-tile of a wave <= s + 1
    // (slot s needs waves <= s - 1 of every XCD: two waves of slack for
    // XCDs that run behind this one)
    const int last = S.loc_pre[s + 2 < W ? s + 2 : W] - 1;
    int at = last >= 0 ? last + L : 0;
    // and not before this stream's own work reaches the time by which the
    // slowest XCD ends the waves the slot waits for (an XCD carrying a hot
    // expert ends them late; its partners run their later GEMM2 tiles first)
    const int need = S.need[s < W ? s : W];
    while (p_time < npos - 1 &&
           2 * (p_time + 1 < loc ? p_time + 1 : loc) + (p_time + 1 - L > 0 ? p_time + 1 - L : 0) < need)
      ++p_time;
    at = at > p_time ? at : p_time;
    S.cb_pos[at + 1] += mine;  // counted from position at + 1 on
  }
  S.cb_pre[W + 1] = cb;
}

// First ticket of position i, once cb_pos[i] = combine tasks at positions
// < i: every position j < i holds NT1 GEMM1 tiles when j < n, NT2 GEMM2
// tiles when j >= L, and its combine tasks.
__host__ __device__ inline int sched_pos_of(const WaveSchedule& S, int i) {
  const int n = S.n_local, L = S.lag;
  return S.NT1 * (i < n ? i : n) + S.NT2 * (i > L ? i - L : 0) + S.cb_pos[i];
}

__host__ __device__ inline void sched_build_positions(WaveSchedule& S) {
  const int npos = S.n_local + S.lag;
  for (int i = 1; i <= npos; ++i) S.cb_pos[i] += S.cb_pos[i - 1];
  for (int i = 0; i <= npos; ++i) S.pos[i] = sched_pos_of(S, i);
  S.total = S.pos[npos];
}

__host__ __device__ inline void sched_build(WaveSchedule& S, const int32_t* offsets,
                                            const int32_t* ready_off, int E_local, int G, int BT,
                                            int NT1, int NT2, int cb_parts, int xcd, int lag,
                                            bool whole_experts) {
  sched_build_tables(S, offsets, ready_off, E_local, G, BT, NT1, NT2, cb_parts, xcd, lag, whole_experts, false);
  if (S.err == 0) sched_build_positions(S);
}

// The prefix of sched_build_positions by one wavefront (all 64 lanes of the
// calling wave; lane l sums a contiguous chunk, the chunk sums are scanned
// across lanes, then each lane writes its chunk's running sums).
__device__ inline void sched_scan_cb_pos_wave(WaveSchedule& S) {
  const int lane = static_cast<int>(threadIdx.x) & 63;
  const int len = S.n_local + S.lag + 1;
  const int per = (len + 63) / 64;
  const int b = lane * per, e = b + per < len ? b + per : len;
  int sum = 0;
  for (int i = b; i < e; ++i) sum += S.cb_pos[i];
  int incl = sum;
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  int run = incl - sum;
  for (int i = b; i < e; ++i) {
    run += S.cb_pos[i];
    S.cb_pos[i] = run;
  }
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
