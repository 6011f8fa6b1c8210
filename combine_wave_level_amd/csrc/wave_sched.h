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
// When the m-tiles of a weight-streaming shape do not divide evenly over the
// XCDs, each XCD instead takes an eighth of the output tiles of every m-tile
// ("spread", see sched_spreads).
//
// Inside one XCD's stream the XCD's m-tiles are taken in wave order,
// m_0 .. m_{n-1}, and the tickets run through positions i = 0 .. n+L-1:
//   the GEMM1 tiles of m_i (i < n; their operand loads are the dispatch
//   pulls),
//   the GEMM2 tiles of m_{i-L} (i >= L),
//   the XCD's share of the combine chunks of every ready slot s < W whose
//   position is i (tokens whose last local wave is s-1; slot 0 = tokens with
//   no local pick): the position of the GEMM2 tiles of the XCD's last m-tile
//   of a wave <= s + 1.
// The last slot (W: tokens whose last local wave is the last one, most of
// the tokens once k is a few waves' worth of experts) is in no stream: a
// workgroup whose stream is exhausted takes chunks of that slot from its
// XCD's pool counter (XCD x takes chunks x, x + 8, ...), waiting once for
// every wave on every XCD before its first chunk, so every workgroup of the
// chip works on it, each as soon as it is free.  One counter per XCD keeps
// the claims of 256 workgroups off a single address.
// The GEMM2 tiles of consecutive m-tiles of one expert are dealt in groups
// of up to min(kSchedGroup, L) m-tiles (a group never crosses an expert, so
// never a wave, and starts at a multiple of that size or at the expert's
// first local m-tile): the group's tiles fill the positions of its m-tiles
// in output-tile-major order, (m_a, n), (m_a+1, n), ..., (m_a, n+1), ...,
// so an XCD runs every m-tile's use of a W2 tile at about the same time and
// the tile is read from HBM once into the L2.  A group of g <= L m-tiles
// starting at m_a has its GEMM2 tiles at positions >= a + L > a + g - 1,
// after the GEMM1 tiles of all its m-tiles.
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
constexpr int kCusPerXcd = 32;          // compute units of one XCD
constexpr int kSchedMaxExperts = 256;
constexpr int kSchedMaxWaves = 256;
constexpr int kSchedMaxLocal = 512;     // m-tiles of one XCD
constexpr int kSchedMaxLag = 64;       // GEMM2 lag, in m-tiles
constexpr int kCombineTokens = 8;       // tokens per combine task
constexpr int kCtrPad = 64;             // int32 words (256 B) between counters of different XCDs
constexpr int kSchedGroup = 8;          // m-tiles whose GEMM2 tiles interleave (at most the lag)

struct WaveSchedule {
  int W, G, NT1, NT2, total, xcd, n_local, lag, err;
  // spread: every m-tile's output tiles are split over the 8 XCDs (NT1 / NT2
  // = this stream's share per m-tile, starting at nt1_base / nt2_base of the
  // NT1_all / NT2_all tiles); else an m-tile lives on one XCD
  int spread, nt1_base, nt2_base, NT1_all, NT2_all;
  int32_t mt_pre[kSchedMaxExperts + 1];  // first m-tile of each local expert
  int32_t loc_mt[kSchedMaxLocal];        // global m-tile of this XCD's j-th m-tile (ascending)
  int32_t grp[kSchedMaxLocal];           // GEMM2 group of local m-tile j: first | size << 16
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
//
// The build is cut into steps that the kernel runs in parallel where it can
// (sched_build runs them in order on the host):
//   sched_init              header fields
//   sched_mtiles            m-tiles of one expert (the kernel's wavefront
//                           takes their prefix sum into mt_pre)
//   sched_deal_whole        whole-expert dealing, sequential (one thread)
//   sched_deal_single       single-m-tile dealing in closed form, any
//                           index range (every thread a share)
//   sched_place             combine placement, one slot at a time, any
//                           range; leaves the slot's task count in
//                           cb_pre[s + 1] and adds it to cb_pos[at + 1]
//   exclusive prefix of cb_pre, then sched_build_positions.
// Every step is exact integer arithmetic, so the order of the threads never
// changes the schedule.

__host__ __device__ inline void sched_init(WaveSchedule& S, int E_local, int G, int NT1, int NT2, int xcd,
                                           int lag) {
  S.W = E_local / G;
  S.lag = lag < 1 ? 1 : (lag > kSchedMaxLag ? kSchedMaxLag : lag);
  S.G = G;
  S.NT1 = S.NT1_all = NT1;
  S.NT2 = S.NT2_all = NT2;
  S.spread = S.nt1_base = S.nt2_base = 0;
  S.xcd = xcd;
  S.err = 0;
}

__host__ __device__ inline int sched_mtiles(const int32_t* offsets, int e, int BT) {
  return (offsets[e + 1] - offsets[e] + BT - 1) / BT;
}

// Rooms of the XCDs: the first n % 8 take floor(n / 8) + 1 m-tiles, the
// others floor(n / 8).
__host__ __device__ inline int sched_cap(int n, int y) { return n / kXcds + (y < n % kXcds ? 1 : 0); }

// Work model for placing the combine (an m-tile's GEMM1 tiles cost 2 units:
// K = d over 2I features; its GEMM2 tiles 1 unit: K = I over d features):
// XCD y's stream ends the GEMM2 tiles of its first c of cap m-tiles after
// 2 min(c + L, cap) + c units; need[s] = the largest such time over the
// XCDs for the m-tiles of waves < s.
__host__ __device__ inline int sched_work_of(int c, int cap, int L) {
  return c > 0 ? 2 * (c + L < cap ? c + L : cap) + c : 0;
}

// Whole-expert dealing: each deal goes to the XCD with the most room
// (lowest id on ties) and takes as much of the expert as fits; the rooms
// sum to the m-tiles still to deal, so every deal finds room.  Needs the
// header and mt_pre; writes loc_mt, loc_pre, need, n_local (err on
// overflow).
__host__ __device__ inline void sched_deal_whole(WaveSchedule& S, int E_local) {
  const int W = S.W, G = S.G, L = S.lag, xcd = S.xcd;  // in registers: stores into S may alias
  const int run = S.mt_pre[E_local];
  int room[kXcds], cap[kXcds], cnt[kXcds];
#pragma unroll
  for (int y = 0; y < kXcds; ++y) {
    cap[y] = room[y] = sched_cap(run, y);
    cnt[y] = 0;
  }
  S.need[0] = 0;
  int loc = 0, w_next = 0;
  int w_e = 0, in_wave = 0;  // wave of expert e and its rank in the wave (no integer division)
  for (int e = 0; e < E_local; ++e) {
    while (w_next <= w_e && w_next < W) S.loc_pre[w_next++] = loc;
    int first = S.mt_pre[e];
    int n = S.mt_pre[e + 1] - first;
    while (n > 0) {
      // the argmax and the update index the arrays with constants only (an
      // index held in a register makes every access a chain of selects)
      int x = 0, rx = room[0];
#pragma unroll
      for (int y = 1; y < kXcds; ++y) {
        if (room[y] > rx) {
          rx = room[y];
          x = y;
        }
      }
      const int take = n < rx ? n : rx;
#pragma unroll
      for (int y = 0; y < kXcds; ++y) {
        if (y == x) {
          room[y] -= take;
          cnt[y] += take;
        }
      }
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
#pragma unroll
      for (int y = 0; y < kXcds; ++y) {
        const int ty = sched_work_of(cnt[y], cap[y], L);
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
  }
}

// Single-m-tile dealing in closed form.  Dealing one m-tile at a time to the
// XCD with the most room (lowest id on ties), from rooms floor(n/8) + 1 for
// the first r = n % 8 XCDs and floor(n/8) for the others, sends m-tile j to
// XCD j for j < r and to XCD (j - r) % 8 after (the first r deals level the
// rooms, then the deals go round the XCDs in id order).
//   Deals to XCD x among the first M m-tiles:
__host__ __device__ inline int sched_single_count(int x, int M, int r) {
  return (x < r && x < M ? 1 : 0) + (M > r + x ? (M - r - x + kXcds - 1) / kXcds : 0);
}
//   Global index of XCD x's i-th m-tile:
__host__ __device__ inline int sched_single_local(int x, int i, int r) {
  return x < r ? (i == 0 ? x : r + x + kXcds * (i - 1)) : r + x + kXcds * i;
}

// Spreading: when the m-tiles do not divide evenly over the XCDs (r != 0)
// and both GEMMs' output tiles do, every XCD takes an eighth of every
// m-tile's GEMM1 and GEMM2 tiles instead, so that the weight-streaming
// shapes load every XCD equally.  The GEMM1 -> GEMM2 hand-off of an m-tile
// then crosses XCDs (a device-wide counter per m-tile; the kernel writes the
// L2 back before publishing and reads the activations with device-coherent
// loads).  Each stream holds every m-tile, in order.
__host__ __device__ inline bool sched_spreads(int run, int NT1_all, int NT2_all) {
  return run % kXcds != 0 && NT1_all % kXcds == 0 && NT2_all % kXcds == 0 && run <= kSchedMaxLocal;
}

// The thread's share (indices begin, begin + step, ...) of loc_mt, loc_pre
// and need for single-m-tile dealing (or spreading).  Needs the header and
// mt_pre; every thread sets the same header fields, n_local and err.
__host__ __device__ inline void sched_deal_single(WaveSchedule& S, int E_local, int begin, int step) {
  const int W = S.W, G = S.G, L = S.lag, xcd = S.xcd;
  const int run = S.mt_pre[E_local], r = run % kXcds;
  if (sched_spreads(run, S.NT1_all, S.NT2_all)) {
    const int nt1 = S.NT1_all / kXcds, nt2 = S.NT2_all / kXcds;
    S.spread = 1;
    S.NT1 = nt1;
    S.NT2 = nt2;
    S.nt1_base = xcd * nt1;
    S.nt2_base = xcd * nt2;
    S.n_local = run;
    for (int i = begin; i < run; i += step) S.loc_mt[i] = i;
    for (int w = begin; w <= W; w += step) {
      const int M = S.mt_pre[w * G];
      S.loc_pre[w] = M;
      S.need[w] = w > 0 ? sched_work_of(M, run, L) : 0;
    }
    return;
  }
  const int n = sched_cap(run, xcd);
  if (n > kSchedMaxLocal) {
    S.err = 1;
    S.n_local = 0;
    S.total = 0;
    return;
  }
  S.n_local = n;
  for (int i = begin; i < n; i += step) S.loc_mt[i] = sched_single_local(xcd, i, r);
  for (int w = begin; w <= W; w += step) {
    const int M = S.mt_pre[w * G];
    S.loc_pre[w] = w == W ? n : sched_single_count(xcd, M, r);
    int t = 0;
    if (w > 0) {
#pragma unroll
      for (int y = 0; y < kXcds; ++y) {
        const int ty = sched_work_of(sched_single_count(y, M, r), sched_cap(run, y), L);
        t = ty > t ? ty : t;
      }
    }
    S.need[w] = t;
  }
}

// GEMM2 groups of local m-tiles begin, begin + step, ... (needs the dealt
// tables: loc_mt, mt_pre, n_local).  Local m-tiles j - 1 and j share a group
// when they are consecutive m-tiles of one expert and j is not a multiple
// of the group size.
__host__ __device__ inline bool sched_same_run(const WaveSchedule& S, int j) {
  if (j <= 0 || S.loc_mt[j] != S.loc_mt[j - 1] + 1) return false;
  const int E = S.W * S.G;
  return sched_expert_of(S.mt_pre, 0, E, S.loc_mt[j]) == sched_expert_of(S.mt_pre, 0, E, S.loc_mt[j - 1]);
}
__host__ __device__ inline void sched_groups(WaveSchedule& S, int begin, int step) {
  const int C = kSchedGroup < S.lag ? kSchedGroup : S.lag, n = S.n_local;
  for (int j = begin; j < n; j += step) {
    const int a0 = (j / C) * C, a1 = a0 + C < n ? a0 + C : n;
    int c0 = j, c1 = j + 1;
    while (c0 > a0 && sched_same_run(S, c0)) --c0;
    while (c1 < a1 && sched_same_run(S, c1)) ++c1;
    S.grp[j] = c0 | ((c1 - c0) << 16);
  }
}

// Work of this XCD's stream through position q: 2 units per m-tile of
// GEMM1 (q <= n of them), 1 per m-tile of GEMM2 (positions >= L).
__host__ __device__ inline int sched_stream_work(int q, int n, int L) {
  return 2 * (q < n ? q : n) + (q - L > 0 ? q - L : 0);
}

// First position p in [0, npos - 1] whose next position's work reaches
// need (npos - 1 if none does); sched_stream_work grows with q.
__host__ __device__ inline int sched_p_time(int need, int n, int L, int npos) {
  int lo = 0, hi = npos - 1;  // answer in [lo, hi]
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (sched_stream_work(mid + 1, n, L) >= need) hi = mid; else lo = mid + 1;
  }
  return lo;
}

// Combine placement of slots begin, begin + step, ... <= W (tokens whose
// last local wave is s - 1): this XCD's share of the slot's chunks sits at
// the position of the GEMM2 tiles of its last m-tile of a wave <= s + 1
// (slot s needs waves <= s - 1 of every XCD: two waves of slack for XCDs
// that run behind this one), and not before this stream's own work reaches
// need[s], the time by which the slowest XCD ends those waves (an XCD
// carrying a hot expert ends them late; its partners run their later GEMM2
// tiles first).  need grows with s, so the positions do too.  Writes the
// slot's task count to cb_pre[s + 1] and adds it to cb_pos[at + 1] with
// add(), which must be atomic when threads share the work.
template <class Add>
__host__ __device__ inline void sched_place(WaveSchedule& S, const int32_t* ready_off, int cb_parts, int begin,
                                            int step, Add add) {
  const int W = S.W, L = S.lag, xcd = S.xcd, n = S.n_local;
  const int npos = n + L;  // positions 0 .. npos - 1
  for (int s = begin; s <= W; s += step) {
    // the last slot is combined from the device-wide pool (no stream tasks)
    const int chunks =
        s == W ? 0 : cb_parts * ((ready_off[s + 1] - ready_off[s] + kCombineTokens - 1) / kCombineTokens);
    const int mine = chunks > xcd ? (chunks - xcd + kXcds - 1) / kXcds : 0;
    const int last = S.loc_pre[s + 2 < W ? s + 2 : W] - 1;
    int at = last >= 0 ? last + L : 0;
    const int p_time = sched_p_time(S.need[s < W ? s : W], n, L, npos);
    at = at > p_time ? at : p_time;
    S.cb_pre[s + 1] = mine;
    if (mine > 0) add(&S.cb_pos[at + 1], mine);
  }
}

// The host composition of the steps (cb_pos must hold zeros).
__host__ __device__ inline void sched_build_tables(WaveSchedule& S, const int32_t* offsets,
                                                   const int32_t* ready_off, int E_local, int G, int BT,
                                                   int NT1, int NT2, int cb_parts, int xcd, int lag,
                                                   bool whole_experts) {
  sched_init(S, E_local, G, NT1, NT2, xcd, lag);
  int run = 0;
  for (int e = 0; e < E_local; ++e) {
    S.mt_pre[e] = run;
    run += sched_mtiles(offsets, e, BT);
  }
  S.mt_pre[E_local] = run;
  if (whole_experts)
    sched_deal_whole(S, E_local);
  else
    sched_deal_single(S, E_local, 0, 1);
  if (S.err) return;
  sched_groups(S, 0, 1);
  for (int i = 0; i <= S.n_local + S.lag; ++i) S.cb_pos[i] = 0;
  sched_place(S, ready_off, cb_parts, 0, 1, [](int32_t* p, int v) { *p += v; });
  S.cb_pre[0] = 0;
  for (int s = 1; s <= S.W + 1; ++s) S.cb_pre[s] += S.cb_pre[s - 1];
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
  sched_build_tables(S, offsets, ready_off, E_local, G, BT, NT1, NT2, cb_parts, xcd, lag, whole_experts);
  if (S.err == 0) sched_build_positions(S);
}

// In-place inclusive prefix sum of a[0 .. len) by one wavefront (all 64
// lanes of the calling wave; lane l sums a contiguous chunk, the chunk sums
// are scanned across lanes, then each lane writes its chunk's running sums).
// The kernel's form of the host loops over mt_pre, cb_pre and cb_pos.
__device__ inline void sched_scan_wave(int32_t* a, int len) {
  const int lane = static_cast<int>(threadIdx.x) & 63;
  const int per = (len + 63) / 64;
  const int b = lane * per, e = b + per < len ? b + per : len;
  int sum = 0;
  for (int i = b; i < e; ++i) sum += a[i];
  int incl = sum;
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  int run = incl - sum;
  for (int i = b; i < e; ++i) {
    run += a[i];
    a[i] = run;
  }
}

// GEMM2 tiles of wave w on this XCD.
__host__ __device__ inline int sched_g2_of_wave(const WaveSchedule& S, int w) {
  return (S.loc_pre[w + 1] - S.loc_pre[w]) * S.NT2;
}
// GEMM2 tiles of wave w over all XCDs.
__host__ __device__ inline int sched_g2_all(const WaveSchedule& S, int w) {
  return (S.mt_pre[(w + 1) * S.G] - S.mt_pre[w * S.G]) * S.NT2_all;
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
      t.nt = S.nt1_base + o;
      sched_local_mtile(S, i, t);
      return t;
    }
    o -= S.NT1;
  }
  if (i >= L) {
    if (o < S.NT2) {
      // position i's share of its m-tile's group, output-tile-major
      const int j = i - L, c0 = S.grp[j] & 0xffff, cs = S.grp[j] >> 16;
      const int g = (j - c0) * S.NT2 + o;
      t.kind = kTaskGemm2;
      t.nt = S.nt2_base + g / cs;
      sched_local_mtile(S, c0 + g % cs, t);
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

// The last ready slot's pool: column parts of a chunk (at least two, so
// each wavefront's share of a token is one pass of its loads for d = 4096)
// and chunks of kCombineTokens tokens x parts.
__host__ __device__ inline int sched_pool_parts(int cb_parts) { return cb_parts > 2 ? cb_parts : 2; }
__host__ __device__ inline int sched_pool_chunks(int ntok, int pparts) {
  return pparts * ((ntok + kCombineTokens - 1) / kCombineTokens);
}
// Chunks of XCD x's share (chunks x, x + kXcds, ...).
__host__ __device__ inline int sched_pool_share(int nchunks, int x) {
  return nchunks > x ? (nchunks - x + kXcds - 1) / kXcds : 0;
}

// Counter layout (int32 words) of the persistent kernel.  Counters touched
// by different XCDs never share a 256-byte span:
//   [x * kCtrPad]                   ticket of XCD x
//   region(x) = kXcds * kCtrPad + x * region_words:
//     region(x) + w                 GEMM2 tiles of wave w finished on XCD x
//     region(x) + W + j             GEMM1 tiles finished of XCD x's m-tile j
//   kXcds * (kCtrPad + region_words) + w   GEMM2 tiles of wave w finished, all XCDs
//   that + pad(W) + j               spread schedules: GEMM1 tiles of m-tile j
//                                   finished, all XCDs
//   that + pad(W) + kSchedMaxLocal + x * kCtrPad   XCD x's pool counter of
//                                   the last ready slot
// region_words >= W + kSchedMaxLocal, rounded up to kCtrPad (pad).
__host__ __device__ inline int sched_region_words(int W) {
  return ((W + kSchedMaxLocal + kCtrPad - 1) / kCtrPad) * kCtrPad;
}
__host__ __device__ inline int sched_pad_words(int n) { return ((n + kCtrPad - 1) / kCtrPad) * kCtrPad; }
__host__ __device__ inline size_t sched_counter_words(int W) {
  return static_cast<size_t>(kXcds) * (kCtrPad + sched_region_words(W)) + sched_pad_words(W) + kSchedMaxLocal +
         static_cast<size_t>(kXcds) * kCtrPad;
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
// spread schedules: GEMM1 tiles of m-tile j finished, all XCDs
__host__ __device__ inline int sched_g1all_index(const WaveSchedule& S, int rw, int j) {
  return kXcds * (kCtrPad + rw) + sched_pad_words(S.W) + j;
}
__host__ __device__ inline int sched_pool_index(int W, int xcd) {
  return kXcds * (kCtrPad + sched_region_words(W)) + sched_pad_words(W) + kSchedMaxLocal + xcd * kCtrPad;
}

// ---------------------------------------------------------------- phase kernels

// XCD-affine tile order of the phase kernels (the large tile shapes, when
// the routed-to experts average at least two m-tiles).  The tiles are
// listed expert by expert, n-tile-major inside an expert (the m-tiles of an
// expert that read one weight tile are adjacent), and the list is cut into
// 8 contiguous runs of equal length; workgroup b runs tiles of run b % 8,
// since the dispatcher deals consecutive workgroups to the 8 XCDs in turn
// (only locality depends on that, never correctness).  So an m-tile's token
// rows are fetched by one or two XCDs instead of by every XCD that holds one
// of its n-tiles, and the m-tiles of an expert that read the same weight
// tile run side by side under one L2.  Measured on MI355X against the plain
// order (m-tile-major over the whole grid), FFN on the phase kernels: mid
// layer T=4096 (4.5 m-tiles per expert) 1.4% faster, stress layer T=4096
// (2.1) 2.9% and T=16384 (6.4) 3 to 5% faster; the V3/V4-scale share
// (1.6 m-tiles per expert, most experts one full m-tile and a short tail)
// 1.6% slower, so there the plain order stays.  The backward's products
// (g, the h recompute, the dx rows) walk their tiles the same way, under
// the same rule (stress layer T=16384: g 13%, the recompute 8%, the dx rows
// 2.5% faster; mid layer within the run-to-run spread).
__host__ __device__ inline bool phase_xcd_order(const int32_t* mt_pre, int E_local) {
  int routed = 0;
  for (int e = 0; e < E_local; ++e) routed += mt_pre[e + 1] > mt_pre[e];
  return mt_pre[E_local] >= 2 * routed;
}
struct PhaseTiles {
  int begin, end, first, stride;  // run [begin, end) of the list; tiles begin + first + j * stride
};
__host__ __device__ inline PhaseTiles phase_tiles(int total, bool xcd_order, int block, int grid) {
  if (!xcd_order || grid % kXcds != 0) return {0, total, block, grid};
  const int x = block % kXcds;
  const long long t = total;
  return {static_cast<int>(t * x / kXcds), static_cast<int>(t * (x + 1) / kXcds), block / kXcds, grid / kXcds};
}
// Tile g of the list (NT n-tiles per m-tile): its expert e, m-tile mt and
// n-tile nt.  The plain order: m-tile g / NT, n-tile g % NT.
__host__ __device__ inline void phase_tile(const int32_t* mt_pre, int E_local, int NT, int g, bool xcd_order, int& e,
                                           int& mt, int& nt) {
  e = sched_expert_of(mt_pre, 0, E_local, g / NT);
  if (!xcd_order) {
    mt = g / NT;
    nt = g % NT;
    return;
  }
  const int n = mt_pre[e + 1] - mt_pre[e];
  const int r = g - NT * mt_pre[e];
  nt = r / n;
  mt = mt_pre[e] + r % n;
}

}  // namespace moe
