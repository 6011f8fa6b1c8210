// CPU check of the persistent expert-wave kernel's task order
// (combine_wave_level_amd/csrc/wave_sched.h): the same host+device schedule
// functions and counter layout the kernel uses, driven by host threads
// (grouped into the 8 per-XCD streams) with std::atomic counters in place of
// the device counters.
//
// stdin: E_local G BT NT1 NT2 cb_parts threads_per_xcd seed lag whole_experts   (cb_parts 0: no combine)
//        offsets[E_local + 1]  ready_off[W + 2]
// Checks (exit status 0 = all hold):
//   1. structure (spread schedules: every stream holds every m-tile and an
//      eighth of its output tiles; otherwise:) every expert with at most an eighth of all m-tiles lives
//      on one XCD, the XCDs' m-tile counts differ by at most the largest
//      dealt chunk; over the 8 streams every GEMM1 / GEMM2 tile (m-tile x
//      output tile) and every combine chunk of the slots before the last
//      has exactly one ticket (the last slot is in no stream); both
//      GEMM tiles of an m-tile live in the stream of the XCD owning it;
//      decoded experts own their m-tiles and belong to the decoded wave;
//      every XCD's counters fit its region;
//   2. every GEMM2 tile waits only on smaller tickets of its own stream, and
//      every combine task of slot s comes after all of its stream's GEMM2
//      tiles of waves < s (no stream can block on its own later tickets);
//   3. an emulated run completes (a thread whose stream is exhausted then
//      takes its XCD's share of the last slot's chunks from that XCD's pool
//      counter once every wave of every XCD is done), every counter ends at
//      its target and every pool chunk is combined once;
//   4. the schedule equals the one a plain sequential greedy builds (the
//      definition: every deal to the XCD with the most room, lowest id on
//      ties, the combine placed by walking the positions), and the kernel's
//      split of the build over threads (strided index ranges taken in any
//      order) gives the same schedule.
#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <thread>
#include <vector>

#include "../../combine_wave_level_amd/csrc/wave_sched.h"

using namespace moe;

static int fail(const char* msg, long a = 0, long b = 0) {
  std::printf("FAIL %s (%ld, %ld)\n", msg, a, b);
  std::fflush(stdout);
  std::exit(1);
}

// The sequential definition of the dealing and the combine placement, one
// m-tile or expert piece and one position at a time.
static void reference_tables(WaveSchedule& S, const int32_t* offsets, const int32_t* ready_off, int E_local, int G,
                             int BT, int NT1, int NT2, int cb_parts, int xcd, int lag, bool whole_experts) {
  const bool cb_pos_zeroed = false;
  S.W = E_local / G;
  const int W = S.W;  // loop bounds in registers (stores into S may alias its fields)
  S.lag = lag < 1 ? 1 : (lag > kSchedMaxLag ? kSchedMaxLag : lag);
  S.G = G;
  S.NT1 = NT1;
  S.NT2 = NT2;
  S.NT1_all = NT1;
  S.NT2_all = NT2;
  S.spread = S.nt1_base = S.nt2_base = 0;
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
  // GEMM2 groups, in one pass: a group ends at an expert change, a break in
  // the global m-tile numbering, or when it holds min(kSchedGroup, L) m-tiles
  // counted from a multiple of that size
  {
    const int C = kSchedGroup < L ? kSchedGroup : L;
    auto expert_of = [&](int mt) {
      int e = 0;
      while (S.mt_pre[e + 1] <= mt) ++e;
      return e;
    };
    int start = 0;
    for (int j = 0; j <= loc; ++j) {
      const bool cut = j == loc || j % C == 0 || S.loc_mt[j] != S.loc_mt[j - 1] + 1 ||
                       expert_of(S.loc_mt[j]) != expert_of(S.loc_mt[j - 1]);
      if (cut && j > start) {
        for (int q = start; q < j; ++q) S.grp[q] = start | ((j - start) << 16);
        start = j;
      }
    }
  }
  // combine tasks of this XCD per slot, and the position of each slot
  const int npos = loc + L;  // positions 0 .. npos - 1
  int cb = 0;
  if (!cb_pos_zeroed)
    for (int i = 0; i <= npos; ++i) S.cb_pos[i] = 0;
  int p_time = 0;  // first position whose work reaches need[s] (need grows with s)
  for (int s = 0; s <= W; ++s) {
    S.cb_pre[s] = cb;
    // the last slot is combined from the device-wide pool, in no stream
    const int chunks = s == W ? 0 : cb_parts * ((ready_off[s + 1] - ready_off[s] + kCombineTokens - 1) / kCombineTokens);
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


// The build as the kernel splits it: strided ranges of the parallel steps,
// the ranges taken in a shuffled order.
static void strided_tables(WaveSchedule& S, const int32_t* offsets, const int32_t* ready_off, int E_local, int G,
                           int BT, int NT1, int NT2, int cb_parts, int xcd, int lag, bool whole, int step,
                           std::mt19937& rng) {
  sched_init(S, E_local, G, NT1, NT2, xcd, lag);
  S.mt_pre[0] = 0;
  for (int e = 0; e < E_local; ++e) S.mt_pre[e + 1] = sched_mtiles(offsets, e, BT);
  for (int e = 1; e <= E_local; ++e) S.mt_pre[e] += S.mt_pre[e - 1];
  std::vector<int> order(step);
  for (int b = 0; b < step; ++b) order[b] = b;
  std::shuffle(order.begin(), order.end(), rng);
  if (whole)
    sched_deal_whole(S, E_local);
  else
    for (int b : order) sched_deal_single(S, E_local, b, step);
  if (S.err) return;
  std::shuffle(order.begin(), order.end(), rng);
  for (int b : order) sched_groups(S, b, step);
  for (int i = 0; i <= kSchedMaxLocal + kSchedMaxLag; ++i) S.cb_pos[i] = 0;
  S.cb_pre[0] = 0;
  std::shuffle(order.begin(), order.end(), rng);
  for (int b : order) sched_place(S, ready_off, cb_parts, b, step, [](int32_t* p, int v) { *p += v; });
  for (int s = 1; s <= S.W + 1; ++s) S.cb_pre[s] += S.cb_pre[s - 1];
  sched_build_positions(S);
}

static void same_schedule(const WaveSchedule& a, const WaveSchedule& b, int E_local, const char* what, int x) {
  if (a.err != b.err) fail(what, x, 0);
  if (a.err) return;
  bool ok = a.W == b.W && a.G == b.G && a.NT1 == b.NT1 && a.NT2 == b.NT2 && a.lag == b.lag &&
            a.n_local == b.n_local && a.total == b.total && a.spread == b.spread && a.nt1_base == b.nt1_base &&
            a.nt2_base == b.nt2_base && a.NT1_all == b.NT1_all && a.NT2_all == b.NT2_all;
  for (int e = 0; ok && e <= E_local; ++e) ok = a.mt_pre[e] == b.mt_pre[e];
  for (int j = 0; ok && j < a.n_local; ++j) ok = a.loc_mt[j] == b.loc_mt[j] && a.grp[j] == b.grp[j];
  for (int w = 0; ok && w <= a.W; ++w) ok = a.loc_pre[w] == b.loc_pre[w] && a.need[w] == b.need[w];
  for (int s = 0; ok && s <= a.W + 1; ++s) ok = a.cb_pre[s] == b.cb_pre[s];
  for (int i = 0; ok && i <= a.n_local + a.lag; ++i) ok = a.cb_pos[i] == b.cb_pos[i] && a.pos[i] == b.pos[i];
  if (!ok) fail(what, x, 1);
}

int main() {
  int E_local, G, BT, NT1, NT2, cb_parts, per_xcd, lag, whole;
  unsigned seed;
  if (std::scanf("%d %d %d %d %d %d %d %u %d %d", &E_local, &G, &BT, &NT1, &NT2, &cb_parts, &per_xcd, &seed, &lag, &whole) != 10)
    return fail("input");
  const int W = E_local / G;
  std::vector<int32_t> offsets(E_local + 1), ready_off(W + 2);
  for (auto& v : offsets) if (std::scanf("%d", &v) != 1) return fail("offsets");
  for (auto& v : ready_off) if (std::scanf("%d", &v) != 1) return fail("ready_off");
  static WaveSchedule S[kXcds];
  for (int x = 0; x < kXcds; ++x)
    sched_build(S[x], offsets.data(), ready_off.data(), E_local, G, BT, NT1, NT2, cb_parts, x, lag, whole != 0);
  for (int x = 0; x < kXcds; ++x)
    if (S[x].err) fail("schedule overflow", x, S[x].n_local);
  {
    // ---- 4. the sequential definition and the kernel's split of the build
    static WaveSchedule R, P;
    std::mt19937 rng(seed);
    for (int x = 0; x < kXcds; ++x) {
      if (S[x].spread) {
        // spreading replaces the deal: every m-tile in order, an eighth of
        // its output tiles, the same work model on every XCD
        const int run = S[x].mt_pre[E_local];
        if (whole || !sched_spreads(run, NT1, NT2) || S[x].n_local != run || S[x].NT1 * kXcds != NT1 ||
            S[x].NT2 * kXcds != NT2 || S[x].nt1_base != x * S[x].NT1 || S[x].nt2_base != x * S[x].NT2)
          fail("spread header", x, run);
        for (int j = 0; j < run; ++j)
          if (S[x].loc_mt[j] != j) fail("spread local m-tiles", x, j);
        R = S[x];
      } else {
        if (!whole && sched_spreads(S[x].mt_pre[E_local], NT1, NT2)) fail("should spread", x, 0);
        reference_tables(R, offsets.data(), ready_off.data(), E_local, G, BT, NT1, NT2, cb_parts, x, lag,
                         whole != 0);
        if (R.err == 0) sched_build_positions(R);
      }
      same_schedule(R, S[x], E_local, "schedule differs from the sequential definition", x);
      for (int step : {1, 3, 64, 256}) {
        strided_tables(P, offsets.data(), ready_off.data(), E_local, G, BT, NT1, NT2, cb_parts, x, lag, whole != 0,
                       step, rng);
        same_schedule(R, P, E_local, "strided build differs", x);
      }
    }
  }
  const int nmt = S[0].mt_pre[E_local];
  const int rw = sched_region_words(W);

  // ---- 1. structure, 2. in-stream dependencies
  std::vector<int> g1_owner(static_cast<size_t>(nmt) * NT1, -1), g2_owner(static_cast<size_t>(nmt) * NT2, -1);
  std::vector<int> g1_ticket(g1_owner.size(), -1), g2_ticket(g2_owner.size(), -1);
  std::vector<std::vector<int>> cb_seen(W + 1);
  for (int s = 0; s <= W; ++s) {
    const int chunks = s == W ? 0 : cb_parts * ((ready_off[s + 1] - ready_off[s] + kCombineTokens - 1) / kCombineTokens);
    cb_seen[s].assign(chunks, 0);
  }
  // the last slot's pool chunks (only with a fused combine)
  const int pool_chunks = cb_parts > 0 ? sched_pool_chunks(ready_off[W + 1] - ready_off[W], sched_pool_parts(cb_parts)) : 0;
  std::vector<std::atomic<int>> pool_seen(pool_chunks);
  for (auto& c : pool_seen) c.store(0);
  const bool spread = S[0].spread != 0;
  for (int x = 1; x < kXcds; ++x)
    if ((S[x].spread != 0) != spread) fail("spread differs between XCDs", x);
  if (!spread) {
    // owner XCD of every m-tile, from the local lists
    std::vector<int> owner(nmt, -1);
    for (int x = 0; x < kXcds; ++x)
      for (int j = 0; j < S[x].n_local; ++j) {
        const int mt = S[x].loc_mt[j];
        if (mt < 0 || mt >= nmt || owner[mt] != -1) fail("m-tile dealt twice or out of range", x, mt);
        if (j > 0 && S[x].loc_mt[j - 1] >= mt) fail("local m-tiles not ascending", x, j);
        owner[mt] = x;
      }
    // every m-tile dealt; whole-expert deals split an expert only when an
    // XCD fills up (each XCD fills once), so there are at most
    // E_local + kXcds - 1 (expert, XCD) pieces
    int pieces = 0;
    for (int e = 0; e < E_local; ++e) {
      const int a = S[0].mt_pre[e], b = S[0].mt_pre[e + 1];
      for (int mt = a; mt < b; ++mt) {
        if (owner[mt] < 0) fail("m-tile not dealt", e, mt);
        if (mt == a || owner[mt] != owner[mt - 1]) ++pieces;
      }
    }
    if (whole && pieces > E_local + kXcds - 1) fail("experts split more than XCD fills allow", pieces, E_local);
    int lo = 1 << 30, hi = -1;
    for (int x = 0; x < kXcds; ++x) {
      lo = S[x].n_local < lo ? S[x].n_local : lo;
      hi = S[x].n_local > hi ? S[x].n_local : hi;
      for (int w = 0; w < W; ++w)
        for (int j = S[x].loc_pre[w]; j < S[x].loc_pre[w + 1]; ++j)
          if (S[0].mt_pre[w * G] > S[x].loc_mt[j] || S[x].loc_mt[j] >= S[0].mt_pre[(w + 1) * G])
            fail("local wave prefix", x, j);
    }
    if (hi - lo > 1) fail("XCD loads differ by more than one m-tile", lo, hi);
  }
  for (int x = 0; x < kXcds; ++x)
    if (W + S[x].n_local > rw) fail("counter region too small", x, S[x].n_local);
  for (int x = 0; x < kXcds; ++x) {
    for (int tk = 0; tk < S[x].total; ++tk) {
      const Task t = sched_decode(S[x], tk);
      if (t.kind == kTaskCombine) {
        if (t.slot < 0 || t.slot > W || t.chunk < 0 || t.chunk >= static_cast<int>(cb_seen[t.slot].size()))
          fail("combine range", tk, t.chunk);
        if (cb_seen[t.slot][t.chunk]++) fail("combine chunk twice", t.slot, t.chunk);
        continue;
      }
      if (t.loc < S[x].loc_pre[t.wave] || t.loc >= S[x].loc_pre[t.wave + 1] || S[x].loc_mt[t.loc] != t.mt)
        fail("m-tile not this XCD's m-tile of the decoded wave", x, t.mt);
      if (t.mt < S[x].mt_pre[t.expert] || t.mt >= S[x].mt_pre[t.expert + 1]) fail("expert does not own m-tile", tk, t.mt);
      if (t.expert / G != t.wave) fail("expert not in wave", tk, t.expert);
      const int NT = t.kind == kTaskGemm1 ? NT1 : NT2;
      if (t.nt < 0 || t.nt >= NT) fail("nt range", tk, t.nt);
      const size_t id = static_cast<size_t>(t.mt) * NT + t.nt;
      auto& own = t.kind == kTaskGemm1 ? g1_owner : g2_owner;
      auto& tck = t.kind == kTaskGemm1 ? g1_ticket : g2_ticket;
      if (own[id] != -1) fail("tile twice", tk, t.mt);
      own[id] = x;
      tck[id] = tk;
    }
  }
  for (int x = 0; x < kXcds; ++x) {
    std::vector<int> last_g2(W, -1);
    for (int tk = 0; tk < S[x].total; ++tk) {
      const Task t = sched_decode(S[x], tk);
      if (t.kind == kTaskGemm2) last_g2[t.wave] = tk;
    }
    for (int tk = 0; tk < S[x].total; ++tk) {
      const Task t = sched_decode(S[x], tk);
      if (t.kind != kTaskCombine) continue;
      for (int w = 0; w < t.slot; ++w)
        if (last_g2[w] > tk) fail("combine task before its stream's GEMM2 of an earlier wave", x, tk);
    }
  }
  for (int v : g1_owner) if (v < 0) fail("GEMM1 tile without ticket");
  for (int v : g2_owner) if (v < 0) fail("GEMM2 tile without ticket");
  for (int s = 0; s <= W; ++s)
    for (int c : cb_seen[s]) if (c != 1) fail("combine chunk not covered once", s);
  if (!spread) {
    for (int mt = 0; mt < nmt; ++mt)
      for (int nt = 0; nt < NT2; ++nt) {
        const size_t i2 = static_cast<size_t>(mt) * NT2 + nt;
        for (int n1 = 0; n1 < NT1; ++n1) {
          const size_t i1 = static_cast<size_t>(mt) * NT1 + n1;
          if (g1_owner[i1] != g2_owner[i2]) fail("GEMM1 and GEMM2 of an m-tile on different XCDs", mt);
          if (g1_ticket[i1] >= g2_ticket[i2]) fail("GEMM2 waits on a later ticket", mt, nt);
        }
      }
  } else {
    // a GEMM2 tile waits on every stream's GEMM1 tiles of its m-tile: they
    // sit at an earlier position (m-tile j at position j, its GEMM2 at
    // j + L) in every stream, and GEMM1 tiles wait on nothing
    for (int x = 0; x < kXcds; ++x) {
      std::vector<int> g1_last(nmt, -1);
      for (int tk = 0; tk < S[x].total; ++tk) {
        const Task t = sched_decode(S[x], tk);
        if (t.kind == kTaskGemm1) g1_last[t.mt] = tk;
        if (t.kind == kTaskGemm2 && g1_last[t.mt] < 0) fail("spread GEMM2 before its stream's GEMM1 tiles", x, tk);
      }
    }
  }

  // ---- 3. emulated run
  const size_t nctr = sched_counter_words(W) + 1;  // + the kernel's exit count
  for (int x = 0; x < kXcds; ++x)
    if (static_cast<size_t>(sched_pool_index(W, x)) >= nctr - 1) fail("pool counter outside the counters", x);
  for (int x = 1; x < kXcds; ++x)
    if (sched_pool_index(W, x) - sched_pool_index(W, x - 1) < kCtrPad) fail("pool counters share a span", x);
  {
    int sum = 0;
    for (int x = 0; x < kXcds; ++x) sum += sched_pool_share(pool_chunks, x);
    if (sum != pool_chunks) fail("pool shares do not cover the chunks", sum, pool_chunks);
  }
  std::vector<std::atomic<int>> ctr(nctr);
  for (auto& c : ctr) c.store(0);
  std::atomic<int> done_tasks{0};
  auto wait_geq = [&](int idx, int target) {
    const auto t0 = std::chrono::steady_clock::now();
    while (ctr[idx].load(std::memory_order_acquire) < target) {
      if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(20)) fail("wait never satisfied", idx, target);
      std::this_thread::yield();
    }
  };
  auto worker = [&](int x, int id) {
    const WaveSchedule& s = S[x];
    std::mt19937 rng(seed * 7919u + id);
    for (;;) {
      const int tk = ctr[sched_ticket_index(x)].fetch_add(1, std::memory_order_relaxed);
      if (tk >= s.total) break;
      const Task t = sched_decode(s, tk);
      if (rng() % 4 == 0) std::this_thread::sleep_for(std::chrono::microseconds(rng() % 200));
      if (t.kind == kTaskGemm1) {
        const int done = ctr[sched_g1done_index(s, rw, t.loc)].fetch_add(1, std::memory_order_release) + 1;
        if (s.spread && done == s.NT1) ctr[sched_g1all_index(s, rw, t.loc)].fetch_add(s.NT1);
      } else if (t.kind == kTaskGemm2) {
        if (s.spread)
          wait_geq(sched_g1all_index(s, rw, t.loc), s.NT1_all);
        else
          wait_geq(sched_g1done_index(s, rw, t.loc), s.NT1);
        const int done = ctr[sched_g2local_index(s, rw, t.wave)].fetch_add(1) + 1;
        if (done == sched_g2_of_wave(s, t.wave)) ctr[sched_g2all_index(s, rw, t.wave)].fetch_add(done);
      } else {
        for (int w = 0; w < t.slot; ++w) wait_geq(sched_g2all_index(s, rw, w), sched_g2_all(s, w));
      }
      done_tasks.fetch_add(1);
    }
    // the stream is exhausted: the last slot from the pool (a thread that
    // claims a chunk waits once for every wave of every XCD)
    if (pool_chunks == 0) return;
    bool waited = false;
    const int mine = sched_pool_share(pool_chunks, x);
    for (;;) {
      const int j = ctr[sched_pool_index(W, x)].fetch_add(1, std::memory_order_relaxed);
      if (j >= mine) break;
      const int c = x + kXcds * j;
      if (!waited)
        for (int w = 0; w < W; ++w) wait_geq(sched_g2all_index(s, rw, w), sched_g2_all(s, w));
      waited = true;
      if (rng() % 4 == 0) std::this_thread::sleep_for(std::chrono::microseconds(rng() % 100));
      pool_seen[c].fetch_add(1);
    }
  };
  std::vector<std::thread> th;
  for (int x = 0; x < kXcds; ++x)
    for (int i = 0; i < per_xcd; ++i) th.emplace_back(worker, x, x * per_xcd + i);
  for (auto& t : th) t.join();
  int total = 0;
  for (int x = 0; x < kXcds; ++x) total += S[x].total;
  if (done_tasks.load() != total) fail("tasks done", done_tasks.load(), total);
  for (int x = 0; x < kXcds; ++x)
    for (int j = 0; j < S[x].n_local; ++j)
      if (ctr[sched_g1done_index(S[x], rw, j)].load() != S[x].NT1) fail("g1done count", x, j);
  if (spread)
    for (int j = 0; j < nmt; ++j)
      if (ctr[sched_g1all_index(S[0], rw, j)].load() != NT1) fail("g1all count", j);
  for (int w = 0; w < W; ++w)
    if (ctr[sched_g2all_index(S[0], rw, w)].load() != sched_g2_all(S[0], w)) fail("g2 all count", w);
  for (int c = 0; c < pool_chunks; ++c)
    if (pool_seen[c].load() != 1) fail("pool chunk not combined once", c);
  int max_group = 0;
  for (int x = 0; x < kXcds; ++x)
    for (int j = 0; j < S[x].n_local; ++j) max_group = std::max(max_group, S[x].grp[j] >> 16);
  std::printf("OK total=%d W=%d mtiles=%d spread=%d max_group=%d\n", total, W, nmt, spread ? 1 : 0, max_group);
  return 0;
}
