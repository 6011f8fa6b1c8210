// CPU check of the persistent expert-wave kernel's task order
// (combine_wave_level_amd/csrc/wave_sched.h): the same host+device schedule
// functions the kernel calls, driven by host threads with std::atomic
// counters in place of the device counters.
//
// stdin: E_local G BT NT1 NT2 with_combine nthreads seed
//        offsets[E_local + 1]  ready_off[W + 2]
// Checks (exit status 0 = all hold):
//   1. structure: every GEMM1 / GEMM2 tile (m-tile x output tile) and every
//      combine chunk has exactly one ticket; decoded experts own their
//      m-tiles and belong to the decoded wave;
//   2. every wait of a ticket is on tickets smaller than itself (the
//      deadlock-freedom argument);
//   3. an emulated run with nthreads workers (random delays) completes and
//      each wait target is reached.
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

int main() {
  int E_local, G, BT, NT1, NT2, with_cb, nthreads;
  unsigned seed;
  if (std::scanf("%d %d %d %d %d %d %d %u", &E_local, &G, &BT, &NT1, &NT2, &with_cb, &nthreads, &seed) != 8)
    return fail("input");
  const int W = E_local / G;
  std::vector<int32_t> offsets(E_local + 1), ready_off(W + 2);
  for (auto& v : offsets) if (std::scanf("%d", &v) != 1) return fail("offsets");
  for (auto& v : ready_off) if (std::scanf("%d", &v) != 1) return fail("ready_off");
  static WaveSchedule S;
  sched_build(S, offsets.data(), ready_off.data(), E_local, G, BT, NT1, NT2, with_cb);
  const int nmt = S.mt_pre[E_local];

  // ---- 1. structure
  std::vector<int> g1_ticket(static_cast<size_t>(nmt) * NT1, -1), g2_ticket(static_cast<size_t>(nmt) * NT2, -1);
  std::vector<std::vector<int>> cb_ticket(W + 1);
  for (int s = 0; s <= W; ++s) cb_ticket[s].assign(S.n_cb[s], -1);
  for (int tk = 0; tk < S.total; ++tk) {
    const Task t = sched_decode(S, tk);
    if (t.kind == kTaskCombine) {
      if (t.slot < 0 || t.slot > W || t.chunk < 0 || t.chunk >= S.n_cb[t.slot]) fail("combine range", tk);
      if (cb_ticket[t.slot][t.chunk] != -1) fail("combine chunk twice", tk);
      cb_ticket[t.slot][t.chunk] = tk;
      continue;
    }
    if (t.mt < S.mt_pre[t.expert] || t.mt >= S.mt_pre[t.expert + 1]) fail("expert does not own m-tile", tk, t.mt);
    if (t.expert / G != t.wave) fail("expert not in wave", tk, t.expert);
    const int NT = t.kind == kTaskGemm1 ? NT1 : NT2;
    if (t.nt < 0 || t.nt >= NT) fail("nt range", tk, t.nt);
    auto& slot = (t.kind == kTaskGemm1 ? g1_ticket : g2_ticket)[static_cast<size_t>(t.mt) * NT + t.nt];
    if (slot != -1) fail("tile twice", tk, t.mt);
    slot = tk;
  }
  for (int v : g1_ticket) if (v < 0) fail("GEMM1 tile without ticket");
  for (int v : g2_ticket) if (v < 0) fail("GEMM2 tile without ticket");
  for (int s = 0; s <= W; ++s) {
    for (int v : cb_ticket[s]) if (v < 0) fail("combine chunk without ticket", s);
    const int want = with_cb ? (ready_off[s + 1] - ready_off[s] + kCombineTokens - 1) / kCombineTokens : 0;
    if (static_cast<int>(cb_ticket[s].size()) != want) fail("combine chunk count", s);
  }

  // ---- 2. waits only on smaller tickets
  for (int mt = 0; mt < nmt; ++mt)
    for (int nt = 0; nt < NT2; ++nt) {
      const int tk = g2_ticket[static_cast<size_t>(mt) * NT2 + nt];
      for (int n1 = 0; n1 < NT1; ++n1)
        if (g1_ticket[static_cast<size_t>(mt) * NT1 + n1] >= tk) fail("GEMM2 waits on a later ticket", tk);
    }
  for (int s = 0; s <= W; ++s)
    for (int tk : cb_ticket[s])
      for (int w = 0; w < s; ++w)
        for (int mt = S.mt_pre[w * G]; mt < S.mt_pre[(w + 1) * G]; ++mt)
          for (int nt = 0; nt < NT2; ++nt)
            if (g2_ticket[static_cast<size_t>(mt) * NT2 + nt] >= tk) fail("combine waits on a later ticket", tk);

  // ---- 3. emulated run
  std::vector<std::atomic<int>> cnt(1 + W + nmt + 1);
  for (auto& c : cnt) c.store(0);
  std::atomic<int> done_tasks{0};
  auto wait_geq = [&](int idx, int target) {
    const auto t0 = std::chrono::steady_clock::now();
    while (cnt[idx].load(std::memory_order_acquire) < target) {
      if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(20)) fail("wait never satisfied", idx, target);
      std::this_thread::yield();
    }
  };
  auto worker = [&](int id) {
    std::mt19937 rng(seed * 7919u + id);
    for (;;) {
      const int tk = cnt[0].fetch_add(1, std::memory_order_relaxed);
      if (tk >= S.total) break;
      const Task t = sched_decode(S, tk);
      if (rng() % 4 == 0) std::this_thread::sleep_for(std::chrono::microseconds(rng() % 200));
      if (t.kind == kTaskGemm1) {
        cnt[sched_g1done_index(S, t.mt)].fetch_add(1, std::memory_order_release);
      } else if (t.kind == kTaskGemm2) {
        wait_geq(sched_g1done_index(S, t.mt), S.NT1);
        cnt[sched_g2done_index(S, t.wave)].fetch_add(1, std::memory_order_release);
      } else {
        for (int w = 0; w < t.slot; ++w) wait_geq(sched_g2done_index(S, w), S.n_g2[w]);
      }
      done_tasks.fetch_add(1);
    }
  };
  std::vector<std::thread> th;
  for (int i = 0; i < nthreads; ++i) th.emplace_back(worker, i);
  for (auto& x : th) x.join();
  if (done_tasks.load() != S.total) fail("tasks done", done_tasks.load(), S.total);
  for (int mt = 0; mt < nmt; ++mt)
    if (cnt[sched_g1done_index(S, mt)].load() != NT1) fail("g1done count", mt);
  for (int w = 0; w < W; ++w)
    if (cnt[sched_g2done_index(S, w)].load() != S.n_g2[w]) fail("g2done count", w);
  std::printf("OK total=%d W=%d mtiles=%d\n", S.total, W, nmt);
  return 0;
}
