// Host simulation of the persistent forward driver's work plan
// (mixture_experts_layer_30_amd/csrc/persist_plan.h, compiled here for the
// CPU): worker threads play the workgroups, each serving queue (id mod 8),
// taking tickets from per-queue atomic counters, mapping them to items with
// the plan code the kernel uses, waiting on the same dependency counters
// (bounded: a wait over 5 s reports a deadlock) and signalling completion.
// Random delays vary the interleavings. Checked per case:
//  - every item of the layer runs exactly once, no ticket maps outside it;
//  - a D item starts only after all U items of its row tile, and a U item of
//    minibatch m >= N_s only after all D items of minibatch m - N_s;
//  - the U and D items of one row tile run in the same queue;
//  - groups of 4 row tiles stay in one queue, and the queues' group counts
//    differ by at most one.
// Prints "ok <cases>" on success, a diagnosis and exit status 1 otherwise.
#define MOK_HD inline
#include "../mixture_experts_layer_30_amd/csrc/persist_plan.h"

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <memory>
#include <random>
#include <thread>
#include <vector>

using namespace mok;

namespace {

struct Case {
  int n_mb, n_slots, ntu, ntd, per_queue;
  std::vector<int32_t> mbs;
};

std::atomic<int> g_fail{0};

void fail(const char* what, int a, int b, int c) {
  if (g_fail.exchange(1) == 0) std::fprintf(stderr, "FAIL: %s (%d %d %d)\n", what, a, b, c);
}

bool wait_for(const std::atomic<int>& c, int64_t target) {
  const auto t0 = std::chrono::steady_clock::now();
  while (c.load(std::memory_order_acquire) < target) {
    if (g_fail.load()) return false;
    if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(5)) {
      fail("wait did not end (deadlock)", (int)target, c.load(), 0);
      return false;
    }
    std::this_thread::yield();
  }
  return true;
}

bool run_case(const Case& k, uint64_t seed) {
  const int ntiles = k.mbs[k.n_mb];
  PersistPlan P{k.mbs.data(), k.n_mb, k.n_slots, k.ntu, k.ntd};
  std::unique_ptr<std::atomic<int>[]> tick(new std::atomic<int>[kPlanQueues]);
  std::unique_ptr<std::atomic<int>[]> ddone(new std::atomic<int>[k.n_mb]);
  std::unique_ptr<std::atomic<int>[]> udone(new std::atomic<int>[ntiles]);
  std::unique_ptr<std::atomic<int>[]> ran_u(new std::atomic<int>[(size_t)ntiles * k.ntu]);
  std::unique_ptr<std::atomic<int>[]> ran_d(new std::atomic<int>[(size_t)ntiles * k.ntd]);
  std::unique_ptr<std::atomic<int>[]> queue_u(new std::atomic<int>[ntiles]);
  std::unique_ptr<std::atomic<int>[]> queue_d(new std::atomic<int>[ntiles]);
  for (int q = 0; q < kPlanQueues; ++q) tick[q] = 0;
  for (int m = 0; m < k.n_mb; ++m) ddone[m] = 0;
  for (int t = 0; t < ntiles; ++t) { udone[t] = 0; queue_u[t] = -1; queue_d[t] = -1; }
  for (int64_t i = 0; i < (int64_t)ntiles * k.ntu; ++i) ran_u[i] = 0;
  for (int64_t i = 0; i < (int64_t)ntiles * k.ntd; ++i) ran_d[i] = 0;

  auto tile_mb = [&](int ti) {
    int m = 0;
    while (m < k.n_mb && k.mbs[m + 1] <= ti) ++m;
    return m;
  };

  const int workers = kPlanQueues * k.per_queue;
  std::vector<std::thread> th;
  for (int w = 0; w < workers; ++w) {
    th.emplace_back([&, w] {
      const int q = w % kPlanQueues;
      std::mt19937_64 rng(seed * 7919 + w);
      PlanCursor cur;
      plan_cursor_init(cur);
      for (;;) {
        if (g_fail.load()) return;
        const int t = tick[q].fetch_add(1);
        PlanItem it;
        if (!plan_item(P, cur, q, t, it)) return;
        if (it.m < 0 || it.m >= k.n_mb || it.ti < k.mbs[it.m] || it.ti >= k.mbs[it.m + 1]) {
          fail("item outside its minibatch", it.m, it.ti, t);
          return;
        }
        if (tile_mb(it.ti) != it.m) { fail("tile of another minibatch", it.m, it.ti, 0); return; }
        if (rng() % 4 == 0) std::this_thread::sleep_for(std::chrono::microseconds(rng() % 50));
        if (it.down) {
          if (it.col < 0 || it.col >= k.ntd) { fail("D column", it.col, k.ntd, 0); return; }
          if (!wait_for(udone[it.ti], k.ntu)) return;
          for (int c = 0; c < k.ntu; ++c)
            if (ran_u[(size_t)it.ti * k.ntu + c].load() != 1) { fail("D before its U items", it.ti, c, 0); return; }
          int exp = -1;
          if (!queue_d[it.ti].compare_exchange_strong(exp, q) && exp != q) { fail("D items in two queues", it.ti, exp, q); return; }
          if (queue_u[it.ti].load() != q) { fail("D in another queue than U", it.ti, queue_u[it.ti].load(), q); return; }
          if (rng() % 3 == 0) std::this_thread::yield();
          ran_d[(size_t)it.ti * k.ntd + it.col] += 1;
          ddone[it.m].fetch_add(1, std::memory_order_release);
        } else {
          if (it.col < 0 || it.col >= k.ntu) { fail("U column", it.col, k.ntu, 0); return; }
          if (it.m >= k.n_slots) {
            const int mp = it.m - k.n_slots;
            if (!wait_for(ddone[mp], P.down_items(mp))) return;
            for (int ti = k.mbs[mp]; ti < k.mbs[mp + 1]; ++ti)
              for (int c = 0; c < k.ntd; ++c)
                if (ran_d[(size_t)ti * k.ntd + c].load() != 1) { fail("slot reused before its D items", it.m, ti, c); return; }
          }
          int exp = -1;
          if (!queue_u[it.ti].compare_exchange_strong(exp, q) && exp != q) { fail("U items in two queues", it.ti, exp, q); return; }
          if (rng() % 3 == 0) std::this_thread::yield();
          ran_u[(size_t)it.ti * k.ntu + it.col] += 1;
          udone[it.ti].fetch_add(1, std::memory_order_release);
        }
      }
    });
  }
  for (auto& t : th) t.join();
  if (g_fail.load()) return false;
  for (int ti = 0; ti < ntiles; ++ti) {
    for (int c = 0; c < k.ntu; ++c)
      if (ran_u[(size_t)ti * k.ntu + c].load() != 1) { fail("U item not run exactly once", ti, c, ran_u[(size_t)ti * k.ntu + c].load()); return false; }
    for (int c = 0; c < k.ntd; ++c)
      if (ran_d[(size_t)ti * k.ntd + c].load() != 1) { fail("D item not run exactly once", ti, c, ran_d[(size_t)ti * k.ntd + c].load()); return false; }
  }
  // balance: the groups (4 consecutive row tiles of a minibatch) of the
  // whole layer are dealt round-robin, so the queues' group counts differ by
  // at most one
  std::vector<int> groups(kPlanQueues, 0);
  for (int m = 0; m < k.n_mb; ++m)
    for (int ti = k.mbs[m]; ti < k.mbs[m + 1]; ti += kPlanGroup) {
      const int q = queue_u[ti].load();
      for (int u = ti; u < std::min(ti + kPlanGroup, k.mbs[m + 1]); ++u)
        if (queue_u[u].load() != q) { fail("group split over queues", m, ti, u); return false; }
      groups[q] += 1;
    }
  const auto mm = std::minmax_element(groups.begin(), groups.end());
  if (*mm.second - *mm.first > 1) { fail("queues unbalanced (groups)", *mm.first, *mm.second, 0); return false; }
  return true;
}

}  // namespace

int main(int argc, char** argv) {
  const int ncases = argc > 1 ? std::atoi(argv[1]) : 200;
  std::mt19937_64 rng(12345);
  int done = 0;
  // fixed cases first: one minibatch and one slot with a partial group; one
  // slot reused by many minibatches; more slots than needed
  std::vector<Case> cases;
  cases.push_back({1, 1, 2, 1, 1, {0, 5}});
  cases.push_back({6, 1, 3, 4, 2, {0, 2, 3, 9, 9 + 1, 14, 20}});
  cases.push_back({5, 3, 1, 1, 1, {0, 33, 66, 67, 100, 101}});
  cases.push_back({8, 4, 16, 28, 4, {0, 36, 72, 108, 144, 180, 216, 252, 288}});
  for (int i = 0; i < ncases; ++i) {
    Case k;
    k.n_mb = 1 + (int)(rng() % 12);
    k.n_slots = 1 + (int)(rng() % std::min(k.n_mb, 5));
    k.ntu = 1 + (int)(rng() % 9);
    k.ntd = 1 + (int)(rng() % 11);
    k.per_queue = 1 + (int)(rng() % 3);
    k.mbs.assign(1, 0);
    for (int m = 0; m < k.n_mb; ++m) k.mbs.push_back(k.mbs.back() + 1 + (int)(rng() % 40));
    cases.push_back(k);
  }
  for (size_t i = 0; i < cases.size(); ++i) {
    if (!run_case(cases[i], i + 1)) {
      const Case& k = cases[i];
      std::fprintf(stderr, "case %zu: n_mb %d n_slots %d ntu %d ntd %d per_queue %d tiles %d\n", i, k.n_mb,
                   k.n_slots, k.ntu, k.ntd, k.per_queue, k.mbs[k.n_mb]);
      return 1;
    }
    ++done;
  }
  std::printf("ok %d\n", done);
  return 0;
}
