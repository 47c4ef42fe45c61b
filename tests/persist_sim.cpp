// Host simulation of the persistent forward driver's work plan
// (mixture_experts_layer_30_amd/csrc/persist_plan.h, compiled here for the
// CPU): worker threads play the workgroups, each serving queue (id mod 8),
// taking tickets from per-queue atomic counters, mapping them to items with
// the plan code the kernel uses, waiting on the same dependency counters
// (bounded: a wait over 5 s reports a deadlock) and signalling completion the
// way the kernel does (U items per row tile; D items per row tile, the last
// one retiring the tile). Random delays vary the interleavings. Row-tile
// tables are built like the schedule's: expert segments of the permuted rows
// cut at multiples of M and into pieces of at most bm rows, invalid rows
// (untiled) at the end. Checked per case:
//  - every item of the layer runs exactly once, no ticket maps outside it;
//  - a D item starts only after all U items of its row tile;
//  - a U item of minibatch m >= N_s starts only after every D item of each
//    row tile of minibatch m - N_s whose slot rows overlap its own (found by
//    brute force here) is done, and plan_first_overlap / plan_overlaps name
//    exactly those tiles;
//  - the U and D items of one row tile run in the same queue;
//  - a queue's row tiles of one minibatch are contiguous, and the queues'
//    tile counts over the layer differ by at most one.
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

struct Tile {
  int32_t p0, p1;
};

struct Case {
  int n_slots, ntu, ntd, per_queue;
  int64_t M;
  std::vector<Tile> tiles;
  std::vector<int32_t> mbs;   // [n_mb + 1]
  int n_mb() const { return (int)mbs.size() - 1; }
};

// tiles of the valid rows [0, nvalid) with the given expert segment sizes,
// as the schedule cuts them; R rows in all (R - nvalid invalid)
Case make_case(int64_t R, int64_t M, const std::vector<int>& seg, int bm, int n_slots, int ntu, int ntd,
               int per_queue) {
  Case k;
  k.M = M; k.n_slots = n_slots; k.ntu = ntu; k.ntd = ntd; k.per_queue = per_queue;
  const int n_mb = (int)((R + M - 1) / M);
  int64_t lo = 0;
  for (int c : seg) {
    const int64_t hi = lo + c;
    for (int64_t p = lo; p < hi;) {
      const int64_t end = std::min(hi, (p / M + 1) * M);
      for (int64_t q = p; q < end; q += bm) k.tiles.push_back({(int32_t)q, (int32_t)std::min<int64_t>(q + bm, end)});
      p = end;
    }
    lo = hi;
  }
  const int64_t nvalid = lo;
  k.mbs.assign(n_mb + 1, (int32_t)k.tiles.size());
  for (int m = 0; m < n_mb; ++m) {
    if ((int64_t)m * M >= nvalid) continue;
    int u = 0;
    while (u < (int)k.tiles.size() && k.tiles[u].p0 < (int64_t)m * M) ++u;
    k.mbs[m] = u;
  }
  return k;
}

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
  const int n_mb = k.n_mb();
  const int ntiles = k.mbs[n_mb];
  PersistPlan P{k.mbs.data(), n_mb, k.n_slots, k.ntu, k.ntd};
  std::unique_ptr<std::atomic<int>[]> tick(new std::atomic<int>[kPlanQueues]);
  std::unique_ptr<std::atomic<int>[]> udone(new std::atomic<int>[ntiles + 1]);
  std::unique_ptr<std::atomic<int>[]> dcnt(new std::atomic<int>[ntiles + 1]);
  std::unique_ptr<std::atomic<int>[]> retired(new std::atomic<int>[ntiles + 1]);
  std::unique_ptr<std::atomic<int>[]> ran_u(new std::atomic<int>[(size_t)ntiles * k.ntu + 1]);
  std::unique_ptr<std::atomic<int>[]> ran_d(new std::atomic<int>[(size_t)ntiles * k.ntd + 1]);
  std::unique_ptr<std::atomic<int>[]> queue_u(new std::atomic<int>[ntiles + 1]);
  std::unique_ptr<std::atomic<int>[]> queue_d(new std::atomic<int>[ntiles + 1]);
  for (int q = 0; q < kPlanQueues; ++q) tick[q] = 0;
  for (int t = 0; t < ntiles; ++t) { udone[t] = 0; dcnt[t] = 0; retired[t] = 0; queue_u[t] = -1; queue_d[t] = -1; }
  for (int64_t i = 0; i < (int64_t)ntiles * k.ntu; ++i) ran_u[i] = 0;
  for (int64_t i = 0; i < (int64_t)ntiles * k.ntd; ++i) ran_d[i] = 0;

  auto tile_mb = [&](int ti) {
    int m = 0;
    while (m < n_mb && k.mbs[m + 1] <= ti) ++m;
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
        if (it.m < 0 || it.m >= n_mb || it.ti < k.mbs[it.m] || it.ti >= k.mbs[it.m + 1]) {
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
          if (dcnt[it.ti].fetch_add(1, std::memory_order_acq_rel) == k.ntd - 1)
            retired[it.ti].store(1, std::memory_order_release);
        } else {
          if (it.col < 0 || it.col >= k.ntu) { fail("U column", it.col, k.ntu, 0); return; }
          if (it.m >= k.n_slots) {
            const int mp = it.m - k.n_slots;
            const int64_t o0 = k.tiles[it.ti].p0 - (int64_t)it.m * k.M, o1 = k.tiles[it.ti].p1 - (int64_t)it.m * k.M;
            // the plan's overlap range against brute force
            int u = plan_first_overlap(P, k.tiles.data(), k.M, mp, o0);
            const int u0 = u;
            for (; plan_overlaps(P, k.tiles.data(), k.M, mp, u, o1); ++u)
              if (!wait_for(retired[u], 1)) return;
            for (int v = k.mbs[mp]; v < k.mbs[mp + 1]; ++v) {
              const bool ov = k.tiles[v].p0 - mp * k.M < o1 && k.tiles[v].p1 - mp * k.M > o0;
              if (ov != (v >= u0 && v < u)) { fail("overlap range differs from brute force", it.ti, v, mp); return; }
              if (ov)
                for (int c = 0; c < k.ntd; ++c)
                  if (ran_d[(size_t)v * k.ntd + c].load() != 1) { fail("slot rows reused before their D items", it.ti, v, c); return; }
            }
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
  // balance: each queue's tiles of a minibatch are one contiguous chunk, and
  // the queues' tile counts over the layer differ by at most one
  std::vector<int> tiles_q(kPlanQueues, 0);
  for (int m = 0; m < n_mb; ++m) {
    std::vector<int> seen(kPlanQueues, 0);
    int prev = -1;
    for (int ti = k.mbs[m]; ti < k.mbs[m + 1]; ++ti) {
      const int q = queue_u[ti].load();
      if (q != prev) {
        if (seen[q]) { fail("chunk of a queue not contiguous", m, ti, q); return false; }
        seen[q] = 1;
        prev = q;
      }
      tiles_q[q] += 1;
    }
  }
  const auto mm = std::minmax_element(tiles_q.begin(), tiles_q.end());
  if (*mm.second - *mm.first > 1) { fail("queues unbalanced (tiles)", *mm.first, *mm.second, 0); return false; }
  return true;
}

}  // namespace

int main(int argc, char** argv) {
  const int ncases = argc > 1 ? std::atoi(argv[1]) : 200;
  std::mt19937_64 rng(12345);
  int done = 0;
  // fixed cases first: one minibatch and one slot with a partial group; one
  // slot reused by many minibatches; more slots than needed; 1-row experts
  // (many tiles per slot window); invalid rows at the end
  std::vector<Case> cases;
  cases.push_back(make_case(74, 128, {20, 14, 30, 6, 4}, 16, 1, 2, 1, 1));
  cases.push_back(make_case(600, 64, {100, 3, 200, 97, 200}, 16, 1, 3, 4, 2));
  cases.push_back(make_case(500, 100, {250, 250}, 8, 3, 1, 1, 1));
  cases.push_back(make_case(1024, 128, std::vector<int>(512, 2), 16, 2, 4, 3, 2));
  cases.push_back(make_case(700, 96, {300, 200, 50}, 32, 2, 2, 2, 1));
  for (int i = 0; i < ncases; ++i) {
    const int64_t M = 16 * (1 + (int64_t)(rng() % 16));
    const int n_mb = 1 + (int)(rng() % 12);
    const int64_t R = (n_mb - 1) * M + 1 + (int64_t)(rng() % M);
    const int E = 1 + (int)(rng() % 40);
    const int64_t nvalid = R - (rng() % 3 == 0 ? (int64_t)(rng() % (R / 4 + 1)) : 0);
    // random segment sizes summing to nvalid (some empty)
    std::vector<int64_t> cuts;
    for (int e = 0; e < E - 1; ++e) cuts.push_back((int64_t)(rng() % (nvalid + 1)));
    std::sort(cuts.begin(), cuts.end());
    std::vector<int> seg;
    int64_t prev = 0;
    for (int64_t c : cuts) { seg.push_back((int)(c - prev)); prev = c; }
    seg.push_back((int)(nvalid - prev));
    const int bm = 8 << (rng() % 3);
    const int n_slots = 1 + (int)(rng() % std::min(n_mb, 5));
    cases.push_back(make_case(R, M, seg, bm, n_slots, 1 + (int)(rng() % 9), 1 + (int)(rng() % 11),
                              1 + (int)(rng() % 3)));
  }
  for (size_t i = 0; i < cases.size(); ++i) {
    if (!run_case(cases[i], i + 1)) {
      const Case& k = cases[i];
      std::fprintf(stderr, "case %zu: n_mb %d n_slots %d ntu %d ntd %d per_queue %d tiles %d M %lld\n", i,
                   k.n_mb(), k.n_slots, k.ntu, k.ntd, k.per_queue, k.mbs[k.n_mb()], (long long)k.M);
      return 1;
    }
    ++done;
  }
  std::printf("ok %d\n", done);
  return 0;
}
