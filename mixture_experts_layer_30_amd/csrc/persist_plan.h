// Work plan of the persistent forward driver.
//
// [MoK clip] Key points, bullets 3-5, How-to items 3-4 and the key chart's
// ring token buffer: routed rows flow through the expert FFN one minibatch
// at a time, minibatch m in ring slot m mod N_s, and a slot is refilled as
// soon as the work that read it has retired, the stages signalling each other
// through counters in device memory instead of kernel boundaries.
//
// Items. Minibatch m has nr(m) row tiles (mb_tile_start[m] .. [m+1]) and
//   U(m, ti, c)  gate/up + SwiGLU of row tile ti, h-column tile c < ntu,
//                writing the tile's h rows into slot m mod N_s;
//   D(m, ti, c)  down GEMM of row tile ti, output column tile c < ntd,
//                reading those h rows.
// D(m, ti, *) needs every U(m, ti, *); U(m, *, *) needs every D(m - N_s, *, *)
// (the previous user of its slot) when m >= N_s.
//
// Queues. There is one queue per XCD (workgroup wg serves queue wg mod 8).
// Each minibatch's row tiles are cut into groups of 4 consecutive tiles, and
// the groups of all minibatches, in order, are dealt to the queues round-robin
// (group g of minibatch m to queue (groups before m + g) mod 8), so the queues
// get equal work over the layer whatever the tile count of one minibatch. Both
// the U and the D items of a row tile are in the queue of its group: h never
// crosses an XCD. Within a group the items run column by column, so the 32 or
// so tiles in flight on an XCD share 4 row panels and 8 column panels in its
// L2 (the row-tile order of the one-launch-per-stage kernels).
//
// Order. Queue q lists stage s = 0 .. n_mb as [U(s) items, D(s-1) items]
// (its own groups only), or [D(s-1), U(s)] with a single ring slot. Every item
// then depends only on items earlier in this stage order: D(s-1) on U(s-1),
// one stage back; U(s) on D(s - N_s), which sits in stage s - N_s + 1 < s for
// N_s >= 2, and in stage s before the U block for N_s = 1. Workgroups take
// tickets from their queue in increasing order, so the earliest unfinished
// item in the stage order has finished dependencies, and it is either held by
// a running workgroup or is the next ticket of its queue, whose workgroups are
// all free to take it (any of them holding an earlier item would contradict
// its being the earliest). With the grid no larger than the resident
// workgroups, every wait therefore ends.
//
// Which workgroup runs an item never changes what it computes: the layer's
// results are bitwise those of one launch per stage.
//
// These functions are also compiled for the host, where a simulation with
// threads checks the plan and its waits.
#pragma once
#include <stdint.h>

#ifndef MOK_HD
#define MOK_HD __host__ __device__ __forceinline__
#endif

namespace mok {

constexpr int kPlanQueues = 8;   // one per XCD
constexpr int kPlanGroup = 4;    // row tiles per group

struct PlanItem {
  int down;   // 1: D item, 0: U item
  int m;      // minibatch
  int ti;     // row tile (index into the forward tile table)
  int col;    // column tile
};

struct PersistPlan {
  const int32_t* mbs;   // mb_tile_start [n_mb + 1]
  int n_mb, n_slots, ntu, ntd;

  MOK_HD int nr(int m) const { return (m < 0 || m >= n_mb) ? 0 : mbs[m + 1] - mbs[m]; }
  MOK_HD static int ngroups(int nr) { return (nr + kPlanGroup - 1) / kPlanGroup; }
  // first group of a minibatch (gb groups before it) that queue q takes
  MOK_HD static int first_group(int gb, int q) {
    return ((q - gb) % kPlanQueues + kPlanQueues) % kPlanQueues;
  }
  // row tiles of a minibatch (nr tiles, gb groups before it) in queue q
  MOK_HD static int rows_q(int nr, int gb, int q) {
    const int ng = ngroups(nr), g0 = first_group(gb, q);
    if (g0 >= ng) return 0;
    const int cnt = (ng - 1 - g0) / kPlanQueues + 1;
    const int last = g0 + kPlanQueues * (cnt - 1);
    return kPlanGroup * cnt - (last == ng - 1 ? kPlanGroup * ng - nr : 0);
  }
  MOK_HD bool down_first() const { return n_slots == 1; }
  // completed D items of minibatch m that free its slot
  MOK_HD int64_t down_items(int m) const { return (int64_t)ntd * nr(m); }
};

// A workgroup's position in its queue. Its tickets increase, so the stage
// only moves forward: walking the stages costs n_mb + 1 steps per workgroup
// over the whole launch.
struct PlanCursor {
  int s;          // stage
  int64_t base;   // items of the queue before stage s
  int gbu;        // groups of the minibatches before s (U block: minibatch s)
  int gbd;        // groups of the minibatches before s - 1 (D block: minibatch s - 1)
};

MOK_HD void plan_cursor_init(PlanCursor& c) {
  c.s = 0;
  c.base = 0;
  c.gbu = 0;
  c.gbd = 0;
}

MOK_HD int64_t plan_stage_items(const PersistPlan& P, const PlanCursor& c, int q) {
  return (int64_t)P.ntd * PersistPlan::rows_q(P.nr(c.s - 1), c.gbd, q) +
         (int64_t)P.ntu * PersistPlan::rows_q(P.nr(c.s), c.gbu, q);
}

// Item of ticket t of queue q (t not below any earlier ticket of this
// cursor); false once the queue is exhausted.
MOK_HD bool plan_item(const PersistPlan& P, PlanCursor& c, int q, int64_t t, PlanItem& it) {
  if (t < c.base) return false;
  for (;;) {
    if (c.s > P.n_mb) return false;
    const int64_t n = plan_stage_items(P, c, q);
    if (t < c.base + n) break;
    c.base += n;
    c.gbd = c.gbu;
    c.gbu += PersistPlan::ngroups(P.nr(c.s));
    ++c.s;
  }
  int64_t o = t - c.base;
  const int64_t nd = (int64_t)P.ntd * PersistPlan::rows_q(P.nr(c.s - 1), c.gbd, q);
  const int64_t nu = (int64_t)P.ntu * PersistPlan::rows_q(P.nr(c.s), c.gbu, q);
  int down;
  if (P.down_first()) {
    down = o < nd;
    if (!down) o -= nd;
  } else {
    down = o >= nu;
    if (down) o -= nu;
  }
  const int m = down ? c.s - 1 : c.s;
  const int nc = down ? P.ntd : P.ntu;
  const int gb = down ? c.gbd : c.gbu;
  const int nr = P.nr(m);
  // the queue's groups of minibatch m in ascending order, kPlanGroup * nc
  // items per group (only the minibatch's last group may be shorter, and it
  // comes last)
  const int j = (int)(o / ((int64_t)kPlanGroup * nc));
  const int g = PersistPlan::first_group(gb, q) + kPlanQueues * j;
  const int rem = nr - kPlanGroup * g;
  const int hg = rem < kPlanGroup ? rem : kPlanGroup;
  const int jj = (int)(o - (int64_t)j * kPlanGroup * nc);
  it.down = down;
  it.m = m;
  it.col = jj / hg;
  it.ti = P.mbs[m] + kPlanGroup * g + jj % hg;
  return true;
}

}  // namespace mok
