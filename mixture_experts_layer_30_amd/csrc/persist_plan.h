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
// D(m, ti, *) needs every U(m, ti, *). A row tile is retired once all its D
// items are done. U(m, ti, *) with m >= N_s needs the row tiles of minibatch
// m - N_s (the previous users of slot m mod N_s) whose slot rows overlap
// ti's to be retired: a few tiles, found by plan_first_overlap.
//
// Queues. There is one queue per XCD (workgroup wg serves queue wg mod 8).
// Minibatch m's nr row tiles are cut into 8 contiguous chunks, one per
// queue, of nr / 8 tiles, the nr mod 8 extra tiles going one each to the
// queues that follow the previous minibatch's extras (the chunks of queue
// rank j = (q - mb_tile_start[m]) mod 8; mb_tile_start[m] is the count of
// all tiles before m, so the extras are dealt round-robin over the whole
// layer and any two queues' tile counts differ by at most one). Both the U
// and the D items of a row tile are in the queue of its chunk: h never
// crosses an XCD. A chunk runs in groups of 4 tiles, each group column by
// column, so the 32 or so tiles in flight on an XCD share 4 row panels and 8
// column panels in its L2 (the row-tile order of the one-launch-per-stage
// kernels).
//
// Order. Queue q lists stage s = 0 .. n_mb as [U(s) items, D(s-1) items]
// (its own chunks only), or [D(s-1), U(s)] with a single ring slot. Every item
// then depends only on items earlier in this stage order: D(s-1) on U(s-1),
// one stage back; U(s) on D(s - N_s) items, which sit in stage s - N_s + 1 < s
// for N_s >= 2, and in stage s before the U block for N_s = 1. Workgroups take
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
  // queue q's chunk of minibatch m: tiles [mbs[m] + first, + count)
  MOK_HD void chunk(int m, int q, int& first, int& count) const {
    const int n = nr(m);
    if (n == 0) { first = 0; count = 0; return; }
    const int j = ((q - mbs[m]) % kPlanQueues + kPlanQueues) % kPlanQueues;
    const int base = n / kPlanQueues, extra = n % kPlanQueues;
    first = j * base + (j < extra ? j : extra);
    count = base + (j < extra ? 1 : 0);
  }
  MOK_HD int chunk_size(int m, int q) const {
    int f, c;
    chunk(m, q, f, c);
    return c;
  }
  MOK_HD bool down_first() const { return n_slots == 1; }
};

// A workgroup's position in its queue. Its tickets increase, so the stage
// only moves forward: walking the stages costs n_mb + 1 steps per workgroup
// over the whole launch.
struct PlanCursor {
  int s;          // stage
  int64_t base;   // items of the queue before stage s
};

MOK_HD void plan_cursor_init(PlanCursor& c) {
  c.s = 0;
  c.base = 0;
}

MOK_HD int64_t plan_stage_items(const PersistPlan& P, const PlanCursor& c, int q) {
  return (int64_t)P.ntd * P.chunk_size(c.s - 1, q) + (int64_t)P.ntu * P.chunk_size(c.s, q);
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
    ++c.s;
  }
  int64_t o = t - c.base;
  const int64_t nd = (int64_t)P.ntd * P.chunk_size(c.s - 1, q);
  const int64_t nu = (int64_t)P.ntu * P.chunk_size(c.s, q);
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
  int first, count;
  P.chunk(m, q, first, count);
  // groups of kPlanGroup tiles of the chunk in ascending order, kPlanGroup *
  // nc items per group (only the last group may be shorter)
  const int g = (int)(o / ((int64_t)kPlanGroup * nc));
  const int rem = count - kPlanGroup * g;
  const int hg = rem < kPlanGroup ? rem : kPlanGroup;
  const int jj = (int)(o - (int64_t)g * kPlanGroup * nc);
  it.down = down;
  it.m = m;
  it.col = jj / hg;
  it.ti = P.mbs[m] + first + kPlanGroup * g + jj % hg;
  return true;
}

// Completion counters in device memory (ints, zero at the launch).
constexpr int kPlanHeader = 16;   // [0, 8) ticket per queue, 8 stop flag,
                                  // 9 arrivals, 10 misplaced workgroups
struct PersistCounters {
  int* ticket;      // [kPlanQueues]
  int* stop;
  int* arrived;
  int* misplaced;
  int* udone;       // [max_tiles] U items done per row tile
  int* dcnt;        // [max_tiles] D items done per row tile
  int* retired;     // [max_tiles] 1 once the row tile's slot rows may be rewritten
};
MOK_HD int64_t persist_counter_count(int max_tiles) { return kPlanHeader + 3 * (int64_t)max_tiles; }
MOK_HD PersistCounters persist_counters(int* c, int max_tiles) {
  PersistCounters k;
  k.ticket = c;
  k.stop = c + kPlanQueues;
  k.arrived = c + kPlanQueues + 1;
  k.misplaced = c + kPlanQueues + 2;
  k.udone = c + kPlanHeader;
  k.dcnt = k.udone + max_tiles;
  k.retired = k.dcnt + max_tiles;
  return k;
}

// Slot-reuse dependencies. The row tiles of one minibatch are consecutive in
// the table and ascending and contiguous in the permuted row p; minibatch mp
// holds rows [mp*M, ...) at slot offsets p - mp*M. The tiles of minibatch mp
// whose slot rows overlap slot offsets [o0, o1) are u = plan_first_overlap(..,
// o0) onwards while plan_overlaps(.., u, o1).
template <class Tile>
MOK_HD int plan_first_overlap(const PersistPlan& P, const Tile* tiles, int64_t M, int mp, int64_t o0) {
  int l = P.mbs[mp], r = P.mbs[mp + 1];
  const int64_t lo = (int64_t)mp * M + o0;
  while (l < r) {                      // first tile with p1 > lo
    const int h = (l + r) >> 1;
    if (tiles[h].p1 > lo) r = h;
    else l = h + 1;
  }
  return l;
}
template <class Tile>
MOK_HD bool plan_overlaps(const PersistPlan& P, const Tile* tiles, int64_t M, int mp, int u, int64_t o1) {
  return u < P.mbs[mp + 1] && tiles[u].p0 < (int64_t)mp * M + o1;
}

}  // namespace mok
