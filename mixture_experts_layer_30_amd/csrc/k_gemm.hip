// Grouped GEMMs of the expert SwiGLU FFN on gfx950 matrix cores.
//
// [MoK clip] Key points, bullet 5 and the key chart: the expert FFN with its
// SwiGLU is the compute stage between dispatch and combine; bullet 3: it runs
// as a grouped GEMM per expert over a minibatch of routed rows.
// [MoK card] "Core concepts": MXFP8 weights are pre-quantized; here both GEMM
// operands are MXFP8 (E4M3 + one E8M0 scale per 32 along K) on the scaled
// MFMA, accumulating in fp32.
//
// Each output element is owned by exactly one workgroup and summed over K in
// ascending order: results are bitwise reproducible (no split-K, no atomics).
// Tile machinery (LDS layout, loaders, MFMA stage) lives in gemm_core.h.
#include "gemm_core.h"
#include "mok_launch.h"
#include "persist_plan.h"
#include "rows_core.h"
#include "sched_core.h"

using namespace mok;

namespace {

using G256 = Geo<256, 256, 2, 2>;

// ================================================================== forward
// A forward tile: row tile ti, of minibatch m = tiles[ti].m (rows in ring
// slot m mod N_s).
struct FwdTile {
  mok_tile t;
  int nrows;
  int64_t slot_row0;     // ring row of the tile's first row
};

MOK_DEV void fwd_tile_at(const mok_fwd_args& a, int ti, FwdTile& ft) {
  ft.t = a.tiles[ti];
  ft.nrows = ft.t.p1 - ft.t.p0;
  const int m = ft.t.m;
  ft.slot_row0 = (int64_t)(m % a.n_slots) * a.M + (ft.t.p0 - (int64_t)m * a.M);
}

// gate/up GEMM + SwiGLU of one row tile x 128 h-columns. The A operand is the
// tile's x rows read in place through the token table (the dispatch gather
// fused into the operand copies). The B tile holds 32-row
// groups alternating Wg and Wu, so accumulator column blocks j = 2jj (gate) and
// 2jj + 1 (up) cover the same 32 h-columns.
template <bool F8>
MOK_DEV void gateup_tile(const mok_fwd_args& a, uint8_t* lds_raw, int ti, int ny) {
  using G = G256;
  Smem<G, F8>& sm = *reinterpret_cast<Smem<G, F8>*>(lds_raw);
  FwdTile ft;
  fwd_tile_at(a, ti, ft);
  const int64_t H = a.H, I = a.I;
  const int n0 = ny * (G::BN / 2);
  const int64_t xrow = F8 ? H : 2 * H;                       // bytes per X row
  const int64_t wrow = F8 ? H : 2 * H;                       // bytes per weight row
  const int64_t eoff = (int64_t)ft.t.e * I * wrow;
  const LoadKDG<G::BM> la(a.x, a.tok + ft.t.p0, xrow, ft.nrows);
  LoadKD<G::BN, RowsGateUp> lb{{(const uint8_t*)a.wg + eoff, (const uint8_t*)a.wu + eoff, wrow, n0, (int)I}};
  Acc<G::FM, G::FN> acc;
  if constexpr (F8) {
    const int64_t sx = H / 32;
    const LoadScalesDG<G::BM> lsa(a.xs, a.tok + ft.t.p0, sx, ft.nrows);
    const int64_t se = (int64_t)ft.t.e * I * sx;
    LoadScalesD<G::BN, RowsGateUp> lsb{{a.sg + se, a.su + se, sx, n0, (int)I}};
    mainloop_rows<false, G, true>(sm, la, lb, lsa, lsb, (int)(H / 64), ft.nrows, acc);
  } else {
    NoScales ns;
    mainloop_rows<false, G, false>(sm, la, lb, ns, ns, (int)(H / 32), ft.nrows, acc);
  }

  // SwiGLU on the accumulators; h (and a, b) staged in LDS for row-wise stores.
  constexpr int HW = G::BN / 2;                               // 128 h columns
  uint8_t* st = lds_raw;
  if constexpr (!F8) {
    // h = silu(a) * b per element from an fp32 half-tile in LDS. Tile column
    // (c/32)*64 + c%32 holds gate column c of the tile, +32 its up column.
    using HS = HalfF32<G>;
    bf16_t* hs = reinterpret_cast<bf16_t*>(a.ring_h) + ft.slot_row0 * I + n0;
    bf16_t* abp = a.ab ? a.ab + (int64_t)ft.t.p0 * 2 * I + n0 : nullptr;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (half) barrier_lds_only();
      HS::put(st, acc, half);
      barrier_lds_only();
      const int rows = min(128, ft.nrows - 128 * half);
      for (int idx = threadIdx.x; idx < 128 * (HW / 8); idx += kThreads) {
        const int r = idx / (HW / 8), c = (idx % (HW / 8)) * 8;
        if (r >= rows || n0 + c >= I) continue;
        float av[8], bv[8], h[8];
        const int tc = (c >> 5) * 64 + (c & 31);
        HS::get8(st, r, tc, av);
        HS::get8(st, r, tc + 32, bv);
#pragma unroll
        for (int u = 0; u < 8; ++u) h[u] = av[u] * sigmoidf_(av[u]) * bv[u];
        const int64_t rr = 128 * half + r;
        store_nt(hs + rr * I + c, pack_bf16x8(h));
        if (abp) {
          store_nt(abp + rr * 2 * I + c, pack_bf16x8(av));
          store_nt(abp + rr * 2 * I + I + c, pack_bf16x8(bv));
        }
      }
    }
  } else {
    // MXFP8 h: one E8M0 scale per 32 h-columns of a row. Each thread takes one
    // 32-column block of one row from the fp32 half-tile: amax, scale byte,
    // 32 E4M3 codes (two 16-byte stores) and the scale. A store instruction
    // here covers pieces of 16 rows, so these stores stay cached (the L2
    // merges them into whole lines; nontemporal they would leave as partial
    // lines, measured 28% slower for the kernel).
    using HS = HalfF32<G>;
    uint8_t* hq = a.ring_h + ft.slot_row0 * I + n0;
    uint8_t* hsc = a.ring_hs + ft.slot_row0 * (I / 32) + n0 / 32;
    bf16_t* abp = a.ab ? a.ab + (int64_t)ft.t.p0 * 2 * I + n0 : nullptr;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (half) barrier_lds_only();
      HS::put(st, acc, half);
      barrier_lds_only();
      const int rows = min(128, ft.nrows - 128 * half);
      for (int idx = threadIdx.x; idx < 128 * (HW / 32); idx += kThreads) {
        const int r = idx / (HW / 32), blk = idx % (HW / 32);
        if (r >= rows || n0 + blk * 32 >= I) continue;
        float h[32];
        float amax = 0.f;
#pragma unroll
        for (int u = 0; u < 32; u += 8) {
          float av[8], bv[8];
          HS::get8(st, r, blk * 64 + u, av);
          HS::get8(st, r, blk * 64 + 32 + u, bv);
#pragma unroll
          for (int v = 0; v < 8; ++v) {
            h[u + v] = av[v] * sigmoidf_(av[v]) * bv[v];
            amax = fmaxf(amax, fabsf(h[u + v]));
          }
        }
        const int sc = mx_scale_byte(amax);
        const float inv = mx_inv_scale(sc);
        uint32_t w[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          w[u] = e4m3_pack4(h[4 * u] * inv, h[4 * u + 1] * inv, h[4 * u + 2] * inv,
                          h[4 * u + 3] * inv);
        const int64_t rr = 128 * half + r;
        uint4* d = reinterpret_cast<uint4*>(hq + rr * I + blk * 32);
        d[0] = make_uint4(w[0], w[1], w[2], w[3]);
        d[1] = make_uint4(w[4], w[5], w[6], w[7]);
        hsc[rr * (I / 32) + blk] = (uint8_t)sc;
      }
      // a, b saved for the backward: one 8-column chunk per thread, 16 threads
      // per row, so each store instruction writes whole row segments and can
      // carry the nontemporal hint
      if (abp) {
        for (int idx = threadIdx.x; idx < 128 * (HW / 8); idx += kThreads) {
          const int r = idx / (HW / 8), c = (idx % (HW / 8)) * 8;
          if (r >= rows || n0 + c >= I) continue;
          float av[8], bv[8];
          const int tc = (c >> 5) * 64 + (c & 31);
          HS::get8(st, r, tc, av);
          HS::get8(st, r, tc + 32, bv);
          const int64_t rr = 128 * half + r;
          store_nt(abp + rr * 2 * I + c, pack_bf16x8(av));
          store_nt(abp + rr * 2 * I + I + c, pack_bf16x8(bv));
        }
      }
    }
  }
}

// Kernels whose tile ends in a plain bf16 row store can run the main loop with
// the operands exchanged and store the transposed accumulators directly
// (store_tile_bf16_t); chosen per kernel family from measurements.
constexpr bool kTrDown = true, kTrDx = true, kTrDw = true;

// (na: valid rows of la, the tile's row operand)
template <bool TR, class G, bool F8, class LA, class LB, class SA, class SB>
MOK_DEV void mainloop_x(Smem<G, F8>& sm, const LA& la, const LB& lb, const SA& sa, const SB& sb, int nk,
                        int na, Acc<G::FM, G::FN>& acc) {
  if constexpr (TR) mainloop_rows<true, G, F8>(sm, lb, la, sb, sa, nk, na, acc);
  else mainloop_rows<false, G, F8>(sm, la, lb, sa, sb, nk, na, acc);
}

template <bool TR, class G, class Dst>
MOK_DEV void store_bf16_x(uint8_t* lds, const Acc<G::FM, G::FN>& acc, int nrows, int ncols, Dst dst) {
  if constexpr (TR) store_tile_bf16_t<G>(lds, acc, nrows, ncols, dst);
  else store_tile_bf16<G>(lds, acc, nrows, ncols, dst);
}

// down GEMM of one row tile x 256 output columns; each row is pushed to its
// flat position perm[p] of obuf (unique destinations, no atomics).
template <bool F8>
MOK_DEV void down_tile(const mok_fwd_args& a, uint8_t* lds_raw, int ti, int ny) {
  using G = G256;
  Smem<G, F8>& sm = *reinterpret_cast<Smem<G, F8>*>(lds_raw);
  FwdTile ft;
  fwd_tile_at(a, ti, ft);
  const int64_t H = a.H, I = a.I;
  const int n0 = ny * G::BN;
  const int64_t hrow = F8 ? I : 2 * I;
  LoadKD<G::BM, RowsStrided> la{{a.ring_h + ft.slot_row0 * hrow, hrow, ft.nrows}};
  LoadKD<G::BN, RowsStrided> lb{{(const uint8_t*)a.wd + ((int64_t)ft.t.e * H + n0) * hrow, hrow,
                                (int)(H - n0)}};
  Acc<G::FM, G::FN> acc;
  if constexpr (F8) {
    const int64_t sx = I / 32;
    LoadScalesD<G::BM, RowsStrided> lsa{{a.ring_hs + ft.slot_row0 * sx, sx, ft.nrows}};
    LoadScalesD<G::BN, RowsStrided> lsb{{a.sd + ((int64_t)ft.t.e * H + n0) * sx, sx, (int)(H - n0)}};
    mainloop_x<kTrDown, G, true>(sm, la, lb, lsa, lsb, (int)(I / 64), ft.nrows, acc);
  } else {
    NoScales ns;
    mainloop_x<kTrDown, G, false>(sm, la, lb, ns, ns, (int)(I / 32), ft.nrows, acc);
  }
  // destination rows, staged in the top 1 KiB of LDS once every wavefront
  // has left the main loop
  int* rows = tile_rows<Smem<G, F8>>(lds_raw);
  barrier_lds_only();
  for (int r = threadIdx.x; r < G::BM; r += kThreads) rows[r] = r < ft.nrows ? a.perm[ft.t.p0 + r] : 0;
  bf16_t* ob = a.obuf + n0;
  store_bf16_x<kTrDown, G>(lds_raw, acc, ft.nrows, (int)(H - n0),
                           [&](int r) { return ob + (int64_t)rows[r] * H; });
}

// One launch covers the tiles of minibatches [m0, m1). Launch grids are 1-D
// upper bounds; the tile count is read on the device and the tile order is
// XCD-aware (xcd_swizzle: 4 x 8 blocks of row x column tiles per XCD).
template <bool F8>
__global__ __launch_bounds__(kThreads, 1) void gateup_kernel(mok_fwd_args a, int m0, int m1, int ncol) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[tile_lds_bytes<Smem<G256, F8>>()];
  const int t0 = a.mb_tile_start[m0];
  int row, col;
  if (!xcd_swizzle(a.mb_tile_start[m1] - t0, ncol, row, col)) return;
  gateup_tile<F8>(a, lds_raw, t0 + row, col);
}

template <bool F8>
__global__ __launch_bounds__(kThreads, 1) void down_kernel(mok_fwd_args a, int m0, int m1, int ncol) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[tile_lds_bytes<Smem<G256, F8>>()];
  const int t0 = a.mb_tile_start[m0];
  int row, col;
  if (!xcd_swizzle(a.mb_tile_start[m1] - t0, ncol, row, col)) return;
  down_tile<F8>(a, lds_raw, t0 + row, col);
}

// ================================================================== persistent driver
// One launch runs the forward's gate/up and down tiles (gateup_tile and
// down_tile, unchanged) as items taken from per-XCD queues in the order of
// persist_plan.h, which also states why every wait ends. Completion travels
// through counters per row tile: a U item adds one to udone[tile], a D item
// to dcnt[tile], and the last D item of a tile marks it retired. A D item
// waits for all U items of its row tile; a U item of minibatch m >= N_s
// waits until every row tile of minibatch m - N_s whose ring rows overlap
// its own is retired (the previous users of those slot rows).
//
// Bounded by construction: each workgroup's loop ends when its queue is
// exhausted (tickets only grow), a wait gives up after ps.spin_limit ticks
// of the real-time counter, and a give-up (or a tile table that fails the
// checks below) sets ps.give_up_bit in the status word and a stop flag that
// ends every workgroup's loop at its next item. The outputs are then
// incomplete; the status word says so.
//
// Visibility. Each XCD has its own L2; the L2s are not coherent with each
// other. The U and D items of a row tile share a queue, and queue q is
// served by the workgroups that run on XCD q, so h goes from its writer to
// its readers through one L2: the writer waits until its stores are in the
// L2 before its counter moves, and the reader invalidates its CU's L1 after
// the wait. A D item's obuf rows are read only after the item loop, so it
// signals without waiting for its stores. The hazard across XCDs is the
// reuse of ring rows: dirty h lines of minibatch m left in one XCD's L2
// must reach memory before another XCD writes the same rows for minibatch
// m + N_s, so the last D item of a row tile writes its XCD's L2 back
// (agent-scope release) before it marks the tile retired, and the reuse
// waits on retired tiles. At the start every
// workgroup checks the XCD it runs on (HW_REG_XCC_ID) against its queue and
// the grid agrees on the result (one arrival counter); if any workgroup is
// elsewhere, every signal releases and every wait acquires at agent scope.

MOK_DEV uint32_t xcc_id() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 0xf;
}

// thread 0 spins until *c >= target (false: stopped or gave up)
MOK_DEV bool persist_spin(const int* c, int target, int* stop, const mok_persist_args& ps) {
  if (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) return true;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
    if (__hip_atomic_load(stop, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return false;
    if (__builtin_amdgcn_s_memrealtime() - t0 > ps.spin_limit) {
      __hip_atomic_fetch_or(ps.status, ps.give_up_bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(stop, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  return true;
}

// the workgroup learns thread 0's verdict
MOK_DEV bool wg_agree(bool ok, int* s_ok) {
  if (threadIdx.x == 0) *s_ok = ok ? 1 : 0;
  __syncthreads();
  return *s_ok != 0;
}

// this thread's stores are in its XCD's L2 (all of them, with `agent`: in
// memory) once the workgroup passes the barrier
MOK_DEV void persist_release(bool agent) {
  if (agent) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// after a wait: the CU's L1 holds no line older than the wait (`agent`: nor
// the L2)
MOK_DEV void persist_acquire(bool agent) {
  if (agent) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  else asm volatile("buffer_inv sc0" ::: "memory");
}

// The tiles run as calls: inlined into the item loop, the lane-dependent
// address arithmetic of both tile kinds is hoisted out of the loop and kept
// live across it, and the registers spill inside the main loops. A call keeps
// each tile's code as in its one-stage kernel. The kernel passes its kernarg
// segment pointer (valid only in the kernel itself: the call convention does
// not hand it to callees, where the builtin yields a null pointer) and the
// callee reads the forward arguments there (they come first) with scalar
// loads; the LDS goes in as an LDS pointer. Neither goes through private
// memory.
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef const __attribute__((address_space(4))) mok_fwd_args* fwd_args_cptr;

MOK_DEV const mok_fwd_args& persist_fwd_args(fwd_args_cptr ap) {
  // the pointer arrives in vector registers; it is the same in every lane
  const uint64_t v = (uint64_t)ap;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return *(const mok_fwd_args*)(fwd_args_cptr)(((uint64_t)hi << 32) | lo);
}

template <bool F8>
__device__ __noinline__ void persist_gateup(fwd_args_cptr ap, lds_u8* lds, int ti, int col) {
  gateup_tile<F8>(persist_fwd_args(ap), (uint8_t*)lds, ti, col);
}

template <bool F8>
__device__ __noinline__ void persist_down(fwd_args_cptr ap, lds_u8* lds, int ti, int col) {
  down_tile<F8>(persist_fwd_args(ap), (uint8_t*)lds, ti, col);
}

// The tile table (written by the schedule) must fit the bounds the counters
// and the host's item count were sized for; every workgroup reads the same
// table and reaches the same verdict. On failure the give-up bit and the
// stop flag are set.
MOK_DEV bool persist_table_valid(const mok_fwd_args& a, const PersistPlan& P, const mok_persist_args& ps,
                                 const PersistCounters& C) {
  bool valid = P.mbs[0] == 0 && P.mbs[a.n_mb] <= ps.max_tiles;
  for (int m = 0; m < a.n_mb && valid; ++m) {
    const int n = P.nr(m);
    valid = n >= 0 && n <= ps.max_mb_tiles;
  }
  if (!valid && threadIdx.x == 0) {
    __hip_atomic_fetch_or(ps.status, ps.give_up_bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(C.stop, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return valid;
}

MOK_DEV PersistPlan persist_plan(const mok_fwd_args& a) {
  PersistPlan P;
  P.mbs = a.mb_tile_start;
  P.n_mb = a.n_mb;
  P.n_slots = a.n_slots;
  P.ntu = (int)((a.I + G256::BN / 2 - 1) / (G256::BN / 2));
  P.ntd = (int)((a.H + G256::BN - 1) / G256::BN);
  return P;
}

// Thread 0 of every workgroup: records whether it runs on the XCD of its
// queue q (misplaced flag; set regardless with force_agent) and arrives at
// counter `arrived`.
MOK_DEV void persist_arrive(const PersistCounters& C, int* arrived, int q, bool force_agent) {
  if (force_agent || xcc_id() != (uint32_t)q)
    __hip_atomic_fetch_or(C.misplaced, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_fetch_add(arrived, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// The item loop of the persistent forward (queue q; s_ticket, s_ok: LDS
// words of the workgroup). False if a wait gave up or the launch stopped.
template <bool F8>
MOK_DEV bool persist_item_loop(const mok_fwd_args& a, fwd_args_cptr ap, const mok_persist_args& ps,
                               const PersistCounters& C, const PersistPlan& P, int q, bool agent,
                               uint8_t* lds_raw, int* s_ticket, int* s_ok) {
  PlanCursor cur;
  plan_cursor_init(cur);
  for (;;) {
    if (threadIdx.x == 0) {
      int t = -1;
      if (__hip_atomic_load(C.stop, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0)
        t = __hip_atomic_fetch_add(C.ticket + q, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *s_ticket = t;
    }
    __syncthreads();
    const int t = *s_ticket;
    __syncthreads();                                   // s_ticket is free for the next item
    if (t < 0) return false;
    PlanItem it;
    if (!plan_item(P, cur, q, t, it)) return true;
    if (it.down) {
      bool w = true;
      if (threadIdx.x == 0) w = persist_spin(C.udone + it.ti, P.ntu, C.stop, ps);
      if (!wg_agree(w, s_ok)) return false;
      persist_acquire(agent);
      persist_down<F8>(ap, (lds_u8*)lds_raw, it.ti, it.col);
      // the obuf stores need no agent-scope release (they are read after the
      // item loop only); the tile's h reads are complete (its main loop
      // consumed every copy)
      __syncthreads();
      if (threadIdx.x == 0) {
        const int done = __hip_atomic_fetch_add(C.dcnt + it.ti, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (done == P.ntd - 1) {
          // the tile's last reader: its XCD's dirty h lines go to memory
          // before another XCD may write these ring rows
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
          __builtin_amdgcn_s_waitcnt(0);               // the write-back finished
          __hip_atomic_store(C.retired + it.ti, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    } else {
      bool w = true;
      if (it.m >= a.n_slots && threadIdx.x == 0) {
        const mok_tile cur_t = a.tiles[it.ti];
        const int mp = it.m - a.n_slots;
        const int64_t o0 = cur_t.p0 - (int64_t)it.m * a.M, o1 = cur_t.p1 - (int64_t)it.m * a.M;
        int u = plan_first_overlap(P, a.tiles, a.M, mp, o0);
        for (; w && plan_overlaps(P, a.tiles, a.M, mp, u, o1); ++u)
          w = persist_spin(C.retired + u, 1, C.stop, ps);
      }
      if (!wg_agree(w, s_ok)) return false;
      persist_gateup<F8>(ap, (lds_u8*)lds_raw, it.ti, it.col);
      persist_release(agent);
      if (threadIdx.x == 0)
        __hip_atomic_fetch_add(C.udone + it.ti, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <bool F8>
__global__ __launch_bounds__(kThreads, 1) void fwd_persistent_kernel(mok_fwd_args a, mok_persist_args ps) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[tile_lds_bytes<Smem<G256, F8>>()];
  __shared__ int s_ticket, s_ok, s_agent;
  const int q = (int)blockIdx.x % kPlanQueues;
  const PersistPlan P = persist_plan(a);
  // the kernel's own arguments, for the tile calls: `a` is the first one
  const fwd_args_cptr ap = (fwd_args_cptr)__builtin_amdgcn_kernarg_segment_ptr();
  const PersistCounters C = persist_counters(ps.ctr, ps.max_tiles);
  if (!persist_table_valid(a, P, ps, C)) return;

  // placement: every workgroup on the XCD of its queue, or agent-scope sync
  if (threadIdx.x == 0) {
    persist_arrive(C, C.arrived, q, ps.force_agent != 0);
    int agent_sync = -1;   // -1: the grid did not gather (stop)
    if (persist_spin(C.arrived, (int)gridDim.x, C.stop, ps)) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      agent_sync = __hip_atomic_load(C.misplaced, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
    }
    s_agent = agent_sync;
  }
  __syncthreads();
  if (s_agent < 0) return;
  persist_item_loop<F8>(a, ap, ps, C, P, q, s_agent != 0, lds_raw, &s_ticket, &s_ok);
}

// ================================================================== single-launch layer
// [MoK card] "What it is": the whole forward in one kernel; [MoK clip] Key
// points 4-5 and the key chart: schedule generation on the GPU, then the
// dispatch -> expert FFN -> combine pipeline, stages waking each other through
// counters. One resident grid (a workgroup per CU) runs, separated by grid-
// wide counter waits:
//   1. (MXFP8) x quantized along H, and the schedule's chunk histograms;
//   2. workgroup 0: the schedule scan (totals, offsets, chunk bases, tiles);
//   3. the schedule scatter (perm, dest, tok);
//   4. the gate/up and down items of the persistent forward (the gather is
//      the gate/up tiles' operand copies through tok);
//   5. the weighted combine of the obuf rows into y.
// Each step's results are published at agent scope (every workgroup writes
// its XCD's L2 back before it arrives, every waiter invalidates after the
// wait). The schedule written here is the one mok_build_schedule writes (the
// same steps, sched_core.h), so the backward can use it; y and fwd_ctx are
// bitwise those of mok_build_schedule + mok_forward.
template <bool F8>
__global__ __launch_bounds__(kThreads, 1) void layer_fwd_kernel(mok_fwd_args a, mok_persist_args ps, mok_layer_args L) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[tile_lds_bytes<Smem<G256, F8>>()];
  __shared__ int s_ticket, s_ok, s_agent;
  static_assert(sizeof(mok_sched::ChunkLds) <= sizeof(lds_raw), "chunk LDS");
  static_assert(sizeof(mok_sched::ScanLds<kThreads>) <= sizeof(lds_raw), "scan LDS");
  const int q = (int)blockIdx.x % kPlanQueues;
  const int G = (int)gridDim.x, g = (int)blockIdx.x;
  const fwd_args_cptr ap = (fwd_args_cptr)__builtin_amdgcn_kernarg_segment_ptr();
  const PersistCounters C = persist_counters(ps.ctr, ps.max_tiles);
  int* const step = C.misplaced + 1;                 // [0] hist done, [1] scan done, [2] scatter done, [3] GEMMs done

  // 1. MXFP8 x, chunk histograms
  if constexpr (F8) {
    constexpr int NB = 4;
    const int64_t nblk = a.T * (a.H / 32), S = (int64_t)G * kThreads;
    for (int64_t i = (int64_t)g * kThreads + threadIdx.x; i < nblk; i += NB * S)
      mx_quantize_batch<NB>(L.x, a.H, i, S, nblk, const_cast<uint8_t*>(a.x), const_cast<uint8_t*>(a.xs));
  }
  for (int c = g; c < L.nchunks; c += G) {
    mok_sched::sched_hist_chunk(L.ids, L.R, a.E, L.chunk, c, L.bh, *reinterpret_cast<mok_sched::ChunkLds*>(lds_raw));
    __syncthreads();
  }
  persist_release(true);
  if (threadIdx.x == 0) persist_arrive(C, step + 0, q, ps.force_agent != 0);

  // 2. the scan
  if (g == 0) {
    bool ok = true;
    if (threadIdx.x == 0) ok = persist_spin(step + 0, G, C.stop, ps);
    if (!wg_agree(ok, &s_ok)) return;
    persist_acquire(true);
    // (a give-up of another workgroup may already be in the status word,
    // which the host cleared before the launch)
    mok_sched::sched_scan<kThreads>(L.s, L.R, a.E, L.nchunks, L.bh, a.M, L.bm_f, L.bm_b, a.n_mb, L.max_f,
                                    L.max_b, *reinterpret_cast<mok_sched::ScanLds<kThreads>*>(lds_raw),
                                    ps.give_up_bit);
    persist_release(true);
    if (threadIdx.x == 0) __hip_atomic_store(step + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // 3. the scatter
  {
    bool ok = true;
    if (threadIdx.x == 0) ok = persist_spin(step + 1, 1, C.stop, ps);
    if (!wg_agree(ok, &s_ok)) return;
    persist_acquire(true);
  }
  for (int c = g; c < L.nchunks; c += G) {
    mok_sched::sched_scatter_chunk(L.ids, L.s, L.R, a.E, a.topk, L.chunk, c, L.bh,
                                   *reinterpret_cast<mok_sched::ChunkLds*>(lds_raw));
    __syncthreads();
  }
  persist_release(true);
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(step + 2, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    int agent_sync = -1;
    if (persist_spin(step + 2, G, C.stop, ps)) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      agent_sync = __hip_atomic_load(C.misplaced, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
    }
    s_agent = agent_sync;
  }
  __syncthreads();
  if (s_agent < 0) return;
  persist_acquire(true);

  // 4. the expert FFN
  const PersistPlan P = persist_plan(a);
  if (!persist_table_valid(a, P, ps, C)) return;
  if (!persist_item_loop<F8>(a, ap, ps, C, P, q, s_agent != 0, lds_raw, &s_ticket, &s_ok)) return;
  persist_release(true);                               // this XCD's obuf rows, in memory
  if (threadIdx.x == 0) __hip_atomic_fetch_add(step + 3, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);

  // 5. the combine
  {
    bool ok = true;
    if (threadIdx.x == 0) ok = persist_spin(step + 3, G, C.stop, ps);
    if (!wg_agree(ok, &s_ok)) return;
    persist_acquire(true);
  }
  // one token per wavefront at a time
  const int nvalid = L.s.offsets[a.E];
  const int nw = kThreads / 64;
  for (int64_t t = (int64_t)g * nw + wave_id(); t < a.T; t += (int64_t)G * nw)
    combine_token_wave<4>(a.obuf, L.topk_w, L.s.dest, nvalid, t, a.topk, a.H, L.y);
}

// ================================================================== backward
// Backward row-tile kernels: 1-D grid over (row tile, column tile) in the
// XCD-aware order of xcd_swizzle; ny receives the column tile.
MOK_DEV bool bwd_tile(const mok_bwd_args& a, int ncol, mok_tile& t, int& ny) {
  int row;
  if (!xcd_swizzle(*a.n_tiles, ncol, row, ny)) return false;
  t = a.tiles[row];
  return true;
}

// dh = dO . Wd[e] (K = H), then the SwiGLU backward from the saved a, b:
// dA = dh*b*s*(1 + a*(1-s)), dB = dh*a*s, h = a*s*b with s = sigmoid(a).
// dO row p is w_p * dy[tok[p]] (w_p = topk_w at the row's flat position): the
// A operand is the dy rows read in place and w_p scales the fp32 dh row in
// the epilogue. h is stored as w_p * h, the operand that takes w_p's place in
// dWd = sum_p dO[p]^T h[p] = sum_p dy[tok[p]]^T (w_p h[p]).
__global__ __launch_bounds__(kThreads, 1) void bwd_dh_kernel(mok_bwd_args a, int ncol) {
  using G = G256;
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[tile_lds_bytes<Smem<G, false>>()];
  Smem<G, false>& sm = *reinterpret_cast<Smem<G, false>*>(lds_raw);
  mok_tile t;
  int ny;
  if (!bwd_tile(a, ncol, t, ny)) return;
  const int nrows = t.p1 - t.p0;
  const int64_t H = a.H, I = a.I;
  const int n0 = ny * G::BN;
  const LoadKDG<G::BM> la(reinterpret_cast<const uint8_t*>(a.dy), a.tok + t.p0, 2 * H, nrows);
  const LoadKO<G::BN> lb{reinterpret_cast<const uint8_t*>(a.wd + (int64_t)t.e * H * I + n0),
                        reinterpret_cast<const uint8_t*>(a.wd + (int64_t)t.e * H * I + n0), 0x7FFFFFFF,
                        2 * I, (int)H, (int)min<int64_t>(G::BN, I - n0)};
  NoScales ns;
  Acc<G::FM, G::FN> acc;
  mainloop_rows<false, G, false>(sm, la, lb, ns, ns, (int)(H / 32), nrows, acc);
  // Epilogue: dA, dB and h per element from an fp32 half-tile of dh in LDS,
  // the saved a, b and w_p (16-byte loads and stores along the rows). A
  // thread keeps one 8-column chunk c and takes rows r0, r0 + 8, ..., r0 +
  // 120 of each half, in two groups of 8 rows whose a, b loads are all
  // issued before the group's stores (the first group's before the staging):
  // a wait for a load issued after stores also waits for those stores, so
  // loads interleaved with the stores would serialise every row. The
  // barriers wait for LDS operations only, so the loads stay in flight
  // through the staging. w_p per permuted row comes from wperm (loaded with
  // the first group) into the top 1 KiB of LDS, outside the fp32 half-tile.
  using HS = HalfF32<G>;
  float* wrow = reinterpret_cast<float*>(tile_rows<Smem<G, false>>(lds_raw));
  const int tid = (int)threadIdx.x;                    // (kThreads == G::BM: one row each)
  float wmine = a.wperm[t.p0 + min(tid, nrows - 1)];
  wmine = tid < nrows ? wmine : 0.f;
  const int c = (tid % (G::BN / 8)) * 8, r0 = tid / (G::BN / 8);
  const bool colok = n0 + c < I;
  const bf16_t* abt = a.ab + (int64_t)t.p0 * 2 * I + n0 + c;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int rows = min(128, nrows - 128 * half);
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
      uint4 va[8], vb[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int r = r0 + 64 * grp + 8 * u;
        if (colok && r < rows) {
          const bf16_t* q = abt + (int64_t)(128 * half + r) * 2 * I;
          va[u] = *reinterpret_cast<const uint4*>(q);
          vb[u] = *reinterpret_cast<const uint4*>(q + I);
        }
      }
      if (grp == 0) {
        barrier_lds_only();               // the main loop's (half 1: half 0's) LDS reads are done
        HS::put(lds_raw, acc, half);
        if (half == 0) wrow[tid] = wmine;
        barrier_lds_only();
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int r = r0 + 64 * grp + 8 * u;
        if (!colok || r >= rows) continue;
        const int64_t p = t.p0 + 128 * half + r;
        const float wp = wrow[128 * half + r];
        float dh[8], av[8], bv[8], da[8], db[8], h[8];
        HS::get8(lds_raw, r, c, dh);
        unpack_bf16x8(va[u], av);
        unpack_bf16x8(vb[u], bv);
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const float sg = sigmoidf_(av[v]);
          const float d = wp * dh[v];
          da[v] = d * bv[v] * sg * (1.0f + av[v] * (1.0f - sg));
          db[v] = d * av[v] * sg;
          h[v] = wp * (av[v] * sg * bv[v]);
        }
        store_nt(a.dab + p * 2 * I + n0 + c, pack_bf16x8(da));
        store_nt(a.dab + p * 2 * I + I + n0 + c, pack_bf16x8(db));
        store_nt(a.hb + p * I + n0 + c, pack_bf16x8(h));
      }
    }
  }
}

// dX rows = [dA | dB] . [Wg[e]; Wu[e]] (K = 2I); row p goes to flat row perm[p].
__global__ __launch_bounds__(kThreads, 1) void bwd_dx_kernel(mok_bwd_args a, int ncol) {
  using G = G256;
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[tile_lds_bytes<Smem<G, false>>()];
  Smem<G, false>& sm = *reinterpret_cast<Smem<G, false>*>(lds_raw);
  mok_tile t;
  int ny;
  if (!bwd_tile(a, ncol, t, ny)) return;
  const int nrows = t.p1 - t.p0;
  const int64_t H = a.H, I = a.I;
  const int n0 = ny * G::BN;
  LoadKD<G::BM, RowsStrided> la{{reinterpret_cast<const uint8_t*>(a.dab + (int64_t)t.p0 * 2 * I), 4 * I, nrows}};
  // row k of [Wg[e]; Wu[e]]: Wg row k for k < I, Wu row k - I beyond
  const LoadKO<G::BN> lb{reinterpret_cast<const uint8_t*>(a.wg + (int64_t)t.e * I * H + n0),
                        reinterpret_cast<const uint8_t*>(a.wu + (int64_t)t.e * I * H + n0), (int)I,
                        2 * H, (int)(2 * I), (int)min<int64_t>(G::BN, H - n0)};
  NoScales ns;
  Acc<G::FM, G::FN> acc;
  mainloop_x<kTrDx, G, false>(sm, la, lb, ns, ns, (int)(2 * I / 32), nrows, acc);
  int* rows = tile_rows<Smem<G, false>>(lds_raw);
  barrier_lds_only();
  for (int r = threadIdx.x; r < G::BM; r += kThreads) rows[r] = r < nrows ? a.perm[t.p0 + r] : 0;
  bf16_t* d = a.dxrows + n0;
  store_bf16_x<kTrDx, G>(lds_raw, acc, nrows, (int)(H - n0),
                         [&](int r) { return d + (int64_t)rows[r] * H; });
}

// Weight gradients out[m][n] = sum over the expert's rows p (ascending) of
// A[p][m] * B[p][n]; both operands K-outer (one of them gathered: its k-row p
// is a token row of dy or x, read in place through the token table).
template <class LA, class LB>
MOK_DEV void dw_tile(uint8_t* lds_raw, const LA& la, int mlimit, const LB& lb, int nlimit, int K,
                     bf16_t* out, int64_t ldo) {
  using G = G256;
  Smem<G, false>& sm = *reinterpret_cast<Smem<G, false>*>(lds_raw);
  NoScales ns;
  Acc<G::FM, G::FN> acc;
  mainloop_x<kTrDw, G, false>(sm, la, lb, ns, ns, (K + 31) / 32, mlimit, acc);
  store_bf16_x<kTrDw, G>(lds_raw, acc, mlimit, nlimit, [&](int r) { return out + (int64_t)r * ldo; });
}

// dWd[e] = sum_p dO[p]^T h[p] = sum_p dy[tok[p]]^T (w_p h[p]) (hb holds w_p h)
__global__ __launch_bounds__(kThreads, 1) void bwd_dwd_kernel(mok_bwd_args a, int ntm, int ry) {
  using G = G256;
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[tile_lds_bytes<Smem<G, false>>()];
  int e, mt_, nt_;
  if (!dw_tile_of(a.E, a.eorder, ntm, (int)((a.I + G::BN - 1) / G::BN), ry, e, mt_, nt_)) return;
  const int tl = mt_ * (int)((a.I + G::BN - 1) / G::BN) + nt_;
  const int64_t H = a.H, I = a.I;
  const int ntn = (int)((I + G::BN - 1) / G::BN);
  const int m0 = (tl / ntn) * G::BM, n0 = (tl % ntn) * G::BN;
  const int o = a.offsets[e], c = a.offsets[e + 1] - o;
  const int mlim = (int)min<int64_t>(G::BM, H - m0), nlim = (int)min<int64_t>(G::BN, I - n0);
  const LoadKOG<G::BM> la(reinterpret_cast<const uint8_t*>(a.dy + m0), a.tok + o, 2 * H, c, mlim);
  const uint8_t* hp = reinterpret_cast<const uint8_t*>(a.hb + (int64_t)o * I + n0);
  const LoadKO<G::BN> lb{hp, hp, 0x7FFFFFFF, 2 * I, c, nlim};
  dw_tile(lds_raw, la, mlim, lb, nlim, c, a.dwd + (int64_t)e * H * I + (int64_t)m0 * I + n0, I);
}

// [dWg; dWu][e] = sum_p [dA dB][p]^T x[tok[p]]
__global__ __launch_bounds__(kThreads, 1) void bwd_dwgu_kernel(mok_bwd_args a, int ntm, int ry) {
  using G = G256;
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[tile_lds_bytes<Smem<G, false>>()];
  int e, mt_, nt_;
  if (!dw_tile_of(a.E, a.eorder, ntm, (int)((a.H + G::BN - 1) / G::BN), ry, e, mt_, nt_)) return;
  const int tl = mt_ * (int)((a.H + G::BN - 1) / G::BN) + nt_;
  const int64_t H = a.H, I = a.I;
  const int ntn = (int)((H + G::BN - 1) / G::BN);
  const int mt = tl / ntn;
  const int n0 = (tl % ntn) * G::BN;
  // rows [0, I) of the stacked [dWg; dWu] are dWg, [I, 2I) dWu; a tile never
  // straddles the two because I is a multiple of 128 and tiles of 256 rows are
  // split at I.
  const int tiles_g = (int)((I + G::BM - 1) / G::BM);
  const bool up = mt >= tiles_g;
  const int m0 = (up ? mt - tiles_g : mt) * G::BM;
  const int mlim = (int)min<int64_t>(G::BM, I - m0), nlim = (int)min<int64_t>(G::BN, H - n0);
  const int o = a.offsets[e], c = a.offsets[e + 1] - o;
  bf16_t* out = (up ? a.dwu : a.dwg) + (int64_t)e * I * H + (int64_t)m0 * H + n0;
  const uint8_t* dp = reinterpret_cast<const uint8_t*>(a.dab + (int64_t)o * 2 * I + (up ? I : 0) + m0);
  const LoadKO<G::BM> la{dp, dp, 0x7FFFFFFF, 4 * I, c, mlim};
  const LoadKOG<G::BN> lb(reinterpret_cast<const uint8_t*>(a.x + n0), a.tok + o, 2 * H, c, nlim);
  dw_tile(lds_raw, la, mlim, lb, nlim, c, out, H);
}

// ================================================================== MXFP8 backward
// The backward GEMMs with MXFP8 operands on the scaled MFMA ([MoK card]
// "What it is": forward and backward in BF16 and MXFP8). Every operand is
// K-contiguous: the weights come transposed and quantized along the
// contraction axis, the activations are quantized along it (rows) or
// token-blocked (weight gradients, K = an expert's rows).

// dh = dO . Wd[e] (K = H) from dO rows and Wd^T rows, then the SwiGLU
// backward; writes dA|dB rows quantized along 2I (for dX), dA|dB token-blocked
// (for dWg/dWu) and h (bf16, token-blocked by token_quantize_kernel). dA and dB
// are rounded to bf16 once and both of their quantizations take those values.
__global__ __launch_bounds__(kThreads, 1) void bwd_dh8_kernel(mok_bwd_args a, int ncol) {
  using G = G256;
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[tile_lds_bytes<Smem<G, true>>()];
  Smem<G, true>& sm = *reinterpret_cast<Smem<G, true>*>(lds_raw);
  mok_tile t;
  int ny;
  if (!bwd_tile(a, ncol, t, ny)) return;
  const int nrows = t.p1 - t.p0;
  const int64_t H = a.H, I = a.I, sH = H / 32, s2I = 2 * I / 32;
  const int n0 = ny * G::BN;
  const int64_t wrow = (int64_t)t.e * I + n0;           // first Wd^T row of the tile
  const LoadKD<G::BM, RowsStrided> la{{a.dOq + (int64_t)t.p0 * H, H, nrows}};
  const LoadKD<G::BN, RowsStrided> lb{{a.wdt + wrow * H, H, (int)(I - n0)}};
  const LoadScalesD<G::BM, RowsStrided> lsa{{a.dOs + (int64_t)t.p0 * sH, sH, nrows}};
  const LoadScalesD<G::BN, RowsStrided> lsb{{a.wdt_s + wrow * sH, sH, (int)(I - n0)}};
  Acc<G::FM, G::FN> acc;
  mainloop_rows<false, G, true>(sm, la, lb, lsa, lsb, (int)(H / 64), nrows, acc);
  // per row and 32-column block: dA, dB, h from dh and the saved a, b;
  // the 32 dA (and dB) values of the block share one scale along I
  using HS = HalfF32<G>;
  // a thread keeps one 32-column block and takes rows r0, r0 + 32, r0 + 64,
  // r0 + 96 of each half, in two groups of 2 rows whose a, b loads are issued
  // before the group's stores (see bwd_dh_kernel); the stores cover pieces of
  // many rows per instruction and stay cached (see gateup_tile)
  const int blk = threadIdx.x % (G::BN / 32), r0 = threadIdx.x / (G::BN / 32), c0 = blk * 32;
  const bool colok = n0 + c0 < I;
  const bf16_t* abt = a.ab + (int64_t)t.p0 * 2 * I + n0 + c0;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int rows = min(128, nrows - 128 * half);
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
      uint4 va[2][4], vb[2][4];
#pragma unroll
      for (int i2 = 0; i2 < 2; ++i2) {
        const int r = r0 + 32 * (2 * grp + i2);
        if (colok && r < rows) {
          const bf16_t* q = abt + (int64_t)(128 * half + r) * 2 * I;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            va[i2][u] = *reinterpret_cast<const uint4*>(q + 8 * u);
            vb[i2][u] = *reinterpret_cast<const uint4*>(q + I + 8 * u);
          }
        }
      }
      if (grp == 0) {
        if (half) barrier_lds_only();
        HS::put(lds_raw, acc, half);
        barrier_lds_only();
      }
#pragma unroll
      for (int i2 = 0; i2 < 2; ++i2) {
        const int r = r0 + 32 * (2 * grp + i2);
        if (!colok || r >= rows) continue;
        const int64_t p = t.p0 + 128 * half + r;
        float da[32], db[32];
        float amaxa = 0.f, amaxb = 0.f;
#pragma unroll
        for (int u = 0; u < 32; u += 8) {
          float dh[8], av[8], bv[8], h[8];
          HS::get8(lds_raw, r, c0 + u, dh);
          unpack_bf16x8(va[i2][u / 8], av);
          unpack_bf16x8(vb[i2][u / 8], bv);
#pragma unroll
          for (int v = 0; v < 8; ++v) {
            const float sg = sigmoidf_(av[v]);
            da[u + v] = dh[v] * bv[v] * sg * (1.0f + av[v] * (1.0f - sg));
            db[u + v] = dh[v] * av[v] * sg;
            h[v] = av[v] * sg * bv[v];
          }
          *reinterpret_cast<uint4*>(a.hb + p * I + n0 + c0 + u) = pack_bf16x8(h);
          // dA and dB are bf16 values before either of their quantizations
          unpack_bf16x8(pack_bf16x8(da + u), da + u);
          unpack_bf16x8(pack_bf16x8(db + u), db + u);
#pragma unroll
          for (int v = 0; v < 8; ++v) {
            amaxa = fmaxf(amaxa, fabsf(da[u + v]));
            amaxb = fmaxf(amaxb, fabsf(db[u + v]));
          }
        }
        // the row's bf16 dA and dB values replace its fp32 dh block in the
        // staging area (this thread alone reads that block): 64 bytes of dA,
        // then 64 of dB, for the token-blocked pass below
        {
          uint4* stash = reinterpret_cast<uint4*>(lds_raw + r * HS::PITCH + c0 * 4);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            stash[u] = pack_bf16x8(da + 8 * u);
            stash[4 + u] = pack_bf16x8(db + 8 * u);
          }
        }
#pragma unroll
        for (int side = 0; side < 2; ++side) {
          const float* v = side ? db : da;
          const int sc = mx_scale_byte(side ? amaxb : amaxa);
          const float inv = mx_inv_scale(sc);
          uint32_t w[8];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            w[u] = e4m3_pack4(v[4 * u] * inv, v[4 * u + 1] * inv, v[4 * u + 2] * inv,
                          v[4 * u + 3] * inv);
          const int64_t col = (side ? I : 0) + n0 + c0;
          uint4* d = reinterpret_cast<uint4*>(a.dabq + p * 2 * I + col);
          d[0] = make_uint4(w[0], w[1], w[2], w[3]);
          d[1] = make_uint4(w[4], w[5], w[6], w[7]);
          a.dabs[p * s2I + col / 32] = (uint8_t)sc;
        }
      }
    }
    // token-blocked dA | dB of this half ([MoK card] MXFP8 backward operands
    // of dWg/dWu, blocked by 32 along the expert's rows counted from its
    // first row): one 32-row block x two adjacent columns per item, read from
    // the stashed bf16 values; rows past the tile's end are zero up to the
    // expert's padded length. Same bits as quantizing stored bf16 rows.
    barrier_lds_only();
    const int64_t N = 2 * I;
    const int koffe = a.koff[t.e], kp = a.koff[t.e + 1] - koffe;
    const int rbase = t.p0 - a.offsets[t.e] + 128 * half;   // padded-axis position of row 0 of the half
    for (int item = threadIdx.x; item < 4 * 256; item += kThreads) {
      const int rb = item >> 8, cpair = item & 255;
      const int q = cpair >> 7, cc = (cpair & 127) * 2;     // q: dA or dB; tile columns cc, cc + 1
      const int pos0 = rbase + 32 * rb;
      if (pos0 >= kp || n0 + cc >= I) continue;
      float x0[32], x1[32];
      float m0 = 0.f, m1 = 0.f;
#pragma unroll
      for (int rr = 0; rr < 32; ++rr) {
        const int row = 32 * rb + rr;
        uint32_t wv = 0u;
        if (row < rows)
          wv = *reinterpret_cast<const uint32_t*>(lds_raw + row * HS::PITCH + (cc >> 5) * 128 + q * 64 +
                                                  (cc & 31) * 2);
        x0[rr] = __uint_as_float(wv << 16);
        x1[rr] = __uint_as_float(wv & 0xFFFF0000u);
        m0 = fmaxf(m0, fabsf(x0[rr]));
        m1 = fmaxf(m1, fabsf(x1[rr]));
      }
#pragma unroll
      for (int side = 0; side < 2; ++side) {
        const float* v = side ? x1 : x0;
        const int sc = mx_scale_byte(side ? m1 : m0);
        const float inv = mx_inv_scale(sc);
        uint32_t wds[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          wds[u] = e4m3_pack4(v[4 * u] * inv, v[4 * u + 1] * inv, v[4 * u + 2] * inv, v[4 * u + 3] * inv);
        const int64_t n = (int64_t)q * I + n0 + cc + side;
        uint4* d = reinterpret_cast<uint4*>(a.dabT + N * koffe + n * kp + pos0);
        d[0] = make_uint4(wds[0], wds[1], wds[2], wds[3]);
        d[1] = make_uint4(wds[4], wds[5], wds[6], wds[7]);
        a.dabTs[N * (koffe / 32) + n * (kp / 32) + pos0 / 32] = (uint8_t)sc;
      }
    }
  }
}

// dX rows = [dA | dB] . [Wg[e]; Wu[e]] (K = 2I) from quantized dA|dB rows and
// [Wg; Wu]^T rows; row p goes to flat row perm[p].
__global__ __launch_bounds__(kThreads, 1) void bwd_dx8_kernel(mok_bwd_args a, int ncol) {
  using G = G256;
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[tile_lds_bytes<Smem<G, true>>()];
  Smem<G, true>& sm = *reinterpret_cast<Smem<G, true>*>(lds_raw);
  mok_tile t;
  int ny;
  if (!bwd_tile(a, ncol, t, ny)) return;
  const int nrows = t.p1 - t.p0;
  const int64_t H = a.H, I = a.I, K = 2 * I, sK = K / 32;
  const int n0 = ny * G::BN;
  const int64_t wrow = (int64_t)t.e * H + n0;
  const LoadKD<G::BM, RowsStrided> la{{a.dabq + (int64_t)t.p0 * K, K, nrows}};
  const LoadKD<G::BN, RowsStrided> lb{{a.wgut + wrow * K, K, (int)(H - n0)}};
  const LoadScalesD<G::BM, RowsStrided> lsa{{a.dabs + (int64_t)t.p0 * sK, sK, nrows}};
  const LoadScalesD<G::BN, RowsStrided> lsb{{a.wgut_s + wrow * sK, sK, (int)(H - n0)}};
  Acc<G::FM, G::FN> acc;
  mainloop_x<kTrDx, G, true>(sm, la, lb, lsa, lsb, (int)(K / 64), nrows, acc);
  int* rows = tile_rows<Smem<G, true>>(lds_raw);
  barrier_lds_only();
  for (int r = threadIdx.x; r < G::BM; r += kThreads) rows[r] = r < nrows ? a.perm[t.p0 + r] : 0;
  bf16_t* d = a.dxrows + n0;
  store_bf16_x<kTrDx, G>(lds_raw, acc, nrows, (int)(H - n0), [&](int r) { return d + (int64_t)rows[r] * H; });
}

// Weight gradient out[m][n] = sum over the expert's rows of A[m][k] B[n][k],
// both operands token-blocked MXFP8 rows of the expert (K = tok_pad(rows)).
MOK_DEV void dw8_tile(uint8_t* lds_raw, const uint8_t* A, const uint8_t* As, int mlim, const uint8_t* B,
                      const uint8_t* Bs, int nlim, int kp, bf16_t* out, int64_t ldo) {
  using G = G256;
  Smem<G, true>& sm = *reinterpret_cast<Smem<G, true>*>(lds_raw);
  const LoadKD<G::BM, RowsStrided> la{{A, kp, mlim}};
  const LoadKD<G::BN, RowsStrided> lb{{B, kp, nlim}};
  const LoadScalesD<G::BM, RowsStrided> lsa{{As, kp / 32, mlim}};
  const LoadScalesD<G::BN, RowsStrided> lsb{{Bs, kp / 32, nlim}};
  Acc<G::FM, G::FN> acc;
  mainloop_x<kTrDw, G, true>(sm, la, lb, lsa, lsb, kp / 64, mlim, acc);
  store_bf16_x<kTrDw, G>(lds_raw, acc, mlim, nlim, [&](int r) { return out + (int64_t)r * ldo; });
}

__global__ __launch_bounds__(kThreads, 1) void bwd_dwd8_kernel(mok_bwd_args a, int ntm, int ry) {
  using G = G256;
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[tile_lds_bytes<Smem<G, true>>()];
  int e, mt_, nt_;
  if (!dw_tile_of(a.E, a.eorder, ntm, (int)((a.I + G::BN - 1) / G::BN), ry, e, mt_, nt_)) return;
  const int tl = mt_ * (int)((a.I + G::BN - 1) / G::BN) + nt_;
  const int64_t H = a.H, I = a.I;
  const int ntn = (int)((I + G::BN - 1) / G::BN);
  const int m0 = (tl / ntn) * G::BM, n0 = (tl % ntn) * G::BN;
  // wave-uniform: kept in scalar registers
  const int64_t koff = __builtin_amdgcn_readfirstlane(a.koff[e]);
  const int kp = __builtin_amdgcn_readfirstlane(a.koff[e + 1]) - (int)koff;
  dw8_tile(lds_raw, a.dOT + H * koff + (int64_t)m0 * kp, a.dOTs + H * (koff / 32) + (int64_t)m0 * (kp / 32),
           (int)min<int64_t>(G::BM, H - m0), a.hT + I * koff + (int64_t)n0 * kp,
           a.hTs + I * (koff / 32) + (int64_t)n0 * (kp / 32), (int)min<int64_t>(G::BN, I - n0), kp,
           a.dwd + (int64_t)e * H * I + (int64_t)m0 * I + n0, I);
}

__global__ __launch_bounds__(kThreads, 1) void bwd_dwgu8_kernel(mok_bwd_args a, int ntm, int ry) {
  using G = G256;
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[tile_lds_bytes<Smem<G, true>>()];
  int e, mt_, nt_;
  if (!dw_tile_of(a.E, a.eorder, ntm, (int)((a.H + G::BN - 1) / G::BN), ry, e, mt_, nt_)) return;
  const int tl = mt_ * (int)((a.H + G::BN - 1) / G::BN) + nt_;
  const int64_t H = a.H, I = a.I;
  const int ntn = (int)((H + G::BN - 1) / G::BN);
  const int mt = tl / ntn;
  const int n0 = (tl % ntn) * G::BN;
  // stacked [dWg; dWu] rows; tiles split at I (I is a multiple of 128)
  const int tiles_g = (int)((I + G::BM - 1) / G::BM);
  const bool up = mt >= tiles_g;
  const int m0 = (up ? mt - tiles_g : mt) * G::BM;
  const int64_t arow = (up ? I : 0) + m0;               // row of the token-blocked dA|dB
  // wave-uniform: kept in scalar registers
  const int64_t koff = __builtin_amdgcn_readfirstlane(a.koff[e]);
  const int kp = __builtin_amdgcn_readfirstlane(a.koff[e + 1]) - (int)koff;
  bf16_t* out = (up ? a.dwu : a.dwg) + (int64_t)e * I * H + (int64_t)m0 * H + n0;
  dw8_tile(lds_raw, a.dabT + 2 * I * koff + arow * kp, a.dabTs + 2 * I * (koff / 32) + arow * (kp / 32),
           (int)min<int64_t>(G::BM, I - m0), a.xT + H * koff + (int64_t)n0 * kp,
           a.xTs + H * (koff / 32) + (int64_t)n0 * (kp / 32), (int)min<int64_t>(G::BN, H - n0), kp, out, H);
}

unsigned cdivu(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

}  // namespace

// grid of the row-tile kernels (see xcd_swizzle)
unsigned rt_grid(int64_t max_tiles, int ncol) {
  return (unsigned)((int64_t)kXcds * ((max_tiles + kXcds - 1) / kXcds) * ncol);
}
// blocks of the weight-gradient grids (see dw_tile_of): kXcds = ry x (kXcds/ry)
// blocks per expert, ry chosen so that the blocks are closest to square
// without an empty block (an empty block would idle an XCD)
int dw_ry(int ntm, int ntn) {
  int best = 1;
  double bs = 1e30;
  for (int ry = 1; ry <= kXcds; ry *= 2) {
    const int cx = kXcds / ry;
    if (ry > ntm || cx > ntn) continue;
    const double h = (double)ntm / ry, w = (double)ntn / cx;
    const double sq = h > w ? h / w : w / h;
    if (sq < bs) {
      bs = sq;
      best = ry;
    }
  }
  return best;
}
unsigned dw_grid(int E, int ntm, int ntn, int ry) {
  const int cx = kXcds / ry;
  return (unsigned)((int64_t)kXcds * E * ((ntm + ry - 1) / ry) * ((ntn + cx - 1) / cx));
}

hipError_t mok_launch_gateup(const mok_fwd_args& a, int m0, int m1, int max_tiles, bool mxfp8,
                             hipStream_t st) {
  const int ncol = (int)cdivu(a.I, G256::BN / 2);
  const dim3 grid(rt_grid(max_tiles, ncol));
  if (mxfp8) hipLaunchKernelGGL(gateup_kernel<true>, grid, dim3(kThreads), 0, st, a, m0, m1, ncol);
  else hipLaunchKernelGGL(gateup_kernel<false>, grid, dim3(kThreads), 0, st, a, m0, m1, ncol);
  return hipGetLastError();
}

hipError_t mok_launch_down(const mok_fwd_args& a, int m0, int m1, int max_tiles, bool mxfp8,
                           hipStream_t st) {
  const int ncol = (int)cdivu(a.H, G256::BN);
  const dim3 grid(rt_grid(max_tiles, ncol));
  if (mxfp8) hipLaunchKernelGGL(down_kernel<true>, grid, dim3(kThreads), 0, st, a, m0, m1, ncol);
  else hipLaunchKernelGGL(down_kernel<false>, grid, dim3(kThreads), 0, st, a, m0, m1, ncol);
  return hipGetLastError();
}


hipError_t mok_launch_fwd_persistent(const mok_fwd_args& a, const mok_persist_args& ps, int grid,
                                     bool mxfp8, hipStream_t st) {
  if (grid <= 0 || grid % kPlanQueues != 0) return hipErrorInvalidValue;
  if (mxfp8) hipLaunchKernelGGL(fwd_persistent_kernel<true>, dim3(grid), dim3(kThreads), 0, st, a, ps);
  else hipLaunchKernelGGL(fwd_persistent_kernel<false>, dim3(grid), dim3(kThreads), 0, st, a, ps);
  return hipGetLastError();
}

hipError_t mok_launch_layer_fwd(const mok_fwd_args& a, const mok_persist_args& ps, const mok_layer_args& L,
                                int grid, bool mxfp8, hipStream_t st) {
  if (grid <= 0 || grid % kPlanQueues != 0) return hipErrorInvalidValue;
  if (mxfp8) hipLaunchKernelGGL(layer_fwd_kernel<true>, dim3(grid), dim3(kThreads), 0, st, a, ps, L);
  else hipLaunchKernelGGL(layer_fwd_kernel<false>, dim3(grid), dim3(kThreads), 0, st, a, ps, L);
  return hipGetLastError();
}

hipError_t mok_launch_bwd_dh(const mok_bwd_args& a, hipStream_t st) {
  const int ncol = (int)cdivu(a.I, G256::BN);
  hipLaunchKernelGGL(bwd_dh_kernel, dim3(rt_grid(a.max_tiles, ncol)), dim3(kThreads), 0, st, a, ncol);
  return hipGetLastError();
}

hipError_t mok_launch_bwd_dh8(const mok_bwd_args& a, hipStream_t st) {
  const int ncol = (int)cdivu(a.I, G256::BN);
  hipLaunchKernelGGL(bwd_dh8_kernel, dim3(rt_grid(a.max_tiles, ncol)), dim3(kThreads), 0, st, a, ncol);
  return hipGetLastError();
}

hipError_t mok_launch_bwd_dx8(const mok_bwd_args& a, hipStream_t st) {
  const int ncol = (int)cdivu(a.H, G256::BN);
  hipLaunchKernelGGL(bwd_dx8_kernel, dim3(rt_grid(a.max_tiles, ncol)), dim3(kThreads), 0, st, a, ncol);
  return hipGetLastError();
}

hipError_t mok_launch_bwd_dwd8(const mok_bwd_args& a, hipStream_t st) {
  const int ntm = (int)(cdivu(a.H, G256::BM)), ntn = (int)cdivu(a.I, G256::BN);
  hipLaunchKernelGGL(bwd_dwd8_kernel, dim3(dw_grid(a.E, ntm, ntn, dw_ry(ntm, ntn))), dim3(kThreads), 0, st, a, ntm,
                     dw_ry(ntm, ntn));
  return hipGetLastError();
}

hipError_t mok_launch_bwd_dwgu8(const mok_bwd_args& a, hipStream_t st) {
  const int ntm = (int)(2 * cdivu(a.I, G256::BM)), ntn = (int)cdivu(a.H, G256::BN);
  hipLaunchKernelGGL(bwd_dwgu8_kernel, dim3(dw_grid(a.E, ntm, ntn, dw_ry(ntm, ntn))), dim3(kThreads), 0, st, a, ntm,
                     dw_ry(ntm, ntn));
  return hipGetLastError();
}

hipError_t mok_launch_bwd_dx(const mok_bwd_args& a, hipStream_t st) {
  const int ncol = (int)cdivu(a.H, G256::BN);
  hipLaunchKernelGGL(bwd_dx_kernel, dim3(rt_grid(a.max_tiles, ncol)), dim3(kThreads), 0, st, a, ncol);
  return hipGetLastError();
}

hipError_t mok_launch_bwd_dwd(const mok_bwd_args& a, hipStream_t st) {
  const int ntm = (int)(cdivu(a.H, G256::BM)), ntn = (int)cdivu(a.I, G256::BN);
  hipLaunchKernelGGL(bwd_dwd_kernel, dim3(dw_grid(a.E, ntm, ntn, dw_ry(ntm, ntn))), dim3(kThreads), 0, st, a, ntm,
                     dw_ry(ntm, ntn));
  return hipGetLastError();
}

hipError_t mok_launch_bwd_dwgu(const mok_bwd_args& a, hipStream_t st) {
  const int ntm = (int)(2 * cdivu(a.I, G256::BM)), ntn = (int)cdivu(a.H, G256::BN);
  hipLaunchKernelGGL(bwd_dwgu_kernel, dim3(dw_grid(a.E, ntm, ntn, dw_ry(ntm, ntn))), dim3(kThreads), 0, st, a, ntm,
                     dw_ry(ntm, ntn));
  return hipGetLastError();
}
