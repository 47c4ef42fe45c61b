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

using namespace mok;

namespace {

using G256 = Geo<256, 256, 2, 2>;

// ================================================================== forward
// A forward tile: row tile ti of minibatch m (rows in ring slot m mod N_s).
struct FwdTile {
  mok_tile t;
  int nrows;
  int64_t slot_row0;     // ring row of the tile's first row
};

MOK_DEV void fwd_tile_at(const mok_fwd_args& a, int m, int ti, FwdTile& ft) {
  ft.t = a.tiles[ti];
  ft.nrows = ft.t.p1 - ft.t.p0;
  ft.slot_row0 = (int64_t)(m % a.n_slots) * a.M + (ft.t.p0 - (int64_t)m * a.M);
}

// gate/up GEMM + SwiGLU of one row tile x 128 h-columns. The B tile holds 32-row
// groups alternating Wg and Wu, so accumulator column blocks j = 2jj (gate) and
// 2jj + 1 (up) cover the same 32 h-columns.
template <bool F8>
MOK_DEV void gateup_tile(const mok_fwd_args& a, uint8_t* lds_raw, int m, int ti, int ny) {
  using G = G256;
  Smem<G>& sm = *reinterpret_cast<Smem<G>*>(lds_raw);
  FwdTile ft;
  fwd_tile_at(a, m, ti, ft);
  const int64_t H = a.H, I = a.I;
  const int n0 = ny * (G::BN / 2);
  const int64_t xrow = F8 ? H : 2 * H;                       // bytes per X row
  const int64_t wrow = F8 ? H : 2 * H;                       // bytes per weight row
  const int64_t eoff = (int64_t)ft.t.e * I * wrow;
  LoadKD<G::BM, RowsStrided> la{{a.ring_x + ft.slot_row0 * xrow, xrow, ft.nrows}};
  LoadKD<G::BN, RowsGateUp> lb{{(const uint8_t*)a.wg + eoff, (const uint8_t*)a.wu + eoff, wrow, n0, (int)I}};
  Acc<G::FM, G::FN> acc;
  if constexpr (F8) {
    const int64_t sx = H / 32;
    LoadScalesD<G::BM, RowsStrided> lsa{{a.ring_xs + ft.slot_row0 * sx, sx, ft.nrows}};
    const int64_t se = (int64_t)ft.t.e * I * sx;
    LoadScalesD<G::BN, RowsGateUp> lsb{{a.sg + se, a.su + se, sx, n0, (int)I}};
    mainloop<G, true>(sm, la, lb, lsa, lsb, (int)(H / 64), acc);
  } else {
    NoScales ns;
    mainloop<G, false>(sm, la, lb, ns, ns, (int)(H / 32), acc);
  }

  // SwiGLU on the accumulators; h (and a, b) staged in LDS for row-wise stores.
  constexpr int HW = G::BN / 2;                               // 128 h columns
  uint8_t* st = lds_raw;
  const int hcol0 = G::wn() * (G::WTN / 2);
  if constexpr (!F8) {
    // h = silu(a) * b per element from an fp32 half-tile in LDS. Tile column
    // (c/32)*64 + c%32 holds gate column c of the tile, +32 its up column.
    using HS = HalfF32<G>;
    bf16_t* hs = reinterpret_cast<bf16_t*>(a.ring_h) + ft.slot_row0 * I + n0;
    bf16_t* abp = a.ab ? a.ab + (int64_t)ft.t.p0 * 2 * I + n0 : nullptr;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (half) __syncthreads();
      HS::put(st, acc, half);
      __syncthreads();
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
        *reinterpret_cast<uint4*>(hs + rr * I + c) = pack_bf16x8(h);
        if (abp) {
          *reinterpret_cast<uint4*>(abp + rr * 2 * I + c) = pack_bf16x8(av);
          *reinterpret_cast<uint4*>(abp + rr * 2 * I + I + c) = pack_bf16x8(bv);
        }
      }
    }
  } else {
    // MXFP8 h: one E8M0 scale per 32 h-columns of a row. Each thread takes one
    // 32-column block of one row from the fp32 half-tile: amax, scale byte,
    // 32 E4M3 codes (two 16-byte stores) and the scale.
    using HS = HalfF32<G>;
    uint8_t* hq = a.ring_h + ft.slot_row0 * I + n0;
    uint8_t* hsc = a.ring_hs + ft.slot_row0 * (I / 32) + n0 / 32;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (half) __syncthreads();
      HS::put(st, acc, half);
      __syncthreads();
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
          w[u] = e4m3_encode(h[4 * u] * inv) | (e4m3_encode(h[4 * u + 1] * inv) << 8) |
                 (e4m3_encode(h[4 * u + 2] * inv) << 16) | (e4m3_encode(h[4 * u + 3] * inv) << 24);
        const int64_t rr = 128 * half + r;
        uint4* d = reinterpret_cast<uint4*>(hq + rr * I + blk * 32);
        d[0] = make_uint4(w[0], w[1], w[2], w[3]);
        d[1] = make_uint4(w[4], w[5], w[6], w[7]);
        hsc[rr * (I / 32) + blk] = (uint8_t)sc;
      }
    }
  }
}

// down GEMM of one row tile x 256 output columns; each row is pushed to its
// flat position perm[p] of obuf (unique destinations, no atomics).
template <bool F8>
MOK_DEV void down_tile(const mok_fwd_args& a, uint8_t* lds_raw, int* rows, int m, int ti, int ny) {
  using G = G256;
  Smem<G>& sm = *reinterpret_cast<Smem<G>*>(lds_raw);
  FwdTile ft;
  fwd_tile_at(a, m, ti, ft);
  const int64_t H = a.H, I = a.I;
  const int n0 = ny * G::BN;
  const int64_t hrow = F8 ? I : 2 * I;
  for (int r = threadIdx.x; r < G::BM; r += kThreads) rows[r] = r < ft.nrows ? a.perm[ft.t.p0 + r] : 0;
  LoadKD<G::BM, RowsStrided> la{{a.ring_h + ft.slot_row0 * hrow, hrow, ft.nrows}};
  LoadKD<G::BN, RowsStrided> lb{{(const uint8_t*)a.wd + ((int64_t)ft.t.e * H + n0) * hrow, hrow,
                                (int)(H - n0)}};
  Acc<G::FM, G::FN> acc;
  if constexpr (F8) {
    const int64_t sx = I / 32;
    LoadScalesD<G::BM, RowsStrided> lsa{{a.ring_hs + ft.slot_row0 * sx, sx, ft.nrows}};
    LoadScalesD<G::BN, RowsStrided> lsb{{a.sd + ((int64_t)ft.t.e * H + n0) * sx, sx, (int)(H - n0)}};
    mainloop<G, true>(sm, la, lb, lsa, lsb, (int)(I / 64), acc);
  } else {
    NoScales ns;
    mainloop<G, false>(sm, la, lb, ns, ns, (int)(I / 32), acc);
  }
  bf16_t* ob = a.obuf + n0;
  store_tile_bf16<G>(lds_raw, acc, ft.nrows, (int)(H - n0),
                     [&](int r) { return ob + (int64_t)rows[r] * H; });
}

// Launch grids are 1-D upper bounds; the tile count of minibatch m is read
// on the device and the logical tile order is XCD-aware (xcd_tile), row-major
// over (row tile, column tile).
template <bool F8>
__global__ __launch_bounds__(kThreads, 1) void gateup_kernel(mok_fwd_args a, int m, int ncol) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[sizeof(Smem<G256>)];
  const int t0 = a.mb_tile_start[m];
  const int L = xcd_tile((a.mb_tile_start[m + 1] - t0) * ncol);
  if (L < 0) return;
  gateup_tile<F8>(a, lds_raw, m, t0 + L / ncol, L % ncol);
}

template <bool F8>
__global__ __launch_bounds__(kThreads, 1) void down_kernel(mok_fwd_args a, int m, int ncol) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[sizeof(Smem<G256>)];
  __shared__ int rows[G256::BM];
  const int t0 = a.mb_tile_start[m];
  const int L = xcd_tile((a.mb_tile_start[m + 1] - t0) * ncol);
  if (L < 0) return;
  down_tile<F8>(a, lds_raw, rows, m, t0 + L / ncol, L % ncol);
}

// ================================================================== persistent driver
// [MoK clip] Key points, bullets 3-5, and How-to items 3-4: minibatches of
// routed rows flow through a fixed ring of token slots on the device; a slot
// is refilled as soon as the work that read it has retired, and completion
// is signalled through counters in memory rather than by kernel boundaries.
//
// One persistent launch runs every work item of the forward's expert stage:
//   G(m, c)  gather rows [m*M + c*GR, +GR) into ring slot m mod N_s
//   U(m, r, n) gate/up tile (row tile r of minibatch m, h-column tile n)
//   D(m, r, n) down tile
// Items are numbered in one global order, stage by stage: stage s holds
// D(s - dl), then G(s), then U(s - ul), with (dl, ul) = (2, 1) when N_s >= 2
// and (1, 0) when N_s = 1. Every item depends only on items numbered before
// it (G(m) on all D(m - N_s), U on G of its minibatch, D on all U of its row
// tile). Workgroups take item numbers from an atomic ticket in increasing
// order, so every item an item waits for is held by a workgroup that is
// already running: the waits always end. A wait that exceeds about two
// seconds sets MOK_STATUS_WATCHDOG and gives up instead of hanging.
// Which workgroup runs an item never changes what it computes, so the result
// is bitwise the same as with one launch per stage.
constexpr int kGatherRows = 64;

struct FwdPlan {
  int n_mb, M, R, dl, ul, ntu, ntd, gi_full, n_stages;
  const int* mbs;                      // mb_tile_start
  MOK_DEV int tiles_before(int m) const { return mbs[m < 0 ? 0 : (m > n_mb ? n_mb : m)]; }
  MOK_DEV int gi(int m) const {        // gather items of minibatch m
    if (m < 0 || m >= n_mb) return 0;
    return (min(M, R - m * M) + kGatherRows - 1) / kGatherRows;
  }
  MOK_DEV int64_t gsum(int m) const {  // gather items of minibatches < m
    if (m <= 0) return 0;
    if (m >= n_mb) return (int64_t)(n_mb - 1) * gi_full + gi(n_mb - 1);
    return (int64_t)m * gi_full;
  }
  MOK_DEV int64_t cum(int s) const {   // items in stages < s
    return (int64_t)ntd * tiles_before(s - dl) + gsum(s) + (int64_t)ntu * tiles_before(s - ul);
  }
};

struct mok_persist_args {
  int* ctr;          // [0] ticket, [1 .. n_mb] gather done, [1+n_mb .. 2 n_mb] down done,
                     // [1 + 2 n_mb ..] gate/up tiles done per forward row tile
  int32_t* status;   // schedule status word (watchdog bit)
  const uint8_t* xsrc;
  const uint8_t* xscales;
  const int32_t* offsets_E;
};

MOK_DEV void signal_done(int* c) {
  __threadfence();                     // this thread's results are visible device-wide
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(c, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

MOK_DEV void wait_for(const int* c, int target, int32_t* status) {
  if (threadIdx.x == 0 && target > 0) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (__hip_atomic_load(c, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(2);
      // once any wait has timed out, no later wait blocks: the launch drains
      if (__hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 2) break;
      if (__builtin_amdgcn_s_memrealtime() - t0 > 200000000ull) {   // 2 s at 100 MHz
        __hip_atomic_fetch_or(status, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

MOK_DEV void gather_item(const mok_fwd_args& a, const mok_persist_args& ps, bool f8, int m, int c) {
  const int64_t xrow = f8 ? a.H : 2 * a.H, srow = a.H / 32;
  const int64_t mb0 = (int64_t)m * a.M;
  const int64_t rows_m = min((int64_t)a.M, (int64_t)a.T * a.topk - mb0);
  const int nvalid = *ps.offsets_E;
  const int64_t slot0 = (int64_t)(m % a.n_slots) * a.M;
  const int w = threadIdx.x >> 6, l = lane_id();
  for (int rr = w; rr < kGatherRows; rr += 4) {
    const int64_t r = (int64_t)c * kGatherRows + rr;
    if (r >= rows_m || mb0 + r >= nvalid) break;
    const int64_t tok = a.perm[mb0 + r] / a.topk;
    const uint4* src = reinterpret_cast<const uint4*>(ps.xsrc + tok * xrow);
    uint4* dst = reinterpret_cast<uint4*>(a.ring_x + (slot0 + r) * xrow);
    for (int64_t q = l; q < xrow / 16; q += 64) dst[q] = src[q];
    if (f8) {
      const uint32_t* ss = reinterpret_cast<const uint32_t*>(ps.xscales + tok * srow);
      uint32_t* ds = reinterpret_cast<uint32_t*>(a.ring_xs + (slot0 + r) * srow);
      for (int64_t q = l; q < srow / 4; q += 64) ds[q] = ss[q];
    }
  }
}

template <bool F8>
__global__ __launch_bounds__(kThreads, 1) void fwd_persistent_kernel(mok_fwd_args a, mok_persist_args ps) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[sizeof(Smem<G256>)];
  __shared__ int rows[G256::BM];
  __shared__ int s_ticket;
  FwdPlan P;
  P.n_mb = a.n_mb;
  P.M = a.M;
  P.R = (int)(a.T * a.topk);
  P.dl = a.n_slots >= 2 ? 2 : 1;
  P.ul = P.dl - 1;
  P.ntu = (int)((a.I + G256::BN / 2 - 1) / (G256::BN / 2));
  P.ntd = (int)((a.H + G256::BN - 1) / G256::BN);
  P.gi_full = (a.M + kGatherRows - 1) / kGatherRows;
  P.n_stages = a.n_mb + P.dl;
  P.mbs = a.mb_tile_start;
  int* gdone = ps.ctr + 1;
  int* ddone = ps.ctr + 1 + a.n_mb;
  int* udone = ps.ctr + 1 + 2 * a.n_mb;
  const int64_t total = P.cum(P.n_stages);
  for (;;) {
    if (threadIdx.x == 0) s_ticket = __hip_atomic_fetch_add(ps.ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int64_t t = s_ticket;
    if (t >= total) break;
    // stage s with cum(s) <= t < cum(s + 1)
    int lo = 0, hi = P.n_stages - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (P.cum(mid) <= t) lo = mid; else hi = mid - 1;
    }
    const int s = lo;
    int64_t o = t - P.cum(s);
    const int md = s - P.dl;
    const int64_t nd = (md >= 0 && md < P.n_mb) ? (int64_t)P.ntd * (P.tiles_before(md + 1) - P.tiles_before(md)) : 0;
    if (o < nd) {                                                  // D(md, r, n)
      const int ti = P.tiles_before(md) + (int)(o / P.ntd);
      wait_for(udone + ti, P.ntu, ps.status);
      down_tile<F8>(a, lds_raw, rows, md, ti, (int)(o % P.ntd));
      signal_done(ddone + md);
      continue;
    }
    o -= nd;
    const int ng = P.gi(s);
    if (o < ng) {                                                  // G(s, c)
      const int mp = s - a.n_slots;
      if (mp >= 0) wait_for(ddone + mp, P.ntd * (P.tiles_before(mp + 1) - P.tiles_before(mp)), ps.status);
      gather_item(a, ps, F8, s, (int)o);
      signal_done(gdone + s);
      continue;
    }
    o -= ng;                                                       // U(mu, r, n)
    const int mu = s - P.ul;
    const int ti = P.tiles_before(mu) + (int)(o / P.ntu);
    wait_for(gdone + mu, P.gi(mu), ps.status);
    gateup_tile<F8>(a, lds_raw, mu, ti, (int)(o % P.ntu));
    signal_done(udone + ti);
  }
}

// ================================================================== backward
// Backward row-tile kernels: 1-D grid, logical tile L = (row tile, column
// tile) row-major in XCD-aware order; ny receives the column tile.
MOK_DEV bool bwd_tile(const mok_bwd_args& a, int ncol, mok_tile& t, int& ny) {
  const int L = xcd_tile(*a.n_tiles * ncol);
  if (L < 0) return false;
  t = a.tiles[L / ncol];
  ny = L % ncol;
  return true;
}

// dh = dO . Wd[e] (K = H), then the SwiGLU backward from the saved a, b:
// dA = dh*b*s*(1 + a*(1-s)), dB = dh*a*s, h = a*s*b with s = sigmoid(a).
__global__ __launch_bounds__(kThreads, 1) void bwd_dh_kernel(mok_bwd_args a, int ncol) {
  using G = G256;
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[sizeof(Smem<G>)];
  Smem<G>& sm = *reinterpret_cast<Smem<G>*>(lds_raw);
  mok_tile t;
  int ny;
  if (!bwd_tile(a, ncol, t, ny)) return;
  const int nrows = t.p1 - t.p0;
  const int64_t H = a.H, I = a.I;
  const int n0 = ny * G::BN;
  LoadKD<G::BM, RowsStrided> la{{reinterpret_cast<const uint8_t*>(a.dO + (int64_t)t.p0 * H), 2 * H, nrows}};
  const LoadKO<G::BN> lb{reinterpret_cast<const uint8_t*>(a.wd + (int64_t)t.e * H * I + n0),
                        reinterpret_cast<const uint8_t*>(a.wd + (int64_t)t.e * H * I + n0), 0x7FFFFFFF,
                        2 * I, (int)H, (int)min<int64_t>(G::BN, I - n0)};
  NoScales ns;
  Acc<G::FM, G::FN> acc;
  mainloop<G, false>(sm, la, lb, ns, ns, (int)(H / 32), acc);
  // dA, dB and h per element from an fp32 half-tile of dh in LDS and the
  // saved a, b (16-byte loads and stores along the row).
  using HS = HalfF32<G>;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (half) __syncthreads();
    HS::put(lds_raw, acc, half);
    __syncthreads();
    const int rows = min(128, nrows - 128 * half);
    for (int idx = threadIdx.x; idx < 128 * (G::BN / 8); idx += kThreads) {
      const int r = idx / (G::BN / 8), c = (idx % (G::BN / 8)) * 8;
      if (r >= rows || n0 + c >= I) continue;
      const int64_t p = t.p0 + 128 * half + r;
      float dh[8], av[8], bv[8], da[8], db[8], h[8];
      HS::get8(lds_raw, r, c, dh);
      unpack_bf16x8(*reinterpret_cast<const uint4*>(a.ab + p * 2 * I + n0 + c), av);
      unpack_bf16x8(*reinterpret_cast<const uint4*>(a.ab + p * 2 * I + I + n0 + c), bv);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float sg = sigmoidf_(av[u]);
        da[u] = dh[u] * bv[u] * sg * (1.0f + av[u] * (1.0f - sg));
        db[u] = dh[u] * av[u] * sg;
        h[u] = av[u] * sg * bv[u];
      }
      *reinterpret_cast<uint4*>(a.dab + p * 2 * I + n0 + c) = pack_bf16x8(da);
      *reinterpret_cast<uint4*>(a.dab + p * 2 * I + I + n0 + c) = pack_bf16x8(db);
      *reinterpret_cast<uint4*>(a.hb + p * I + n0 + c) = pack_bf16x8(h);
    }
  }
}

// dX rows = [dA | dB] . [Wg[e]; Wu[e]] (K = 2I); row p goes to flat row perm[p].
__global__ __launch_bounds__(kThreads, 1) void bwd_dx_kernel(mok_bwd_args a, int ncol) {
  using G = G256;
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[sizeof(Smem<G>)];
  __shared__ int rows[G::BM];
  Smem<G>& sm = *reinterpret_cast<Smem<G>*>(lds_raw);
  mok_tile t;
  int ny;
  if (!bwd_tile(a, ncol, t, ny)) return;
  const int nrows = t.p1 - t.p0;
  const int64_t H = a.H, I = a.I;
  const int n0 = ny * G::BN;
  for (int r = threadIdx.x; r < G::BM; r += kThreads) rows[r] = r < nrows ? a.perm[t.p0 + r] : 0;
  LoadKD<G::BM, RowsStrided> la{{reinterpret_cast<const uint8_t*>(a.dab + (int64_t)t.p0 * 2 * I), 4 * I, nrows}};
  // row k of [Wg[e]; Wu[e]]: Wg row k for k < I, Wu row k - I beyond
  const LoadKO<G::BN> lb{reinterpret_cast<const uint8_t*>(a.wg + (int64_t)t.e * I * H + n0),
                        reinterpret_cast<const uint8_t*>(a.wu + (int64_t)t.e * I * H + n0), (int)I,
                        2 * H, (int)(2 * I), (int)min<int64_t>(G::BN, H - n0)};
  NoScales ns;
  Acc<G::FM, G::FN> acc;
  mainloop<G, false>(sm, la, lb, ns, ns, (int)(2 * I / 32), acc);
  bf16_t* d = a.dxrows + n0;
  store_tile_bf16<G>(lds_raw, acc, nrows, (int)(H - n0),
                     [&](int r) { return d + (int64_t)rows[r] * H; });
}

// Weight gradients out[m][n] = sum over the expert's rows p (ascending) of
// A[p][m] * B[p][n]; both operands K-outer.
MOK_DEV void dw_tile(uint8_t* lds_raw, const bf16_t* A, int64_t lda, int mlimit, const bf16_t* B,
                     int64_t ldb, int nlimit, int K, bf16_t* out, int64_t ldo) {
  using G = G256;
  Smem<G>& sm = *reinterpret_cast<Smem<G>*>(lds_raw);
  const LoadKO<G::BM> la{reinterpret_cast<const uint8_t*>(A), reinterpret_cast<const uint8_t*>(A),
                        0x7FFFFFFF, 2 * lda, K, mlimit};
  const LoadKO<G::BN> lb{reinterpret_cast<const uint8_t*>(B), reinterpret_cast<const uint8_t*>(B),
                        0x7FFFFFFF, 2 * ldb, K, nlimit};
  NoScales ns;
  Acc<G::FM, G::FN> acc;
  mainloop<G, false>(sm, la, lb, ns, ns, (K + 31) / 32, acc);
  store_tile_bf16<G>(lds_raw, acc, mlimit, nlimit, [&](int r) { return out + (int64_t)r * ldo; });
}

__global__ __launch_bounds__(kThreads, 1) void bwd_dwd_kernel(mok_bwd_args a, int tiles_per_e) {
  using G = G256;
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[sizeof(Smem<G>)];
  const int L = xcd_tile(a.E * tiles_per_e);
  if (L < 0) return;
  const int e = L / tiles_per_e, tl = L % tiles_per_e;
  const int64_t H = a.H, I = a.I;
  const int ntn = (int)((I + G::BN - 1) / G::BN);
  const int m0 = (tl / ntn) * G::BM, n0 = (tl % ntn) * G::BN;
  const int o = a.offsets[e], c = a.offsets[e + 1] - o;
  dw_tile(lds_raw, a.dO + (int64_t)o * H + m0, H, (int)min<int64_t>(G::BM, H - m0),
          a.hb + (int64_t)o * I + n0, I, (int)min<int64_t>(G::BN, I - n0), c,
          a.dwd + (int64_t)e * H * I + (int64_t)m0 * I + n0, I);
}

__global__ __launch_bounds__(kThreads, 1) void bwd_dwgu_kernel(mok_bwd_args a, int tiles_per_e) {
  using G = G256;
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[sizeof(Smem<G>)];
  const int L = xcd_tile(a.E * tiles_per_e);
  if (L < 0) return;
  const int e = L / tiles_per_e, tl = L % tiles_per_e;
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
  const int mlim = (int)min<int64_t>(G::BM, I - m0);
  const int o = a.offsets[e], c = a.offsets[e + 1] - o;
  bf16_t* out = (up ? a.dwu : a.dwg) + (int64_t)e * I * H + (int64_t)m0 * H + n0;
  dw_tile(lds_raw, a.dab + (int64_t)o * 2 * I + (up ? I : 0) + m0, 2 * I, mlim,
          a.xg + (int64_t)o * H + n0, H, (int)min<int64_t>(G::BN, H - n0), c, out, H);
}

unsigned cdivu(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

}  // namespace

unsigned grid8(int64_t n) { return (unsigned)((n + kXcds - 1) / kXcds * kXcds); }

hipError_t mok_launch_gateup(const mok_fwd_args& a, int m, int max_tiles_mb, bool mxfp8,
                             hipStream_t st) {
  const int ncol = (int)cdivu(a.I, G256::BN / 2);
  const dim3 grid(grid8((int64_t)max_tiles_mb * ncol));
  if (mxfp8) hipLaunchKernelGGL(gateup_kernel<true>, grid, dim3(kThreads), 0, st, a, m, ncol);
  else hipLaunchKernelGGL(gateup_kernel<false>, grid, dim3(kThreads), 0, st, a, m, ncol);
  return hipGetLastError();
}

hipError_t mok_launch_down(const mok_fwd_args& a, int m, int max_tiles_mb, bool mxfp8,
                           hipStream_t st) {
  const int ncol = (int)cdivu(a.H, G256::BN);
  const dim3 grid(grid8((int64_t)max_tiles_mb * ncol));
  if (mxfp8) hipLaunchKernelGGL(down_kernel<true>, grid, dim3(kThreads), 0, st, a, m, ncol);
  else hipLaunchKernelGGL(down_kernel<false>, grid, dim3(kThreads), 0, st, a, m, ncol);
  return hipGetLastError();
}

hipError_t mok_launch_fwd_persistent(const mok_fwd_args& a, int* counters, int32_t* status,
                                     const void* xsrc, const uint8_t* xscales,
                                     const int32_t* offsets_E, int grid, bool mxfp8, hipStream_t st) {
  mok_persist_args ps;
  ps.ctr = counters;
  ps.status = status;
  ps.xsrc = static_cast<const uint8_t*>(xsrc);
  ps.xscales = xscales;
  ps.offsets_E = offsets_E;
  if (mxfp8) hipLaunchKernelGGL(fwd_persistent_kernel<true>, dim3(grid), dim3(kThreads), 0, st, a, ps);
  else hipLaunchKernelGGL(fwd_persistent_kernel<false>, dim3(grid), dim3(kThreads), 0, st, a, ps);
  return hipGetLastError();
}

hipError_t mok_launch_bwd_dh(const mok_bwd_args& a, hipStream_t st) {
  const int ncol = (int)cdivu(a.I, G256::BN);
  hipLaunchKernelGGL(bwd_dh_kernel, dim3(grid8((int64_t)a.max_tiles * ncol)), dim3(kThreads), 0, st, a, ncol);
  return hipGetLastError();
}

hipError_t mok_launch_bwd_dx(const mok_bwd_args& a, hipStream_t st) {
  const int ncol = (int)cdivu(a.H, G256::BN);
  hipLaunchKernelGGL(bwd_dx_kernel, dim3(grid8((int64_t)a.max_tiles * ncol)), dim3(kThreads), 0, st, a, ncol);
  return hipGetLastError();
}

hipError_t mok_launch_bwd_dwd(const mok_bwd_args& a, hipStream_t st) {
  const int tpe = (int)(cdivu(a.H, G256::BM) * cdivu(a.I, G256::BN));
  hipLaunchKernelGGL(bwd_dwd_kernel, dim3(grid8((int64_t)a.E * tpe)), dim3(kThreads), 0, st, a, tpe);
  return hipGetLastError();
}

hipError_t mok_launch_bwd_dwgu(const mok_bwd_args& a, hipStream_t st) {
  const int tpe = (int)(2 * cdivu(a.I, G256::BM) * cdivu(a.H, G256::BN));
  hipLaunchKernelGGL(bwd_dwgu_kernel, dim3(grid8((int64_t)a.E * tpe)), dim3(kThreads), 0, st, a, tpe);
  return hipGetLastError();
}
