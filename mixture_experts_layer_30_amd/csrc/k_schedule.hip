// Routing schedule on the device, no host synchronisation.
//
// [MoK clip] Key points, bullet 4: the schedule table is generated entirely on
// the GPU and routed-token counts never travel to the CPU. [MoK card] "Using
// the functional API": the schedule is built from the top-k expert choices.
//
// One workgroup of 16 wavefronts does the whole job:
//   1. each wave owns a contiguous chunk of flat rows and builds a histogram
//      of expert ids in LDS; ties inside a 64-row step are ranked with
//      wavefront ballots (no atomics, so ranks are stable by row index);
//   2. per-expert totals, their exclusive scan (offsets) and each wave's base
//      position inside every expert segment;
//   3. the ranking is replayed to scatter perm[p] = i and dest[i] = p;
//   4. the row-tile tables for the grouped GEMMs.
// Rows whose id lies outside [0, E) go to an extra bucket E placed after all
// valid rows; they set status bit 0.
#include "mok_device.h"
#include "mok_launch.h"

namespace {

constexpr int kWaves = 16;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxBuckets = 513;   // E <= 512 plus the invalid bucket

MOK_DEV uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Mask of active lanes that hold the same bucket as this lane.
MOK_DEV uint64_t match_mask(int v, bool active, int nbits) {
  uint64_t m = __ballot(active);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (v >> b) & 1;
    const uint64_t bb = __ballot(active && bit);
    m &= bit ? bb : ~bb;
  }
  return m;
}

// Exclusive scan of one int per thread over the whole 1024-thread block.
MOK_DEV int block_exclusive_scan(int v, int* sums, int* total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  int incl = v;
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  if (lane == 63) sums[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int s = lane < kWaves ? sums[lane] : 0;
    int si = s;
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(si, d);
      if (lane >= d) si += o;
    }
    if (lane < kWaves) sums[kWaves + lane] = si - s;
    if (lane == kWaves - 1) sums[2 * kWaves] = si;
  }
  __syncthreads();
  const int r = incl - v + sums[kWaves + wave];
  if (total) *total = sums[2 * kWaves];
  __syncthreads();
  return r;
}

// Number of row tiles of the segment [lo, hi) when cut at multiples of `cut`
// and split into pieces of at most `bm` rows.
MOK_DEV int count_tiles(int lo, int hi, int cut, int bm) {
  int n = 0;
  for (int p = lo; p < hi;) {
    const int end = min(hi, (p / cut + 1) * cut);
    n += (end - p + bm - 1) / bm;
    p = end;
  }
  return n;
}

MOK_DEV void write_tiles(mok_tile* out, int room, int e, int lo, int hi, int cut, int bm) {
  int n = 0;
  for (int p = lo; p < hi;) {
    const int end = min(hi, (p / cut + 1) * cut);
    for (int q = p; q < end && n < room; q += bm) {
      mok_tile t;
      t.e = e; t.p0 = q; t.p1 = min(q + bm, end); t.m = q / cut;
      out[n++] = t;
    }
    p = end;
  }
}

__global__ __launch_bounds__(kThreads) void schedule_kernel(const int32_t* __restrict__ ids,
                                                          mok_sched_ptrs s, int R, int E,
                                                          int M, int bm_f, int bm_b, int n_mb,
                                                          int max_f, int max_b) {
  __shared__ int hist[kWaves][kMaxBuckets];
  __shared__ int sums[2 * kWaves + 1];
  __shared__ int s_off[kMaxBuckets];
  __shared__ int s_flag;

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int nb = E + 1;                                  // buckets incl. invalid
  const int nbits = 32 - __clz(E);                       // bits for values 0..E
  for (int v = tid; v < kWaves * kMaxBuckets; v += kThreads) (&hist[0][0])[v] = 0;
  if (tid == 0) s_flag = 0;
  __syncthreads();

  const int chunk = ((R + kWaves - 1) / kWaves + 63) & ~63;
  const int lo = min(R, wave * chunk), hi = min(R, lo + chunk);

  // 1. histogram per wave chunk
  for (int base = lo; base < hi; base += 64) {
    const int i = base + lane;
    const bool act = i < hi;
    int v = 0;
    if (act) {
      const int id = ids[i];
      v = (id >= 0 && id < E) ? id : E;
    }
    const uint64_t m = match_mask(v, act, nbits);
    if (act && (m & lanemask_lt()) == 0) hist[wave][v] += __popcll(m);
  }
  __syncthreads();

  // 2. totals, exclusive scan over buckets, per-wave bases
  int my_count = 0;
  if (tid < nb) {
    int run = 0;
    for (int w = 0; w < kWaves; ++w) {
      const int c = hist[w][tid];
      hist[w][tid] = run;
      run += c;
    }
    my_count = run;
  }
  int nvalid_total = 0;
  const int excl = block_exclusive_scan(tid < nb ? my_count : 0, sums, &nvalid_total);
  if (tid < nb) {
    s_off[tid] = excl;
    if (tid < E) s.counts[tid] = my_count;
    s.offsets[tid] = excl;                                // offsets[E] = valid rows
    if (tid == E && my_count > 0) s_flag = 1;
    for (int w = 0; w < kWaves; ++w) hist[w][tid] += excl;
  }
  __syncthreads();

  // 3. replay the ranking and scatter
  for (int base = lo; base < hi; base += 64) {
    const int i = base + lane;
    const bool act = i < hi;
    int v = 0;
    if (act) {
      const int id = ids[i];
      v = (id >= 0 && id < E) ? id : E;
    }
    const uint64_t m = match_mask(v, act, nbits);
    int p = 0;
    if (act) p = hist[wave][v] + __popcll(m & lanemask_lt());
    if (act && (m & lanemask_lt()) == 0) hist[wave][v] += __popcll(m);
    if (act && (unsigned)p < (unsigned)R) {   // always true for a consistent ranking
      s.perm[p] = i;
      s.dest[i] = p;
    }
  }

  // 4. row tiles: forward tiles are cut at minibatch boundaries, backward not
  int nf = 0, nbk = 0;
  int lo_e = 0, hi_e = 0;
  if (tid < E) {
    lo_e = s_off[tid];
    hi_e = s_off[tid + 1];
    nf = count_tiles(lo_e, hi_e, M, bm_f);
    nbk = (hi_e - lo_e + bm_b - 1) / bm_b;
  }
  int total_f = 0, total_b = 0;
  const int start_f = block_exclusive_scan(nf, sums, &total_f);
  const int start_b = block_exclusive_scan(nbk, sums, &total_b);
  if (tid < E) {
    write_tiles(s.fwd_tiles + start_f, max_f - start_f, tid, lo_e, hi_e, M, bm_f);
    write_tiles(s.bwd_tiles + start_b, max_b - start_b, tid, lo_e, hi_e, 0x7FFFFFFF, bm_b);
  }
  total_f = min(total_f, max_f);
  total_b = min(total_b, max_b);
  if (tid == 0) {
    *s.n_fwd_tiles = total_f;
    *s.n_bwd_tiles = total_b;
    *s.status = s_flag ? 1 : 0;
  }
  __syncthreads();
  __threadfence_block();
  // first forward tile of each minibatch: tiles are in ascending p0
  for (int m = tid; m <= n_mb; m += kThreads) {
    const long long target = (long long)m * M;
    int a = 0, b = total_f;
    while (a < b) {
      const int c = (a + b) >> 1;
      if ((long long)s.fwd_tiles[c].p0 < target) a = c + 1; else b = c;
    }
    s.mb_tile_start[m] = a;
  }
}

}  // namespace

hipError_t mok_launch_schedule(const int32_t* ids, const mok_sched_ptrs& s, int R, int E,
                               int M, int bm_f, int bm_b, int n_mb, int max_f, int max_b,
                               hipStream_t st) {
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kThreads), 0, st, ids, s, R, E, M, bm_f,
                     bm_b, n_mb, max_f, max_b);
  return hipGetLastError();
}
