// Routing schedule on the device, no host synchronisation.
//
// [MoK clip] Key points, bullet 4: the schedule table is generated entirely on
// the GPU and routed-token counts never travel to the CPU. [MoK card] "Using
// the functional API": the schedule is built from the top-k expert choices.
//
// Three launches, each deterministic (no atomics; ties ranked by row index):
//   1. hist:    the rows are cut into chunks of equal size; each workgroup
//               counts the expert ids of its chunk (wavefront ballots group
//               equal ids inside a 64-row step);
//   2. scan:    one workgroup turns the chunk counts into per-expert totals,
//               their exclusive scan (offsets) and the base position of every
//               chunk inside every expert segment, then writes the row-tile
//               tables for the grouped GEMMs;
//   3. scatter: each workgroup replays the ranking of its chunk and writes
//               perm[p] = i and dest[i] = p.
// Rows whose id lies outside [0, E) go to an extra bucket E placed after all
// valid rows; they set status bit 0.
#include "mok_device.h"
#include "mok_launch.h"

#include <algorithm>

namespace {

constexpr int kScanThreads = 1024;
constexpr int kScanWaves = kScanThreads / 64;
constexpr int kChunkThreads = 256;               // 4 wavefronts per chunk
constexpr int kChunkWaves = kChunkThreads / 64;
constexpr int kMaxBuckets = 513;                 // E <= 512 plus the invalid bucket

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

// Exclusive scan of one int per thread over a 1024-thread block.
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
    int s = lane < kScanWaves ? sums[lane] : 0;
    int si = s;
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(si, d);
      if (lane >= d) si += o;
    }
    if (lane < kScanWaves) sums[kScanWaves + lane] = si - s;
    if (lane == kScanWaves - 1) sums[2 * kScanWaves] = si;
  }
  __syncthreads();
  const int r = incl - v + sums[kScanWaves + wave];
  if (total) *total = sums[2 * kScanWaves];
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

// Writes the tiles of one expert segment; with mb_start, a tile that begins
// at a multiple of `cut` records its table index (first + n) there.
MOK_DEV void write_tiles(mok_tile* out, int room, int e, int lo, int hi, int cut, int bm,
                         int32_t* mb_start, int first) {
  int n = 0;
  for (int p = lo; p < hi;) {
    const int end = min(hi, (p / cut + 1) * cut);
    for (int q = p; q < end && n < room; q += bm) {
      mok_tile t;
      t.e = e; t.p0 = q; t.p1 = min(q + bm, end); t.m = q / cut;
      if (mb_start && q % cut == 0) mb_start[q / cut] = first + n;
      out[n++] = t;
    }
    p = end;
  }
}

MOK_DEV int bucket_of(int id, int E) { return (id >= 0 && id < E) ? id : E; }

// Rows of chunk c handled by wavefront w: [lo, hi), contiguous, in order.
MOK_DEV void wave_rows(int c, int w, int R, int chunk, int& lo, int& hi) {
  const int per = chunk / kChunkWaves;           // chunk is a multiple of 256
  lo = min(R, c * chunk + w * per);
  hi = min(R, lo + per);
}

// Per-wavefront histograms of one chunk in LDS: h[w][v] += count.
MOK_DEV void chunk_histogram(const int32_t* ids, int R, int E, int chunk, int nbits,
                             int (*h)[kMaxBuckets]) {
  const int lane = lane_id(), w = threadIdx.x >> 6;
  int lo, hi;
  wave_rows(blockIdx.x, w, R, chunk, lo, hi);
  for (int base = lo; base < hi; base += 256) {
    int v[4];
    bool act[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {                // loads of 4 steps first
      const int i = base + 64 * u + lane;
      act[u] = i < hi;
      v[u] = act[u] ? bucket_of(ids[i], E) : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint64_t m = match_mask(v[u], act[u], nbits);
      if (act[u] && (m & lanemask_lt()) == 0) h[w][v[u]] += __popcll(m);
    }
  }
}

// 1. chunk counts: bh[c * nb + v] = rows of chunk c in bucket v
__global__ __launch_bounds__(kChunkThreads) void sched_hist_kernel(const int32_t* __restrict__ ids,
                                                                 int R, int E, int chunk,
                                                                 int32_t* __restrict__ bh) {
  __shared__ int h[kChunkWaves][kMaxBuckets];
  const int nb = E + 1, nbits = 32 - __clz(E);
  for (int v = threadIdx.x; v < kChunkWaves * kMaxBuckets; v += kChunkThreads) (&h[0][0])[v] = 0;
  __syncthreads();
  chunk_histogram(ids, R, E, chunk, nbits, h);
  __syncthreads();
  for (int v = threadIdx.x; v < nb; v += kChunkThreads) {
    int t = 0;
#pragma unroll
    for (int w = 0; w < kChunkWaves; ++w) t += h[w][v];
    bh[(int64_t)blockIdx.x * nb + v] = t;
  }
}

// 2. totals, offsets, chunk bases (bh becomes the base of chunk c in bucket
// v), tile tables
__global__ __launch_bounds__(kScanThreads) void sched_scan_kernel(mok_sched_ptrs s, int R, int E,
                                                                int nchunks, int32_t* __restrict__ bh,
                                                                int M, int bm_f, int bm_b, int n_mb,
                                                                int max_f, int max_b) {
  __shared__ int sums[2 * kScanWaves + 1];
  __shared__ int s_off[kMaxBuckets];
  __shared__ int s_flag;
  const int tid = threadIdx.x, nb = E + 1;
  if (tid == 0) s_flag = 0;
  constexpr int kBatch = 16;                     // chunk counts loaded per round trip
  int run = 0;
  if (tid < nb) {
    for (int c0 = 0; c0 < nchunks; c0 += kBatch) {
      int n[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) n[u] = c0 + u < nchunks ? bh[(int64_t)(c0 + u) * nb + tid] : 0;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) run += n[u];
    }
  }
  __syncthreads();
  int nvalid_total = 0;
  const int excl = block_exclusive_scan(tid < nb ? run : 0, sums, &nvalid_total);
  if (tid < nb) {
    s_off[tid] = excl;
    if (tid < E) s.counts[tid] = run;
    s.offsets[tid] = excl;                       // offsets[E] = valid rows
    if (tid == E && run > 0) s_flag = 1;
    int base = excl;
    for (int c0 = 0; c0 < nchunks; c0 += kBatch) {
      int n[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) n[u] = c0 + u < nchunks ? bh[(int64_t)(c0 + u) * nb + tid] : 0;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (c0 + u < nchunks) bh[(int64_t)(c0 + u) * nb + tid] = base;
        base += n[u];
      }
    }
  }
  __syncthreads();

  // row tiles: forward tiles are cut at minibatch boundaries, backward not
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
  total_f = min(total_f, max_f);
  total_b = min(total_b, max_b);
  // First forward tile of each minibatch m: every m*M below the valid-row
  // count starts a tile (forward tiles are cut at multiples of M and expert
  // segments tile [0, valid rows)); minibatches past the valid rows start at
  // the end of the table.
  const int nvalid = s_off[E];
  for (int m = tid; m <= n_mb; m += kScanThreads)
    if ((int64_t)m * M >= nvalid) s.mb_tile_start[m] = total_f;
  if (tid < E) {
    write_tiles(s.fwd_tiles + start_f, max_f - start_f, tid, lo_e, hi_e, M, bm_f, s.mb_tile_start,
                start_f);
    write_tiles(s.bwd_tiles + start_b, max_b - start_b, tid, lo_e, hi_e, 0x7FFFFFFF, bm_b, nullptr, 0);
  }
  for (int q = tid; q < kTokPad; q += kScanThreads) s.tok[R + q] = 0;
  if (tid == 0) {
    *s.n_fwd_tiles = total_f;
    *s.n_bwd_tiles = total_b;
    *s.status = s_flag ? 1 : 0;
  }
}

// 3. scatter: replay the chunk's ranking from its bases
__global__ __launch_bounds__(kChunkThreads) void sched_scatter_kernel(const int32_t* __restrict__ ids,
                                                                    mok_sched_ptrs s, int R, int E,
                                                                    int topk, int chunk,
                                                                    const int32_t* __restrict__ bh) {
  __shared__ int h[kChunkWaves][kMaxBuckets];
  const int nb = E + 1, nbits = 32 - __clz(E);
  const int lane = lane_id(), w = threadIdx.x >> 6;
  for (int v = threadIdx.x; v < kChunkWaves * kMaxBuckets; v += kChunkThreads) (&h[0][0])[v] = 0;
  __syncthreads();
  chunk_histogram(ids, R, E, chunk, nbits, h);
  __syncthreads();
  // h[w][v] <- base of wavefront w's rows in bucket v
  for (int v = threadIdx.x; v < nb; v += kChunkThreads) {
    int run = bh[(int64_t)blockIdx.x * nb + v];
#pragma unroll
    for (int ww = 0; ww < kChunkWaves; ++ww) {
      const int c = h[ww][v];
      h[ww][v] = run;
      run += c;
    }
  }
  __syncthreads();
  int lo, hi;
  wave_rows(blockIdx.x, w, R, chunk, lo, hi);
  for (int base = lo; base < hi; base += 256) {
    int v[4];
    bool act[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = base + 64 * u + lane;
      act[u] = i < hi;
      v[u] = act[u] ? bucket_of(ids[i], E) : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = base + 64 * u + lane;
      const uint64_t m = match_mask(v[u], act[u], nbits);
      int p = 0;
      if (act[u]) p = h[w][v[u]] + __popcll(m & lanemask_lt());
      if (act[u] && (m & lanemask_lt()) == 0) h[w][v[u]] += __popcll(m);
      if (act[u] && (unsigned)p < (unsigned)R) {   // always true for a consistent ranking
        s.perm[p] = i;
        s.dest[i] = p;
        s.tok[p] = i / topk;
      }
    }
  }
}

}  // namespace

int mok_schedule_chunk_rows(int64_t R) {
  // rows per chunk: a multiple of 256 rows, at least 1024, at most 2048 chunks
  const int64_t per = (R + 2047) / 2048;
  return (int)std::max<int64_t>(1024, (per + 255) / 256 * 256);
}

hipError_t mok_launch_schedule(const int32_t* ids, const mok_sched_ptrs& s, int R, int E,
                               int topk, int M, int bm_f, int bm_b, int n_mb, int max_f, int max_b,
                               int32_t* chunk_counts, hipStream_t st) {
  const int chunk = mok_schedule_chunk_rows(R);
  const int nchunks = (R + chunk - 1) / chunk;
  if (nchunks > 0)
    hipLaunchKernelGGL(sched_hist_kernel, dim3(nchunks), dim3(kChunkThreads), 0, st, ids, R, E, chunk,
                       chunk_counts);
  hipLaunchKernelGGL(sched_scan_kernel, dim3(1), dim3(kScanThreads), 0, st, s, R, E, nchunks,
                     chunk_counts, M, bm_f, bm_b, n_mb, max_f, max_b);
  if (nchunks > 0)
    hipLaunchKernelGGL(sched_scatter_kernel, dim3(nchunks), dim3(kChunkThreads), 0, st, ids, s, R, E,
                       topk, chunk, chunk_counts);
  return hipGetLastError();
}
