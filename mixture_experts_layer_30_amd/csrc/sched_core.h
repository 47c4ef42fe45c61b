// Device code of the routing schedule, shared by the three schedule launches
// (k_schedule.hip) and the single-launch layer (k_gemm.hip), which runs the
// same steps inside one persistent grid.
//
// [MoK clip] Key points, bullet 4: the schedule table is generated entirely on
// the GPU and routed-token counts never travel to the CPU. Deterministic: no
// atomics; ties are ranked by row index.
//   1. hist:    the rows are cut into chunks of equal size; chunk c's
//               workgroup counts the expert ids of its rows (wavefront
//               ballots group equal ids inside a 64-row step);
//   2. scan:    one workgroup turns the chunk counts into per-expert totals,
//               their exclusive scan (offsets) and the base position of every
//               chunk inside every expert segment, then writes the row-tile
//               tables for the grouped GEMMs;
//   3. scatter: chunk c's workgroup replays the ranking of its rows and writes
//               perm[p] = i and dest[i] = p.
// Rows whose id lies outside [0, E) go to an extra bucket E placed after all
// valid rows; they set status bit 0.
#pragma once
#include "mok_device.h"
#include "mok_launch.h"

namespace mok_sched {

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

// Exclusive scan of one int per thread over an NT-thread block (sums: at
// least 2 * NT / 64 + 1 ints of LDS).
template <int NT>
MOK_DEV int block_exclusive_scan(int v, int* sums, int* total) {
  constexpr int kWaves = NT / 64;
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

// LDS of the chunk steps (per-wavefront bucket counts)
struct ChunkLds {
  int h[kChunkWaves][kMaxBuckets];
};

// Per-wavefront histograms of chunk c in LDS: h[w][v] += count.
MOK_DEV void chunk_histogram(const int32_t* ids, int R, int E, int chunk, int c, int nbits,
                             int (*h)[kMaxBuckets]) {
  const int lane = lane_id(), w = threadIdx.x >> 6;
  int lo, hi;
  wave_rows(c, w, R, chunk, lo, hi);
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

// 1. chunk counts: bh[c * nb + v] = rows of chunk c in bucket v (a
// kChunkThreads-thread workgroup)
MOK_DEV void sched_hist_chunk(const int32_t* __restrict__ ids, int R, int E, int chunk, int c,
                              int32_t* __restrict__ bh, ChunkLds& L) {
  const int nb = E + 1, nbits = 32 - __clz(E);
  for (int v = threadIdx.x; v < kChunkWaves * kMaxBuckets; v += kChunkThreads) (&L.h[0][0])[v] = 0;
  __syncthreads();
  chunk_histogram(ids, R, E, chunk, c, nbits, L.h);
  __syncthreads();
  for (int v = threadIdx.x; v < nb; v += kChunkThreads) {
    int t = 0;
#pragma unroll
    for (int w = 0; w < kChunkWaves; ++w) t += L.h[w][v];
    bh[(int64_t)c * nb + v] = t;
  }
}

// LDS of the scan step for an NT-thread workgroup
template <int NT>
struct ScanLds {
  int sums[2 * (NT / 64) + 1];
  int s_off[kMaxBuckets + 1];
  int s_cnt[kMaxBuckets];
  int s_flag;
};

// 2. totals, offsets, chunk bases (bh becomes the base of chunk c in bucket
// v), tile tables; one NT-thread workgroup. Thread tid owns the BPT
// consecutive buckets (and experts) from tid * BPT: with NT = 1024 one each.
// The status word gets bit 0 (bad expert ids); the bits in keep_bits that
// other workgroups may already have set in it (atomically, in a launch that
// also runs this scan, after clearing the word beforehand) are kept.
template <int NT>
MOK_DEV void sched_scan(const mok_sched_ptrs& s, int R, int E, int nchunks, int32_t* __restrict__ bh, int M,
                        int bm_f, int bm_b, int n_mb, int max_f, int max_b, ScanLds<NT>& L,
                        int32_t keep_bits = 0) {
  constexpr int BPT = (kMaxBuckets + NT - 1) / NT;
  const int tid = threadIdx.x, nb = E + 1;
  if (tid == 0) L.s_flag = 0;
  constexpr int kBatch = 16;                     // chunk counts loaded per round trip
  // the loads of a round cover all BPT buckets of the thread
  int run[BPT];
#pragma unroll
  for (int b = 0; b < BPT; ++b) run[b] = 0;
  if (tid * BPT < nb) {
    for (int c0 = 0; c0 < nchunks; c0 += kBatch) {
      int n[BPT][kBatch];
#pragma unroll
      for (int b = 0; b < BPT; ++b) {
        const int v = tid * BPT + b;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) n[b][u] = (v < nb && c0 + u < nchunks) ? bh[(int64_t)(c0 + u) * nb + v] : 0;
      }
#pragma unroll
      for (int b = 0; b < BPT; ++b)
#pragma unroll
        for (int u = 0; u < kBatch; ++u) run[b] += n[b][u];
    }
  }
  __syncthreads();
  int own = 0;
#pragma unroll
  for (int b = 0; b < BPT; ++b) own += run[b];
  int nvalid_total = 0;
  const int excl0 = block_exclusive_scan<NT>(own, L.sums, &nvalid_total);
  int base[BPT];
  {
    int excl = excl0;
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      const int v = tid * BPT + b;
      base[b] = excl;
      if (v < nb) {
        L.s_off[v] = excl;
        L.s_cnt[v] = run[b];
        if (v < E) s.counts[v] = run[b];
        s.offsets[v] = excl;                     // offsets[E] = valid rows
        if (v == E && run[b] > 0) L.s_flag = 1;
      }
      excl += run[b];
    }
  }
  if (tid * BPT < nb) {
    for (int c0 = 0; c0 < nchunks; c0 += kBatch) {
      int n[BPT][kBatch];
#pragma unroll
      for (int b = 0; b < BPT; ++b) {
        const int v = tid * BPT + b;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) n[b][u] = (v < nb && c0 + u < nchunks) ? bh[(int64_t)(c0 + u) * nb + v] : 0;
      }
#pragma unroll
      for (int b = 0; b < BPT; ++b) {
        const int v = tid * BPT + b;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          if (v < nb && c0 + u < nchunks) bh[(int64_t)(c0 + u) * nb + v] = base[b];
          base[b] += n[b][u];
        }
      }
    }
  }
  __syncthreads();

  // row tiles: forward tiles are cut at minibatch boundaries, backward not
  int nf[BPT], nbk[BPT], lo_e[BPT], hi_e[BPT];
  int own_f = 0, own_b = 0;
#pragma unroll
  for (int b = 0; b < BPT; ++b) {
    const int e = tid * BPT + b;
    nf[b] = nbk[b] = lo_e[b] = hi_e[b] = 0;
    if (e < E) {
      lo_e[b] = L.s_off[e];
      hi_e[b] = L.s_off[e + 1];
      nf[b] = count_tiles(lo_e[b], hi_e[b], M, bm_f);
      nbk[b] = (hi_e[b] - lo_e[b] + bm_b - 1) / bm_b;
    }
    own_f += nf[b];
    own_b += nbk[b];
  }
  int total_f = 0, total_b = 0;
  int start_f = block_exclusive_scan<NT>(own_f, L.sums, &total_f);
  int start_b = block_exclusive_scan<NT>(own_b, L.sums, &total_b);
  total_f = min(total_f, max_f);
  total_b = min(total_b, max_b);
  // First forward tile of each minibatch m: every m*M below the valid-row
  // count starts a tile (forward tiles are cut at multiples of M and expert
  // segments tile [0, valid rows)); minibatches past the valid rows start at
  // the end of the table.
  const int nvalid = L.s_off[E];
  for (int m = tid; m <= n_mb; m += NT)
    if ((int64_t)m * M >= nvalid) s.mb_tile_start[m] = total_f;
#pragma unroll
  for (int b = 0; b < BPT; ++b) {
    const int e = tid * BPT + b;
    if (e < E) {
      write_tiles(s.fwd_tiles + start_f, max_f - start_f, e, lo_e[b], hi_e[b], M, bm_f, s.mb_tile_start,
                  start_f);
      write_tiles(s.bwd_tiles + start_b, max_b - start_b, e, lo_e[b], hi_e[b], 0x7FFFFFFF, bm_b, nullptr, 0);
    }
    start_f += nf[b];
    start_b += nbk[b];
  }
  for (int q = tid; q < kTokPad; q += NT) s.tok[R + q] = 0;
  // experts by descending count, ties to the lower id: the rank of e is the
  // number of experts before it in that order
  for (int e = tid; e < E; e += NT) {
    const int ce = L.s_cnt[e];
    int rank = 0;
    for (int f = 0; f < E; ++f) {
      const int cf = L.s_cnt[f];
      rank += (cf > ce || (cf == ce && f < e)) ? 1 : 0;
    }
    s.eorder[rank] = e;
  }
  if (tid == 0) {
    *s.n_fwd_tiles = total_f;
    *s.n_bwd_tiles = total_b;
    if (keep_bits) {
      __hip_atomic_fetch_and(s.status, keep_bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_or(s.status, L.s_flag ? 1 : 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      *s.status = L.s_flag ? 1 : 0;
    }
  }
}

// 3. scatter: replay chunk c's ranking from its bases (a kChunkThreads-thread
// workgroup)
MOK_DEV void sched_scatter_chunk(const int32_t* __restrict__ ids, const mok_sched_ptrs& s, int R, int E,
                                 int topk, int chunk, int c, const int32_t* __restrict__ bh, ChunkLds& L) {
  const int nb = E + 1, nbits = 32 - __clz(E);
  const int lane = lane_id(), w = threadIdx.x >> 6;
  for (int v = threadIdx.x; v < kChunkWaves * kMaxBuckets; v += kChunkThreads) (&L.h[0][0])[v] = 0;
  __syncthreads();
  chunk_histogram(ids, R, E, chunk, c, nbits, L.h);
  __syncthreads();
  // h[w][v] <- base of wavefront w's rows in bucket v
  for (int v = threadIdx.x; v < nb; v += kChunkThreads) {
    int run = bh[(int64_t)c * nb + v];
#pragma unroll
    for (int ww = 0; ww < kChunkWaves; ++ww) {
      const int cnt = L.h[ww][v];
      L.h[ww][v] = run;
      run += cnt;
    }
  }
  __syncthreads();
  int lo, hi;
  wave_rows(c, w, R, chunk, lo, hi);
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
      if (act[u]) p = L.h[w][v[u]] + __popcll(m & lanemask_lt());
      if (act[u] && (m & lanemask_lt()) == 0) L.h[w][v[u]] += __popcll(m);
      if (act[u] && (unsigned)p < (unsigned)R) {   // always true for a consistent ranking
        s.perm[p] = i;
        s.dest[i] = p;
        s.tok[p] = i / topk;
      }
    }
  }
}

}  // namespace mok_sched
