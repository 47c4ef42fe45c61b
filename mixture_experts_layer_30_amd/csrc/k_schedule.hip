// Routing schedule on the device, no host synchronisation: three launches
// (hist, scan, scatter) of the steps in sched_core.h.
//
// [MoK clip] Key points, bullet 4: the schedule table is generated entirely on
// the GPU and routed-token counts never travel to the CPU. [MoK card] "Using
// the functional API": the schedule is built from the top-k expert choices.
#include "mok_device.h"
#include "mok_launch.h"
#include "sched_core.h"

#include <algorithm>

namespace {

using namespace mok_sched;

constexpr int kScanThreads = 1024;

// 1. chunk counts, one workgroup per chunk
__global__ __launch_bounds__(kChunkThreads) void sched_hist_kernel(const int32_t* __restrict__ ids,
                                                                 int R, int E, int chunk,
                                                                 int32_t* __restrict__ bh) {
  __shared__ ChunkLds L;
  sched_hist_chunk(ids, R, E, chunk, blockIdx.x, bh, L);
}

// 2. totals, offsets, chunk bases, tile tables
__global__ __launch_bounds__(kScanThreads) void sched_scan_kernel(mok_sched_ptrs s, int R, int E,
                                                                int nchunks, int32_t* __restrict__ bh,
                                                                int M, int bm_f, int bm_b, int n_mb,
                                                                int max_f, int max_b) {
  __shared__ ScanLds<kScanThreads> L;
  sched_scan<kScanThreads>(s, R, E, nchunks, bh, M, bm_f, bm_b, n_mb, max_f, max_b, L);
}

// 3. scatter, one workgroup per chunk
__global__ __launch_bounds__(kChunkThreads) void sched_scatter_kernel(const int32_t* __restrict__ ids,
                                                                    mok_sched_ptrs s, int R, int E,
                                                                    int topk, int chunk,
                                                                    const int32_t* __restrict__ bh) {
  __shared__ ChunkLds L;
  sched_scatter_chunk(ids, s, R, E, topk, chunk, blockIdx.x, bh, L);
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
