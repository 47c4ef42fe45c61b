// Grouped GEMMs of the expert SwiGLU FFN on gfx950 matrix cores (bf16 MFMA).
//
// [MoK clip] Key points, bullet 5 and the key chart: the expert FFN with its
// SwiGLU is the compute stage between dispatch and combine; bullet 3: it runs
// as one grouped GEMM per expert over a minibatch of routed rows.
//
// Every GEMM here is C[BM x BN] = sum_k A[m][k] * B[n][k] on a 128 x 128 tile
// with a K step of 64, four wavefronts in a 2 x 2 grid, each owning a 64 x 64
// block built from 2 x 2 v_mfma_f32_32x32x16_bf16. Operand tiles are staged
// through LDS (double-buffered) as [row][64] bf16 with 16-byte chunks XOR-
// swizzled by row, so both the global->LDS copy and the MFMA operand reads are
// free of bank conflicts. Two loaders fill a tile:
//   LoadK  - the operand is K-contiguous in memory (weights of the forward
//            GEMMs, gathered token rows, dO rows ...): 16-byte row chunks.
//   LoadT  - the operand is K-outer (element (m, k) at base + k*ld + m), as
//            in the backward GEMMs: 4 k-rows x 8 m are loaded and transposed
//            in registers before the LDS write.
// Each output element is owned by exactly one workgroup and summed over K in
// ascending order, so results are bitwise reproducible (no split-K, no
// atomics).
#include "mok_device.h"
#include "mok_launch.h"

namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int NTHR = 256;
constexpr int TILE = BM * BK;            // bf16 elements per operand tile

struct Smem {
  bf16_t a[2][TILE];
  bf16_t b[2][TILE];
  int rows[BM];
};

MOK_DEV int lds_off(int r, int chunk) { return r * BK + ((chunk ^ (r & 7)) << 3); }

// ------------------------------------------------------------------ loaders
struct LoadK {
  const uint8_t* row[4];                 // address of element k = 0 of each of this thread's rows
  uint4 v[4];
  MOK_DEV void fetch(int kt) {
    const int off = kt * (BK * 2) + (threadIdx.x & 7) * 16;
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = *reinterpret_cast<const uint4*>(row[q] + off);
  }
  MOK_DEV void put(bf16_t* t) const {
    const int c = threadIdx.x & 7;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = (threadIdx.x >> 3) + 32 * q;
      *reinterpret_cast<uint4*>(t + lds_off(r, c)) = v[q];
    }
  }
  MOK_DEV static int my_row(int q) { return (threadIdx.x >> 3) + 32 * q; }
};

struct LoadT {
  const bf16_t* base0;                   // used for k < ksplit
  const bf16_t* base1;                   // used for k >= ksplit
  int ksplit;
  int64_t ld;
  int K;                                 // k >= K reads as zero
  uint4 v[4];
  MOK_DEV void fetch(int kt) {
    const int kq = threadIdx.x & 15, mc = threadIdx.x >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = kt * BK + 4 * kq + i;
      if (k < K) {
        const bf16_t* b = k < ksplit ? base0 : base1;
        v[i] = *reinterpret_cast<const uint4*>(b + (int64_t)k * ld + 8 * mc);
      } else {
        v[i] = make_uint4(0, 0, 0, 0);
      }
    }
  }
  MOK_DEV void put(bf16_t* t) const {
    const int kq = threadIdx.x & 15, mc = threadIdx.x >> 4;
    const uint32_t w0[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
    const uint32_t w1[4] = {v[1].x, v[1].y, v[1].z, v[1].w};
    const uint32_t w2[4] = {v[2].x, v[2].y, v[2].z, v[2].w};
    const uint32_t w3[4] = {v[3].x, v[3].y, v[3].z, v[3].w};
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const uint32_t sel = (m & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t lo = __builtin_amdgcn_perm(w1[m >> 1], w0[m >> 1], sel);
      const uint32_t hi = __builtin_amdgcn_perm(w3[m >> 1], w2[m >> 1], sel);
      const int r = 8 * mc + m;
      *reinterpret_cast<uint2*>(t + lds_off(r, kq >> 1) + (kq & 1) * 4) = make_uint2(lo, hi);
    }
  }
};

// ------------------------------------------------------------------ MFMA core
struct Acc {
  f32x16_t c[2][2];
};

MOK_DEV void mma_stage(const bf16_t* ta, const bf16_t* tb, Acc& acc) {
  const int lane = lane_id(), w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;
  const int lr = lane & 31, lk = lane >> 5;
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    bf16x8_t a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = wm * 64 + i * 32 + lr;
      a[i] = *reinterpret_cast<const bf16x8_t*>(ta + lds_off(r, 2 * kk + lk));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = wn * 64 + j * 32 + lr;
      b[j] = *reinterpret_cast<const bf16x8_t*>(tb + lds_off(r, 2 * kk + lk));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc.c[i][j], 0, 0, 0);
  }
}

template <class LA, class LB>
MOK_DEV void mainloop(Smem& sm, LA& la, LB& lb, int nk, Acc& acc) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc.c[i][j][q] = 0.f;
  __syncthreads();                       // sm.rows and previous use of the buffers
  if (nk <= 0) return;
  la.fetch(0);
  lb.fetch(0);
  la.put(sm.a[0]);
  lb.put(sm.b[0]);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      la.fetch(kt + 1);
      lb.fetch(kt + 1);
    }
    mma_stage(sm.a[cur], sm.b[cur], acc);
    if (more) {
      la.put(sm.a[cur ^ 1]);
      lb.put(sm.b[cur ^ 1]);
    }
    __syncthreads();
  }
}

// Output coordinates of accumulator element q of block (i, j) of this lane.
MOK_DEV int out_row(int i, int q) {
  const int w = threadIdx.x >> 6, lane = lane_id();
  return (w >> 1) * 64 + i * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
}
MOK_DEV int out_col(int j) {
  const int w = threadIdx.x >> 6, lane = lane_id();
  return (w & 1) * 64 + j * 32 + (lane & 31);
}

// ================================================================== forward
// gate/up GEMM of one row tile x 64 h-columns. The B tile interleaves 32-row
// groups of Wg and Wu so that wave column wn holds gate (j = 0) and up (j = 1)
// for the same 32 h-columns; the SwiGLU runs on the accumulators.
__global__ __launch_bounds__(NTHR, 2) void gateup_bf16_kernel(mok_fwd_args a, int m) {
  __shared__ Smem sm;
  const int ti = a.mb_tile_start[m] + (int)blockIdx.x;
  if (ti >= a.mb_tile_start[m + 1]) return;
  const mok_tile tile = a.tiles[ti];
  const int nrows = tile.p1 - tile.p0;
  const int64_t H = a.H, I = a.I, M = a.M;
  const int n0 = blockIdx.y * 64;
  const int64_t slot_row0 = (int64_t)(m % a.n_slots) * M + (tile.p0 - (int64_t)m * M);
  const bf16_t* xs = reinterpret_cast<const bf16_t*>(a.ring_x) + slot_row0 * H;
  const bf16_t* wg = reinterpret_cast<const bf16_t*>(a.wg) + (int64_t)tile.e * I * H;
  const bf16_t* wu = reinterpret_cast<const bf16_t*>(a.wu) + (int64_t)tile.e * I * H;
  LoadK la, lb;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = LoadK::my_row(q);
    la.row[q] = reinterpret_cast<const uint8_t*>(xs + (int64_t)min(r, nrows - 1) * H);
    const int g = r >> 5;
    const int col = n0 + (g >> 1) * 32 + (r & 31);
    lb.row[q] = reinterpret_cast<const uint8_t*>(((g & 1) ? wu : wg) + (int64_t)col * H);
  }
  Acc acc;
  mainloop(sm, la, lb, (int)(H / BK), acc);

  bf16_t* hs = reinterpret_cast<bf16_t*>(a.ring_h) + slot_row0 * I;
  const int col = n0 + ((threadIdx.x >> 6) & 1) * 32 + (lane_id() & 31);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int r = out_row(i, q);
      if (r >= nrows) continue;
      const float av = acc.c[i][0][q], bv = acc.c[i][1][q];
      const float h = av * sigmoidf_(av) * bv;
      hs[(int64_t)r * I + col] = f32_to_bf16(h);
      if (a.ab) {
        bf16_t* abr = a.ab + (int64_t)(tile.p0 + r) * 2 * I;
        abr[col] = f32_to_bf16(av);
        abr[I + col] = f32_to_bf16(bv);
      }
    }
}

// down GEMM of one row tile x 128 output columns; each row is pushed to its
// flat position perm[p] of obuf (unique destinations, no atomics).
__global__ __launch_bounds__(NTHR, 2) void down_bf16_kernel(mok_fwd_args a, int m) {
  __shared__ Smem sm;
  const int ti = a.mb_tile_start[m] + (int)blockIdx.x;
  if (ti >= a.mb_tile_start[m + 1]) return;
  const mok_tile tile = a.tiles[ti];
  const int nrows = tile.p1 - tile.p0;
  const int64_t H = a.H, I = a.I, M = a.M;
  const int n0 = blockIdx.y * BN;
  const int64_t slot_row0 = (int64_t)(m % a.n_slots) * M + (tile.p0 - (int64_t)m * M);
  const bf16_t* hs = reinterpret_cast<const bf16_t*>(a.ring_h) + slot_row0 * I;
  const bf16_t* wd = reinterpret_cast<const bf16_t*>(a.wd) + (int64_t)tile.e * H * I;
  if (threadIdx.x < BM) sm.rows[threadIdx.x] = threadIdx.x < nrows ? a.perm[tile.p0 + threadIdx.x] : 0;
  LoadK la, lb;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = LoadK::my_row(q);
    la.row[q] = reinterpret_cast<const uint8_t*>(hs + (int64_t)min(r, nrows - 1) * I);
    lb.row[q] = reinterpret_cast<const uint8_t*>(wd + (int64_t)(n0 + r) * I);
  }
  Acc acc;
  mainloop(sm, la, lb, (int)(I / BK), acc);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int r = out_row(i, q);
      if (r >= nrows) continue;
      bf16_t* orow = a.obuf + (int64_t)sm.rows[r] * H + n0;
#pragma unroll
      for (int j = 0; j < 2; ++j) orow[out_col(j)] = f32_to_bf16(acc.c[i][j][q]);
    }
}

// ================================================================== backward
// dh = dO . Wd[e] (K = H), then the SwiGLU backward from the saved a, b:
// dA = dh*b*s*(1 + a*(1-s)), dB = dh*a*s, h = a*s*b with s = sigmoid(a).
__global__ __launch_bounds__(NTHR, 2) void bwd_dh_kernel(mok_bwd_args a) {
  __shared__ Smem sm;
  const int ti = (int)blockIdx.x;
  if (ti >= *a.n_tiles) return;
  const mok_tile tile = a.tiles[ti];
  const int nrows = tile.p1 - tile.p0;
  const int64_t H = a.H, I = a.I;
  const int n0 = blockIdx.y * BN;
  LoadK la;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = LoadK::my_row(q);
    la.row[q] = reinterpret_cast<const uint8_t*>(a.dO + (int64_t)(tile.p0 + min(r, nrows - 1)) * H);
  }
  LoadT lb;
  lb.base0 = lb.base1 = a.wd + (int64_t)tile.e * H * I + n0;
  lb.ksplit = 0x7FFFFFFF;
  lb.ld = I;
  lb.K = (int)H;
  Acc acc;
  mainloop(sm, la, lb, (int)(H / BK), acc);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int r = out_row(i, q);
      if (r >= nrows) continue;
      const int64_t p = tile.p0 + r;
      const bf16_t* abr = a.ab + p * 2 * I;
      bf16_t* dr = a.dab + p * 2 * I;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = n0 + out_col(j);
        const float av = bf16_to_f32(abr[c]), bv = bf16_to_f32(abr[I + c]);
        const float s = sigmoidf_(av), dh = acc.c[i][j][q];
        dr[c] = f32_to_bf16(dh * bv * s * (1.0f + av * (1.0f - s)));
        dr[I + c] = f32_to_bf16(dh * av * s);
        a.hb[p * I + c] = f32_to_bf16(av * s * bv);
      }
    }
}

// dX rows = [dA | dB] . [Wg[e]; Wu[e]] (K = 2I); row p goes to flat row perm[p].
__global__ __launch_bounds__(NTHR, 2) void bwd_dx_kernel(mok_bwd_args a) {
  __shared__ Smem sm;
  const int ti = (int)blockIdx.x;
  if (ti >= *a.n_tiles) return;
  const mok_tile tile = a.tiles[ti];
  const int nrows = tile.p1 - tile.p0;
  const int64_t H = a.H, I = a.I;
  const int n0 = blockIdx.y * BN;
  if (threadIdx.x < BM) sm.rows[threadIdx.x] = threadIdx.x < nrows ? a.perm[tile.p0 + threadIdx.x] : 0;
  LoadK la;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = LoadK::my_row(q);
    la.row[q] = reinterpret_cast<const uint8_t*>(a.dab + (int64_t)(tile.p0 + min(r, nrows - 1)) * 2 * I);
  }
  LoadT lb;
  lb.base0 = a.wg + (int64_t)tile.e * I * H + n0;
  lb.base1 = a.wu + (int64_t)tile.e * I * H + n0 - I * H;   // row k of [Wg; Wu] for k >= I
  lb.ksplit = (int)I;
  lb.ld = H;
  lb.K = (int)(2 * I);
  Acc acc;
  mainloop(sm, la, lb, (int)(2 * I / BK), acc);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int r = out_row(i, q);
      if (r >= nrows) continue;
      bf16_t* orow = a.dxrows + (int64_t)sm.rows[r] * H + n0;
#pragma unroll
      for (int j = 0; j < 2; ++j) orow[out_col(j)] = f32_to_bf16(acc.c[i][j][q]);
    }
}

// Weight gradients: out[m][n] = sum over the expert's rows p (ascending) of
// A[p][m] * B[p][n]; both operands K-outer. blockIdx.y = expert.
MOK_DEV void dw_tile(Smem& sm, const bf16_t* A, int64_t lda, const bf16_t* B, int64_t ldb,
                     int K, bf16_t* out, int64_t ldo) {
  LoadT la, lb;
  la.base0 = la.base1 = A;
  la.ksplit = 0x7FFFFFFF;
  la.ld = lda;
  la.K = K;
  lb.base0 = lb.base1 = B;
  lb.ksplit = 0x7FFFFFFF;
  lb.ld = ldb;
  lb.K = K;
  Acc acc;
  mainloop(sm, la, lb, (K + BK - 1) / BK, acc);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      bf16_t* orow = out + (int64_t)out_row(i, q) * ldo;
#pragma unroll
      for (int j = 0; j < 2; ++j) orow[out_col(j)] = f32_to_bf16(acc.c[i][j][q]);
    }
}

__global__ __launch_bounds__(NTHR, 2) void bwd_dwd_kernel(mok_bwd_args a) {
  __shared__ Smem sm;
  const int e = blockIdx.y;
  const int64_t H = a.H, I = a.I;
  const int ntn = (int)(I / BN);
  const int m0 = (blockIdx.x / ntn) * BM, n0 = (blockIdx.x % ntn) * BN;
  const int o = a.offsets[e], c = a.offsets[e + 1] - o;
  dw_tile(sm, a.dO + (int64_t)o * H + m0, H, a.hb + (int64_t)o * I + n0, I, c,
          a.dwd + (int64_t)e * H * I + (int64_t)m0 * I + n0, I);
}

__global__ __launch_bounds__(NTHR, 2) void bwd_dwgu_kernel(mok_bwd_args a) {
  __shared__ Smem sm;
  const int e = blockIdx.y;
  const int64_t H = a.H, I = a.I;
  const int ntn = (int)(H / BN);
  const int m0 = (blockIdx.x / ntn) * BM, n0 = (blockIdx.x % ntn) * BN;
  const int o = a.offsets[e], c = a.offsets[e + 1] - o;
  bf16_t* out = (m0 < I ? a.dwg + (int64_t)m0 * H : a.dwu + (int64_t)(m0 - I) * H) +
                (int64_t)e * I * H + n0;
  dw_tile(sm, a.dab + (int64_t)o * 2 * I + m0, 2 * I, a.xg + (int64_t)o * H + n0, H, c, out, H);
}

}  // namespace

hipError_t mok_launch_gateup(const mok_fwd_args& a, int m, int max_tiles_mb, bool mxfp8,
                             hipStream_t st) {
  if (mxfp8) return hipErrorNotSupported;
  hipLaunchKernelGGL(gateup_bf16_kernel, dim3(max_tiles_mb, (unsigned)(a.I / 64)), dim3(NTHR), 0,
                     st, a, m);
  return hipGetLastError();
}

hipError_t mok_launch_down(const mok_fwd_args& a, int m, int max_tiles_mb, bool mxfp8,
                           hipStream_t st) {
  if (mxfp8) return hipErrorNotSupported;
  hipLaunchKernelGGL(down_bf16_kernel, dim3(max_tiles_mb, (unsigned)(a.H / BN)), dim3(NTHR), 0, st,
                     a, m);
  return hipGetLastError();
}

hipError_t mok_launch_bwd_dh(const mok_bwd_args& a, hipStream_t st) {
  hipLaunchKernelGGL(bwd_dh_kernel, dim3(a.max_tiles, (unsigned)(a.I / BN)), dim3(NTHR), 0, st, a);
  return hipGetLastError();
}

hipError_t mok_launch_bwd_dx(const mok_bwd_args& a, hipStream_t st) {
  hipLaunchKernelGGL(bwd_dx_kernel, dim3(a.max_tiles, (unsigned)(a.H / BN)), dim3(NTHR), 0, st, a);
  return hipGetLastError();
}

hipError_t mok_launch_bwd_dwd(const mok_bwd_args& a, hipStream_t st) {
  hipLaunchKernelGGL(bwd_dwd_kernel, dim3((unsigned)((a.H / BM) * (a.I / BN)), a.E), dim3(NTHR), 0,
                     st, a);
  return hipGetLastError();
}

hipError_t mok_launch_bwd_dwgu(const mok_bwd_args& a, hipStream_t st) {
  hipLaunchKernelGGL(bwd_dwgu_kernel, dim3((unsigned)((2 * a.I / BM) * (a.H / BN)), a.E),
                     dim3(NTHR), 0, st, a);
  return hipGetLastError();
}
