// Row-wise, HBM-bound kernels of the MoE layer: weighted combine,
// reverse-combine, reverse-dispatch and MXFP8 quantization.
//
// [MoK clip] How-to item 2: forward = pull dispatch + push combine, backward =
// pull reverse-combine + push reverse-dispatch, all four from one schedule.
// On one GPU the exchange is local: the pull dispatch is fused into the GEMMs'
// operand copies (x and dy rows read in place through the token table), the
// push combine is the down GEMM's row scatter into obuf, and the kernels here
// move whole rows with 16-byte accesses so a wavefront touches contiguous
// 1 KiB spans.
#include "mok_device.h"
#include "mok_launch.h"
#include "rows_core.h"

namespace {

// ------------------------------------------------------------------ combine
// One thread per (token, 8 columns) (combine_elem: y = sum over j ascending
// of w*o in fp32). With WAVE_TOKEN (H/8 a multiple of 64) the 64 lanes of a wavefront share
// one token, which is then read from lane 0 so that its dest and w entries
// are loaded once per wavefront through the scalar unit.
template <bool WAVE_TOKEN>
__global__ __launch_bounds__(256) void combine_kernel(
    const bf16_t* __restrict__ obuf, const float* __restrict__ w,
    const int32_t* __restrict__ dest, const int32_t* __restrict__ offsets_E, int64_t T, int topk,
    int64_t H, bf16_t* __restrict__ y) {
  const int64_t nch = H >> 3;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int64_t t = idx / nch;
  if constexpr (WAVE_TOKEN) t = __builtin_amdgcn_readfirstlane((int)t);
  const int64_t c = idx - t * nch;
  if (t >= T) return;
  combine_elem(obuf, w, dest, *offsets_E, t, c, topk, H, y);
}

// ------------------------------------------------------------------ reverse-combine
// One wavefront per token: dw[t][j] = <dy[t], obuf[t*k+j]> reduced in a fixed
// order (each lane sums its columns in ascending order, then a xor butterfly).
// The k rows go 8 at a time through one pass over the columns, so their loads
// overlap. The bf16 backward needs nothing more (its GEMMs read dy rows in
// place and apply w themselves); the MXFP8 backward (QUANT) also quantizes
// each row dO[dest[i]] = bf16(w[i] * dy[t]) along H from those bf16 values
// into permuted order (a 32-column block is the 4 chunks of 4 adjacent
// lanes); the bf16 dO rows themselves are never stored. With wperm, each
// routed row's weight is also written at its permuted position (wperm[dest[i]]
// = w[i]), the per-row scale the bf16 dh epilogue applies.
template <bool QUANT>
__global__ __launch_bounds__(256) void reverse_combine_kernel(
    const bf16_t* __restrict__ dy, const bf16_t* __restrict__ obuf, const float* __restrict__ w,
    const int32_t* __restrict__ dest, const int32_t* __restrict__ offsets_E, int64_t T, int topk,
    int64_t H, float* __restrict__ dw, float* __restrict__ wperm, uint8_t* __restrict__ dOq,
    uint8_t* __restrict__ dOs) {
  // the token of this wavefront, read from lane 0 so that its dest and w
  // entries are loaded once per wavefront through the scalar unit
  const int64_t t = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * 4 + (threadIdx.x >> 6)));
  const int lane = lane_id();
  if (t >= T) return;
  const int nvalid = *offsets_E;
  const int64_t nch = H >> 3;
  const uint4* dyr = reinterpret_cast<const uint4*>(dy + t * H);
  for (int j0 = 0; j0 < topk; j0 += 8) {
    int64_t row[8];
    int pos[8];
    bool ok[8];
    float wv[8], part[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u;
      row[u] = t * topk + min(j, topk - 1);
      pos[u] = dest[row[u]];
      ok[u] = j < topk && pos[u] < nvalid;
      wv[u] = w[row[u]];
      part[u] = 0.f;
    }
    for (int64_t c = lane; c < nch; c += 64) {
      float g[8];
      unpack8(dyr[c], g);
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = reinterpret_cast<const uint4*>(obuf + row[u] * H)[c];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (!ok[u]) continue;
        float o[8], d[8];
        unpack8(v[u], o);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          part[u] = fmaf(g[q], o[q], part[u]);
          d[q] = wv[u] * g[q];
        }
        if constexpr (QUANT) {
          const uint4 packed = pack8(d);
          float b[8];
          unpack8(packed, b);                    // the bf16 values of the dO row
          float amax = 0.f;
#pragma unroll
          for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(b[q]));
          amax = fmaxf(amax, __shfl_xor(amax, 1));
          amax = fmaxf(amax, __shfl_xor(amax, 2));
          const int sc = mx_scale_byte(amax);
          const float inv = mx_inv_scale(sc);
          const uint32_t lo = e4m3_pack4(b[0] * inv, b[1] * inv, b[2] * inv,
                          b[3] * inv);
          const uint32_t hi = e4m3_pack4(b[4] * inv, b[5] * inv, b[6] * inv,
                          b[7] * inv);
          reinterpret_cast<uint2*>(dOq + (int64_t)pos[u] * H)[c] = make_uint2(lo, hi);
          if ((c & 3) == 0) dOs[(int64_t)pos[u] * (H / 32) + (c >> 2)] = (uint8_t)sc;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float pt = part[u];
#pragma unroll
      for (int s = 32; s >= 1; s >>= 1) pt += __shfl_xor(pt, s);
      if (lane == 0 && j0 + u < topk) {
        dw[t * topk + j0 + u] = ok[u] ? pt : 0.0f;
        if (wperm && ok[u]) wperm[pos[u]] = wv[u];
      }
    }
  }
}

// ------------------------------------------------------------------ MXFP8 quantize
// One thread per 32-element block: amax -> E8M0 scale -> 32 E4M3 codes.
__global__ __launch_bounds__(256) void mxfp8_quantize_kernel(const bf16_t* __restrict__ src,
                                                            int64_t nblocks, int64_t K,
                                                            uint8_t* __restrict__ q,
                                                            uint8_t* __restrict__ scales) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= nblocks) return;
  mx_quantize_block(src, K, idx, q, scales);
}

// ------------------------------------------------------------------ transposing MXFP8 quantize
// q[b][c][col0 + r] = E4M3 code of src[b][r][c], blocked by 32 along r (the
// source rows): the weight copies that the MXFP8 backward contracts over the
// weights' other axis (Wd^T blocked along H, [Wg; Wu]^T along 2I). The codes
// and scale bytes are those mxfp8_quantize_kernel gives for the transposed
// matrix. One workgroup per 64 source rows x 128 source columns of matrix b:
// the tile comes in as 256-byte row segments (16-byte loads) into LDS; each
// thread then takes one source column and one 32-row block (a wavefront's 64
// lanes read 64 adjacent bf16 of one tile row per step, conflict-free) and
// writes its 32 codes as two 16-byte stores along the output row.
__global__ __launch_bounds__(256) void mxfp8_quantize_t_kernel(const bf16_t* __restrict__ src, int64_t rows,
                                                              int64_t cols, uint8_t* __restrict__ q,
                                                              uint8_t* __restrict__ scales, int64_t ld,
                                                              int64_t col0) {
  __shared__ __attribute__((aligned(16))) bf16_t tile[64 * 128];
  const int64_t b = blockIdx.z;
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 128;
  const bf16_t* s = src + b * rows * cols;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int idx = threadIdx.x + 256 * u, row = idx >> 4, ch = idx & 15;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r0 + row < rows && c0 + ch * 8 < cols)
      v = *reinterpret_cast<const uint4*>(s + (r0 + row) * cols + c0 + ch * 8);
    *reinterpret_cast<uint4*>(tile + row * 128 + ch * 8) = v;
  }
  __syncthreads();
  const int c = threadIdx.x & 127, rb = threadIdx.x >> 7;
  if (c0 + c >= cols || r0 + 32 * rb >= rows) return;
  float v[32];
  float amax = 0.f;
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    v[r] = bf16_to_f32(tile[(32 * rb + r) * 128 + c]);
    amax = fmaxf(amax, fabsf(v[r]));
  }
  const int sc = mx_scale_byte(amax);
  const float inv = mx_inv_scale(sc);
  uint32_t wds[8];
#pragma unroll
  for (int u = 0; u < 8; ++u)
    wds[u] = e4m3_pack4(v[4 * u] * inv, v[4 * u + 1] * inv, v[4 * u + 2] * inv, v[4 * u + 3] * inv);
  const int64_t orow = b * cols + c0 + c;
  const int64_t ocol = col0 + r0 + 32 * rb;
  uint4* d = reinterpret_cast<uint4*>(q + orow * ld + ocol);
  d[0] = make_uint4(wds[0], wds[1], wds[2], wds[3]);
  d[1] = make_uint4(wds[4], wds[5], wds[6], wds[7]);
  scales[orow * (ld / 32) + ocol / 32] = (uint8_t)sc;
}

// ------------------------------------------------------------------ token-blocked MXFP8
// For the weight-gradient GEMMs of the MXFP8 backward (contraction over an
// expert's rows): expert e's rows [o_e, o_e + c_e) of the source, transposed
// to [N][Kp_e] and quantized along the rows in blocks of 32 counted from o_e
// (positions past c_e are zero, which decode to zero under the block's
// scale). One workgroup per (COLS columns x 128 positions of the padded
// token axis, which never straddle two experts since every Kp is a multiple
// of 128): it stages the 128 x COLS block in LDS (2*COLS-byte row segments
// in), then 4 adjacent threads per column quantize its four 32-row blocks and
// write them as one 128-byte segment of the transposed row.
// With perm, row p of the source is the token row perm[p] / topk (x, dy read
// in place); with w as well, its values are first scaled by w[perm[p]] and
// rounded to bf16 (the dO rows w * dy, the same bits as a stored dO row).
template <int COLS>
__global__ __launch_bounds__(256) void token_quantize_kernel(
    const bf16_t* __restrict__ src, int64_t ld, const int32_t* __restrict__ perm, int topk,
    const float* __restrict__ w,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ koffs,
    const int32_t* __restrict__ blk_e, int64_t N, uint8_t* __restrict__ dst, uint8_t* __restrict__ dsts) {
  static_assert(COLS == 64 || COLS == 128, "64 or 128 columns per workgroup");
  constexpr int CH = COLS / 8;                   // 16-byte chunks per row
  // the 128 x COLS block as bf16, row pitch 2*COLS bytes; the 8-column chunk
  // ch of row r sits at chunk ch ^ (2 * (r / 32)), so that the four 32-row
  // blocks read by the four threads of one column fall in different banks
  __shared__ __attribute__((aligned(16))) bf16_t tile[128 * COLS];
  // blockIdx.x: COLS-column slice (adjacent workgroups read adjacent slices
  // of the same rows); blockIdx.y: 128 positions of the padded token axis
  const int e = blk_e[blockIdx.y];               // expert owning these positions, -1 past the end
  if (e < 0) return;
  const int koff = koffs[e], kp = koffs[e + 1] - koff;
  const int o = offsets[e], c = offsets[e + 1] - o;
  const int r0 = (int)blockIdx.y * 128 - koff;   // first row of the block within the expert
  const int nrow = min(128, c - r0);             // rows of this block that exist (may be <= 0)
  const int64_t n0 = (int64_t)blockIdx.x * COLS;
  constexpr int NL = 128 * CH / 256;             // 16-byte loads per thread
  uint4 v[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int idx = threadIdx.x + 256 * i, r = idx / CH;
    const int64_t col = n0 + (idx % CH) * 8;
    v[i] = make_uint4(0u, 0u, 0u, 0u);
    if (r < nrow && col < N) {
      const int64_t p = o + r0 + r;
      const int32_t i_flat = perm ? perm[p] : 0;
      const int64_t row = perm ? (int64_t)(i_flat / topk) : p;
      v[i] = *reinterpret_cast<const uint4*>(src + row * ld + col);
      if (w) {
        const float wv = w[i_flat];
        float f[8];
        unpack8(v[i], f);
#pragma unroll
        for (int q = 0; q < 8; ++q) f[q] *= wv;
        v[i] = pack8(f);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int idx = threadIdx.x + 256 * i, r = idx / CH, ch = idx % CH;
    *reinterpret_cast<uint4*>(tile + r * COLS + ((ch ^ (2 * (r >> 5))) << 3)) = v[i];
  }
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < COLS / 64; ++pass) {
    const int cl = (threadIdx.x >> 2) + 64 * pass, qb = threadIdx.x & 3;   // column, 32-row block
    const int64_t n = n0 + cl;
    if (n >= N) continue;
    float x[32];
    float amax = 0.f;
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      x[r] = bf16_to_f32(tile[(32 * qb + r) * COLS + (cl ^ (16 * qb))]);
      amax = fmaxf(amax, fabsf(x[r]));
    }
    const int sc = mx_scale_byte(amax);
    const float inv = mx_inv_scale(sc);
    uint32_t wds[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      wds[u] = e4m3_pack4(x[4 * u] * inv, x[4 * u + 1] * inv, x[4 * u + 2] * inv,
                          x[4 * u + 3] * inv);
    uint4* d = reinterpret_cast<uint4*>(dst + N * koff + n * kp + r0 + 32 * qb);
    d[0] = make_uint4(wds[0], wds[1], wds[2], wds[3]);
    d[1] = make_uint4(wds[4], wds[5], wds[6], wds[7]);
    dsts[N * (koff / 32) + n * (kp / 32) + r0 / 32 + qb] = (uint8_t)sc;
  }
}

// koff[e] = sum over e' < e of tok_pad(rows of e'), e = 0..E, by a Hillis-Steele
// scan of up to kMaxExperts values in one workgroup (integer, exact).
// It also fills blk_e[b] (b < nblk), the expert whose padded positions hold
// [128b, 128b + 128), or -1 past the last expert, by a binary search of koff.
__global__ __launch_bounds__(256) void token_offsets_kernel(const int32_t* __restrict__ offsets, int E,
                                                            int32_t* __restrict__ koff, int nblk,
                                                            int32_t* __restrict__ blk_e) {
  __shared__ int v[2][kMaxExperts + 1];
  for (int i = threadIdx.x; i <= E; i += 256) v[0][i] = i == 0 ? 0 : tok_pad(offsets[i] - offsets[i - 1]);
  __syncthreads();
  int cur = 0;
  for (int d = 1; d <= E; d <<= 1) {
    for (int i = threadIdx.x; i <= E; i += 256) v[cur ^ 1][i] = v[cur][i] + (i >= d ? v[cur][i - d] : 0);
    __syncthreads();
    cur ^= 1;
  }
  for (int i = threadIdx.x; i <= E; i += 256) koff[i] = v[cur][i];
  for (int b = threadIdx.x; b < nblk; b += 256) {
    const int t0 = 128 * b;
    int lo = -1;
    if (t0 < v[cur][E]) {                        // largest e with koff[e] <= t0
      int hi = E;
      lo = 0;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (v[cur][mid] <= t0) lo = mid; else hi = mid;
      }
    }
    blk_e[b] = lo;
  }
}

// clears bytes [0, bytes) of a 16-byte aligned buffer: 16-byte stores, the
// last partial unit byte by byte
__global__ __launch_bounds__(256) void zero_kernel(uint4* p, int64_t bytes) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (16 * i + 16 <= bytes) {
    p[i] = make_uint4(0, 0, 0, 0);
  } else if (16 * i < bytes) {
    uint8_t* b = reinterpret_cast<uint8_t*>(p + i);
    for (int64_t j = 0; j < bytes - 16 * i; ++j) b[j] = 0;
  }
}

inline unsigned grid_for(int64_t n, int64_t per_block) {
  return (unsigned)((n + per_block - 1) / per_block);
}

}  // namespace

hipError_t mok_launch_combine(const bf16_t* obuf, const float* w, const int32_t* dest,
                              const int32_t* offsets_E, int64_t T, int topk, int64_t H,
                              bf16_t* y, hipStream_t st) {
  const int64_t n = T * (H / 8);
  if (n <= 0) return hipSuccess;
  if ((H / 8) % 64 == 0)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(grid_for(n, 256)), dim3(256), 0, st, obuf, w, dest,
                       offsets_E, T, topk, H, y);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(grid_for(n, 256)), dim3(256), 0, st, obuf, w, dest,
                       offsets_E, T, topk, H, y);
  return hipGetLastError();
}

hipError_t mok_launch_reverse_combine(const bf16_t* dy, const bf16_t* obuf, const float* w,
                                      const int32_t* dest, const int32_t* offsets_E, int64_t T,
                                      int topk, int64_t H, float* dw, float* wperm, uint8_t* dOq,
                                      uint8_t* dOs, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  if (dOq)
    hipLaunchKernelGGL(reverse_combine_kernel<true>, dim3(grid_for(T, 4)), dim3(256), 0, st, dy, obuf,
                       w, dest, offsets_E, T, topk, H, dw, wperm, dOq, dOs);
  else
    hipLaunchKernelGGL(reverse_combine_kernel<false>, dim3(grid_for(T, 4)), dim3(256), 0, st, dy,
                       obuf, w, dest, offsets_E, T, topk, H, dw, wperm, dOq, dOs);
  return hipGetLastError();
}

hipError_t mok_launch_reverse_dispatch(const bf16_t* dxrows, const int32_t* dest,
                                       const int32_t* offsets_E, int64_t T, int topk, int64_t H,
                                       bf16_t* dx, hipStream_t st) {
  const int64_t n = T * (H / 8);
  if (n <= 0) return hipSuccess;
  if ((H / 8) % 64 == 0)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(grid_for(n, 256)), dim3(256), 0, st, dxrows,
                       (const float*)nullptr, dest, offsets_E, T, topk, H, dx);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(grid_for(n, 256)), dim3(256), 0, st, dxrows,
                       (const float*)nullptr, dest, offsets_E, T, topk, H, dx);
  return hipGetLastError();
}

hipError_t mok_launch_mxfp8_quantize(const bf16_t* src, int64_t rows, int64_t K, uint8_t* q,
                                     uint8_t* scales, hipStream_t st) {
  const int64_t nblocks = rows * (K / 32);
  if (nblocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(mxfp8_quantize_kernel, dim3(grid_for(nblocks, 256)), dim3(256), 0, st, src,
                     nblocks, K, q, scales);
  return hipGetLastError();
}

hipError_t mok_launch_mxfp8_quantize_t(const bf16_t* src, int64_t batch, int64_t rows, int64_t cols, uint8_t* q,
                                       uint8_t* scales, int64_t ld, int64_t col0, hipStream_t st) {
  if (batch <= 0 || rows <= 0 || cols <= 0) return hipSuccess;
  if (batch > 65535 || (rows + 63) / 64 > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mxfp8_quantize_t_kernel, dim3((unsigned)((cols + 127) / 128), (unsigned)((rows + 63) / 64),
                                                   (unsigned)batch),
                     dim3(256), 0, st, src, rows, cols, q, scales, ld, col0);
  return hipGetLastError();
}

hipError_t mok_launch_token_quantize(const bf16_t* src, int64_t ld, const int32_t* perm, int topk,
                                     const float* w, const int32_t* offsets, const int32_t* koff, int E, int64_t R,
                                     int64_t N, uint8_t* dst, uint8_t* dst_scales, hipStream_t st) {
  if (R <= 0 || N <= 0) return hipSuccess;
  if (E > kMaxExperts) return hipErrorInvalidValue;
  const int nblk = mok_token_blocks(R, E);
  constexpr int kCols = 64;                       // measured: 128 columns per workgroup is 5-15% slower
  hipLaunchKernelGGL(token_quantize_kernel<kCols>, dim3((unsigned)((N + kCols - 1) / kCols), (unsigned)nblk),
                     dim3(256), 0, st, src, ld, perm, topk, w, offsets, koff, koff + E + 1, N, dst, dst_scales);
  return hipGetLastError();
}

hipError_t mok_launch_token_offsets(const int32_t* offsets, int E, int64_t R, int32_t* koff, hipStream_t st) {
  if (E > kMaxExperts) return hipErrorInvalidValue;
  hipLaunchKernelGGL(token_offsets_kernel, dim3(1), dim3(256), 0, st, offsets, E, koff, mok_token_blocks(R, E),
                     koff + E + 1);
  return hipGetLastError();
}

hipError_t mok_launch_zero(void* p, int64_t bytes, hipStream_t st) {
  if (bytes <= 0) return hipSuccess;
  // (16-byte stores need 16-byte alignment; fewer than 16 bytes go byte by byte)
  if (bytes >= 16 && reinterpret_cast<uintptr_t>(p) % 16 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(zero_kernel, dim3(grid_for((bytes + 15) / 16, 256)), dim3(256), 0, st, (uint4*)p, bytes);
  return hipGetLastError();
}
