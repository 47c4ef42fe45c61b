// Host-side launch entry points of the device kernels (internal to libmok).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mok_device.h"
#include "persist_plan.h"

struct mok_sched_ptrs {
  int32_t* status;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* dest;
  int32_t* tok;          // [R + kTokPad]: token of permuted row p (perm[p] / topk), then zeros
  int32_t* n_fwd_tiles;
  mok_tile* fwd_tiles;
  int32_t* mb_tile_start;
  int32_t* n_bwd_tiles;
  mok_tile* bwd_tiles;
  int32_t* eorder;       // [E] experts by descending count, ties to the lower id
};

// Zero entries after the R entries of the token table: the GEMM loaders read
// token indices up to two 64-row pairs of K past an expert's last row.
constexpr int kTokPad = 256;

// Row-tile sizes of the grouped GEMMs.
constexpr int kTileRowsFwd = 256;
constexpr int kTileRowsBwd = 256;

// Rows per chunk of the schedule's count/scatter passes, and the launches.
// chunk_counts holds ceil(R / chunk) * (E + 1) ints.
int mok_schedule_chunk_rows(int64_t R);
hipError_t mok_launch_schedule(const int32_t* ids, const mok_sched_ptrs& s, int R, int E, int topk, int M,
                               int bm_f, int bm_b, int n_mb, int max_f, int max_b,
                               int32_t* chunk_counts, hipStream_t st);

// y[t] = sum_j w[t][j] * obuf[t*k+j] (valid rows only), fp32, j ascending.
hipError_t mok_launch_combine(const bf16_t* obuf, const float* w, const int32_t* dest,
                              const int32_t* offsets_E, int64_t T, int topk, int64_t H,
                              bf16_t* y, hipStream_t st);

// dw[t][j] = <dy[t], obuf[t*k+j]>; with dOq (MXFP8) also the rows
// dO[dest[t*k+j]] = bf16(w[t][j] * dy[t]) quantized along H (dOq, dOs).
hipError_t mok_launch_reverse_combine(const bf16_t* dy, const bf16_t* obuf, const float* w,
                                      const int32_t* dest, const int32_t* offsets_E, int64_t T,
                                      int topk, int64_t H, float* dw, float* wperm, uint8_t* dOq,
                                      uint8_t* dOs, hipStream_t st);

// dx[t] = sum_j dxrows[t*k+j] (valid rows only), fp32, j ascending.
hipError_t mok_launch_reverse_dispatch(const bf16_t* dxrows, const int32_t* dest,
                                       const int32_t* offsets_E, int64_t T, int topk, int64_t H,
                                       bf16_t* dx, hipStream_t st);

hipError_t mok_launch_mxfp8_quantize(const bf16_t* src, int64_t rows, int64_t K, uint8_t* q,
                                     uint8_t* scales, hipStream_t st);

// q[b][c][col0 + r] = E4M3(src[b][r][c]) blocked by 32 along r; scales
// [b][c][ld/32] at (col0 + r)/32. rows % 32 == 0, cols % 8 == 0, ld and col0
// multiples of 32, src and q 16-byte aligned (checked by the caller).
hipError_t mok_launch_mxfp8_quantize_t(const bf16_t* src, int64_t batch, int64_t rows, int64_t cols, uint8_t* q,
                                       uint8_t* scales, int64_t ld, int64_t col0, hipStream_t st);

// Matrix-core peak probe: `workgroups` workgroups of 4 wavefronts, each
// issuing 8 * iters MFMAs back to back on register operands (kind 0: bf16
// 32x32x16, kind 1: scaled fp8 32x32x64), one float per thread to sink.
hipError_t mok_launch_probe_mfma(int kind, int workgroups, int iters, float* sink, hipStream_t st);

// clears `bytes` bytes at p (16-byte aligned)
hipError_t mok_launch_zero(void* p, int64_t bytes, hipStream_t st);

// ---------------------------------------------------------------- grouped GEMMs
struct mok_fwd_args {
  // problem
  int64_t T, H, I;
  int E, topk, M, n_slots, n_mb;
  // schedule
  const int32_t* perm;
  const mok_tile* tiles;
  const int32_t* n_tiles;
  const int32_t* mb_tile_start;
  // weights
  const void* wg;
  const void* wu;
  const void* wd;
  const uint8_t* sg;
  const uint8_t* su;
  const uint8_t* sd;
  // operand rows of the gate/up GEMM: permuted row p is row tok[p] of x (bf16
  // [T][H]) or, for MXFP8, of its E4M3 codes [T][H] with scales xs [T][H/32]
  const int32_t* tok;
  const uint8_t* x;
  const uint8_t* xs;
  // ring: slot s holds the h rows of minibatch m (s = m mod N_s) at
  // ring_h + s*M*hrow_bytes
  uint8_t* ring_h;
  uint8_t* ring_hs;      // MXFP8 scales of ring_h rows
  // outputs
  bf16_t* obuf;          // [R][H], flat row order
  bf16_t* ab;            // [R][2I] saved pre-activations (NULL = none)
};

// gate/up GEMM + SwiGLU epilogue over the row tiles of minibatches
// [m0, m1) (at most max_tiles tiles).
hipError_t mok_launch_gateup(const mok_fwd_args& a, int m0, int m1, int max_tiles, bool mxfp8,
                             hipStream_t st);
// down GEMM over the row tiles of minibatches [m0, m1); writes obuf[perm[p]].
hipError_t mok_launch_down(const mok_fwd_args& a, int m0, int m1, int max_tiles, bool mxfp8,
                           hipStream_t st);

// Persistent forward: one launch runs every gate/up and down tile of the
// layer, minibatch after minibatch through the ring (plan: persist_plan.h).
struct mok_persist_args {
  int* ctr;              // mok_persist_counters ints, zero at the launch (layout:
                         // persist_counters in persist_plan.h)
  int32_t* status;       // schedule status word
  int32_t give_up_bit;   // set in *status when a wait gives up or the tile table is inconsistent
  int max_tiles;         // bound on mb_tile_start[n_mb]
  int max_mb_tiles;      // bound on the row tiles of one minibatch
  uint64_t spin_limit;   // ticks of the 64-bit real-time counter one wait may last
  int force_agent;       // 1: synchronise at agent scope even when every workgroup
                         // runs on the XCD of its queue (the path taken otherwise
                         // only on a different placement; for tests)
};
inline int64_t mok_persist_counters(int max_tiles) { return mok::persist_counter_count(max_tiles); }
// grid: a multiple of 8, at most the workgroups resident at once (one per CU)
hipError_t mok_launch_fwd_persistent(const mok_fwd_args& a, const mok_persist_args& ps, int grid,
                                     bool mxfp8, hipStream_t st);

// Single-launch layer: the schedule steps and the combine around the
// persistent forward, in one grid (layer_fwd_kernel).
struct mok_layer_args {
  const int32_t* ids;    // topk_ids [R]
  mok_sched_ptrs s;      // the schedule being built
  int R, chunk, nchunks; // routed rows; schedule chunk rows and count
  int32_t* bh;           // chunk count table [nchunks][E + 1]
  int bm_f, bm_b, max_f, max_b;
  const bf16_t* x;       // bf16 x [T][H] (quantized into mok_fwd_args.x / xs for MXFP8)
  const float* topk_w;
  bf16_t* y;
};
hipError_t mok_launch_layer_fwd(const mok_fwd_args& a, const mok_persist_args& ps, const mok_layer_args& L,
                                int grid, bool mxfp8, hipStream_t st);

struct mok_bwd_args {
  int64_t T, H, I;
  int E, topk;
  const int32_t* perm;
  const int32_t* offsets;
  const int32_t* eorder;  // experts by descending count (the weight-gradient order)
  const mok_tile* tiles;
  const int32_t* n_tiles;
  int max_tiles;
  const bf16_t* wg;
  const bf16_t* wu;
  const bf16_t* wd;
  const int32_t* tok;     // token of each permuted row (schedule)
  const float* topk_w;    // [T][k] combine weights
  const float* wperm;     // [R] combine weight of each permuted row (bf16 path)
  const bf16_t* dy;       // [T][H] upstream gradient
  const bf16_t* x;        // [T][H] layer input
  const bf16_t* ab;       // [R][2I] permuted (saved by forward)
  bf16_t* dab;           // [R][2I] permuted: dA | dB
  bf16_t* hb;            // [R][I] permuted: recomputed h (bf16: w * h)
  bf16_t* dxrows;        // [R][H] flat row order
  bf16_t* dwg;
  bf16_t* dwu;
  bf16_t* dwd;
  // MXFP8 backward (NULL for bf16). Token-blocked operands of expert e are
  // [N][Kp_e] E4M3 matrices at byte N*koff_e (Kp_e = rows rounded up to 128,
  // koff_e = sum of Kp over experts before e), scales [N][Kp_e/32] at N*koff_e/32.
  const uint8_t* wdt;    // Wd^T [E][I][H], blocks along H
  const uint8_t* wdt_s;
  const uint8_t* wgut;   // [Wg; Wu]^T [E][H][2I], blocks along 2I
  const uint8_t* wgut_s;
  uint8_t* dOq;          // dO rows [R][H], blocks along H
  uint8_t* dOs;
  uint8_t* dabq;         // dA | dB rows [R][2I], blocks along 2I
  uint8_t* dabs;
  uint8_t* dOT;          // token-blocked dO (N = H)
  uint8_t* dOTs;
  uint8_t* hT;           // token-blocked h (N = I)
  uint8_t* hTs;
  uint8_t* dabT;         // token-blocked dA | dB (N = 2I)
  uint8_t* dabTs;
  uint8_t* xT;           // token-blocked x rows (N = H)
  uint8_t* xTs;
  int32_t* koff;         // [E+1] start of each expert on the padded token axis, then the
                         // expert of each 128-position block (mok_launch_token_offsets)
};

hipError_t mok_launch_bwd_dh(const mok_bwd_args& a, hipStream_t st);     // dh, SwiGLU bwd
hipError_t mok_launch_bwd_dwd(const mok_bwd_args& a, hipStream_t st);    // dWd
hipError_t mok_launch_bwd_dwgu(const mok_bwd_args& a, hipStream_t st);   // dWg, dWu
hipError_t mok_launch_bwd_dx(const mok_bwd_args& a, hipStream_t st);     // dX rows
// MXFP8 backward GEMMs (same roles; operands in the MXFP8 fields of mok_bwd_args)
hipError_t mok_launch_bwd_dh8(const mok_bwd_args& a, hipStream_t st);
hipError_t mok_launch_bwd_dx8(const mok_bwd_args& a, hipStream_t st);
hipError_t mok_launch_bwd_dwd8(const mok_bwd_args& a, hipStream_t st);
hipError_t mok_launch_bwd_dwgu8(const mok_bwd_args& a, hipStream_t st);
// Token-blocked MXFP8 copy of the rows of every expert (layout as in
// mok_bwd_args): row p of the source is src + p*ld, or with perm the token
// row src + (perm[p] / topk)*ld, scaled by w[perm[p]] and rounded to bf16
// when w is given; N columns; R routed rows.
hipError_t mok_launch_token_quantize(const bf16_t* src, int64_t ld, const int32_t* perm, int topk,
                                     const float* w, const int32_t* offsets, const int32_t* koff, int E, int64_t R,
                                     int64_t N, uint8_t* dst, uint8_t* dst_scales, hipStream_t st);
// 128-position blocks of the padded token axis (an upper bound: R + 128 E positions)
inline int mok_token_blocks(int64_t R, int E) { return (int)((R + 128 * (int64_t)E + 127) / 128); }
// koff[0..E] of the padded token axis from the expert offsets, followed in the
// same buffer by the expert of each 128-position block (koff + E + 1, one int
// per block, -1 past the end); one workgroup
hipError_t mok_launch_token_offsets(const int32_t* offsets, int E, int64_t R, int32_t* koff, hipStream_t st);

// ---------------------------------------------------------------- router
hipError_t mok_launch_router_forward(const bf16_t* x, const float* wr, const float* bias, int64_t T, int H,
                                     int E, int k, int32_t* ids, float* w, hipStream_t st);
hipError_t mok_launch_router_backward(const bf16_t* x, const float* wr, const int32_t* ids, const float* w,
                                      const float* g, int64_t T, int H, int E, int k,
                                      const int32_t* offsets, const int32_t* perm, const int32_t* tok,
                                      float* d_sel, bf16_t* dx, float* d_wr, hipStream_t st);
