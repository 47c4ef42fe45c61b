// Tile machinery shared by the grouped-GEMM kernels (gfx950 matrix cores).
//
// A workgroup of 256 threads (4 wavefronts in a WM x WN grid) computes a
// BM x BN tile of C = A . B^T over K. K advances in stages of 64 bytes per
// operand row (32 bf16 or 64 fp8); LDS holds two slots, each a pair of
// consecutive stages (128 bytes of K per row). Every operand reaches LDS by
// direct global->LDS copies (global_load_lds); a slot is refilled with the
// pair after next while the other slot's pair is being multiplied.
//
// Why pairs of stages: every copy instruction then reads whole 128-byte lines
// (8 rows x 128 B for K-contiguous operands). On gfx950 a copy costs the
// address unit about one cache line per two clocks, and HBM delivers whole
// lines at full rate; 64-byte half-line reads measured half the L2 rate and
// about 70% of the HBM rate.
//
// Two LDS tile layouts, both 32 KiB per slot for 256 rows or columns:
//  * K-contiguous operands (row r = K vector in memory): [256 rows][128 B].
//    16-byte LDS reads serve 8 lanes per bank half; they are conflict-free
//    when, in every group of 8 lanes, address bit 7 equals lane bit 3 and the
//    16-byte slots (address bits 4-6) differ (measured on gfx950: 64 banks,
//    256 bytes per clock). MFMA lanes 0-31 read 32 consecutive rows, so row
//    r is stored at physical row swap03(r) (row bits 0 and 3 exchanged) and
//    its 16-byte chunk c at c ^ (r & 7).
//  * K-outer operands (element (k, n) at k*ld + n in memory): [64 k][512 B],
//    16-byte chunk c of k-row k stored at c ^ ((k & 3) << 2). Fragments are
//    read with ds_read_b64_tr_b16, which hands a 16-lane group the transpose
//    of the 4 x 16 block its lanes address (lane 4q + p addresses k-row q,
//    columns 4p .. 4p+3; lane i receives column i, k-rows 0 .. 3).
//
// bf16: v_mfma_f32_32x32x16_bf16; lane l supplies row l%32, K elements
//       8*(l/32) .. +8 of a 16-wide K step.
// fp8:  v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 operands; lane l supplies
//       row l%32, bytes 0-15 = K 16*(l/32) .. +16 (scale block 0) and bytes
//       16-31 = K 32 + 16*(l/32) .. +16 (scale block 1); the E8M0 scale of
//       (row l%32, block l/32) comes from lane l (measured on gfx950).
// Accumulator element q of a 32x32 fragment sits at row 8*(q/4) + 4*(l/32) +
// q%4, column l%32.
#pragma once
#include <type_traits>

#include "mok_device.h"

namespace mok {

constexpr int kThreads = 256;
constexpr int kStage = 64;                        // K bytes per row per stage
constexpr int kSlotRow = 128;                     // K bytes per row per LDS slot (2 stages)

MOK_DEV int swap03(int r) { return (r & ~0x9) | ((r >> 3) & 1) | ((r & 1) << 3); }
// byte offset of 16-byte chunk `chunk` (0..7) of row `row` in a K-contiguous slot
MOK_DEV int lds_at(int row, int chunk) { return swap03(row) * kSlotRow + ((chunk ^ (row & 7)) << 4); }
// byte offset of byte `byte` of k-row k (0..63) in a K-outer slot
MOK_DEV int lds_ko(int k, int byte) { return k * 512 + ((((byte >> 4) ^ ((k & 3) << 2))) << 4) + (byte & 15); }

typedef const __attribute__((address_space(3))) uint8_t* lds_cptr;
typedef __attribute__((ext_vector_type(4))) short v4i16_t;

// 512 zero bytes: the source of K-outer rows past the end of K.
__device__ __attribute__((aligned(16))) uint8_t kZeroRow[512];

// Wait until at most N of this wavefront's vector-memory operations are
// outstanding and all of its LDS operations are done (gfx9 s_waitcnt
// encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
MOK_DEV void wait_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

// Direct copy of 16 (or 4) bytes per lane from global memory into LDS:
// lane l's bytes land at LDS byte address lds + 16*l (4*l). Written as inline
// assembly so that the compiler does not track these LDS writes: its
// conservative tracking would add a full vmcnt wait before LDS reads that it
// cannot prove disjoint from every copy in flight, draining the copy
// pipeline. The main loop orders copies and reads with explicit waits and
// barriers instead. The compiler does not count these operations in its own
// vmcnt bookkeeping either; that only makes its waits for ordinary loads
// stricter, never weaker.
// `lds` is the 32-bit LDS byte address (wave-uniform, see lds_addr).
MOK_DEV void copy16_to_lds(const void* g, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(g), "{m0}"(lds) : "memory");
}
MOK_DEV void copy4_to_lds(const void* g, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" :: "v"(g), "{m0}"(lds) : "memory");
}
// 32-bit LDS address of a pointer into a __shared__ array (formed once per
// tile: the generic-to-LDS conversion carries a null check)
MOK_DEV uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(lds_cptr)p);
}

// Workgroup barrier without the memory fence of __syncthreads: a workgroup-
// scope release there waits for every outstanding global->LDS copy, which
// would drain the copy pipeline at each stage. Callers issue the waits that
// make their own LDS writes visible (wait_vm_lds) first; the memory clobber
// keeps the compiler from moving LDS accesses across the barrier.
MOK_DEV void barrier_lds() { asm volatile("s_barrier" ::: "memory"); }

// Workgroup barrier that waits for this wavefront's LDS operations only: its
// global loads and stores stay in flight (the workgroup-scope release of
// __syncthreads would wait for them). For reuse of LDS that holds no copy
// targets; the wait and the barrier are one statement, so no LDS access is
// placed between them.
MOK_DEV void barrier_lds_only() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ------------------------------------------------------------------ row sources
// Byte address of element k = 0 of operand row r (rows past the end clamp).
struct RowsStrided {
  const uint8_t* base;
  int64_t stride;          // bytes between rows
  int nrows;               // valid rows (>= 1)
  MOK_DEV const uint8_t* row(int r) const { return base + (int64_t)min(r, nrows - 1) * stride; }
};

// gate/up B operand: LDS rows come in 32-row groups alternating Wg and Wu, so
// that a wavefront column holds gate and up of the same 32 h-columns.
// (The Wg/Wu choice is address arithmetic, not a select between two fields:
// a select of field addresses keeps the loader object in scratch memory.)
struct RowsGateUp {
  uintptr_t wg;            // address of Wg row 0
  intptr_t du;             // Wu address minus Wg address
  int64_t stride;
  int n0;                  // first h column of the tile
  int ncols;               // I
  MOK_DEV RowsGateUp(const uint8_t* g, const uint8_t* u, int64_t stride_, int n0_, int ncols_)
      : wg((uintptr_t)g), du((intptr_t)((uintptr_t)u - (uintptr_t)g)), stride(stride_), n0(n0_),
        ncols(ncols_) {}
  MOK_DEV const uint8_t* row(int r) const {
    const int col = min(n0 + (r >> 6) * 32 + (r & 31), ncols - 1);
    return reinterpret_cast<const uint8_t*>(wg + (intptr_t)((r >> 5) & 1) * du + (int64_t)col * stride);
  }
};

// ------------------------------------------------------------------ loaders
// Every loader copies one pair of stages (slot j = stages 2j, 2j+1) with kDma
// direct copies per wavefront (dma(j, slot)), and supplies this lane's MFMA
// fragment of 32 rows/columns starting at r0 for half h (stage parity) and
// 16-wide bf16 K step kk (frag). Every wavefront issues exactly kDma copies
// per pair (positions past the end are clamped or read zeros, never skipped).
//
// The copies are spread one per MFMA through the main loop, and with one
// wavefront per SIMD only a few other instructions issue in an MFMA's
// shadow, so a copy has to cost almost nothing besides itself: every loader
// keeps this lane's per-copy address offsets in registers (set up once per
// tile), adds a wave-uniform base for the pair, and takes the LDS address
// (m0) as a 32-bit offset formed on the scalar unit. (Computing the addresses
// per copy measured 20% slower on the K-outer GEMMs.)

MOK_DEV int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// K-contiguous operand. One copy instruction fills a 1 KiB window (8
// physical rows x 128 B); lane l writes bytes 16*l .. +16 of it, so each lane
// fetches the global chunk that the layout places at its LDS position.
template <int R, class Rows>
struct LoadKD {
  static constexpr int kDma = R / 32;
  static constexpr int kReads = 1;               // LDS reads per fragment
  Rows src;
  mutable uint32_t mb;     // LDS address of this wavefront's first window in the pair's slot
  MOK_DEV void dma1(int j, uint32_t slot, int q) const {  // copy q of pair j
    if (q == 0) mb = slot + wave_id() * 1024;
    const int w = (int)(threadIdx.x >> 6), l = lane_id();
    const int g = w + 4 * q;                     // window g = physical rows 8g .. 8g+7
    const int row = swap03(8 * g + (l >> 3));    // logical row stored there
    const int lc = (l & 7) ^ (row & 7);          // logical chunk at physical chunk l&7
    copy16_to_lds(src.row(row) + j * kSlotRow + lc * 16, mb + q * 4096);
  }
  MOK_DEV void dma(int j, uint32_t slot) const {
#pragma unroll
    for (int q = 0; q < kDma; ++q) dma1(j, slot, q);
  }
  MOK_DEV static bf16x8_t frag(const uint8_t* t, int r0, int h, int kk) {
    const int l = lane_id();
    return *reinterpret_cast<const bf16x8_t*>(t + lds_at(r0 + (l & 31), 4 * h + 2 * kk + (l >> 5)));
  }
};

// K-outer bf16 operand: element (k, n) at src0 + k*ld + 2n bytes for k <
// ksplit and src1 + (k - ksplit)*ld + 2n beyond (ksplit a multiple of 64, so
// a pair never straddles it); k-rows >= K read as zero, columns past ncols
// are clamped (their products land in unstored output). A slot is 64 k-rows
// of 256 columns; copy q of wavefront w fills window g = w + 4q, i.e. k-rows
// 2g (lanes 0-31) and 2g+1 (lanes 32-63).
template <int R>
struct LoadKO {
  static_assert(R == 256, "K-outer tiles have 256 columns");
  static constexpr int kDma = 8;
  static constexpr int kReads = 2;               // LDS reads per fragment
  const uint8_t* src0;
  const uint8_t* src1;
  int ksplit;
  int64_t ld;              // bytes between k-rows
  int K;
  int ncols;               // valid columns (multiple of 8, >= 8)
  int64_t off[kDma];       // this lane's byte offset from k-row 0 of the pair, per copy
  mutable const uint8_t* pb;   // k-row 0 of the current pair
  mutable uint32_t mb;         // LDS address of this wavefront's first window in the slot
  mutable int kr;              // k-rows of the current pair inside K
  MOK_DEV LoadKO(const uint8_t* s0, const uint8_t* s1, int ksplit_, int64_t ld_, int K_, int ncols_)
      : src0(s0), src1(s1), ksplit(ksplit_), ld(ld_), K(K_), ncols(ncols_) {
    const int w = (int)(threadIdx.x >> 6), l = lane_id();
#pragma unroll
    for (int q = 0; q < kDma; ++q) {
      const int kl = 2 * (w + 4 * q) + (l >> 5);
      const int c = (l & 31) ^ ((kl & 3) << 2);  // logical chunk at physical chunk l&31
      const int cc = min(c, (ncols >> 3) - 1);   // (< 32: also inside the zero row)
      off[q] = (int64_t)kl * ld + cc * 16;
    }
  }
  // this lane's chunk in the zero row for copy window g (tail pair only)
  MOK_DEV static const uint8_t* zero_chunk(int kl, int ncols) {
    const int c = (lane_id() & 31) ^ ((kl & 3) << 2);
    return kZeroRow + min(c, (ncols >> 3) - 1) * 16;
  }
  MOK_DEV void dma1(int j, uint32_t slot, int q) const {
    if (q == 0) {                                // wave-uniform state of the pair
      const int k0 = j * 64;
      pb = k0 < ksplit ? src0 + (int64_t)k0 * ld : src1 + (int64_t)(k0 - ksplit) * ld;
      mb = slot + wave_id() * 1024;
      kr = K - k0;
    }
    const uint8_t* gp = pb + off[q];
    if (kr < 64) {                               // tail pair (wave-uniform branch)
      asm volatile("");                          // a branch, not a select on every copy
      const int kl = 2 * ((int)(threadIdx.x >> 6) + 4 * q) + (lane_id() >> 5);
      if (kl >= kr) gp = zero_chunk(kl, ncols);
    }
    copy16_to_lds(gp, mb + q * 4096);
  }
  MOK_DEV void dma(int j, uint32_t slot) const {
#pragma unroll
    for (int q = 0; q < kDma; ++q) dma1(j, slot, q);
  }
  MOK_DEV static bf16x8_t frag(const uint8_t* t, int r0, int h, int kk) {
    const int l = lane_id(), g = l >> 4, L = l & 15;
    const int n = r0 + 16 * (g & 1) + 4 * (L & 3);
    const int k = 32 * h + 16 * kk + 8 * (g >> 1) + (L >> 2);
    typedef __attribute__((address_space(3))) v4i16_t* lds_v4_ptr;
    const v4i16_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4_ptr)(t + lds_ko(k, 2 * n)));
    const v4i16_t y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4_ptr)(t + lds_ko(k + 4, 2 * n)));
    typedef __attribute__((ext_vector_type(8))) short v8i16_t;
    const v8i16_t v = v8i16_t{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    return __builtin_bit_cast(bf16x8_t, v);
  }
};

// Gathered operands: the operand's row r (K-contiguous) or k-row k (K-outer)
// is row tok[r] of a token-major source, tok being the schedule's token of
// each permuted row. The GEMMs thereby read x and dY rows in place; no
// gathered copy of them is ever written.

// K-contiguous gathered operand (rows past nrows clamp to the last row):
// this lane's row address per copy is formed once per tile.
template <int R>
struct LoadKDG {
  static constexpr int kDma = R / 32;
  static constexpr int kReads = 1;
  const uint8_t* rowp[kDma];
  mutable uint32_t mb;
  MOK_DEV LoadKDG(const uint8_t* base, const int32_t* tok, int64_t stride, int nrows) {
    const int w = (int)(threadIdx.x >> 6), l = lane_id();
#pragma unroll
    for (int q = 0; q < kDma; ++q) {
      const int row = swap03(8 * (w + 4 * q) + (l >> 3));
      const int lc = (l & 7) ^ (row & 7);
      rowp[q] = base + (int64_t)tok[min(row, nrows - 1)] * stride + lc * 16;
    }
  }
  MOK_DEV void dma1(int j, uint32_t slot, int q) const {
    if (q == 0) mb = slot + wave_id() * 1024;
    copy16_to_lds(rowp[q] + j * kSlotRow, mb + q * 4096);
  }
  MOK_DEV void dma(int j, uint32_t slot) const {
#pragma unroll
    for (int q = 0; q < kDma; ++q) dma1(j, slot, q);
  }
  MOK_DEV static bf16x8_t frag(const uint8_t* t, int r0, int h, int kk) {
    return LoadKD<R, RowsStrided>::frag(t, r0, h, kk);
  }
};

// K-outer gathered bf16 operand: k-row k is src + tok[k]*ld (k < K), zero
// beyond. Wavefront w copies the 16 k-rows 16w .. 16w+15 of a pair (window g
// = 8w + q holds k-rows 2g, 2g+1), so the 16 token indices it needs are one
// wave-uniform scalar load of 64 bytes, issued with the first copy of the
// pair before (pairs are copied in ascending order) and used one pair later,
// when it has long arrived. tok must stay readable 128 entries past K.
typedef __attribute__((ext_vector_type(16))) int i32x16_t;
typedef const __attribute__((address_space(4))) i32x16_t* tok16_cptr;

template <int R>
struct LoadKOG {
  static_assert(R == 256, "K-outer tiles have 256 columns");
  static constexpr int kDma = 8;
  static constexpr int kReads = 2;
  const int32_t* tok;      // token of k-row 0
  uint32_t ld;             // bytes between token rows
  int K;
  int ncols;
  const uint8_t* colp[kDma];   // this lane's column chunk in token row 0, per copy
  mutable i32x16_t cur, nxt;
  mutable uint32_t mb;         // LDS address of this wavefront's first window in the slot
  mutable int kr;              // k-rows of the current pair inside K
  MOK_DEV i32x16_t load16(int j) const {
    return *(tok16_cptr)(const void*)(tok + 64 * j + 16 * wave_id());
  }
  MOK_DEV LoadKOG(const uint8_t* src, const int32_t* tok_, int64_t ld_, int K_, int ncols_)
      : tok(tok_), ld((uint32_t)ld_), K(K_), ncols(ncols_) {
    const int l = lane_id();
#pragma unroll
    for (int q = 0; q < kDma; ++q) {
      const int kl = 2 * q + (l >> 5);           // k-row within the wavefront's 16, mod 4 as 2g+hi
      const int c = (l & 31) ^ ((kl & 3) << 2);
      const int cc = min(c, (ncols >> 3) - 1);
      colp[q] = src + cc * 16;
    }
    nxt = load16(0);
  }
  MOK_DEV void dma1(int j, uint32_t slot, int q) const {
    if (q == 0) {
      cur = nxt;
      nxt = load16(j + 1);
      mb = slot + wave_id() * 8192;
      kr = K - j * 64;
    }
    const int hi = lane_id() >> 5;
    // (readfirstlane keeps the two uniform picks apart: folded into one
    // lane-dependent vector index, the index vector would go to scratch)
    const uint32_t t0 = (uint32_t)__builtin_amdgcn_readfirstlane(cur[2 * q]);
    const uint32_t t1 = (uint32_t)__builtin_amdgcn_readfirstlane(cur[2 * q + 1]);
    const uint8_t* gp = colp[q] + (uint64_t)(hi ? t1 : t0) * ld;
    if (kr < 64) {                               // tail pair (wave-uniform branch)
      asm volatile("");                          // a branch, not a select on every copy
      const int kl = 16 * (int)(threadIdx.x >> 6) + 2 * q + hi;
      if (kl >= kr) gp = LoadKO<R>::zero_chunk(kl, ncols);
    }
    copy16_to_lds(gp, mb + q * 1024);
  }
  MOK_DEV void dma(int j, uint32_t slot) const {
#pragma unroll
    for (int q = 0; q < kDma; ++q) dma1(j, slot, q);
  }
  MOK_DEV static bf16x8_t frag(const uint8_t* t, int r0, int h, int kk) {
    return LoadKO<R>::frag(t, r0, h, kk);
  }
};

// E8M0 block scales of a 256-row fp8 operand, copied into LDS as one 32-bit
// word per row holding the scales of K blocks 4j .. 4j+3 (the two stages of
// slot j; K is a multiple of 128, so the word never runs past the row). Lane
// l of wavefront w copies the word of row 64w + l.
template <int R, class Rows>
struct LoadScalesD {
  static_assert(R == 256, "scale tiles have 256 rows");
  static constexpr int kDma = 1;
  Rows src;                                      // byte address of each row's scale 0
  MOK_DEV void dma(int j, uint32_t slot) const {
    const int w = wave_id(), l = lane_id();
    const uint8_t* gp = src.row(64 * w + l) + j * 4;
    copy4_to_lds(gp, slot + 256 * w);
  }
};

// Scales of a gathered fp8 operand: lane l of wavefront w copies the word of
// row 64w + l, i.e. of source row tok[64w + l] (clamped to nrows - 1).
template <int R>
struct LoadScalesDG {
  static_assert(R == 256, "scale tiles have 256 rows");
  static constexpr int kDma = 1;
  const uint8_t* rowp;
  MOK_DEV LoadScalesDG(const uint8_t* base, const int32_t* tok, int64_t stride, int nrows) {
    rowp = base + (int64_t)tok[min((int)threadIdx.x, nrows - 1)] * stride;
  }
  MOK_DEV void dma(int j, uint32_t slot) const {
    copy4_to_lds(rowp + j * 4, slot + 256 * wave_id());
  }
};

struct NoScales {
  static constexpr int kDma = 0;
  MOK_DEV void dma(int, uint32_t) const {}
};


// ------------------------------------------------------------------ accumulators
template <int FM, int FN>
struct Acc {
  f32x16_t c[FM][FN];
  MOK_DEV void zero() {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) c[i][j][q] = 0.f;
  }
};

// Tile geometry: 4 wavefronts in a WM x WN grid over a BM x BN tile.
template <int BM_, int BN_, int WM_, int WN_>
struct Geo {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static_assert(WM * WN == 4, "four wavefronts");
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  MOK_DEV static int wm() { return (int)(threadIdx.x >> 6) / WN; }
  MOK_DEV static int wn() { return (int)(threadIdx.x >> 6) % WN; }
  // tile coordinates of accumulator element (i, j, q) of this lane
  MOK_DEV static int row(int i, int q) {
    return wm() * WTM + i * 32 + 8 * (q >> 2) + 4 * (lane_id() >> 5) + (q & 3);
  }
  MOK_DEV static int col(int j) { return wn() * WTN + j * 32 + (lane_id() & 31); }
};

// LDS of one tile: two slots per operand (a pair of stages each), plus the
// per-row scale words of each slot for fp8.
template <class G, bool SCALES>
struct SmemT {
  uint8_t a[2][G::BM * kSlotRow];
  uint8_t b[2][G::BN * kSlotRow];
};
template <class G>
struct SmemT<G, true> {
  uint8_t a[2][G::BM * kSlotRow];
  uint8_t b[2][G::BN * kSlotRow];
  uint32_t sa[2][G::BM];
  uint32_t sb[2][G::BN];
};
template <class G, bool F8>
using Smem = SmemT<G, F8>;

// LDS bytes of a tile kernel: the ring, or the epilogue's fp32 half-tile
// (128 rows of BN*4 + 16 bytes) plus a 256-entry row table, if larger.
template <class SM>
constexpr int tile_lds_bytes() {
  return (int)sizeof(SM) > 128 * (256 * 4 + 16) + 1024 ? (int)sizeof(SM) : 128 * (256 * 4 + 16) + 1024;
}
// the row table: the top 1 KiB of a tile's LDS, free once the main loop ends
template <class SM>
MOK_DEV int* tile_rows(uint8_t* lds_raw) {
  return reinterpret_cast<int*>(lds_raw + tile_lds_bytes<SM>() - 1024);
}

// ------------------------------------------------------------------ fragments
// bf16: fragments of one 16-wide K step (kk = 0, 1 within stage half h).
template <class G>
struct FragsB16 {
  bf16x8_t a[G::FM], b[G::FN];
};

// VM x VN: the fragment rows x columns of this wavefront that hold valid
// rows (the others are skipped: no LDS reads, no MFMAs; their accumulators
// stay zero and are never stored).
template <class G, class LA, class LB, int VM = 4, int VN = 4>
MOK_DEV void read_b16(const uint8_t* ta, const uint8_t* tb, int h, int kk, FragsB16<G>& f) {
  const int r0 = G::wm() * G::WTM, c0 = G::wn() * G::WTN;
#pragma unroll
  for (int i = 0; i < G::FM; ++i)
    if (i < VM) f.a[i] = LA::frag(ta, r0 + i * 32, h, kk);
#pragma unroll
  for (int j = 0; j < G::FN; ++j)
    if (j < VN) f.b[j] = LB::frag(tb, c0 + j * 32, h, kk);
}

// LDS read instructions per fragment, averaged over the two operands
template <class LA, class LB>
struct RdPerFrag {
  static constexpr int kAvg = (LA::kReads + LB::kReads + 1) / 2;
};

template <class G, int VM = 4, int VN = 4>
MOK_DEV void mfma_b16_1(const FragsB16<G>& f, int i, int j, Acc<G::FM, G::FN>& acc) {
  if (i < VM && j < VN)
    acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc.c[i][j], 0, 0, 0);
}

template <class G>
MOK_DEV void mfma_b16(const FragsB16<G>& f, Acc<G::FM, G::FN>& acc) {
#pragma unroll
  for (int i = 0; i < G::FM; ++i)
#pragma unroll
    for (int j = 0; j < G::FN; ++j) mfma_b16_1<G>(f, i, j, acc);
}

// fp8: the fragments of one whole stage (one 64-wide scaled K step) and the
// scale words of their rows.
template <class G>
struct FragsF8 {
  i32x8_t a[G::FM], b[G::FN];
  uint32_t as[G::FM], bs[G::FN];
};

MOK_DEV i32x8_t cat8(const bf16x8_t& lo8, const bf16x8_t& hi8) {
  const i32x4_t lo = __builtin_bit_cast(i32x4_t, lo8), hi = __builtin_bit_cast(i32x4_t, hi8);
  return i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

template <class G>
MOK_DEV void read_f8_a(const uint8_t* ta, const uint32_t* sa, int h, int i, FragsF8<G>& f) {
  const int lane = lane_id(), lr = lane & 31, lk = lane >> 5;
  const int r = G::wm() * G::WTM + i * 32 + lr;
  f.a[i] = cat8(*reinterpret_cast<const bf16x8_t*>(ta + lds_at(r, 4 * h + lk)),
                *reinterpret_cast<const bf16x8_t*>(ta + lds_at(r, 4 * h + 2 + lk)));
  f.as[i] = sa[r];
}

template <class G>
MOK_DEV void read_f8_b(const uint8_t* tb, const uint32_t* sb, int h, int j, FragsF8<G>& f) {
  const int lane = lane_id(), lr = lane & 31, lk = lane >> 5;
  const int r = G::wn() * G::WTN + j * 32 + lr;
  f.b[j] = cat8(*reinterpret_cast<const bf16x8_t*>(tb + lds_at(r, 4 * h + lk)),
                *reinterpret_cast<const bf16x8_t*>(tb + lds_at(r, 4 * h + 2 + lk)));
  f.bs[j] = sb[r];
}

// one scaled MFMA of fragment (i, j); sh selects the scale byte of this
// lane's block (stage parity and lane half)
template <class G>
MOK_DEV void mfma_f8(const FragsF8<G>& f, int i, int j, int sh, Acc<G::FM, G::FN>& acc) {
  acc.c[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
      f.a[i], f.b[j], acc.c[i][j], 0, 0, 0, (int)((f.as[i] >> sh) & 0xFFu), 0,
      (int)((f.bs[j] >> sh) & 0xFFu));
}

// ------------------------------------------------------------------ main loop
// nk stages, consumed in pairs from the two LDS slots (pair j in slot j%2).
// Within each stage the MFMAs come in two regions, and the next fragments
// are read from LDS while a region's MFMAs issue:
//
//   stage 2j     region A, region B (no barrier)
//   stage 2j+1   region A; then every wavefront waits for all its copies
//                (pair j+1) and LDS reads, and the workgroup barrier makes
//                pair j+1 visible and guarantees that nobody reads slot j%2
//                any more; the copies of pair j+2 into slot j%2 are issued;
//                region B, reading the first fragments of pair j+1
//
// So each pair has two stages of MFMAs to arrive, and there is one barrier
// per pair.
//
// bf16 regions are the two 16-wide K steps of a stage. fp8 regions are
// fragment rows 0-1 and 2-3 of the one 64-wide K step; the B fragments of the
// next stage are read into each B register as soon as its last MFMA of the
// current stage has issued.
template <class SM, class LA, class LB, class SA, class SB>
struct Pipe {
  static constexpr int kD = LA::kDma + LB::kDma + SA::kDma + SB::kDma;
  const LA& la;
  const LB& lb;
  const SA& sa;
  const SB& sb;
  // LDS addresses of slot 0 of each side; slot b is b slot sizes further
  // (arithmetic, not an array: an array indexed by j & 1 would live in
  // scratch memory)
  uint32_t oa, ob, osa, osb;
  static constexpr uint32_t kSa = sizeof(SM::a[0]), kSb = sizeof(SM::b[0]);
  MOK_DEV Pipe(SM& sm, const LA& la_, const LB& lb_, const SA& sa_, const SB& sb_)
      : la(la_), lb(lb_), sa(sa_), sb(sb_), oa(lds_addr(sm.a[0])), ob(lds_addr(sm.b[0])), osa(0), osb(0) {
    if constexpr (SA::kDma > 0) osa = lds_addr(sm.sa[0]);
    if constexpr (SB::kDma > 0) osb = lds_addr(sm.sb[0]);
  }
  MOK_DEV uint32_t a_at(int b) const { return oa + b * kSa; }
  MOK_DEV uint32_t b_at(int b) const { return ob + b * kSb; }
  MOK_DEV uint32_t sa_at(int b) const { return osa + b * (uint32_t)sizeof(SM::sa[0]); }
  MOK_DEV uint32_t sb_at(int b) const { return osb + b * (uint32_t)sizeof(SM::sb[0]); }
  // pair j into slot j%2; the B side first, so that a gathered A operand's
  // token loads complete while B's copies are issued (prologue only)
  MOK_DEV void dma(int j) const {
    const int b = j & 1;
    lb.dma(j, b_at(b));
    if constexpr (SB::kDma > 0) sb.dma(j, sb_at(b));
    la.dma(j, a_at(b));
    if constexpr (SA::kDma > 0) sa.dma(j, sa_at(b));
  }
  // copy u (0 .. 2*kDma-1) of pair j: A copies first, then B (bf16 only)
  MOK_DEV void dma_unit(int j, int u) const {
    const int b = j & 1;
    if (u < LA::kDma) la.dma1(j, a_at(b), u);
    else lb.dma1(j, b_at(b), u - LA::kDma);
  }
  // fp8: copy u of one side of pair j (u < 8: a K-contiguous window; u == 8:
  // the side's scale words)
  MOK_DEV void dma_a1(int j, int u) const {
    const int s = j & 1;
    if (u < LA::kDma) la.dma1(j, a_at(s), u);
    else if constexpr (SA::kDma > 0) sa.dma(j, sa_at(s));
  }
  MOK_DEV void dma_b1(int j, int u) const {
    const int s = j & 1;
    if (u < LB::kDma) lb.dma1(j, b_at(s), u);
    else if constexpr (SB::kDma > 0) sb.dma(j, sb_at(s));
  }
  MOK_DEV void publish() const {                 // all copies landed, all LDS reads done
    wait_vm_lds<0>();
    barrier_lds();
  }
};

// scheduling-group masks (llvm.amdgcn.sched.group.barrier)
constexpr int kSgMfma = 0x008, kSgDsRead = 0x100;

template <class G, bool F8, int VM = 4, int VN = 4, class LA, class LB, class SA, class SB>
MOK_DEV void mainloop(Smem<G, F8>& sm, const LA& la, const LB& lb, const SA& sa, const SB& sb, int nk,
                      Acc<G::FM, G::FN>& acc) {
  using SM = Smem<G, F8>;
  using P = Pipe<SM, LA, LB, SA, SB>;
  constexpr int kD = P::kD;
  static_assert(kD < 64, "vmcnt range");
  static_assert(G::FM == 4 && G::FN == 4, "schedule written for 4 x 4 fragments");
  const P p(sm, la, lb, sa, sb);
  acc.zero();
  __syncthreads();                               // previous users of the LDS buffers are done
  if (nk <= 0) return;
  const int np = (nk + 1) >> 1;                  // pairs

  // prologue: pairs 0 and 1, wait for pair 0
  p.dma(0);
  if (np > 1) {
    p.dma(1);
    wait_vm_lds<kD>();
  } else {
    wait_vm_lds<0>();
  }
  barrier_lds();

  if constexpr (!F8) {
    static_assert(LA::kDma == 8 && LB::kDma == 8, "16 copies per pair");
    FragsB16<G> f0, f1;
    read_b16<G, LA, LB, VM, VN>(sm.a[0], sm.b[0], 0, 0, f0);
    // One region: the 16 MFMAs of fragments f while the 8 fragments of the
    // next K step are read into n; the reads go with the first 8 MFMAs, and
    // with CP >= 0 copies 8*CP' .. 8*CP'+7 of pair cp follow the last 8, one
    // after each MFMA, so that the copies never stall MFMA issue in a burst.
    auto region = [&](const FragsB16<G>& f, FragsB16<G>& n, const uint8_t* ta, const uint8_t* tb, int h,
                      int kk, int cp, int half) {
      __builtin_amdgcn_sched_barrier(0);
      read_b16<G, LA, LB, VM, VN>(ta, tb, h, kk, n);
#pragma unroll
      for (int t = 0; t < 8; ++t) mfma_b16_1<G, VM, VN>(f, t >> 2, t & 3, acc);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2 * RdPerFrag<LA, LB>::kAvg, 0);
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 2, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        mfma_b16_1<G, VM, VN>(f, 2 + (t >> 2), t & 3, acc);
        if (cp >= 0) p.dma_unit(cp, 8 * half + t);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // stage kt: K steps 0 (f0, read before) and 1 (f1). An odd stage ends its
    // pair j: barrier, then (COPY) the A copies of pair j+2 spread over its
    // second region; the following even stage spreads the B copies of that
    // pair over its first region (PEND).
    auto stage = [&](int kt, bool ODD, bool COPY, bool PEND) {
      const int j = kt >> 1, slot = j & 1;
      region(f0, f1, sm.a[slot], sm.b[slot], ODD ? 1 : 0, 1, PEND ? j + 1 : -1, 1);
      if (ODD) p.publish();
      const int nslot = ODD ? (slot ^ 1) : slot;
      region(f1, f0, sm.a[nslot], sm.b[nslot], ODD ? 0 : 1, 0, COPY ? j + 2 : -1, 0);
    };
    int kt = 0;
    for (; kt + 5 < nk; kt += 2) {               // pair kt/2 + 2 exists
      stage(kt, false, false, kt >= 2);
      stage(kt + 1, true, true, false);
    }
    for (; kt < nk; ++kt) {
      const bool odd = (kt & 1) != 0;
      stage(kt, odd, odd && (kt >> 1) + 2 < np, !odd && kt >= 2 && (kt >> 1) + 1 < np);
    }
  } else {
    static_assert(LA::kDma == 8 && LB::kDma == 8, "8 + 8 window copies per pair");
    const int sh_lane = 8 * (lane_id() >> 5);
    FragsF8<G> f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < VM) read_f8_a<G>(sm.a[0], sm.sa[0], 0, i, f);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      if (jj < VN) read_f8_b<G>(sm.b[0], sm.sb[0], 0, jj, f);
    // the copies of one side of pair cp go one after each of a region's 8
    // MFMAs, the side's scale words with the last (cp < 0: none)
    auto copy_after = [&](int t, int cp, bool bside) {
      if (cp < 0) return;
      if (bside) {
        p.dma_b1(cp, t);
        if (t == 7) p.dma_b1(cp, 8);
      } else {
        p.dma_a1(cp, t);
        if (t == 7) p.dma_a1(cp, 8);
      }
    };
    // stage kt: one 64-wide scaled K step in two regions. An odd stage ends
    // its pair j: barrier, then (COPY) the A side of pair j+2 is copied
    // during its region B; the following even stage copies the B side of
    // that pair during its region A (PEND).
    auto stage = [&](int kt, bool ODD, bool COPY, bool PEND) {
      const int j = kt >> 1, slot = j & 1, h = ODD ? 1 : 0;
      const int sh = 16 * h + sh_lane;
      const int pend = PEND ? j + 1 : -1, cpy = COPY ? j + 2 : -1;
      // region A: rows 0-1; read rows 2-3 of this stage (rows 0-1 and all B
      // fragments were read during the previous stage)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if ((t >> 2) < VM && (t & 3) < VN) mfma_f8<G>(f, t >> 2, t & 3, sh, acc);
        if (t < 2 && 2 + t < VM) read_f8_a<G>(sm.a[slot], sm.sa[slot], h, 2 + t, f);
        copy_after(t, pend, true);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (ODD) p.publish();
      // region B: rows 2-3, column block by column block; each B fragment of
      // the next stage is read once its last MFMA here has issued, rows 0-1
      // of the next stage go into the registers region A freed
      const int nslot = ODD ? (slot ^ 1) : slot, nh = ODD ? 0 : 1;
      const FragsF8<G> g = f;
      if (0 < VM) read_f8_a<G>(sm.a[nslot], sm.sa[nslot], nh, 0, f);
      if (1 < VM) read_f8_a<G>(sm.a[nslot], sm.sa[nslot], nh, 1, f);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        if (2 < VM && jj < VN) mfma_f8<G>(g, 2, jj, sh, acc);
        copy_after(2 * jj, cpy, false);
        if (3 < VM && jj < VN) mfma_f8<G>(g, 3, jj, sh, acc);
        copy_after(2 * jj + 1, cpy, false);
        if (jj < VN) read_f8_b<G>(sm.b[nslot], sm.sb[nslot], nh, jj, f);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    int kt = 0;
    for (; kt + 5 < nk; kt += 2) {               // pair kt/2 + 2 exists
      stage(kt, false, false, kt >= 2);
      stage(kt + 1, true, true, false);
    }
    for (; kt < nk; ++kt) {
      const bool odd = (kt & 1) != 0;
      stage(kt, odd, odd && (kt >> 1) + 2 < np, !odd && kt >= 2 && (kt >> 1) + 1 < np);
    }
  }
}

// The main loop with only this wavefront's fragments that hold valid rows:
// nvalid rows of the A operand (ON_B = false; fragment rows of the
// wavefront's 128) or of the B operand (ON_B = true; fragment columns).
// The last row tile of an expert usually holds few rows; its wavefronts then
// skip the MFMAs and LDS reads of the padding rows (a quarter of the work per
// 32 valid rows) while copies and barriers stay the same in every wavefront.
// The variant is chosen per wavefront from a wave-uniform value, so every
// branch here is a scalar branch.
template <bool ON_B, class G, bool F8, class LA, class LB, class SA, class SB>
MOK_DEV void mainloop_rows(Smem<G, F8>& sm, const LA& la, const LB& lb, const SA& sa, const SB& sb, int nk,
                           int nvalid, Acc<G::FM, G::FN>& acc) {
  static_assert(G::FM == 4 && G::FN == 4, "four fragments per side");
  const int w0 = ON_B ? G::wn() * G::WTN : G::wm() * G::WTM;
  const int v = __builtin_amdgcn_readfirstlane(min(4, max(0, (nvalid - w0 + 31) / 32)));
  if (v >= 4) {
    mainloop<G, F8, 4, 4>(sm, la, lb, sa, sb, nk, acc);
  } else if (v == 3) {
    if constexpr (ON_B) mainloop<G, F8, 4, 3>(sm, la, lb, sa, sb, nk, acc);
    else mainloop<G, F8, 3, 4>(sm, la, lb, sa, sb, nk, acc);
  } else if (v == 2) {
    if constexpr (ON_B) mainloop<G, F8, 4, 2>(sm, la, lb, sa, sb, nk, acc);
    else mainloop<G, F8, 2, 4>(sm, la, lb, sa, sb, nk, acc);
  } else if (v == 1) {
    if constexpr (ON_B) mainloop<G, F8, 4, 1>(sm, la, lb, sa, sb, nk, acc);
    else mainloop<G, F8, 1, 4>(sm, la, lb, sa, sb, nk, acc);
  } else {
    if constexpr (ON_B) mainloop<G, F8, 4, 0>(sm, la, lb, sa, sb, nk, acc);
    else mainloop<G, F8, 0, 4>(sm, la, lb, sa, sb, nk, acc);
  }
}

// ------------------------------------------------------------------ epilogue staging
// fp32 staging of one 128-row half of a 256-row tile (the rows owned by the
// wavefronts with wm() == half), pitch BN*4 + 16 bytes.
template <class G>
struct HalfF32 {
  static_assert(G::BM == 256 && G::WM == 2, "half-tile staging assumes 2 x 128 rows");
  static constexpr int PITCH = G::BN * 4 + 16;
  MOK_DEV static void put(uint8_t* lds, const Acc<G::FM, G::FN>& acc, int half) {
    if (G::wm() != half) return;
#pragma unroll
    for (int i = 0; i < G::FM; ++i)
#pragma unroll
      for (int j = 0; j < G::FN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q)
          *reinterpret_cast<float*>(lds + (G::row(i, q) - 128 * half) * PITCH + G::col(j) * 4) =
              acc.c[i][j][q];
  }
  MOK_DEV static void get8(const uint8_t* lds, int r, int c, float v[8]) {
    const float4 x = *reinterpret_cast<const float4*>(lds + r * PITCH + c * 4);
    const float4 y = *reinterpret_cast<const float4*>(lds + r * PITCH + c * 4 + 16);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w; v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
  }
};

MOK_DEV void unpack_bf16x8(const uint4& v, float f[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f[2 * q] = __uint_as_float(w[q] << 16);
    f[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
  }
}

MOK_DEV uint4 pack_bf16x8(const float f[8]) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                    pack_bf16x2(f[6], f[7]));
}

// Store the accumulator tile as bf16 rows: dst(r) is the address of tile
// column 0 of output row r; rows >= nrows and columns >= ncols are skipped.
// Goes through LDS one 128-row half at a time, 16-byte stores along rows.
template <class G, class Dst>
MOK_DEV void store_tile_bf16(uint8_t* lds, const Acc<G::FM, G::FN>& acc, int nrows, int ncols, Dst dst) {
  using HS = HalfF32<G>;
  constexpr int CPR = G::BN / 8;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    barrier_lds_only();
    HS::put(lds, acc, half);
    barrier_lds_only();
    const int rows = min(128, nrows - 128 * half);
    for (int idx = threadIdx.x; idx < 128 * CPR; idx += kThreads) {
      const int r = idx / CPR, c = (idx % CPR) * 8;
      if (r >= rows || c >= ncols) continue;
      float v[8];
      HS::get8(lds, r, c, v);
      store_nt(dst(128 * half + r) + c, pack_bf16x8(v));
    }
  }
}

// Store a tile accumulated with the operands exchanged (mainloop called with
// the column-side loader first, so acc holds the transpose: accumulator row
// index = output column, accumulator column index = output row) as bf16 rows.
// Each lane then holds 4 adjacent output columns per 4 accumulator elements:
// they are rounded in pairs (v_cvt_pk_bf16_f32, round to nearest even) and
// written as one 8-byte LDS store; the whole 256 x 256 bf16 tile is staged at
// once (128 KiB; 16-byte chunk c of row m at chunk c ^ (m & 15), so the 32 rows
// of one store instruction spread over all banks), then read back and stored
// as 16-byte vectors along rows. dst(r), nrows and ncols as in store_tile_bf16.
template <class G, class Dst>
MOK_DEV void store_tile_bf16_t(uint8_t* lds, const Acc<G::FM, G::FN>& acc, int nrows, int ncols, Dst dst) {
  static_assert(G::BM == 256 && G::BN == 256, "256 x 256 tiles");
  typedef __attribute__((ext_vector_type(2))) float f2_t;
  typedef __attribute__((ext_vector_type(2))) __bf16 b2_t;
  constexpr int PITCH = 512;
  const int l = lane_id();
  barrier_lds_only();
#pragma unroll
  for (int i = 0; i < G::FM; ++i)
#pragma unroll
    for (int j = 0; j < G::FN; ++j) {
      const int m = G::wn() * G::WTN + j * 32 + (l & 31);            // output row
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n0 = G::wm() * G::WTM + i * 32 + 8 * g + 4 * (l >> 5);   // output column
        const b2_t lo = __builtin_convertvector((f2_t){acc.c[i][j][4 * g], acc.c[i][j][4 * g + 1]}, b2_t);
        const b2_t hi = __builtin_convertvector((f2_t){acc.c[i][j][4 * g + 2], acc.c[i][j][4 * g + 3]}, b2_t);
        const int off = m * PITCH + ((((n0 >> 3) ^ (m & 15))) << 4) + ((n0 & 7) << 1);
        *reinterpret_cast<uint2*>(lds + off) =
            make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
      }
    }
  barrier_lds_only();
  constexpr int CPR = G::BN / 8;                                     // 16-byte chunks per row
#pragma unroll 4
  for (int idx = threadIdx.x; idx < G::BM * CPR; idx += kThreads) {
    const int r = idx / CPR, c = idx % CPR;
    if (r >= nrows || 8 * c >= ncols) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(lds + r * PITCH + ((c ^ (r & 15)) << 4));
    store_nt(dst(r) + 8 * c, v);
  }
}

// Consecutive workgroup ids of a 1-D grid are dispatched round-robin over
// the 8 XCDs, each with its own L2: workgroup wg runs on XCD wg mod 8. The
// tile mappings below give each XCD its own set of tiles, ordered so that the
// tiles in flight on one XCD share operand panels in its L2.
constexpr int kXcds = 8;

// Row-tile kernels: nr row tiles (rows of one expert, equal K) x nc column
// tiles. XCD k takes the row tiles [k*rper, (k+1)*rper), rper = ceil(nr / 8),
// and runs them in groups of 4 row tiles, column by column within a group,
// so that the ~32 tiles its CUs run at once form a 4 x 8 block: 12 operand
// panels in flight per XCD (4 A, 8 B) where a row-major order has about 30
// (1-2 A, every B), i.e. 2.5x fewer L2 misses per step of K. Every row tile
// has the same K, so equal row-tile counts per XCD are balanced work.
// Grid: kXcds * ceil(max_nr / 8) * nc. False past the end.
MOK_DEV bool xcd_swizzle(int nr, int nc, int& row, int& col) {
  const int wg = (int)blockIdx.x, k = wg % kXcds, i = wg / kXcds;
  const int rper = (nr + kXcds - 1) / kXcds;
  const int rows_k = min(rper, nr - k * rper);
  if (rows_k <= 0 || i >= rows_k * nc) return false;
  const int gi = i / (4 * nc), hg = min(4, rows_k - 4 * gi), j = i - gi * 4 * nc;
  col = j / hg;
  row = k * rper + 4 * gi + j % hg;
  return true;
}

// Weight-gradient tiles: E experts, each an ntm x ntn grid of output tiles
// whose K loop runs over the expert's routed rows, so a tile's cost follows
// its expert's load. Every expert's grid is cut into kXcds near-square blocks
// (ry rows of blocks x kXcds/ry columns; ry chosen on the host) and XCD k
// runs block k of every expert, expert by expert in the order eorder (the
// schedule's experts by descending count: the longest tiles first, so the
// launch ends on short ones), in groups of 4 tile rows taken column by
// column. Each XCD thereby does 1/8 of every expert's work
// whatever the loads (a contiguous tile range per XCD gave the XCD holding
// the busiest expert 1.7x the mean work on a Zipf(0.8) routing), and the
// tiles in flight on an XCD share their operand panels as in xcd_swizzle.
// Grid: kXcds * E * ceil(ntm / ry) * ceil(ntn / (kXcds / ry)). False past the end.
MOK_DEV bool dw_tile_of(int E, const int32_t* eorder, int ntm, int ntn, int ry, int& e, int& mt, int& nt) {
  const int cx = kXcds / ry;
  const int wg = (int)blockIdx.x, k = wg % kXcds, i = wg / kXcds;
  const int by = k / cx, bx = k % cx;
  const int r0 = by * ntm / ry, r1 = (by + 1) * ntm / ry;
  const int c0 = bx * ntn / cx, c1 = (bx + 1) * ntn / cx;
  const int h = r1 - r0, w = c1 - c0, nb = h * w;
  if (nb <= 0) return false;
  const int pos = i / nb;
  if (pos >= E) return false;
  e = eorder[pos];
  const int j = i - pos * nb;
  const int gi = j / (4 * w), hg = min(4, h - 4 * gi), jj = j - gi * 4 * w;
  nt = c0 + jj / hg;
  mt = r0 + 4 * gi + jj % hg;
  return true;
}

}  // namespace mok
