// Tile machinery shared by the grouped-GEMM kernels (gfx950 matrix cores).
//
// A workgroup of 256 threads (4 wavefronts in a WM x WN grid) computes a
// BM x BN tile of C = A . B^T, where row m of A and row n of B are read as K
// vectors. K advances in stages of 128 bytes per row (64 bf16 or 128 fp8),
// double-buffered through LDS. Each LDS tile is [rows][128 B]; its 16-byte
// chunks are XOR-swizzled with (row ^ row >> 3) & 7, which keeps three access
// patterns free of bank conflicts: 8 lanes writing the 8 chunks of one row
// (row loader), 8 lanes writing one chunk of rows 8 apart (transposing
// loader), and 8 consecutive rows read by the MFMA lanes.
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
#include "mok_device.h"

namespace mok {

constexpr int kThreads = 256;
constexpr int kStage = 128;                       // K bytes per row per stage

MOK_DEV int swz_chunk(int row, int chunk) { return chunk ^ ((row ^ (row >> 3)) & 7); }
MOK_DEV int lds_at(int row, int chunk) { return row * kStage + (swz_chunk(row, chunk) << 4); }

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
struct RowsGateUp {
  const uint8_t* wg;
  const uint8_t* wu;
  int64_t stride;
  int n0;                  // first h column of the tile
  int ncols;               // I
  MOK_DEV const uint8_t* row(int r) const {
    const int col = min(n0 + (r >> 6) * 32 + (r & 31), ncols - 1);
    return (((r >> 5) & 1) ? wu : wg) + (int64_t)col * stride;
  }
};

// ------------------------------------------------------------------ loaders
// K-contiguous operand: R rows x 8 chunks, R*8/256 chunks per thread.
template <int R, class Rows>
struct LoadK {
  static constexpr int N = R * 8 / kThreads;
  Rows src;
  uint4 v[N];
  MOK_DEV static int my_row(int q) { return (int)(threadIdx.x >> 3) + 32 * q; }
  MOK_DEV void fetch(int kt) {
    const int off = kt * kStage + (threadIdx.x & 7) * 16;
#pragma unroll
    for (int q = 0; q < N; ++q) v[q] = *reinterpret_cast<const uint4*>(src.row(my_row(q)) + off);
  }
  MOK_DEV void put(uint8_t* t) const {
    const int c = threadIdx.x & 7;
#pragma unroll
    for (int q = 0; q < N; ++q) *reinterpret_cast<uint4*>(t + lds_at(my_row(q), c)) = v[q];
  }
  MOK_DEV void begin(int kt, uint8_t*) { fetch(kt); }
  MOK_DEV void end(uint8_t* t) const { put(t); }
};

typedef __attribute__((address_space(3))) void* lds_void_ptr;

// K-contiguous operand copied straight from global memory into LDS
// (global_load_lds_dwordx4: lane l of an instruction fills bytes 16*l .. +16
// of a 1 KiB LDS window = 8 tile rows). Each lane fetches the global chunk
// that the swizzle places at its LDS position, so no registers are used.
template <int R, class Rows>
struct LoadKD {
  Rows src;
  MOK_DEV void begin(int kt, uint8_t* t) {
    const int w = (int)(threadIdx.x >> 6), l = lane_id();
#pragma unroll
    for (int q = 0; q < R / 32; ++q) {
      const int g = w + 4 * q;                   // 1 KiB window = rows 8g .. 8g+7
      const int row = 8 * g + (l >> 3);
      const int lc = swz_chunk(row, l & 7);      // logical chunk stored at physical chunk l&7
      const uint8_t* gp = src.row(row) + kt * kStage + lc * 16;
      __builtin_amdgcn_global_load_lds(gp, (lds_void_ptr)(t + g * 1024), 16, 0, 0);
    }
  }
  MOK_DEV void end(uint8_t*) const {}
};

// K-outer bf16 operand: element (m, k) at base + k*ld + m (elements). The tile
// has R rows (m) and 64 k. Each thread loads KR = R/32 k-rows of 8 consecutive
// m and writes them transposed (8 rows of KR k each).
template <int R>
struct LoadT {
  static constexpr int KR = R / 32;
  static constexpr int MC = R / 8;               // m chunks
  const bf16_t* base0;                           // k < ksplit
  const bf16_t* base1;                           // k >= ksplit
  int ksplit;
  int64_t ld;
  int K;                                         // k >= K reads as zero
  int mlimit;                                    // m >= mlimit reads as zero
  uint4 v[KR];
  MOK_DEV void fetch(int kt) {
    const int mc = threadIdx.x % MC, kg = threadIdx.x / MC;
    const bool mok = 8 * mc < mlimit;
#pragma unroll
    for (int i = 0; i < KR; ++i) {
      const int k = kt * 64 + kg * KR + i;
      if (k < K && mok) {
        const bf16_t* b = k < ksplit ? base0 : base1;
        v[i] = *reinterpret_cast<const uint4*>(b + (int64_t)k * ld + 8 * mc);
      } else {
        v[i] = make_uint4(0, 0, 0, 0);
      }
    }
  }
  MOK_DEV void put(uint8_t* t) const {
    const int mc = threadIdx.x % MC, kg = threadIdx.x / MC;
    uint32_t w[KR][4];
#pragma unroll
    for (int i = 0; i < KR; ++i) {
      w[i][0] = v[i].x; w[i][1] = v[i].y; w[i][2] = v[i].z; w[i][3] = v[i].w;
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const uint32_t sel = (m & 1) ? 0x07060302u : 0x05040100u;
      uint32_t o[KR / 2];
#pragma unroll
      for (int i = 0; i < KR / 2; ++i) o[i] = __builtin_amdgcn_perm(w[2 * i + 1][m >> 1], w[2 * i][m >> 1], sel);
      const int r = 8 * mc + m;
      // this thread's KR k values are bytes [kg*KR*2, +KR*2) of the row
      uint8_t* dst = t + lds_at(r, (kg * KR * 2) >> 4) + ((kg * KR * 2) & 15);
      if constexpr (KR == 8) {
        *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
      } else {
        static_assert(KR == 4, "LoadT supports 128 or 256 rows");
        *reinterpret_cast<uint2*>(dst) = make_uint2(o[0], o[1]);
      }
    }
  }
  MOK_DEV void begin(int kt, uint8_t*) { fetch(kt); }
  MOK_DEV void end(uint8_t* t) const { put(t); }
};

// E8M0 scales of an fp8 operand: 4 bytes (blocks) per row per stage.
template <int R>
struct LoadScales {
  const uint8_t* base;     // scale bytes of row 0, block 0
  int64_t stride;          // bytes between rows
  int nrows;
  bool gateup;             // rows follow the RowsGateUp interleave
  const uint8_t* base_u;
  int n0, ncols;
  uint32_t v;
  MOK_DEV void fetch(int kt) {
    const int r = threadIdx.x;
    if (r < R) {
      const uint8_t* p;
      if (gateup) {
        const int col = min(n0 + (r >> 6) * 32 + (r & 31), ncols - 1);
        p = (((r >> 5) & 1) ? base_u : base) + (int64_t)col * stride;
      } else {
        p = base + (int64_t)min(r, nrows - 1) * stride;
      }
      v = *reinterpret_cast<const uint32_t*>(p + kt * 4);
    }
  }
  MOK_DEV void put(uint32_t* t) const {
    if ((int)threadIdx.x < R) t[threadIdx.x] = v;
  }
  MOK_DEV void begin(int kt, uint32_t*) { fetch(kt); }
  MOK_DEV void end(uint32_t* t) const { put(t); }
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

template <class G>
struct Smem {
  uint8_t a[2][G::BM * kStage];
  uint8_t b[2][G::BN * kStage];
  uint32_t sa[2][G::BM];
  uint32_t sb[2][G::BN];
};

// One stage of MFMAs from LDS.
template <class G, bool F8>
MOK_DEV void mma_stage(const uint8_t* ta, const uint8_t* tb, const uint32_t* sa,
                       const uint32_t* sb, Acc<G::FM, G::FN>& acc) {
  const int lane = lane_id(), lr = lane & 31, lk = lane >> 5;
  const int r0 = G::wm() * G::WTM, c0 = G::wn() * G::WTN;
  if constexpr (!F8) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8_t a[G::FM], b[G::FN];
#pragma unroll
      for (int i = 0; i < G::FM; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(ta + lds_at(r0 + i * 32 + lr, 2 * kk + lk));
#pragma unroll
      for (int j = 0; j < G::FN; ++j)
        b[j] = *reinterpret_cast<const bf16x8_t*>(tb + lds_at(c0 + j * 32 + lr, 2 * kk + lk));
#pragma unroll
      for (int i = 0; i < G::FM; ++i)
#pragma unroll
        for (int j = 0; j < G::FN; ++j)
          acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc.c[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);   // keep one K step's fragments live at a time
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      i32x8_t b[G::FN];
      int bs[G::FN];
#pragma unroll
      for (int j = 0; j < G::FN; ++j) {
        const int r = c0 + j * 32 + lr;
        const uint4 lo = *reinterpret_cast<const uint4*>(tb + lds_at(r, 4 * kk + lk));
        const uint4 hi = *reinterpret_cast<const uint4*>(tb + lds_at(r, 4 * kk + 2 + lk));
        b[j] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        bs[j] = (int)((sb[r] >> (8 * (2 * kk + lk))) & 0xFFu);
      }
#pragma unroll
      for (int i = 0; i < G::FM; ++i) {
        const int r = r0 + i * 32 + lr;
        const uint4 lo = *reinterpret_cast<const uint4*>(ta + lds_at(r, 4 * kk + lk));
        const uint4 hi = *reinterpret_cast<const uint4*>(ta + lds_at(r, 4 * kk + 2 + lk));
        const i32x8_t a = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        const int as = (int)((sa[r] >> (8 * (2 * kk + lk))) & 0xFFu);
#pragma unroll
        for (int j = 0; j < G::FN; ++j)
          acc.c[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b[j], acc.c[i][j], 0, 0, 0,
                                                                        as, 0, bs[j]);
      }
      __builtin_amdgcn_sched_barrier(0);   // keep one K step's fragments live at a time
    }
  }
}

struct NoScales {
  MOK_DEV void begin(int, uint32_t*) {}
  MOK_DEV void end(uint32_t*) const {}
};

// Wait for this thread's outstanding global->LDS copies and global loads.
MOK_DEV void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Double-buffered main loop over nk stages. Loaders start stage kt+1 (direct
// copies into the idle LDS buffer, or loads into registers) before the MFMAs
// of stage kt and finish it (register loaders write LDS) after them.
template <class G, bool F8, class LA, class LB, class SA, class SB>
MOK_DEV void mainloop(Smem<G>& sm, LA& la, LB& lb, SA& sa, SB& sb, int nk,
                      Acc<G::FM, G::FN>& acc) {
  acc.zero();
  __syncthreads();                       // previous users of the LDS buffers are done
  if (nk <= 0) return;
  la.begin(0, sm.a[0]);
  lb.begin(0, sm.b[0]);
  sa.begin(0, sm.sa[0]);
  sb.begin(0, sm.sb[0]);
  la.end(sm.a[0]);
  lb.end(sm.b[0]);
  sa.end(sm.sa[0]);
  sb.end(sm.sb[0]);
  wait_vmem();
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1, nxt = cur ^ 1;
    const bool more = kt + 1 < nk;
    if (more) {
      la.begin(kt + 1, sm.a[nxt]);
      lb.begin(kt + 1, sm.b[nxt]);
      sa.begin(kt + 1, sm.sa[nxt]);
      sb.begin(kt + 1, sm.sb[nxt]);
    }
    mma_stage<G, F8>(sm.a[cur], sm.b[cur], sm.sa[cur], sm.sb[cur], acc);
    if (more) {
      la.end(sm.a[nxt]);
      lb.end(sm.b[nxt]);
      sa.end(sm.sa[nxt]);
      sb.end(sm.sb[nxt]);
    }
    wait_vmem();
    __syncthreads();
  }
}

// ------------------------------------------------------------------ epilogue staging
// Output tile staged in LDS as bf16 [BM][W] (row pitch W*2 + 16 bytes), then
// written out as 16-byte row chunks to per-row destinations.
template <int BM, int W>
struct OutStage {
  static constexpr int PITCH = W * 2 + 16;
  MOK_DEV static void put(uint8_t* lds, int r, int c, float v) {
    *reinterpret_cast<bf16_t*>(lds + r * PITCH + c * 2) = f32_to_bf16(v);
  }
  MOK_DEV static void put_bits(uint8_t* lds, int r, int c, bf16_t v) {
    *reinterpret_cast<bf16_t*>(lds + r * PITCH + c * 2) = v;
  }
  // dst(r) = byte address of output row r (column 0 of the tile); rows >= nrows
  // and columns >= ncols are skipped.
  template <class Dst>
  MOK_DEV static void store(const uint8_t* lds, int nrows, int ncols, Dst dst) {
    constexpr int CPR = W / 8;                       // 16-byte chunks per row
    for (int idx = threadIdx.x; idx < BM * CPR; idx += kThreads) {
      const int r = idx / CPR, c = idx % CPR;
      if (r < nrows && c * 8 < ncols)
        *reinterpret_cast<uint4*>(dst(r) + c * 16) = *reinterpret_cast<const uint4*>(lds + r * PITCH + c * 16);
    }
  }
};

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
    __syncthreads();
    HS::put(lds, acc, half);
    __syncthreads();
    const int rows = min(128, nrows - 128 * half);
    for (int idx = threadIdx.x; idx < 128 * CPR; idx += kThreads) {
      const int r = idx / CPR, c = (idx % CPR) * 8;
      if (r >= rows || c >= ncols) continue;
      float v[8];
      HS::get8(lds, r, c, v);
      *reinterpret_cast<uint4*>(dst(128 * half + r) + c) = pack_bf16x8(v);
    }
  }
}

}  // namespace mok
