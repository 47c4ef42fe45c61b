// Router front end: logits, top-k selection and combine weights, and the
// backward from d topk_w.
//
// [MoK clip] key chart, "Router picks top-k": for each token the router
// scores every expert and hands the layer its k experts and their combine
// weights. The pages give no formula; the reading implemented here:
// logits = x . Wr^T (Wr [E][H] fp32, x bf16, fp32 accumulation in a fixed
// order), selection score = logit + bias_e (bias optional), the k largest
// scores in descending order with equal scores in ascending expert id, and
// combine weights = softmax of the k selected unbiased logits (fp32).
// Backward: only the selected logits carry gradient, through the softmax:
// d_sel[t][j] = w_j (g_j - sum_i w_i g_i) with g = d topk_w; then
// dx[t] = sum_j d_sel[t][j] Wr[e_j] and dWr[e] = sum over the rows routed
// to e of d_sel * x[t]. No atomics: every sum has a fixed order.
#include "mok_device.h"
#include "mok_launch.h"

namespace {

constexpr int kRouterTokens = 16;                // tokens per forward workgroup (one 16-row MFMA tile)
constexpr int kRouterWaves = 8;                  // K split across the workgroup's wavefronts
constexpr int kRouterThreads = 64 * kRouterWaves;
constexpr int kRouterMaxE = 512;
constexpr int kRouterGroup = 64;                 // experts per accumulation group (4 column tiles)

typedef __attribute__((ext_vector_type(4))) short rv4i16_t;
typedef __attribute__((address_space(3))) rv4i16_t* lds_rv4_ptr;

MOK_DEV float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
MOK_DEV float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// (score, expert) a beats b: higher score, or equal score and lower id
MOK_DEV bool beats(float sa, int ea, float sb, int eb) { return sa > sb || (sa == sb && ea < eb); }

// Exact three-way split of fp32 values into bf16: w = hi + mid + lo, each
// part the truncation of what remains (8 significant bits each, 24 in all),
// so x * part is exact in fp32 for bf16 x and the MFMA sums exact products.
// Pairs are packed two bf16 per dword (element 2i in the low half).
MOK_DEV void split3(float w0, float w1, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  const uint32_t u0 = __float_as_uint(w0), u1 = __float_as_uint(w1);
  const float r0 = w0 - __uint_as_float(u0 & 0xFFFF0000u), r1 = w1 - __uint_as_float(u1 & 0xFFFF0000u);
  const uint32_t v0 = __float_as_uint(r0), v1 = __float_as_uint(r1);
  const float q0 = r0 - __uint_as_float(v0 & 0xFFFF0000u), q1 = r1 - __uint_as_float(v1 & 0xFFFF0000u);
  hi = (u0 >> 16) | (u1 & 0xFFFF0000u);
  mid = (v0 >> 16) | (v1 & 0xFFFF0000u);
  lo = (__float_as_uint(q0) >> 16) | (__float_as_uint(q1) & 0xFFFF0000u);
}

// Forward: one workgroup per TT tokens (TT = 16, or 64 on large inputs with
// E <= 128). The logits x . Wr^T are a dense contraction (TT token rows x E
// expert columns x H), done on the matrix cores with
// v_mfma_f32_16x16x32_bf16 (lane l supplies row l%16 of a 16-row tile and the
// 8 K values from 8(l/16), so four lanes read one full 128-byte line of a Wr
// row): x is bf16 already and Wr is split exactly into three bf16 parts, so
// every product is exact and the fp32 sums run in the MFMA's fixed order.
// Wave v sums the 32-wide K steps v, v + 8, ... for up to 64 experts at a
// time; the eight partial sums are added in the order v = 0..7 through LDS
// (with TT = 64 one 16-row tile at a time). Each split of a Wr block serves
// the TT/16 row tiles of the workgroup, so larger TT splits and reads Wr
// fewer times per token; every logit is the same sum in the same order
// whatever TT. Then each wavefront selects the top-k of TT/8 tokens: with
// E <= 64 by ranking each lane's expert against all others; otherwise lane
// l holds experts l, l + 64, ... and each of k rounds takes the best
// unselected (score, expert) pair of the wavefront.
template <int TT>
__global__ __launch_bounds__(kRouterThreads) void router_fwd_kernel(
    const bf16_t* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ bias, int64_t T,
    int H, int E, int k, int32_t* __restrict__ ids, float* __restrict__ w) {
  constexpr int NR = TT / 16;                                             // 16-row tiles
  constexpr int LGE = TT == 16 ? kRouterMaxE : 128;                       // logit row length in LDS
  constexpr int NU = TT == 16 ? 4 : 2;                                    // K steps per load batch
  __shared__ float lg[TT * LGE];                                          // [TT][E] logits
  __shared__ float part[kRouterWaves - 1][16 * kRouterGroup];             // waves 1..7 partials
  __shared__ float bsh[kRouterMaxE];                                      // bias (0 if none)
  const int64_t t0 = (int64_t)blockIdx.x * TT;
  const int v = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = lane_id();
  const int r16 = lane & 15, kh = 8 * (lane >> 4);
  const int nsteps = H / 32;                                              // 32-wide K steps
  bool trow[NR];
  const bf16_t* xrow[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    trow[r] = t0 + 16 * r + r16 < T;
    xrow[r] = x + (t0 + (trow[r] ? 16 * r + r16 : 0)) * H + kh;           // row t0 exists: t0 < T
  }
  for (int e = threadIdx.x; e < E; e += kRouterThreads) bsh[e] = bias ? bias[e] : 0.f;
  for (int g0 = 0; g0 < E; g0 += kRouterGroup) {
    const int nb = min(4, (E - g0 + 15) / 16);                           // column tiles in this group
    f32x4_t acc[NR][4];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[r][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // wave v takes the K steps v, v + 8, v + 16, ... in ascending order, in
    // batches of up to NU whose loads are all issued before the first MFMA
    for (int s0 = v; s0 < nsteps; s0 += NU * kRouterWaves) {
      const int nu = min(NU, (nsteps - s0 + kRouterWaves - 1) / kRouterWaves);
      uint4 xa[NU][NR];
      float4 wv[4][NU][2];
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          xa[u][r] = make_uint4(0u, 0u, 0u, 0u);
          if (u < nu && trow[r]) xa[u][r] = *reinterpret_cast<const uint4*>(xrow[r] + 32 * (s0 + kRouterWaves * u));
        }
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int e = g0 + 16 * b + r16;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          wv[b][u][0] = wv[b][u][1] = make_float4(0.f, 0.f, 0.f, 0.f);
          if (b < nb && u < nu && e < E) {
            const float4* src =
                reinterpret_cast<const float4*>(wr + (int64_t)e * H + 32 * (s0 + kRouterWaves * u) + kh);
            wv[b][u][0] = src[0];
            wv[b][u][1] = src[1];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        if (u >= nu) break;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          if (b >= nb) break;
          const float4 p = wv[b][u][0], q = wv[b][u][1];
          uint4 hi, mid, lo;
          split3(p.x, p.y, hi.x, mid.x, lo.x);
          split3(p.z, p.w, hi.y, mid.y, lo.y);
          split3(q.x, q.y, hi.z, mid.z, lo.z);
          split3(q.z, q.w, hi.w, mid.w, lo.w);
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            const bf16x8_t a = __builtin_bit_cast(bf16x8_t, xa[u][r]);
            acc[r][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, hi), acc[r][b], 0, 0, 0);
            acc[r][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, mid), acc[r][b], 0, 0, 0);
            acc[r][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, lo), acc[r][b], 0, 0, 0);
          }
        }
      }
    }
    // accumulator element i: token row 16r + 4(lane/16) + i, expert column
    // lane%16; the partials of one row tile at a time through LDS
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      if (v > 0) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          if (b >= nb) break;
#pragma unroll
          for (int i = 0; i < 4; ++i) part[v - 1][(4 * (lane >> 4) + i) * kRouterGroup + 16 * b + r16] = acc[r][b][i];
        }
      }
      __syncthreads();
      if (v == 0) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          if (b >= nb) break;
          const int e = g0 + 16 * b + r16;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 4 * (lane >> 4) + i;
            const int pi = row * kRouterGroup + 16 * b + r16;
            float sum = acc[r][b][i];
            for (int j = 0; j < kRouterWaves - 1; ++j) sum += part[j][pi];
            if (e < E) lg[(16 * r + row) * E + e] = sum;
          }
        }
      }
      __syncthreads();
    }
  }
  constexpr int TPW = TT / kRouterWaves;                                  // tokens per wavefront
  if (E <= 64) {
    // one expert per lane: its rank is the number of experts that beat it
    // (LDS broadcast reads, no cross-lane traffic); the k lanes of rank < k
    // write their own slot. The softmax runs over the selected experts in
    // ascending id, the same order in every lane.
    for (int q = 0; q < TPW; ++q) {
      const int tt = TPW * v + q;
      const int64_t t = t0 + tt;
      if (t >= T) break;
      const float* row = lg + tt * E;
      const int e = lane < E ? lane : 0;
      const float me = row[e] + bsh[e];
      int rank = 0;
#pragma unroll 8
      for (int e2 = 0; e2 < E; ++e2) rank += beats(row[e2] + bsh[e2], e2, me, e) ? 1 : 0;
      const bool sel = lane < E && rank < k;
      uint64_t msk = __ballot(sel);
      float m = -INFINITY;
      for (uint64_t r = msk; r; r &= r - 1) m = fmaxf(m, row[__builtin_ctzll(r)]);
      float den = 0.f;
      for (uint64_t r = msk; r; r &= r - 1) den += expf(row[__builtin_ctzll(r)] - m);
      if (sel) {
        ids[t * k + rank] = lane;
        w[t * k + rank] = expf(row[lane] - m) / den;
      }
    }
    return;
  }
  for (int q = 0; q < TPW; ++q) {
    const int tt = TPW * v + q;
    const int64_t t = t0 + tt;
    if (t >= T) break;
    uint64_t taken = 0;                          // bit i: expert lane + 64 i selected
    float m = 0.f;                               // max selected logit (set in round 0)
    float sel_l = 0.f;                           // this lane's j-th selected logit (lane j < k)
    int sel_e = 0;
    for (int j = 0; j < k; ++j) {
      float bs = -INFINITY;
      int be = 0x7FFFFFFF;
      for (int i = 0; lane + 64 * i < E; ++i) {
        const int e = lane + 64 * i;
        if ((taken >> i) & 1) continue;
        const float sc = lg[tt * E + e] + bsh[e];
        if (be == 0x7FFFFFFF || beats(sc, e, bs, be)) { bs = sc; be = e; }
      }
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) {
        const float os = __shfl_xor(bs, d);
        const int oe = __shfl_xor(be, d);
        if (be == 0x7FFFFFFF || (oe != 0x7FFFFFFF && beats(os, oe, bs, be))) { bs = os; be = oe; }
      }
      if ((be & 63) == lane) taken |= 1ull << (be >> 6);
      const float l = lg[tt * E + be];
      m = j == 0 ? l : fmaxf(m, l);
      if (lane == j) { sel_l = l; sel_e = be; }
    }
    const float ex = lane < k ? expf(sel_l - m) : 0.f;
    float den = ex;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) den += __shfl_xor(den, d);
    if (lane < k) {
      ids[t * k + lane] = sel_e;
      w[t * k + lane] = ex / den;
    }
  }
}

// Backward, per token: d_sel[t][j] = w_j (g_j - sum_i w_i g_i) (i, j
// ascending), and dx[t] = sum_j d_sel[t][j] Wr[e_j] in fp32, j ascending,
// rounded once to bf16. One wavefront per token: its ids, weights and
// gradients are wave-uniform (scalar loads), lane l takes the 8-column chunks
// l, l + 64, ..., two at a time with all their Wr loads in flight; lane 0
// writes d_sel. Ids outside [0, E) contribute nothing.
__global__ __launch_bounds__(256) void router_bwd_rows_kernel(
    const float* __restrict__ wr, const int32_t* __restrict__ ids, const float* __restrict__ w,
    const float* __restrict__ g, int64_t T, int H, int E, int k, float* __restrict__ d_sel,
    bf16_t* __restrict__ dx) {
  const int64_t t = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * 4 + (threadIdx.x >> 6)));
  const int lane = lane_id();
  if (t >= T) return;
  const int64_t nch = H / 8;
  float s = 0.f;
  for (int j = 0; j < k; ++j) s = fmaf(w[t * k + j], g[t * k + j], s);
  if (lane == 0)
    for (int j = 0; j < k; ++j) d_sel[t * k + j] = w[t * k + j] * (g[t * k + j] - s);
  for (int64_t c0 = lane; c0 < nch; c0 += 128) {
    float acc[2][8];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[b][q] = 0.f;
    const int64_t cb[2] = {c0, min(c0 + 64, nch - 1)};
    for (int j = 0; j < k; ++j) {
      const float dl = w[t * k + j] * (g[t * k + j] - s);
      const int e = ids[t * k + j];
      if (e < 0 || e >= E) continue;
      float4 a[2], b[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float4* wrow = reinterpret_cast<const float4*>(wr + (int64_t)e * H + 8 * cb[u]);
        a[u] = wrow[0];
        b[u] = wrow[1];
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        acc[u][0] = fmaf(dl, a[u].x, acc[u][0]); acc[u][1] = fmaf(dl, a[u].y, acc[u][1]);
        acc[u][2] = fmaf(dl, a[u].z, acc[u][2]); acc[u][3] = fmaf(dl, a[u].w, acc[u][3]);
        acc[u][4] = fmaf(dl, b[u].x, acc[u][4]); acc[u][5] = fmaf(dl, b[u].y, acc[u][5]);
        acc[u][6] = fmaf(dl, b[u].z, acc[u][6]); acc[u][7] = fmaf(dl, b[u].w, acc[u][7]);
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (u == 1 && c0 + 64 >= nch) break;
      reinterpret_cast<uint4*>(dx + t * H)[cb[u]] =
          make_uint4(pack_bf16x2(acc[u][0], acc[u][1]), pack_bf16x2(acc[u][2], acc[u][3]),
                     pack_bf16x2(acc[u][4], acc[u][5]), pack_bf16x2(acc[u][6], acc[u][7]));
    }
  }
}

// dWr[e][h] = sum over the permuted rows p of expert e of d_sel[perm[p]] *
// x[tok[p]][h], fp32. Workgroup (e, 512 columns) of 16 wavefronts:
// wavefront v sums the rows p = o_e + v, o_e + v + 16, ... in ascending
// order (8 columns per lane), then the 16 partial sums are added in the
// order v = 0..15: a fixed partition of the expert's rows, so the result is
// bitwise reproducible. Each wavefront first loads the (d_sel, token) pairs
// of its next 64 rows, one per lane, then walks them in order, so the x row
// loads do not wait on the table loads. Experts with no rows get exact zeros.
constexpr int kDwrWaves = 16;
__global__ __launch_bounds__(64 * kDwrWaves) void router_dwr_kernel(
    const bf16_t* __restrict__ x, const float* __restrict__ d_sel, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ tok, int H, int ncol,
    float* __restrict__ d_wr) {
  __shared__ float part[kDwrWaves - 1][512];
  const int e = (int)blockIdx.x / ncol, cb = (int)blockIdx.x % ncol;
  const int v = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = lane_id();
  const int col = cb * 512 + 8 * lane;
  const bool ok = col < H;
  const int o = offsets[e], n = offsets[e + 1] - o;
  const int nv = n > v ? (n - v + kDwrWaves - 1) / kDwrWaves : 0;      // rows of this wavefront
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int base = 0; base < nv; base += 64) {
    float dl_l = 0.f;
    int tr_l = 0;
    if (base + lane < nv) {
      const int p = o + v + kDwrWaves * (base + lane);
      dl_l = d_sel[perm[p]];
      tr_l = tok[p];
    }
    const int cnt = min(64, nv - base);
#pragma unroll 16
    for (int i = 0; i < cnt; ++i) {
      const float dl = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, dl_l), i));
      const int64_t tr = __builtin_amdgcn_readlane(tr_l, i);
      if (!ok) continue;
      const uint4 xv = *reinterpret_cast<const uint4*>(x + tr * H + col);
      acc[0] = fmaf(dl, bf16_lo(xv.x), acc[0]); acc[1] = fmaf(dl, bf16_hi(xv.x), acc[1]);
      acc[2] = fmaf(dl, bf16_lo(xv.y), acc[2]); acc[3] = fmaf(dl, bf16_hi(xv.y), acc[3]);
      acc[4] = fmaf(dl, bf16_lo(xv.z), acc[4]); acc[5] = fmaf(dl, bf16_hi(xv.z), acc[5]);
      acc[6] = fmaf(dl, bf16_lo(xv.w), acc[6]); acc[7] = fmaf(dl, bf16_hi(xv.w), acc[7]);
    }
  }
  if (v > 0) {
#pragma unroll
    for (int u = 0; u < 8; ++u) part[v - 1][8 * lane + u] = acc[u];
  }
  __syncthreads();
  if (v == 0 && ok) {
    float out[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float s = acc[u];
      for (int i = 0; i < kDwrWaves - 1; ++i) s += part[i][8 * lane + u];
      out[u] = s;
    }
    float4* d = reinterpret_cast<float4*>(d_wr + (int64_t)e * H + col);
    d[0] = make_float4(out[0], out[1], out[2], out[3]);
    d[1] = make_float4(out[4], out[5], out[6], out[7]);
  }
}

// dWr for E <= 128 and k <= 8, as a dense contraction over the tokens on
// the matrix cores: dWr[e][h] = sum over t of D[t][e] x[t][h] with D[t][e] =
// d_sel[t][j] for the j with ids[t][j] == e (0 for the other experts). x is
// read once (the per-expert kernel above reads each token's row k times), at
// the price of E/k times the products, which are cheap here. Workgroup = NW
// wavefronts over 32 output columns of every expert; wavefront v takes the
// 32-token steps v, v + NW, ... in ascending order, each on its own: it
// scatters its 32 tokens' d_sel into its LDS block D^T [EP][32] (cleared
// again after use), stages the tokens' 32 x 32 slice of x in LDS, and runs
// v_mfma_f32_16x16x32_bf16 with D^T split exactly into three bf16 parts (so
// every product d_sel * x is exact and the fp32 sums follow the MFMA's fixed
// order), the x operand read transposed (ds_read_b64_tr_b16). The next
// step's ids, d_sel and x are loaded into registers before the current step
// runs. The NW partial sums are added in the order v = 0 .. NW-1. Bitwise
// reproducible.
template <int EP, int NW>
__global__ __launch_bounds__(64 * NW) void router_dwr_dense_kernel(
    const bf16_t* __restrict__ x, const int32_t* __restrict__ ids, const float* __restrict__ d_sel, int64_t T,
    int H, int E, int k, float* __restrict__ d_wr) {
  constexpr int NC = 32;                          // output columns per workgroup
  constexpr int RT = EP / 16, CT = NC / 16;       // 16 x 16 output tiles
  constexpr int DP = 36;                          // D^T row pitch (floats)
  constexpr int XB = 2 * NC;                      // x slice row bytes
  constexpr int KMAX = 8;
  static_assert((NW - 1) * EP * NC <= NW * EP * DP, "partials fit in the D^T blocks");
  __shared__ __attribute__((aligned(16))) float dT[NW][EP * DP];
  __shared__ __attribute__((aligned(16))) uint8_t xs[NW][32 * XB];
  const int v = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = lane_id();
  const int g = lane >> 4, L = lane & 15;
  const int64_t c0 = (int64_t)blockIdx.x * NC;
  float* dw = dT[v];
  uint8_t* xw = xs[v];
  for (int i = lane; i < EP * DP; i += 64) dw[i] = 0.f;
  f32x4_t acc[RT][CT];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int c = 0; c < CT; ++c) acc[r][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int64_t nsteps = (T + 31) / 32;
  // this lane's share of a step: token t0 + (lane & 31)'s ids and d_sel
  // (lanes < 32), and two 16-byte chunks of the x slice
  int e_n[KMAX];
  float d_n[KMAX];
  uint4 x_n[2];
  auto load = [&](int64_t s) {
    const int64_t t0 = 32 * s, t = t0 + (lane & 31);
    const bool tok_ok = s < nsteps && lane < 32 && t < T;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      e_n[j] = -1;
      d_n[j] = 0.f;
      if (tok_ok && j < k) {
        e_n[j] = ids[t * k + j];
        d_n[j] = d_sel[t * k + j];
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = lane + 64 * u, r = q / (XB / 16), ch = q % (XB / 16);
      x_n[u] = make_uint4(0u, 0u, 0u, 0u);
      if (s < nsteps && t0 + r < T) x_n[u] = *reinterpret_cast<const uint4*>(x + (t0 + r) * H + c0 + 8 * ch);
    }
  };
  load(v);
  for (int64_t s = v; s < nsteps; s += NW) {
    int e_c[KMAX];
    float d_c[KMAX];
    uint4 x_c[2];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) { e_c[j] = e_n[j]; d_c[j] = d_n[j]; }
    x_c[0] = x_n[0];
    x_c[1] = x_n[1];
    load(s + NW);                                // in flight while this step runs
    // scatter (this lane's token; an expert appears once per token, duplicates add)
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (e_c[j] >= 0 && e_c[j] < E) dw[e_c[j] * DP + lane] += d_c[j];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = lane + 64 * u, r = q / (XB / 16), ch = q % (XB / 16);
      *reinterpret_cast<uint4*>(xw + r * XB + 16 * ch) = x_c[u];
    }
    // the wavefront's LDS writes land in order before its reads below
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    bf16x8_t bfr[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      // lane 4q + p of a 16-lane group addresses k-row q, columns 4p..4p+3;
      // lane L receives column L, 4 k-rows; two reads give k-rows 8g .. 8g+7
      const uint8_t* a0 = xw + (8 * g + (L >> 2)) * XB + 2 * (16 * c + 4 * (L & 3));
      const rv4i16_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_rv4_ptr)(a0));
      const rv4i16_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_rv4_ptr)(a0 + 4 * XB));
      typedef __attribute__((ext_vector_type(8))) short v8i16_t;
      bfr[c] = __builtin_bit_cast(bf16x8_t, v8i16_t{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]});
    }
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const float4 p = *reinterpret_cast<const float4*>(dw + (16 * r + L) * DP + 8 * g);
      const float4 q = *reinterpret_cast<const float4*>(dw + (16 * r + L) * DP + 8 * g + 4);
      uint4 hi, mid, lo;
      split3(p.x, p.y, hi.x, mid.x, lo.x);
      split3(p.z, p.w, hi.y, mid.y, lo.y);
      split3(q.x, q.y, hi.z, mid.z, lo.z);
      split3(q.z, q.w, hi.w, mid.w, lo.w);
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        acc[r][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, hi), bfr[c], acc[r][c], 0, 0, 0);
        acc[r][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, mid), bfr[c], acc[r][c], 0, 0, 0);
        acc[r][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, lo), bfr[c], acc[r][c], 0, 0, 0);
      }
    }
    // reads of this step done before the clear and the next step's writes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (e_c[j] >= 0 && e_c[j] < E) dw[e_c[j] * DP + lane] = 0.f;
  }
  // accumulator element i: expert 16r + 4g + i, column 16c + L; the partials
  // of waves 1 .. NW-1 go through the D^T blocks (free now)
  __syncthreads();
  float* part = &dT[0][0];
  if (v > 0) {
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) part[((v - 1) * EP + 16 * r + 4 * g + i) * NC + 16 * c + L] = acc[r][c][i];
  }
  __syncthreads();
  if (v == 0) {
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = 16 * r + 4 * g + i, col = 16 * c + L;
          float sum = acc[r][c][i];
          for (int u = 0; u < NW - 1; ++u) sum += part[(u * EP + e) * NC + col];
          if (e < E) d_wr[(int64_t)e * H + c0 + col] = sum;
        }
  }
}

}  // namespace

hipError_t mok_launch_router_forward(const bf16_t* x, const float* wr, const float* bias, int64_t T, int H,
                                     int E, int k, int32_t* ids, float* w, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  // 64-token workgroups once they still fill every compute unit several
  // times over (and the logits of 64 tokens fit in LDS), else 16
  if (E <= 128 && T >= 64 * 256) {
    const unsigned grid = (unsigned)((T + 63) / 64);
    hipLaunchKernelGGL(router_fwd_kernel<64>, dim3(grid), dim3(kRouterThreads), 0, st, x, wr, bias, T, H, E, k, ids,
                       w);
  } else {
    const unsigned grid = (unsigned)((T + kRouterTokens - 1) / kRouterTokens);
    hipLaunchKernelGGL(router_fwd_kernel<kRouterTokens>, dim3(grid), dim3(kRouterThreads), 0, st, x, wr, bias, T, H,
                       E, k, ids, w);
  }
  return hipGetLastError();
}

hipError_t mok_launch_router_backward(const bf16_t* x, const float* wr, const int32_t* ids, const float* w,
                                      const float* g, int64_t T, int H, int E, int k,
                                      const int32_t* offsets, const int32_t* perm, const int32_t* tok,
                                      float* d_sel, bf16_t* dx, float* d_wr, hipStream_t st) {
  if (T > 0)
    hipLaunchKernelGGL(router_bwd_rows_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, st, wr, ids, w, g, T, H,
                       E, k, d_sel, dx);
  if (E <= 128 && k <= 8 && T > 0) {
    // dense over the tokens (x read once); H is a multiple of 128
    const dim3 grid((unsigned)(H / 32));
    if (E <= 32)
      hipLaunchKernelGGL((router_dwr_dense_kernel<32, 16>), grid, dim3(64 * 16), 0, st, x, ids, d_sel, T, H, E, k,
                         d_wr);
    else if (E <= 64)
      hipLaunchKernelGGL((router_dwr_dense_kernel<64, 8>), grid, dim3(64 * 8), 0, st, x, ids, d_sel, T, H, E, k,
                         d_wr);
    else
      hipLaunchKernelGGL((router_dwr_dense_kernel<128, 4>), grid, dim3(64 * 4), 0, st, x, ids, d_sel, T, H, E, k,
                         d_wr);
    return hipGetLastError();
  }
  const int ncol = (H + 511) / 512;
  hipLaunchKernelGGL(router_dwr_kernel, dim3((unsigned)(E * ncol)), dim3(64 * kDwrWaves), 0, st, x, d_sel, offsets, perm, tok,
                     H, ncol, d_wr);
  return hipGetLastError();
}
