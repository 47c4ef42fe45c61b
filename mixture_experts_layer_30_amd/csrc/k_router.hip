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

constexpr int kRouterTokens = 8;                 // tokens per forward workgroup
constexpr int kRouterThreads = 256;

MOK_DEV float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
MOK_DEV float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// (score, expert) a beats b: higher score, or equal score and lower id
MOK_DEV bool beats(float sa, int ea, float sb, int eb) { return sa > sb || (sa == sb && ea < eb); }

// Forward: one workgroup per 8 tokens. The tokens' x rows sit in LDS; for
// each expert, thread (token = tid / 32, slice = tid % 32) sums its 8-wide
// chunks c = slice, slice + 32, ... in ascending order and the 32 slices are
// combined by a xor butterfly (a fixed tree), so every logit is a fixed
// function of its inputs. Then each wavefront selects the top-k of two
// tokens: lane l holds experts l, l + 64, ...; each of k rounds takes the
// best unselected pair (score, expert) of the wavefront.
__global__ __launch_bounds__(kRouterThreads) void router_fwd_kernel(
    const bf16_t* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ bias, int64_t T,
    int H, int E, int k, int32_t* __restrict__ ids, float* __restrict__ w) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  bf16_t* xs = reinterpret_cast<bf16_t*>(smem);                           // [8][H]
  float* lg = reinterpret_cast<float*>(smem + (size_t)kRouterTokens * H * 2);   // [8][E]
  const int64_t t0 = (int64_t)blockIdx.x * kRouterTokens;
  const int nch = H / 8;                                                  // 16-byte chunks per row
  for (int i = threadIdx.x; i < kRouterTokens * nch; i += kRouterThreads) {
    const int tk = i / nch, c = i % nch;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (t0 + tk < T) v = reinterpret_cast<const uint4*>(x + (t0 + tk) * H)[c];
    reinterpret_cast<uint4*>(xs + (int64_t)tk * H)[c] = v;
  }
  __syncthreads();
  const int tk = threadIdx.x >> 5, sl = threadIdx.x & 31;
  const uint4* xrow = reinterpret_cast<const uint4*>(xs + (int64_t)tk * H);
  for (int e = 0; e < E; ++e) {
    const float4* wrow = reinterpret_cast<const float4*>(wr + (int64_t)e * H);
    float acc = 0.f;
    for (int c = sl; c < nch; c += 32) {
      const uint4 xv = xrow[c];
      const float4 a = wrow[2 * c], b = wrow[2 * c + 1];
      acc = fmaf(bf16_lo(xv.x), a.x, acc);
      acc = fmaf(bf16_hi(xv.x), a.y, acc);
      acc = fmaf(bf16_lo(xv.y), a.z, acc);
      acc = fmaf(bf16_hi(xv.y), a.w, acc);
      acc = fmaf(bf16_lo(xv.z), b.x, acc);
      acc = fmaf(bf16_hi(xv.z), b.y, acc);
      acc = fmaf(bf16_lo(xv.w), b.z, acc);
      acc = fmaf(bf16_hi(xv.w), b.w, acc);
    }
#pragma unroll
    for (int s = 16; s >= 1; s >>= 1) acc += __shfl_xor(acc, s);
    if (sl == 0) lg[tk * E + e] = acc;
  }
  __syncthreads();
  const int wv = threadIdx.x >> 6, lane = lane_id();
  for (int q = 0; q < 2; ++q) {
    const int tt = 2 * wv + q;
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
        const float s = lg[tt * E + e] + (bias ? bias[e] : 0.f);
        if (be == 0x7FFFFFFF || beats(s, e, bs, be)) { bs = s; be = e; }
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
// rounded once to bf16. One thread per (token, 8 columns); the thread of
// column chunk 0 also writes d_sel. Ids outside [0, E) contribute nothing.
__global__ __launch_bounds__(256) void router_bwd_rows_kernel(
    const float* __restrict__ wr, const int32_t* __restrict__ ids, const float* __restrict__ w,
    const float* __restrict__ g, int64_t T, int H, int E, int k, float* __restrict__ d_sel,
    bf16_t* __restrict__ dx) {
  const int64_t nch = H / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t t = idx / nch, c = idx % nch;
  if (t >= T) return;
  float s = 0.f;
  for (int j = 0; j < k; ++j) s = fmaf(w[t * k + j], g[t * k + j], s);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const float dl = w[t * k + j] * (g[t * k + j] - s);
    if (c == 0) d_sel[t * k + j] = dl;
    const int e = ids[t * k + j];
    if (e < 0 || e >= E) continue;
    const float4* wrow = reinterpret_cast<const float4*>(wr + (int64_t)e * H + 8 * c);
    const float4 a = wrow[0], b = wrow[1];
    acc[0] = fmaf(dl, a.x, acc[0]); acc[1] = fmaf(dl, a.y, acc[1]);
    acc[2] = fmaf(dl, a.z, acc[2]); acc[3] = fmaf(dl, a.w, acc[3]);
    acc[4] = fmaf(dl, b.x, acc[4]); acc[5] = fmaf(dl, b.y, acc[5]);
    acc[6] = fmaf(dl, b.z, acc[6]); acc[7] = fmaf(dl, b.w, acc[7]);
  }
  reinterpret_cast<uint4*>(dx + t * H)[c] = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                                       pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
}

// dWr[e][h] = sum over the permuted rows p of expert e of d_sel[perm[p]] *
// x[tok[p]][h], fp32. Workgroup (e, 512 columns): wavefront v sums the rows
// p = o_e + v, o_e + v + 4, ... in ascending order (8 columns per lane), then
// the four partial sums are added in the order v = 0..3: a fixed partition
// of the expert's rows, so the result is bitwise reproducible. Experts with
// no rows get exact zeros.
__global__ __launch_bounds__(256) void router_dwr_kernel(
    const bf16_t* __restrict__ x, const float* __restrict__ d_sel, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ tok, int H, int ncol,
    float* __restrict__ d_wr) {
  __shared__ float part[3][512];
  const int e = (int)blockIdx.x / ncol, cb = (int)blockIdx.x % ncol;
  const int v = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = lane_id();
  const int col = cb * 512 + 8 * lane;
  const bool ok = col < H;
  const int o = offsets[e], n = offsets[e + 1] - o;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int r = v; r < n; r += 4) {
    const int p = o + r;
    const float dl = d_sel[perm[p]];             // wave-uniform loads
    const int64_t tr = tok[p];
    if (!ok) continue;
    const uint4 xv = *reinterpret_cast<const uint4*>(x + tr * H + col);
    acc[0] = fmaf(dl, bf16_lo(xv.x), acc[0]); acc[1] = fmaf(dl, bf16_hi(xv.x), acc[1]);
    acc[2] = fmaf(dl, bf16_lo(xv.y), acc[2]); acc[3] = fmaf(dl, bf16_hi(xv.y), acc[3]);
    acc[4] = fmaf(dl, bf16_lo(xv.z), acc[4]); acc[5] = fmaf(dl, bf16_hi(xv.z), acc[5]);
    acc[6] = fmaf(dl, bf16_lo(xv.w), acc[6]); acc[7] = fmaf(dl, bf16_hi(xv.w), acc[7]);
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
      s += part[0][8 * lane + u];
      s += part[1][8 * lane + u];
      s += part[2][8 * lane + u];
      out[u] = s;
    }
    float4* d = reinterpret_cast<float4*>(d_wr + (int64_t)e * H + col);
    d[0] = make_float4(out[0], out[1], out[2], out[3]);
    d[1] = make_float4(out[4], out[5], out[6], out[7]);
  }
}

}  // namespace

size_t mok_router_lds_bytes(int H, int E) {
  return (size_t)kRouterTokens * H * 2 + (size_t)kRouterTokens * E * 4;
}

hipError_t mok_launch_router_forward(const bf16_t* x, const float* wr, const float* bias, int64_t T, int H,
                                     int E, int k, int32_t* ids, float* w, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  const unsigned grid = (unsigned)((T + kRouterTokens - 1) / kRouterTokens);
  hipLaunchKernelGGL(router_fwd_kernel, dim3(grid), dim3(kRouterThreads), mok_router_lds_bytes(H, E), st, x, wr,
                     bias, T, H, E, k, ids, w);
  return hipGetLastError();
}

hipError_t mok_launch_router_backward(const bf16_t* x, const float* wr, const int32_t* ids, const float* w,
                                      const float* g, int64_t T, int H, int E, int k,
                                      const int32_t* offsets, const int32_t* perm, const int32_t* tok,
                                      float* d_sel, bf16_t* dx, float* d_wr, hipStream_t st) {
  if (T > 0) {
    const int64_t n = T * (H / 8);
    hipLaunchKernelGGL(router_bwd_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, wr, ids, w, g,
                       T, H, E, k, d_sel, dx);
  }
  const int ncol = (H + 511) / 512;
  hipLaunchKernelGGL(router_dwr_kernel, dim3((unsigned)(E * ncol)), dim3(256), 0, st, x, d_sel, offsets, perm, tok,
                     H, ncol, d_wr);
  return hipGetLastError();
}
