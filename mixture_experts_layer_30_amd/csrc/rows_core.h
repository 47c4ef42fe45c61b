// Row-wise device steps shared by the row kernels (k_rows.hip) and the
// single-launch layer (k_gemm.hip): bf16 row chunks, the weighted combine of
// one (token, 8 columns) element, and the MXFP8 quantization of one
// 32-element block.
#pragma once
#include "mok_device.h"

namespace {

MOK_DEV void unpack8(const uint4& v, float f[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f[2 * q] = __uint_as_float(w[q] << 16);
    f[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
  }
}

MOK_DEV uint4 pack8(const float f[8]) {
  uint4 r;
  r.x = pack_bf16x2(f[0], f[1]);
  r.y = pack_bf16x2(f[2], f[3]);
  r.z = pack_bf16x2(f[4], f[5]);
  r.w = pack_bf16x2(f[6], f[7]);
  return r;
}

// y[t][8c .. 8c+8) = sum over j ascending of w[t][j] * obuf[t*k+j] in fp32,
// valid rows only (dest < nvalid); w == nullptr sums with weight 1. The k
// rows are read 8 at a time before any is used, so their loads overlap (rows
// of invalid ids and j >= k read a valid row and are dropped).
MOK_DEV void combine_elem(const bf16_t* __restrict__ obuf, const float* __restrict__ w,
                          const int32_t* __restrict__ dest, int nvalid, int64_t t, int64_t c, int topk,
                          int64_t H, bf16_t* __restrict__ y) {
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < topk; j0 += 8) {
    uint4 v[8];
    float wv[8];
    bool ok[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u;
      const int64_t i = t * topk + min(j, topk - 1);
      ok[u] = j < topk && dest[i] < nvalid;
      wv[u] = w ? w[i] : 1.0f;
      v[u] = reinterpret_cast<const uint4*>(obuf + i * H)[c];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (!ok[u]) continue;
      float o[8];
      unpack8(v[u], o);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = fmaf(wv[u], o[q], acc[q]);
    }
  }
  reinterpret_cast<uint4*>(y + t * H)[c] = pack8(acc);
}

// Block idx of a row-major [rows][K] bf16 matrix (K/32 blocks per row): amax
// -> E8M0 scale -> 32 E4M3 codes.
MOK_DEV void mx_quantize_block(const bf16_t* __restrict__ src, int64_t K, int64_t idx, uint8_t* __restrict__ q,
                               uint8_t* __restrict__ scales) {
  const int64_t nb = K >> 5;
  const int64_t r = idx / nb, b = idx - r * nb;
  const uint4* s = reinterpret_cast<const uint4*>(src + r * K + b * 32);
  float v[32];
#pragma unroll
  for (int u = 0; u < 4; ++u) unpack8(s[u], v + 8 * u);
  float amax = 0.f;
#pragma unroll
  for (int u = 0; u < 32; ++u) amax = fmaxf(amax, fabsf(v[u]));
  const int sc = mx_scale_byte(amax);
  const float inv = mx_inv_scale(sc);
  uint32_t wds[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    wds[u] = e4m3_pack4(v[4 * u] * inv, v[4 * u + 1] * inv, v[4 * u + 2] * inv,
                          v[4 * u + 3] * inv);
  }
  uint4* d = reinterpret_cast<uint4*>(q + r * K + b * 32);
  d[0] = make_uint4(wds[0], wds[1], wds[2], wds[3]);
  d[1] = make_uint4(wds[4], wds[5], wds[6], wds[7]);
  scales[idx] = (uint8_t)sc;
}

// combine_elem for every column chunk of token t, by one wavefront: lane l
// takes chunks l, l + 64, ... (nch = H/8 of them), CU chunks at a time, with
// the loads of 4 rows of each of its CU chunks in flight together. dest, w
// of the token are wave-uniform (scalar loads). Per element the same sum in
// the same order as combine_elem (bitwise equal).
template <int CU>
MOK_DEV void combine_token_wave(const bf16_t* __restrict__ obuf, const float* __restrict__ w,
                                const int32_t* __restrict__ dest, int nvalid, int64_t t, int topk, int64_t H,
                                bf16_t* __restrict__ y) {
  const int lane = lane_id();
  const int64_t nch = H >> 3;
  for (int64_t c0 = lane; c0 < nch; c0 += 64 * CU) {
    float acc[CU][8];
#pragma unroll
    for (int b = 0; b < CU; ++b)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[b][q] = 0.f;
    for (int j0 = 0; j0 < topk; j0 += 4) {
      uint4 v[CU][4];
      float wv[4];
      bool ok[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + u;
        const int64_t i = t * topk + min(j, topk - 1);
        ok[u] = j < topk && dest[i] < nvalid;
        wv[u] = w ? w[i] : 1.0f;
#pragma unroll
        for (int b = 0; b < CU; ++b) {
          const int64_t c = min(c0 + 64 * b, nch - 1);
          v[b][u] = reinterpret_cast<const uint4*>(obuf + i * H)[c];
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (!ok[u]) continue;
#pragma unroll
        for (int b = 0; b < CU; ++b) {
          float o[8];
          unpack8(v[b][u], o);
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[b][q] = fmaf(wv[u], o[q], acc[b][q]);
        }
      }
    }
#pragma unroll
    for (int b = 0; b < CU; ++b)
      if (c0 + 64 * b < nch) reinterpret_cast<uint4*>(y + t * H)[c0 + 64 * b] = pack8(acc[b]);
  }
}

// mx_quantize_block for the NB blocks i0, i0 + stride, ... below n, their
// loads issued together.
template <int NB>
MOK_DEV void mx_quantize_batch(const bf16_t* __restrict__ src, int64_t K, int64_t i0, int64_t stride, int64_t n,
                               uint8_t* __restrict__ q, uint8_t* __restrict__ scales) {
  const int64_t nb = K >> 5;
  uint4 raw[NB][4];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int64_t idx = min(i0 + b * stride, n - 1);
    const int64_t r = idx / nb, bb = idx - r * nb;
    const uint4* sp = reinterpret_cast<const uint4*>(src + r * K + bb * 32);
#pragma unroll
    for (int u = 0; u < 4; ++u) raw[b][u] = sp[u];
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int64_t idx = i0 + b * stride;
    if (idx >= n) continue;
    const int64_t r = idx / nb, bb = idx - r * nb;
    float v[32];
#pragma unroll
    for (int u = 0; u < 4; ++u) unpack8(raw[b][u], v + 8 * u);
    float amax = 0.f;
#pragma unroll
    for (int u = 0; u < 32; ++u) amax = fmaxf(amax, fabsf(v[u]));
    const int sc = mx_scale_byte(amax);
    const float inv = mx_inv_scale(sc);
    uint32_t wds[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      wds[u] = e4m3_pack4(v[4 * u] * inv, v[4 * u + 1] * inv, v[4 * u + 2] * inv, v[4 * u + 3] * inv);
    uint4* d = reinterpret_cast<uint4*>(q + r * K + bb * 32);
    d[0] = make_uint4(wds[0], wds[1], wds[2], wds[3]);
    d[1] = make_uint4(wds[4], wds[5], wds[6], wds[7]);
    scales[idx] = (uint8_t)sc;
  }
}

}  // namespace
