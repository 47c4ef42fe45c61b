// Device-side types and helpers shared by the MoE kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOK_DEV __device__ __forceinline__

typedef uint16_t bf16_t;   // bfloat16 storage (bit pattern)
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(2))) int i32x2_t;

// ------------------------------------------------------------------ schedule layout
// The schedule buffer: a header, then per-expert and per-row arrays, then the
// row-tile tables the grouped GEMMs walk. All offsets are 256-byte aligned and
// computed on the host (mok_layout.h).
struct mok_tile {          // one row tile of one expert: permuted rows [p0, p1)
  int32_t e, p0, p1, m;    // m = minibatch index (p0 / M) for forward tiles
};

// Token-blocked MXFP8 layout of the backward: an expert with c routed rows
// takes tok_pad(c) positions of the padded token axis (c rounded up to 128,
// so its scale words are whole), starting at koff[e] = the sum of tok_pad
// over the experts before it (mok_launch_token_offsets computes koff[0..E]).
MOK_DEV int tok_pad(int c) { return (c + 127) & ~127; }
constexpr int kMaxExperts = 512;

// ------------------------------------------------------------------ bf16 helpers
MOK_DEV float bf16_to_f32(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// fp32 -> bf16, round to nearest even: one v_cvt_pk_bf16_f32 per pair on
// gfx950 (the same result as rounding the bit pattern for finite inputs).
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

MOK_DEV uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

MOK_DEV bf16_t f32_to_bf16(float f) { return (bf16_t)(pack_bf16x2(f, 0.0f) & 0xFFFFu); }

// logistic sigmoid with the hardware reciprocal (about 1 ulp)
MOK_DEV float sigmoidf_(float a) { return __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }

// ------------------------------------------------------------------ MXFP8 (OCP MX v1.0)
// E8M0 scale byte of a 32-element block from its largest magnitude:
// s = clamp(floor(log2 amax) - 8 + 127, 0, 254); 0 for an all-zero block.
MOK_DEV int mx_scale_byte(float amax) {
  uint32_t b = __float_as_uint(amax);
  if (amax == 0.0f) return 0;
  int field = (int)((b >> 23) & 0xFF);
  int e;
  if (field > 0) e = field - 127;
  else e = (31 - __clz((int)(b & 0x7FFFFF))) - 149;   // subnormal amax
  int s = e - 8 + 127;
  return s < 0 ? 0 : (s > 254 ? 254 : s);
}

// E4M3 code of q (|q| < 2^9 after block scaling), round to nearest even,
// saturating to +-448; the sign bit is copied from q (so -0 -> 0x80). The
// kernels encode with e4m3_pack4 (hardware conversion, the same codes); this
// integer form states the rounding and saturation rule it was checked against.
// Branch-free: for |q| >= 2^-6 the float's 23-bit mantissa is rounded to 3
// bits in the integer domain (adding 2^19 - 1 plus the lowest kept bit
// carries exactly when the dropped part is above half, or half with an odd
// kept part; a carry out of the mantissa bumps the exponent), the exponent
// is rebiased from 127 to 7, and codes above 0x7E (448) saturate; below 2^-6
// the value is a multiple of 2^-9, rounded with rint (ties to even, 8 ->
// 0x08 = 2^-6).
MOK_DEV uint32_t e4m3_encode(float q) {
  const uint32_t b = __float_as_uint(q);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t ab = b & 0x7FFFFFFFu;
  const uint32_t r = ab + 0x7FFFFu + ((ab >> 20) & 1u);
  const int32_t nc = min((int32_t)(r >> 20) - (120 << 3), 0x7E);
  const uint32_t sc = (uint32_t)__builtin_rintf(__uint_as_float(ab) * 512.0f);
  return (ab < 0x3C800000u ? sc : (uint32_t)nc) | sign;   // 0x3C800000 = 2^-6
}

// Four E4M3 codes, a in the lowest byte: the same codes as e4m3_encode for
// every finite input, from the hardware conversion (v_cvt_pk_fp8_f32: OCP
// E4M3, round to nearest even, sign kept on zero), which does not saturate
// (out of range it gives NaN), after clamping to +-448. Measured equal to
// e4m3_encode on gfx950 over every code, every midpoint between adjacent
// codes and its two float neighbours (at block scales 2^-7 .. 2^10), values
// far out of range, subnormal inputs, signed zeros and 200k random values.
// NaN inputs are not supported (the hardware keeps them NaN).
MOK_DEV uint32_t e4m3_pack4(float a, float b, float c, float d) {
  const auto sat = [](float v) { return __builtin_fminf(__builtin_fmaxf(v, -448.0f), 448.0f); };
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(sat(a), sat(b), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat(c), sat(d), lo, true);
}

// 2^(127 - s) as a float multiplier (exact; s in 0..254).
MOK_DEV float mx_inv_scale(int s) { return ldexpf(1.0f, 127 - s); }

// ------------------------------------------------------------------ stores
// Global stores with the nontemporal hint (global_store ... nt): GEMM outputs
// are not read again while they would still sit in L2, and with the hint they
// do not evict the operand lines other workgroups are still reading (measured
// on a grouped GEMM with K = 512: main loop 20.6 -> 17.7 us per tile).
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
MOK_DEV void store_nt(void* p, const uint4& v) {
  __builtin_nontemporal_store((u32x4_t){v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(p));
}

// ------------------------------------------------------------------ misc
MOK_DEV int lane_id() { return (int)(threadIdx.x & 63); }

template <typename T>
MOK_DEV T ceil_div(T a, T b) { return (a + b - 1) / b; }
