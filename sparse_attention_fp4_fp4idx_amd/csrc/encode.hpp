// Device helpers for the two FP4 encoders (K writer, Q pack) on gfx950.
//
// One lane owns one 128-element vector in registers, so every step below is
// in-lane and its fp32 operation order is exactly the one stated in
// include/fp4idx.h.  Build flags keep it exact: -ffp-contract=off (no FMA
// formation), default correctly rounded fp32 sqrt/div, fp32 denormals kept.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4idx {

constexpr int kDim = 128;
constexpr int kRope = 64;
constexpr int kPageTokens = 64;
constexpr int kPayloadPage = 4096;  // [1, 4, 64, 16]
constexpr int kScalePage = 256;     // [1, 4, 64]

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (non-temporal: read once, do not keep in cache).
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// 8 bf16 packed in 16 bytes -> 8 fp32 (exact widening).
__device__ __forceinline__ void widen8(uint4 v, float* x) {
  x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
  x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
  x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
  x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}

// 128 bf16 from a 16-byte aligned row.
__device__ __forceinline__ void load_row128(const uint16_t* __restrict__ p, float (&x)[kDim]) {
#pragma unroll
  for (int c = 0; c < kDim / 8; ++c) widen8(ld_stream16(p + 8 * c), x + 8 * c);
}

// RoPE on dims 0..63, rotate-half pairs (j, j+32); cs = 64 bf16 (cos then sin).
// "[AMD] Enable FP4 indexer for Deepseek V4", Modifications: Q and K reuse the
// model's BF16 RoPE cos/sin cache.
__device__ __forceinline__ void rope64(float (&y)[kDim], const uint16_t* __restrict__ cs_row) {
  const uint4* q = reinterpret_cast<const uint4*>(cs_row);
  float cs[kRope];
#pragma unroll
  for (int c = 0; c < kRope / 8; ++c) widen8(q[c], cs + 8 * c);
#pragma unroll
  for (int j = 0; j < kRope / 2; ++j) {
    const float c = cs[j], s = cs[kRope / 2 + j];
    const float a = y[j], b = y[j + kRope / 2];
    const float ac = a * c, bs = b * s, bc = b * c, as = a * s;
    y[j] = ac - bs;
    y[j + kRope / 2] = bc + as;
  }
}

// Normalised Sylvester Hadamard: butterfly stages h = 1, 2, ..., 64, then one
// multiply by fp32(128^-1/2) = 0x3DB504F3.
__device__ __forceinline__ void hadamard128(float (&z)[kDim]) {
#pragma unroll
  for (int h = 1; h < kDim; h <<= 1) {
#pragma unroll
    for (int i = 0; i < kDim; ++i) {
      if (i & h) continue;
      const float u = z[i], v = z[i + h];
      z[i] = u + v;
      z[i + h] = u - v;
    }
  }
  const float C = __uint_as_float(0x3DB504F3u);
#pragma unroll
  for (int i = 0; i < kDim; ++i) z[i] = z[i] * C;
}

// MXFP4 encode of one 128-vector: 4 blocks of 32, each 16 code bytes (element
// 2b in the low nibble of byte b) and one UE8M0 byte.
// Block exponent e = ceil(log2(amax/6)) exactly, from the fp32 bits of amax:
// e = E - 129 + (mantissa > 0x400000), clamped to [-127, 127] (amax = 0 and
// subnormal amax give -127).  The gfx950 packed convert divides by the scale
// 2^e (an exact power of two) and rounds to nearest-even onto the e2m1 grid,
// keeping the sign of zero.
__device__ __forceinline__ void quant128(const float (&z)[kDim], uint4 (&codes)[4], uint32_t& scales) {
  scales = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(z[32 * j + i]));
    const uint32_t bits = __float_as_uint(amax);
    int e = (int)(bits >> 23) - 129 + ((bits & 0x7FFFFFu) > 0x400000u ? 1 : 0);
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
    scales |= (uint32_t)(e + 127) << (8 * j);
    const float sc = (e >= -126) ? __uint_as_float((uint32_t)(e + 127) << 23) : __uint_as_float(0x00400000u);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      const float lo = z[32 * j + 2 * b], hi = z[32 * j + 2 * b + 1];
      switch (b & 3) {
        case 0: w[b >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[b >> 2], lo, hi, sc, 0); break;
        case 1: w[b >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[b >> 2], lo, hi, sc, 1); break;
        case 2: w[b >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[b >> 2], lo, hi, sc, 2); break;
        default: w[b >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[b >> 2], lo, hi, sc, 3); break;
      }
    }
    codes[j] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace fp4idx
