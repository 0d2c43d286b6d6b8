// Device helpers of the K writer and Q pack on gfx950 (FP4 and FP8 caches).
//
// A quad of lanes q = 0..3 owns one 128-vector; lane q holds the 32 elements
//   i = 32*c + 8*q + e,   c = 0..3 (register chunk), e = 0..7.
// Index bits 0-2 (e) and 5-6 (c) are in-lane, bits 3-4 (q) are across the
// quad.  With this placement:
//  * the 16-byte loads are contiguous (chunk c of lane q = bytes 64c + 16q),
//    so a wave's load instruction covers 16 rows x 64 contiguous bytes,
//  * RoPE pairs (j, j+32) are chunks 0 and 1 of the same lane,
//  * Hadamard stages h = 1, 2, 4, 32, 64 are in-lane and h = 8, 16 are one
//    quad-permute DPP exchange each,
//  * a 32-block is chunk c across the quad (amax = 2 DPP max steps) and
//    lane q's 8 codes are bytes 4q..4q+3 of that block's 16 bytes,
//  * the RMSNorm balanced tree is: 8-element subtrees in-lane, then the
//    quad levels (xor 1, xor 2), then the chunk levels in-lane.
// Every floating-point operation is the one of the canonical encoder order
// stated in include/fp4idx.h (one vector evaluated in program order), on the
// same operands and in the same order; additions only ever change operand
// order where IEEE addition is commutative, and u - v is formed as
// v' + (-u') only where that is the identical IEEE operation, so the bytes
// are exactly the canonical ones.  Build flags keep it exact:
// -ffp-contract=off (no FMA formation), default correctly rounded fp32
// sqrt/div, fp32 denormals kept.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4idx {

constexpr int kDim = 128;
constexpr int kRope = 64;
constexpr int kPageTokens = 64;
constexpr int kPayloadPage = 4096;  // [1, 4, 64, 16]
constexpr int kScalePage = 256;     // [1, 4, 64]
constexpr int kFp8Page = 8448;      // [64][128] e4m3 codes, then [64] fp32 scales
constexpr int kFp8ScaleOffset = 8192;

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


// quad_perm DPP controls: xor 1 = [1,0,3,2], xor 2 = [2,3,0,1]
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

struct QuadVec {
  float x[4][8];  // [c][e]
};

// Load the lane's 32 bf16 elements of a 128-row.
__device__ __forceinline__ void quad_load(const uint16_t* __restrict__ row, int q, QuadVec& v) {
  const uint8_t* p = reinterpret_cast<const uint8_t*>(row) + 16 * q;
#pragma unroll
  for (int c = 0; c < 4; ++c) widen8(ld_stream16(p + 64 * c), v.x[c]);
}

// Butterfly across the quad at index bit 3 (CTRL = xor 1) or bit 4 (xor 2):
// the lower-index lane forms u + v, the upper one u - v = (partner) + (-own).
template <int CTRL>
__device__ __forceinline__ void quad_stage(QuadVec& v, bool upper) {
  const uint32_t flip = upper ? 0x80000000u : 0u;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float partner = dpp_f<CTRL>(v.x[c][e]);
      const float own = __uint_as_float(__float_as_uint(v.x[c][e]) ^ flip);
      v.x[c][e] = partner + own;
    }
  }
}

__device__ __forceinline__ void quad_rope(QuadVec& v, const uint16_t* __restrict__ cs_row, int q) {
  const uint8_t* p = reinterpret_cast<const uint8_t*>(cs_row);
  float cs[8], sn[8];
  widen8(*reinterpret_cast<const uint4*>(p + 16 * q), cs);
  widen8(*reinterpret_cast<const uint4*>(p + 64 + 16 * q), sn);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float c = cs[e], s = sn[e];
    const float a = v.x[0][e], b = v.x[1][e];
    const float ac = a * c, bs = b * s, bc = b * c, as = a * s;
    v.x[0][e] = ac - bs;
    v.x[1][e] = bc + as;
  }
}

__device__ __forceinline__ void quad_hadamard(QuadVec& v, int q) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (e & h) continue;
        const float u = v.x[c][e], w = v.x[c][e + h];
        v.x[c][e] = u + w;
        v.x[c][e + h] = u - w;
      }
    }
  }
  quad_stage<kDppXor1>(v, (q & 1) != 0);
  quad_stage<kDppXor2>(v, (q & 2) != 0);
#pragma unroll
  for (int hc = 1; hc < 4; hc <<= 1) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (c & hc) continue;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float u = v.x[c][e], w = v.x[c + hc][e];
        v.x[c][e] = u + w;
        v.x[c + hc][e] = u - w;
      }
    }
  }
  const float C = __uint_as_float(0x3DB504F3u);
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) v.x[c][e] = v.x[c][e] * C;
}

// RMSNorm factor r = 1 / sqrt(S/128 + eps), S by the balanced tree.
__device__ __forceinline__ float quad_rms_factor(const QuadVec& v, float eps) {
  float t[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float s[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = v.x[c][e] * v.x[c][e];
    const float a0 = s[0] + s[1], a1 = s[2] + s[3], a2 = s[4] + s[5], a3 = s[6] + s[7];
    const float b0 = a0 + a1, b1 = a2 + a3;
    t[c] = b0 + b1;
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) t[c] = t[c] + dpp_f<kDppXor1>(t[c]);
#pragma unroll
  for (int c = 0; c < 4; ++c) t[c] = t[c] + dpp_f<kDppXor2>(t[c]);
  const float lo = t[0] + t[1], hi = t[2] + t[3];
  const float S = lo + hi;
  const float ms = S * 0.0078125f;
  return 1.0f / sqrtf(ms + eps);
}

// MXFP4 encode: lane q gets the dword holding its 8 codes of every block
// (word[c]) and the 4 scale bytes of the vector (scales, byte j = block j).
__device__ __forceinline__ void quad_quant(const QuadVec& v, uint32_t (&word)[4], uint32_t& scales) {
  scales = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v.x[c][e]));
    amax = fmaxf(amax, dpp_f<kDppXor1>(amax));
    amax = fmaxf(amax, dpp_f<kDppXor2>(amax));
    const uint32_t bits = __float_as_uint(amax);
    int e = (int)(bits >> 23) - 129 + ((bits & 0x7FFFFFu) > 0x400000u ? 1 : 0);
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
    scales |= (uint32_t)(e + 127) << (8 * c);
    const float sc = (e >= -126) ? __uint_as_float((uint32_t)(e + 127) << 23) : __uint_as_float(0x00400000u);
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v.x[c][0], v.x[c][1], sc, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v.x[c][2], v.x[c][3], sc, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v.x[c][4], v.x[c][5], sc, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v.x[c][6], v.x[c][7], sc, 3);
    word[c] = w;
  }
}

// FP8 encode of the whole vector with one power-of-two scale 2^e, e the
// smallest integer with 448 * 2^e >= amax, clamped to [-127, 127] (448 is the
// largest finite OCP E4M3 value): amax = m 2^E with m in [1, 2) gives
// e = E - 8, plus one when m > 1.75; a zero or subnormal amax gives -127.
// Each code is the e4m3 value nearest to z / 2^e, ties to even, sign kept
// (the hardware convert divides by the scale exactly and rounds to nearest
// even).  The scale handed to the convert is kept a normal number: for
// e < -64 the inputs are first multiplied by 2^64 (exact) and the scale by
// the same.  codes[c] = the lane's 8 codes of chunk c, i.e. bytes
// 32c + 8q .. +7 of the vector; scale = 2^e as stored (2^-127 subnormal).
__device__ __forceinline__ void quad_quant_fp8(const QuadVec& v, uint2 (&codes)[4], float& scale) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v.x[c][e]));
  amax = fmaxf(amax, dpp_f<kDppXor1>(amax));
  amax = fmaxf(amax, dpp_f<kDppXor2>(amax));
  const uint32_t bits = __float_as_uint(amax);
  int e = (int)(bits >> 23) - 135 + ((bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  e = e < -127 ? -127 : (e > 127 ? 127 : e);
  scale = e >= -126 ? __uint_as_float((uint32_t)(e + 127) << 23) : __uint_as_float(0x00400000u);
  const bool tiny = e < -64;
  const float pre = tiny ? __uint_as_float(0x5F800000u) : 1.0f;  // 2^64
  const float sc = __uint_as_float((uint32_t)((tiny ? e + 64 : e) + 127) << 23);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    v2s lo = {0, 0}, hi = {0, 0};
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, v.x[c][0] * pre, v.x[c][1] * pre, sc, false);
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, v.x[c][2] * pre, v.x[c][3] * pre, sc, true);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, v.x[c][4] * pre, v.x[c][5] * pre, sc, false);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, v.x[c][6] * pre, v.x[c][7] * pre, sc, true);
    codes[c] = make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
  }
}

}  // namespace fp4idx
