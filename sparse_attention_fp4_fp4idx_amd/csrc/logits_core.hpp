// Device pieces of the paged indexer logits on gfx950 (FP4 and FP8 caches),
// shared by the logits kernel and the fused logits + top-k kernel: the cache
// format types, the MFMA operands, the ReLU / head-weight epilogue and the
// lane reduction that turns a page's four 16-token tiles into its 64 logits
// in lane order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace fp4idx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte page load: non-temporal (NT) where each page is read once, plain
// where other work-groups re-read it soon and it should stay in L2.
template <bool NT>
__device__ __forceinline__ uint4 ld_page16(const void* p) {
  u32x4 v;
  if constexpr (NT)
    v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  else
    v = *reinterpret_cast<const u32x4*>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
typedef float v4f __attribute__((ext_vector_type(4)));

// ReLU on the bit pattern: every negative float (and -0) is a negative int32,
// so max(bits, 0) gives +0 for them and leaves non-negative values unchanged.
// One integer max instead of the quieting and comparing pair fmaxf needs.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Sum p[j] over the four 16-lane groups; afterwards lane l holds slot
// (l/16)'s total.  permlane32_swap(a, b): a <- [a.lo32, b.lo32], b <- [a.hi32, b.hi32];
// permlane16_swap(a, b): swaps rows 1 and 3 of a with rows 0 and 2 of b.
__device__ __forceinline__ float reduce4(float p0, float p1, float p2, float p3) {
  auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p2), false, false);
  auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p1), __float_as_uint(p3), false, false);
  const float a = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);
  const float b = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);
  auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// FP4 split pools: payload [page][block][token][16 B], scale [page][block][token].
// B lane l = (token l%16, block l/16): exactly the 16-byte payload chunk at
// [page][block][token] and its UE8M0 byte; A lane l = (head l%16, block l/16).
struct Fp4Split {
  // Launch shapes (64 heads or fewer for the wave counts): rows per wave
  // at most (kRowsCapWide past 64 heads), and per rows-per-wave class the
  // resident waves per SIMD asked of the compiler, the pages per wave and
  // the pages in flight.
  static constexpr int kRowsCap = 4, kRowsCapWide = 4;
  static constexpr int kWaves1 = 4, kPpw1 = 4, kD1 = 4;  // one row per wave (decode)
  static constexpr int kWaves2 = 1, kPpw2 = 4, kD2 = 4;  // two rows
  static constexpr int kPpwMany = 8, kDMany = 4;         // three or four rows
  struct Page {  // 4 tiles of 16 tokens
    uint4 b[4];
    uint32_t s[4];
  };
  typedef uint4 QOp;
  static __device__ __forceinline__ uint32_t lane_pay(int li, int lg) { return (uint32_t)(lg * 1024 + li * 16); }
  static __device__ __forceinline__ uint32_t lane_sc(int li, int lg) { return (uint32_t)(lg * 64 + li); }
  template <bool NT>
  static __device__ __forceinline__ void load_page(Page& pr, const uint8_t* __restrict__ payload,
                                                   const uint8_t* __restrict__ scale, int64_t pid, uint32_t lp,
                                                   uint32_t ls) {
    const uint8_t* pp = payload + pid * 4096 + lp;
    const uint8_t* sp = scale + pid * 256 + ls;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      pr.b[t] = ld_page16<NT>(pp + t * 256);
      pr.s[t] = sp[t * 16];
    }
  }
  static __device__ __forceinline__ QOp load_q(const uint8_t* __restrict__ q, int64_t hrow, int lg) {
    return *reinterpret_cast<const uint4*>(q + hrow * 64 + lg * 16);
  }
  static __device__ __forceinline__ uint32_t q_scale_byte(const uint8_t* __restrict__ qs, int64_t hrow, int lg) {
    return qs[hrow * 4 + lg];
  }
  template <int OPA>
  static __device__ __forceinline__ v4f mfma(const QOp& a, const Page& p, int t, uint32_t sa) {
    const v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    const v8i bv = {(int)p.b[t].x, (int)p.b[t].y, (int)p.b[t].z, (int)p.b[t].w, 0, 0, 0, 0};
    const v4f z = {0.f, 0.f, 0.f, 0.f};
    // cbsz = blgp = 4: both operands FP4 (e2m1); op_sel picks the scale byte.
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, z, 4, 4, OPA, (int)sa, 0, (int)p.s[t]);
  }
};

// An FP4 page staged in LDS by the shared-page logits kernel: the payload in
// pool order, the scale bytes of a lane's four tiles in one word (byte t =
// tile t, picked by the MFMA's B op_sel).  The MFMA operands are those of
// Fp4Split, so every logit is computed by the same operations.
struct Fp4Lds {
  struct Page {
    uint4 b[4];
    uint32_t s;
  };
  typedef uint4 QOp;
  template <int OPA>
  static __device__ __forceinline__ v4f mfma(const QOp& a, const Page& p, int t, uint32_t sa) {
    const v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    const v8i bv = {(int)p.b[t].x, (int)p.b[t].y, (int)p.b[t].z, (int)p.b[t].w, 0, 0, 0, 0};
    const v4f z = {0.f, 0.f, 0.f, 0.f};
    switch (t) {  // t is a compile-time constant at every call
      case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, z, 4, 4, OPA, (int)sa, 0, (int)p.s);
      case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, z, 4, 4, OPA, (int)sa, 1, (int)p.s);
      case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, z, 4, 4, OPA, (int)sa, 2, (int)p.s);
      default: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, z, 4, 4, OPA, (int)sa, 3, (int)p.s);
    }
  }
};

// FP8 fused pool: page = [64 tokens][128 e4m3 codes] then [64] fp32 scales
// (powers of two), 8448 bytes.  The fp8 operand holds 32 bytes per lane;
// A lane l = (head l%16, bytes 32(l/16)..+31 of the head's codes), B lane
// l = (token l%16, the same bytes of the token): A and B place code i in the
// same K slot, so the dot product is the plain one whatever order the MFMA
// gives the 128 slots.  One scale per token and per (row, head) makes all
// four block scales of an operand row equal: the MFMA scale is the fp32
// scale's exponent field (an E8M0 byte).
struct Fp8Fused {
  // launch shapes as for Fp4Split; 8-register operands and 36-register pages
  // need more registers per row and per page in flight
  static constexpr int kRowsCap = 4, kRowsCapWide = 2;   // 3+ rows past 64 heads spill
  static constexpr int kWaves1 = 2, kPpw1 = 4, kD1 = 4;
  static constexpr int kWaves2 = 1, kPpw2 = 4, kD2 = 4;
  static constexpr int kPpwMany = 8, kDMany = 4;
  // operands are held as native 8-register vectors (a two-member struct read
  // as one vector keeps the compiler from splitting it into registers)
  struct Page {
    v8i b[4];
    uint32_t s[4];
  };
  typedef v8i QOp;
  static __device__ __forceinline__ v8i join(uint4 lo, uint4 hi) {
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
  static __device__ __forceinline__ uint32_t lane_pay(int li, int lg) { return (uint32_t)(li * 128 + lg * 32); }
  static __device__ __forceinline__ uint32_t lane_sc(int li, int) { return (uint32_t)(8192 + li * 4); }
  template <bool NT>
  static __device__ __forceinline__ void load_page(Page& pr, const uint8_t* __restrict__ pool, const uint8_t*,
                                                   int64_t pid, uint32_t lp, uint32_t ls) {
    const uint8_t* pp = pool + pid * 8448;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      pr.b[t] = join(ld_page16<NT>(pp + lp + t * 2048), ld_page16<NT>(pp + lp + t * 2048 + 16));
      pr.s[t] = (*reinterpret_cast<const uint32_t*>(pp + ls + t * 64) >> 23) & 0xFFu;
    }
  }
  static __device__ __forceinline__ QOp load_q(const uint8_t* __restrict__ q, int64_t hrow, int lg) {
    const uint4* p = reinterpret_cast<const uint4*>(q + hrow * 128 + lg * 32);
    return join(p[0], p[1]);
  }
  static __device__ __forceinline__ uint32_t q_scale_byte(const uint8_t* __restrict__ qs, int64_t hrow, int) {
    return (reinterpret_cast<const uint32_t*>(qs)[hrow] >> 23) & 0xFFu;
  }
  template <int OPA>
  static __device__ __forceinline__ v4f mfma(const QOp& a, const Page& p, int t, uint32_t sa) {
    const v4f z = {0.f, 0.f, 0.f, 0.f};
    // cbsz = blgp = 0: both operands FP8 e4m3.
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, p.b[t], z, 0, 0, OPA, (int)sa, 0, (int)p.s[t]);
  }
};

// Calls f(std::integral_constant<int, I>{}) for I = 0 .. N-1: loop indices
// known at compile time, so the register arrays they index (pages, page ids,
// rows) stay in registers whatever the unroller decides.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// The logits of one query row for one page, token `lane` of the page in
// lane `lane`: per 16-token tile NMT MFMAs, then the ReLU / weight epilogue
// in one fixed-order FMA chain, then the lane reduction.
// Every (row, token) is formed by exactly this sequence whichever kernel
// calls it, so the logits do not depend on the launch shape.  ONE_TILE keeps
// a single tile's MFMA results live at a time (register budget for four
// waves per SIMD).
template <typename FMT, int NMT, bool ONE_TILE>
__device__ __forceinline__ float row_page_logits(const typename FMT::QOp (&aq)[NMT],
                                                 const uint32_t (&asc)[(NMT + 3) / 4], const float (&wv)[NMT][4],
                                                 const typename FMT::Page& pg) {
  // the tile index is a compile-time constant (tile<0..3>), so the page's
  // registers are always indexed statically (a runtime index would put the
  // page in scratch memory)
  auto tile = [&](auto tc) __attribute__((always_inline)) {
    constexpr int t = decltype(tc)::value;
    v4f d[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      switch (mt & 3) {
        case 0: d[mt] = FMT::template mfma<0>(aq[mt], pg, t, asc[mt >> 2]); break;
        case 1: d[mt] = FMT::template mfma<1>(aq[mt], pg, t, asc[mt >> 2]); break;
        case 2: d[mt] = FMT::template mfma<2>(aq[mt], pg, t, asc[mt >> 2]); break;
        default: d[mt] = FMT::template mfma<3>(aq[mt], pg, t, asc[mt >> 2]); break;
      }
    }
    // one fixed-order chain over the M-tiles (the four tiles' chains are
    // independent of each other)
    float r = 0.f;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
      for (int e = 0; e < 4; ++e) r = __builtin_fmaf(wv[mt][e], relu(d[mt][e]), r);
    }
    if constexpr (ONE_TILE) __builtin_amdgcn_sched_barrier(0);
    return r;
  };
  const float p0 = tile(std::integral_constant<int, 0>{});
  const float p1 = tile(std::integral_constant<int, 1>{});
  const float p2 = tile(std::integral_constant<int, 2>{});
  const float p3 = tile(std::integral_constant<int, 3>{});
  // lane l now gets tile l/16's total for token l%16: 64 consecutive tokens
  return reduce4(p0, p1, p2, p3);
}

}  // namespace fp4idx
