// Microbenchmarks of the peaks the roofline fractions are taken against
// (measurement support, not part of the method): FP4 block-scaled MFMA
// throughput, fp32 VALU FMA throughput and streaming HBM read bandwidth on the
// current device, so that a kernel's fraction can be stated against measured
// as well as vendor peaks.
#include "launch.hpp"

namespace fp4idx {

typedef int v8i_p __attribute__((ext_vector_type(8)));
typedef float v4f_p __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_p __attribute__((ext_vector_type(4)));

// Every wave runs `iters` rounds of four independent accumulator chains of
// V_MFMA_SCALE_F32_16X16X128_F8F6F4 with e2m1 operands (the logits kernel's
// instruction), i.e. 4 * iters MFMAs of 65,536 flop.  Operands depend on the
// lane so nothing folds; the sums reach memory only for an impossible value.
__global__ __launch_bounds__(256) void peak_mfma_fp4_kernel(int iters, float* sink) {
  const int l = threadIdx.x;
  const v8i_p a = {l, l ^ 0x5A5A, l * 3, l + 7, 0, 0, 0, 0};
  const v8i_p b = {l * 5, l ^ 0x3C3C, l + 11, l * 9, 0, 0, 0, 0};
  v4f_p c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0;
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c0, 4, 4, 0, 127, 0, 127);
    c1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c1, 4, 4, 0, 127, 0, 127);
    c2 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c2, 4, 4, 0, 127, 0, 127);
    c3 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c3, 4, 4, 0, 127, 0, 127);
  }
  const float s = c0[0] + c1[1] + c2[2] + c3[3];
  if (s == -1.2345e-37f) sink[0] = s;
}

// Every lane runs `iters` rounds of 16 independent fp32 FMA chains
// (acc = acc * a + 0.5 with a uniform `a`: one vector register read per
// instruction, so no register-bank conflicts), i.e. 16 * iters FMA lane-ops.
__global__ __launch_bounds__(256) void peak_valu_fp32_kernel(int iters, float a, float* sink) {
  float acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = (float)(threadIdx.x + j);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = __builtin_fmaf(acc[j], a, 0.5f);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += acc[j];
  if (s == -1.2345e-37f) sink[0] = s;
}

// MFMA / VALU co-execution: per round a wave issues 8 block-scaled FP4 MFMAs
// (8 accumulator chains, the peak kernel's form) and/or 32 fp32 FMAs (8
// chains of the VALU peak kernel's form), MODE 0 the MFMAs only, 1 the FMAs
// only, 2 both, interleaved one MFMA : four FMAs.  Every chain carries across
// rounds, so nothing can be hoisted.  If the matrix and vector pipes of a SIMD
// overlapped, mode 2 would take about the longer of modes 0 and 1; if they
// take turns, about their sum.
template <int MODE>
__global__ __launch_bounds__(256) void peak_mix_kernel(int iters, float a, float* sink) {
  const int l = threadIdx.x;
  const v8i_p av = {l, l ^ 0x5A5A, l * 3, l + 7, 0, 0, 0, 0};
  const v8i_p bv = {l * 5, l ^ 0x3C3C, l + 11, l * 9, 0, 0, 0, 0};
  v4f_p c[8];
  float x[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    c[m] = v4f_p{0.f, 0.f, 0.f, 0.f};
    x[m] = (float)(l + m);
  }
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      if constexpr (MODE != 1) c[m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c[m], 4, 4, 0, 127, 0, 127);
      if constexpr (MODE != 0) {
#pragma unroll
        for (int u = 0; u < 4; ++u) x[(4 * m + u) & 7] = __builtin_fmaf(x[(4 * m + u) & 7], a, 0.5f);
      }
      if constexpr (MODE == 2) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int m = 0; m < 8; ++m) s += c[m][m & 3] + x[m];
  if (s == -1.2345e-37f) sink[0] = s;
}

// Grid-stride read of `n16` 16-byte units (non-temporal loads, eight in
// flight per lane), folded into one word per thread that reaches memory only
// for an impossible value.
__global__ __launch_bounds__(256) void peak_read_kernel(const u32x4_p* __restrict__ src, int64_t n16,
                                                        uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4_p v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4_p v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

constexpr int kPeakMfmaBlocks = 1024;  // x 4 waves: four waves on each of the 1,024 SIMDs
constexpr int kPeakReadBlocks = 2048;

hipError_t launch_peak_mfma_fp4(int32_t iters, float* sink, hipStream_t stream) {
  return launch(peak_mfma_fp4_kernel, dim3(kPeakMfmaBlocks), dim3(256), 0, stream, iters, sink);
}

hipError_t launch_peak_valu_fp32(int32_t iters, float* sink, hipStream_t stream) {
  return launch(peak_valu_fp32_kernel, dim3(kPeakMfmaBlocks), dim3(256), 0, stream, iters, 0.999f, sink);
}

hipError_t launch_peak_mix(int32_t mode, int32_t iters, float* sink, hipStream_t stream) {
  switch (mode) {
    case 0: return launch(peak_mix_kernel<0>, dim3(kPeakMfmaBlocks), dim3(256), 0, stream, iters, 0.999f, sink);
    case 1: return launch(peak_mix_kernel<1>, dim3(kPeakMfmaBlocks), dim3(256), 0, stream, iters, 0.999f, sink);
    default: return launch(peak_mix_kernel<2>, dim3(kPeakMfmaBlocks), dim3(256), 0, stream, iters, 0.999f, sink);
  }
}

hipError_t launch_peak_read(const uint8_t* buf, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  return launch(peak_read_kernel, dim3(kPeakReadBlocks), dim3(256), 0, stream,
                reinterpret_cast<const u32x4_p*>(buf), bytes / 16, sink);
}

}  // namespace fp4idx
