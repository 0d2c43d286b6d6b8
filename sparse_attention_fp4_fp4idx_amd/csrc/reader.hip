// Split-pool reader for gfx950: pool tokens back to fp32 values.
//
// "dsv4.1-amd: KV cache layouts, FP4 indexer, ..." Summary and "[AMD] Enable
// FP4 indexer for Deepseek V4" Device memory: the FP4 pool comes with a split
// writer and reader.  Token s of the pool is page s/64, in-page index s%64;
// its block j is 16 payload bytes at [page][j][token] (element 32j + 2b in the
// low nibble of byte b, 32j + 2b + 1 in the high nibble) scaled by
// 2^(scale[page][j][token] - 127).
//
// Sixteen lanes per token: lane u = 4j + c holds bytes 4c .. 4c + 3 of block
// j, i.e. elements 32j + 8c .. + 7, and writes them as two 16-byte stores.
// Each e2m1 code is converted exactly (scale 1.0) and the block exponent is
// applied with ldexp, which is exact for every result fp32 can represent
// (products below 2^-126 are exact subnormals) and gives +-inf above.
#include "launch.hpp"

namespace fp4idx {

typedef float v2f __attribute__((ext_vector_type(2)));

__global__ __launch_bounds__(256) void read_k_kernel(const uint8_t* __restrict__ payload,
                                                     const uint8_t* __restrict__ scale, int64_t num_pages,
                                                     const int32_t* __restrict__ slot, int64_t n_tokens,
                                                     float* __restrict__ out, int64_t out_stride) {
  const int64_t gl = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t i = gl >> 4;
  if (i >= n_tokens) return;
  const int u = (int)(gl & 15);
  const int j = u >> 2, c = u & 3;
  const int64_t s = slot[i];
  float4 lo = make_float4(0.f, 0.f, 0.f, 0.f), hi = lo;
  if (s >= 0 && s < num_pages * 64) {  // a slot outside the pool (padding) reads as zeros
    const int64_t page = s >> 6;
    const int t = (int)(s & 63);
    const uint32_t w = *reinterpret_cast<const uint32_t*>(payload + page * 4096 + j * 1024 + t * 16 + 4 * c);
    const int e = (int)scale[page * 256 + j * 64 + t] - 127;
    const v2f p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const v2f p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const v2f p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const v2f p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    lo = make_float4(__builtin_ldexpf(p0.x, e), __builtin_ldexpf(p0.y, e), __builtin_ldexpf(p1.x, e),
                     __builtin_ldexpf(p1.y, e));
    hi = make_float4(__builtin_ldexpf(p2.x, e), __builtin_ldexpf(p2.y, e), __builtin_ldexpf(p3.x, e),
                     __builtin_ldexpf(p3.y, e));
  }
  float4* o = reinterpret_cast<float4*>(out + i * out_stride + 32 * j + 8 * c);
  o[0] = lo;
  o[1] = hi;
}

hipError_t launch_read_k(const uint8_t* payload, const uint8_t* scale, int64_t num_pages, const int32_t* slot,
                         int64_t n_tokens, float* out, int64_t out_stride, hipStream_t stream) {
  if (n_tokens == 0) return hipSuccess;
  const int64_t blocks = (16 * n_tokens + 255) / 256;
  return launch(read_k_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, payload, scale, num_pages, slot,
                n_tokens, out, out_stride);
}

}  // namespace fp4idx
