// Fused K writer and index-Q pack for gfx950.
//
// "[AMD] Enable FP4 indexer for Deepseek V4", Modifications / FP4 kernel
// adapters: the K path is RMSNorm -> RoPE -> Hadamard -> FP4 quantisation ->
// paged cache write into separate payload and UE8M0-scale buffers (Motivation:
// payload [num_pages, 1, 4, 64, 16], scale [num_pages, 1, 4, 64]).
// "dsv4.1-amd: KV cache layouts, FP4 indexer, ..." Summary: index-Q and the
// head weights are packed in one launch.
//
// Four lanes per 128-vector (encode_quad.hpp): a quarter of the serial
// instruction chain per lane, and each load instruction of a wave covers 16
// rows x 64 contiguous bytes.  (One lane per vector, with the whole vector in
// one lane's registers, measured 1.5-2x slower at every batch size: its loads
// touch 64 rows per instruction.)
#include "encode_quad.hpp"
#include "launch.hpp"

namespace fp4idx {

__global__ __launch_bounds__(256) void write_k_quad_kernel(const uint16_t* __restrict__ k, int64_t n_tokens,
                                                           int64_t k_row_stride, const int32_t* __restrict__ pos,
                                                           const int32_t* __restrict__ slot,
                                                           const uint16_t* __restrict__ norm_w, float eps,
                                                           const uint16_t* __restrict__ cos_sin,
                                                           uint8_t* __restrict__ payload,
                                                           uint8_t* __restrict__ scale) {
  __shared__ float g[kDim];
  if (threadIdx.x < kDim) g[threadIdx.x] = __uint_as_float((uint32_t)norm_w[threadIdx.x] << 16);
  __syncthreads();
  const int64_t gl = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t i = gl >> 2;  // token; its four lanes leave or stay together
  const int q = (int)(gl & 3);
  if (i >= n_tokens) return;
  const int32_t s = slot[i];
  if (s < 0) return;
  const int32_t p = pos[i];

  QuadVec v;
  quad_load(k + i * k_row_stride, q, v);
  const float r = quad_rms_factor(v, eps);
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float xr = v.x[c][e] * r;
      v.x[c][e] = xr * g[32 * c + 8 * q + e];
    }
  quad_rope(v, cos_sin + (int64_t)p * kRope, q);
  quad_hadamard(v, q);
  uint32_t word[4], sc;
  quad_quant(v, word, sc);

  const int64_t page = s >> 6;
  const int tok = s & 63;
  uint8_t* pp = payload + page * kPayloadPage + tok * 16 + 4 * q;
#pragma unroll
  for (int c = 0; c < 4; ++c) *reinterpret_cast<uint32_t*>(pp + c * 1024) = word[c];
  scale[page * kScalePage + q * 64 + tok] = (uint8_t)(sc >> (8 * q));
}

__global__ __launch_bounds__(256) void pack_q_quad_kernel(const uint16_t* __restrict__ q_in, int64_t n_rows,
                                                          int n_heads, int64_t q_row_stride,
                                                          const int32_t* __restrict__ pos,
                                                          const uint16_t* __restrict__ cos_sin,
                                                          const float* __restrict__ w_in, float w_scale,
                                                          uint8_t* __restrict__ q_fp4, uint8_t* __restrict__ q_scale,
                                                          float* __restrict__ w_out) {
  const int64_t gl = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t idx = gl >> 2;  // (row, head)
  const int q = (int)(gl & 3);
  if (idx >= n_rows * n_heads) return;
  const int64_t row = idx / n_heads;
  const int h = (int)(idx - row * n_heads);
  const int32_t p = pos[row];

  QuadVec v;
  quad_load(q_in + row * q_row_stride + (int64_t)h * kDim, q, v);
  quad_rope(v, cos_sin + (int64_t)p * kRope, q);
  quad_hadamard(v, q);
  uint32_t word[4], sc;
  quad_quant(v, word, sc);

  uint8_t* out = q_fp4 + idx * 64 + 4 * q;
#pragma unroll
  for (int c = 0; c < 4; ++c) *reinterpret_cast<uint32_t*>(out + 16 * c) = word[c];
  q_scale[idx * 4 + q] = (uint8_t)(sc >> (8 * q));
  if (q == 0) w_out[idx] = w_in[idx] * w_scale;
}

hipError_t launch_write_k(const uint16_t* k, int64_t n_tokens, int64_t k_row_stride, const int32_t* pos,
                          const int32_t* slot, const uint16_t* norm_w, float eps, const uint16_t* cos_sin,
                          uint8_t* payload, uint8_t* scale, hipStream_t stream) {
  if (n_tokens == 0) return hipSuccess;
  const int64_t blocks = (4 * n_tokens + 255) / 256;
  return launch(write_k_quad_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, k, n_tokens, k_row_stride, pos, slot,
                norm_w, eps, cos_sin, payload, scale);
}

hipError_t launch_pack_q(const uint16_t* q, int64_t n_rows, int n_heads, int64_t q_row_stride, const int32_t* pos,
                         const uint16_t* cos_sin, const float* w_in, float w_scale, uint8_t* q_fp4,
                         uint8_t* q_scale, float* w_out, hipStream_t stream) {
  const int64_t n = n_rows * n_heads;
  if (n == 0) return hipSuccess;
  const int64_t blocks = (4 * n + 255) / 256;
  return launch(pack_q_quad_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, q, n_rows, n_heads, q_row_stride, pos,
                cos_sin, w_in, w_scale, q_fp4, q_scale, w_out);
}

}  // namespace fp4idx
