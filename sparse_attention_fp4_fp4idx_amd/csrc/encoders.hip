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

// Arguments of the two encoders (kernel arguments by value).
struct WriteKArgs {
  const uint16_t* k;
  int64_t n_tokens;
  int64_t k_row_stride;
  const int32_t* pos;
  const int32_t* slot;
  const uint16_t* norm_w;
  float eps;
  const uint16_t* cos_sin;
  uint8_t* payload;
  uint8_t* scale;
};

struct PackQArgs {
  const uint16_t* q;
  int64_t n_rows;
  int n_heads;
  int64_t q_row_stride;
  const int32_t* pos;
  const uint16_t* cos_sin;
  const float* w_in;
  float w_scale;
  uint8_t* q_fp4;
  uint8_t* q_scale;
  float* w_out;
};

// Block b of the K writer: tokens 64 b .. 64 b + 63, four lanes each.
__device__ __forceinline__ void write_k_block(const WriteKArgs& a, int64_t b) {
  __shared__ float g[kDim];
  if (threadIdx.x < kDim) g[threadIdx.x] = __uint_as_float((uint32_t)a.norm_w[threadIdx.x] << 16);
  __syncthreads();
  const int64_t gl = b * 256 + threadIdx.x;
  const int64_t i = gl >> 2;  // token; its four lanes leave or stay together
  const int q = (int)(gl & 3);
  if (i >= a.n_tokens) return;
  const int32_t s = a.slot[i];
  if (s < 0) return;
  const int32_t p = a.pos[i];

  QuadVec v;
  quad_load(a.k + i * a.k_row_stride, q, v);
  const float r = quad_rms_factor(v, a.eps);
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float xr = v.x[c][e] * r;
      v.x[c][e] = xr * g[32 * c + 8 * q + e];
    }
  quad_rope(v, a.cos_sin + (int64_t)p * kRope, q);
  quad_hadamard(v, q);
  uint32_t word[4], sc;
  quad_quant(v, word, sc);

  const int64_t page = s >> 6;
  const int tok = s & 63;
  uint8_t* pp = a.payload + page * kPayloadPage + tok * 16 + 4 * q;
#pragma unroll
  for (int c = 0; c < 4; ++c) *reinterpret_cast<uint32_t*>(pp + c * 1024) = word[c];
  a.scale[page * kScalePage + q * 64 + tok] = (uint8_t)(sc >> (8 * q));
}

// Block b of the Q pack: (row, head) vectors 64 b .. 64 b + 63, four lanes each.
__device__ __forceinline__ void pack_q_block(const PackQArgs& a, int64_t b) {
  const int64_t gl = b * 256 + threadIdx.x;
  const int64_t idx = gl >> 2;  // (row, head)
  const int q = (int)(gl & 3);
  if (idx >= a.n_rows * a.n_heads) return;
  const int64_t row = idx / a.n_heads;
  const int h = (int)(idx - row * a.n_heads);
  const int32_t p = a.pos[row];

  QuadVec v;
  quad_load(a.q + row * a.q_row_stride + (int64_t)h * kDim, q, v);
  quad_rope(v, a.cos_sin + (int64_t)p * kRope, q);
  quad_hadamard(v, q);
  uint32_t word[4], sc;
  quad_quant(v, word, sc);

  uint8_t* out = a.q_fp4 + idx * 64 + 4 * q;
#pragma unroll
  for (int c = 0; c < 4; ++c) *reinterpret_cast<uint32_t*>(out + 16 * c) = word[c];
  a.q_scale[idx * 4 + q] = (uint8_t)(sc >> (8 * q));
  if (q == 0) a.w_out[idx] = a.w_in[idx] * a.w_scale;
}

__global__ __launch_bounds__(256) void write_k_quad_kernel(WriteKArgs a) { write_k_block(a, blockIdx.x); }

__global__ __launch_bounds__(256) void pack_q_quad_kernel(PackQArgs a) { pack_q_block(a, blockIdx.x); }

// One launch for a decode step's two independent encodes: the first
// k_blocks work-groups write K, the rest pack Q (the branch is uniform per
// work-group).
__global__ __launch_bounds__(256) void write_k_pack_q_kernel(WriteKArgs ka, PackQArgs qa, int64_t k_blocks) {
  const int64_t b = blockIdx.x;
  if (b < k_blocks)
    write_k_block(ka, b);
  else
    pack_q_block(qa, b - k_blocks);
}

static inline int64_t quad_blocks(int64_t n) { return (4 * n + 255) / 256; }

hipError_t launch_write_k(const uint16_t* k, int64_t n_tokens, int64_t k_row_stride, const int32_t* pos,
                          const int32_t* slot, const uint16_t* norm_w, float eps, const uint16_t* cos_sin,
                          uint8_t* payload, uint8_t* scale, hipStream_t stream) {
  if (n_tokens == 0) return hipSuccess;
  const WriteKArgs a{k, n_tokens, k_row_stride, pos, slot, norm_w, eps, cos_sin, payload, scale};
  return launch(write_k_quad_kernel, dim3((unsigned)quad_blocks(n_tokens)), dim3(256), 0, stream, a);
}

hipError_t launch_pack_q(const uint16_t* q, int64_t n_rows, int n_heads, int64_t q_row_stride, const int32_t* pos,
                         const uint16_t* cos_sin, const float* w_in, float w_scale, uint8_t* q_fp4,
                         uint8_t* q_scale, float* w_out, hipStream_t stream) {
  const int64_t n = n_rows * n_heads;
  if (n == 0) return hipSuccess;
  const PackQArgs a{q, n_rows, n_heads, q_row_stride, pos, cos_sin, w_in, w_scale, q_fp4, q_scale, w_out};
  return launch(pack_q_quad_kernel, dim3((unsigned)quad_blocks(n)), dim3(256), 0, stream, a);
}

hipError_t launch_write_k_pack_q(const uint16_t* k, int64_t n_tokens, int64_t k_row_stride, const int32_t* pos_k,
                                 const int32_t* slot, const uint16_t* norm_w, float eps, const uint16_t* cos_sin,
                                 uint8_t* payload, uint8_t* scale, const uint16_t* q, int64_t n_rows, int n_heads,
                                 int64_t q_row_stride, const int32_t* pos_q, const float* w_in, float w_scale,
                                 uint8_t* q_fp4, uint8_t* q_scale, float* w_out, hipStream_t stream) {
  const int64_t kb = quad_blocks(n_tokens), qb = quad_blocks(n_rows * n_heads);
  if (kb + qb == 0) return hipSuccess;
  if (kb + qb > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  const WriteKArgs ka{k, n_tokens, k_row_stride, pos_k, slot, norm_w, eps, cos_sin, payload, scale};
  const PackQArgs qa{q, n_rows, n_heads, q_row_stride, pos_q, cos_sin, w_in, w_scale, q_fp4, q_scale, w_out};
  return launch(write_k_pack_q_kernel, dim3((unsigned)(kb + qb)), dim3(256), 0, stream, ka, qa, kb);
}

}  // namespace fp4idx
