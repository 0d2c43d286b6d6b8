// Fused K writer and index-Q pack for gfx950, into the FP4 cache (split
// payload / scale pools) or the FP8 cache (one fused pool).
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

// Arguments of the encoders (kernel arguments by value).  For the FP8 cache
// `payload` is the fused pool and `scale` is unused.
struct WriteKArgs {
  const uint16_t* k;
  int64_t n_tokens;
  int64_t k_row_stride;
  const int32_t* pos;
  const int32_t* slot;
  const uint16_t* norm_w;
  float eps;
  const uint16_t* cos_sin;
  int32_t max_pos;
  uint8_t* payload;
  uint8_t* scale;
  int64_t num_pages;
};

struct PackQArgs {
  const uint16_t* q;
  int64_t n_rows;
  int n_heads;
  int64_t q_row_stride;
  const int32_t* pos;
  const uint16_t* cos_sin;
  int32_t max_pos;
  const float* w_in;
  float w_scale;
  uint8_t* q_out;
  void* q_scale;  // FP4: uint8 UE8M0 [rows*heads*4]; FP8: fp32 [rows*heads]
  float* w_out;
};

enum class Cache { kFp4, kFp8 };

// Block b of the K writer: tokens 64 b .. 64 b + 63, four lanes each.  A
// token whose slot lies outside [0, num_pages*64) or whose position lies
// outside [0, max_pos) is skipped (negative slots are padding; the others
// break the call's contract, and skipping keeps every access in bounds).
template <Cache C>
__device__ __forceinline__ void write_k_block(const WriteKArgs& a, int64_t b) {
  __shared__ float g[kDim];
  if (threadIdx.x < kDim) g[threadIdx.x] = __uint_as_float((uint32_t)a.norm_w[threadIdx.x] << 16);
  __syncthreads();
  const int64_t gl = b * 256 + threadIdx.x;
  const int64_t i = gl >> 2;  // token; its four lanes leave or stay together
  const int q = (int)(gl & 3);
  if (i >= a.n_tokens) return;
  const int32_t s = a.slot[i];
  const int32_t p = a.pos[i];
  if (s < 0 || (int64_t)s >= a.num_pages * kPageTokens || p < 0 || p >= a.max_pos) return;

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

  const int64_t page = s >> 6;
  const int tok = s & 63;
  if constexpr (C == Cache::kFp4) {
    uint32_t word[4], sc;
    quad_quant(v, word, sc);
    uint8_t* pp = a.payload + page * kPayloadPage + tok * 16 + 4 * q;
#pragma unroll
    for (int c = 0; c < 4; ++c) *reinterpret_cast<uint32_t*>(pp + c * 1024) = word[c];
    a.scale[page * kScalePage + q * 64 + tok] = (uint8_t)(sc >> (8 * q));
  } else {
    uint2 codes[4];
    float sc;
    quad_quant_fp8(v, codes, sc);
    uint8_t* pg = a.payload + page * kFp8Page;
#pragma unroll
    for (int c = 0; c < 4; ++c) *reinterpret_cast<uint2*>(pg + tok * kDim + 32 * c + 8 * q) = codes[c];
    if (q == 0) *reinterpret_cast<float*>(pg + kFp8ScaleOffset + tok * 4) = sc;
  }
}

// Block b of the Q pack: (row, head) vectors 64 b .. 64 b + 63, four lanes
// each.  A row whose position lies outside [0, max_pos) is encoded as the
// zero vector (no table read).
template <Cache C>
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
  if (p >= 0 && p < a.max_pos) {
    quad_rope(v, a.cos_sin + (int64_t)p * kRope, q);
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) v.x[c][e] = 0.0f;
  }
  quad_hadamard(v, q);

  if constexpr (C == Cache::kFp4) {
    uint32_t word[4], sc;
    quad_quant(v, word, sc);
    uint8_t* out = a.q_out + idx * 64 + 4 * q;
#pragma unroll
    for (int c = 0; c < 4; ++c) *reinterpret_cast<uint32_t*>(out + 16 * c) = word[c];
    static_cast<uint8_t*>(a.q_scale)[idx * 4 + q] = (uint8_t)(sc >> (8 * q));
  } else {
    uint2 codes[4];
    float sc;
    quad_quant_fp8(v, codes, sc);
    uint8_t* out = a.q_out + idx * kDim + 8 * q;
#pragma unroll
    for (int c = 0; c < 4; ++c) *reinterpret_cast<uint2*>(out + 32 * c) = codes[c];
    if (q == 0) static_cast<float*>(a.q_scale)[idx] = sc;
  }
  if (q == 0) a.w_out[idx] = a.w_in[idx] * a.w_scale;
}

template <Cache C>
__global__ __launch_bounds__(256) void write_k_quad_kernel(WriteKArgs a) {
  write_k_block<C>(a, blockIdx.x);
}

template <Cache C>
__global__ __launch_bounds__(256) void pack_q_quad_kernel(PackQArgs a) {
  pack_q_block<C>(a, blockIdx.x);
}

// One launch for a decode step's two independent encodes: the first
// k_blocks work-groups write K, the rest pack Q (the branch is uniform per
// work-group).
template <Cache C>
__global__ __launch_bounds__(256) void write_k_pack_q_kernel(WriteKArgs ka, PackQArgs qa, int64_t k_blocks) {
  const int64_t b = blockIdx.x;
  if (b < k_blocks)
    write_k_block<C>(ka, b);
  else
    pack_q_block<C>(qa, b - k_blocks);
}

static inline int64_t quad_blocks(int64_t n) { return (4 * n + 255) / 256; }

template <Cache C>
static hipError_t launch_write_k_any(const WriteKArgs& a, hipStream_t stream) {
  if (a.n_tokens == 0) return hipSuccess;
  return launch(write_k_quad_kernel<C>, dim3((unsigned)quad_blocks(a.n_tokens)), dim3(256), 0, stream, a);
}

template <Cache C>
static hipError_t launch_pack_q_any(const PackQArgs& a, hipStream_t stream) {
  const int64_t n = a.n_rows * a.n_heads;
  if (n == 0) return hipSuccess;
  return launch(pack_q_quad_kernel<C>, dim3((unsigned)quad_blocks(n)), dim3(256), 0, stream, a);
}

template <Cache C>
static hipError_t launch_both(const WriteKArgs& ka, const PackQArgs& qa, hipStream_t stream) {
  const int64_t kb = quad_blocks(ka.n_tokens), qb = quad_blocks(qa.n_rows * qa.n_heads);
  if (kb + qb == 0) return hipSuccess;
  if (kb + qb > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  return launch(write_k_pack_q_kernel<C>, dim3((unsigned)(kb + qb)), dim3(256), 0, stream, ka, qa, kb);
}

hipError_t launch_write_k(const uint16_t* k, int64_t n_tokens, int64_t k_row_stride, const int32_t* pos,
                          const int32_t* slot, const uint16_t* norm_w, float eps, const uint16_t* cos_sin,
                          int32_t max_pos, uint8_t* payload, uint8_t* scale, int64_t num_pages, hipStream_t stream) {
  const WriteKArgs a{k, n_tokens, k_row_stride, pos, slot, norm_w, eps, cos_sin, max_pos, payload, scale, num_pages};
  return launch_write_k_any<Cache::kFp4>(a, stream);
}

hipError_t launch_pack_q(const uint16_t* q, int64_t n_rows, int n_heads, int64_t q_row_stride, const int32_t* pos,
                         const uint16_t* cos_sin, int32_t max_pos, const float* w_in, float w_scale, uint8_t* q_fp4,
                         uint8_t* q_scale, float* w_out, hipStream_t stream) {
  const PackQArgs a{q, n_rows, n_heads, q_row_stride, pos, cos_sin, max_pos, w_in, w_scale, q_fp4, q_scale, w_out};
  return launch_pack_q_any<Cache::kFp4>(a, stream);
}

hipError_t launch_write_k_pack_q(const uint16_t* k, int64_t n_tokens, int64_t k_row_stride, const int32_t* pos_k,
                                 const int32_t* slot, const uint16_t* norm_w, float eps, const uint16_t* cos_sin,
                                 int32_t max_pos, uint8_t* payload, uint8_t* scale, int64_t num_pages,
                                 const uint16_t* q, int64_t n_rows, int n_heads, int64_t q_row_stride,
                                 const int32_t* pos_q, const float* w_in, float w_scale, uint8_t* q_fp4,
                                 uint8_t* q_scale, float* w_out, hipStream_t stream) {
  const WriteKArgs ka{k, n_tokens, k_row_stride, pos_k, slot, norm_w, eps, cos_sin, max_pos, payload, scale, num_pages};
  const PackQArgs qa{q, n_rows, n_heads, q_row_stride, pos_q, cos_sin, max_pos, w_in, w_scale, q_fp4, q_scale, w_out};
  return launch_both<Cache::kFp4>(ka, qa, stream);
}

hipError_t launch_write_k_fp8(const uint16_t* k, int64_t n_tokens, int64_t k_row_stride, const int32_t* pos,
                              const int32_t* slot, const uint16_t* norm_w, float eps, const uint16_t* cos_sin,
                              int32_t max_pos, uint8_t* pool, int64_t num_pages, hipStream_t stream) {
  const WriteKArgs a{k, n_tokens, k_row_stride, pos, slot, norm_w, eps, cos_sin, max_pos, pool, nullptr, num_pages};
  return launch_write_k_any<Cache::kFp8>(a, stream);
}

hipError_t launch_pack_q_fp8(const uint16_t* q, int64_t n_rows, int n_heads, int64_t q_row_stride,
                             const int32_t* pos, const uint16_t* cos_sin, int32_t max_pos, const float* w_in,
                             float w_scale, uint8_t* q_fp8, float* q_scale, float* w_out, hipStream_t stream) {
  const PackQArgs a{q, n_rows, n_heads, q_row_stride, pos, cos_sin, max_pos, w_in, w_scale, q_fp8, q_scale, w_out};
  return launch_pack_q_any<Cache::kFp8>(a, stream);
}

hipError_t launch_write_k_pack_q_fp8(const uint16_t* k, int64_t n_tokens, int64_t k_row_stride,
                                     const int32_t* pos_k, const int32_t* slot, const uint16_t* norm_w, float eps,
                                     const uint16_t* cos_sin, int32_t max_pos, uint8_t* pool, int64_t num_pages,
                                     const uint16_t* q, int64_t n_rows, int n_heads, int64_t q_row_stride,
                                     const int32_t* pos_q, const float* w_in, float w_scale, uint8_t* q_fp8,
                                     float* q_scale, float* w_out, hipStream_t stream) {
  const WriteKArgs ka{k, n_tokens, k_row_stride, pos_k, slot, norm_w, eps, cos_sin, max_pos, pool, nullptr, num_pages};
  const PackQArgs qa{q, n_rows, n_heads, q_row_stride, pos_q, cos_sin, max_pos, w_in, w_scale, q_fp8, q_scale, w_out};
  return launch_both<Cache::kFp8>(ka, qa, stream);
}

}  // namespace fp4idx
