// Fused paged FP4 logits + top-k on gfx950: the selection without writing
// the logits to memory.
//
// "[AMD] DeepSeek-V4.1-Flash on MI350X (gfx950)", Changes (sorted top-k
// selection) over the FP4 paged-MQA logits of "[AMD] Enable FP4 indexer for
// Deepseek V4" (Modifications / decode logits dispatch).
//
// One work-group of 1024 threads per query row.  Phase 1: the 16 waves
// score the row's pages (wave w takes pages w, w + 16, ...; three or four
// in flight at a time) with exactly the per-(row, token) arithmetic of the logits
// kernel (row_page_logits), and each page's 64 logits go to an LDS row of
// up to 32,768 values.  Phase 2: slot j of thread t takes position
// t + 1024 j from LDS, and the register selection of the top-k kernel
// (topk_select) picks the row's k positions.  The result is bit-for-bit the
// one of the logits kernel followed by the top-k kernel.
//
// Where it pays: a row's whole epilogue runs on one CU, and rows of one
// request each read the request's pages, so it suits batches of
// single-row requests (decode); the two-kernel path shares each page among
// up to four rows of a request and spreads one row over many CUs.
#include "launch.hpp"
#include "logits_core.hpp"
#include "topk_core.hpp"

namespace fp4idx {

constexpr int kFusedThreads = 1024;
constexpr int kFusedWaves = kFusedThreads / 64;
// pages in flight per wave: four, three at 64 heads (register budget of
// four waves per SIMD)
template <int NMT>
constexpr int kFusedPagesInFlight = NMT >= 4 ? 3 : 4;

template <int NMT, int J>
__global__ __launch_bounds__(kFusedThreads) void mqa_logits_topk_kernel(
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ indptr, const int32_t* __restrict__ row_ctx,
    const uint8_t* __restrict__ payload, const uint8_t* __restrict__ scale, int64_t num_pages, int32_t bt_stride,
    const uint8_t* __restrict__ q_fp4, const uint8_t* __restrict__ q_scale, const float* __restrict__ w, int k,
    int32_t* __restrict__ out_idx, int32_t n_rows) {
  using FMT = Fp4Split;
  constexpr int NT = kFusedThreads;
  constexpr int H = NMT * 16;
  constexpr int NSC = (NMT + 3) / 4;
  constexpr int D = kFusedPagesInFlight<NMT>;
  __shared__ float stage[NT * J];
  __shared__ TopkRegShared<NT, J> sh;

  // grid: x = row within the request, y = request
  const int req = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the request's rows, kept inside [0, n_rows) whatever indptr holds
  const int ip0 = min(max(indptr[req], 0), n_rows), ip1 = min(max(indptr[req + 1], ip0), n_rows);
  const int64_t row = (int64_t)ip0 + blockIdx.x;
  if (row >= ip1) return;
  // a context length beyond the table or the LDS row is cut to what both hold
  const int ctx = min(max(row_ctx[row], 0), (int)min((int64_t)bt_stride * 64, (int64_t)NT * J));
  const int K = min(k, ctx);
  int32_t* o = out_idx + row * (int64_t)k;
  if (K == ctx) {  // everything is selected (includes ctx == 0)
    for (int i = tid; i < k; i += NT) o[i] = i < ctx ? i : -1;
    return;
  }

  // 1. the row's logits into LDS
  const int li = lane & 15, lg = lane >> 4;
  typename FMT::QOp aq[NMT];
  uint32_t asc[NSC];
  float wv[NMT][4];
#pragma unroll
  for (int c = 0; c < NSC; ++c) asc[c] = 0;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    const int64_t hrow = row * H + mt * 16 + li;
    aq[mt] = FMT::load_q(q_fp4, hrow, lg);
    asc[mt >> 2] |= FMT::q_scale_byte(q_scale, hrow, lg) << (8 * (mt & 3));
    const float4 w4 = *reinterpret_cast<const float4*>(w + row * H + mt * 16 + lg * 4);
    wv[mt][0] = w4.x;
    wv[mt][1] = w4.y;
    wv[mt][2] = w4.z;
    wv[mt][3] = w4.w;
  }
  const uint32_t lane_pay = FMT::lane_pay(li, lg);
  const uint32_t lane_sc = FMT::lane_sc(li, lg);
  const int32_t* bt = block_table + (int64_t)req * bt_stride;
  const int n_pages = (ctx + 63) >> 6;
  for (int p0 = wave; p0 < n_pages; p0 += kFusedWaves * D) {
    typename FMT::Page pg[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int p = p0 + kFusedWaves * d;
      if (p < n_pages) {
        const int32_t id = bt[p];
        // an id outside the pool (a broken contract) reads page 0; its
        // tokens' results are then unspecified but every access in bounds
        FMT::template load_page<true>(pg[d], payload, scale, (id >= 0 && id < num_pages) ? id : 0, lane_pay, lane_sc);
      }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int p = p0 + kFusedWaves * d;
      if (p < n_pages) {
        const float tot = row_page_logits<FMT, NMT, true>(aq, asc, wv, pg[d]);
        const int tok = p * 64 + lane;
        if (tok < ctx) stage[tok] = tot;
      }
    }
  }
  __syncthreads();

  // 2. selection: slots past the row end take a copy of the row's last value
  float v[J];
#pragma unroll
  for (int j = 0; j < J; ++j) v[j] = stage[min(tid + NT * j, ctx - 1)];
  topk_select<NT, J>(v, ctx, K, k, o, sh, [&](int p) { return stage[p]; });
}

template <int NMT, int J>
static hipError_t launch_fused_j(const uint8_t* q_fp4, const uint8_t* q_scale, const float* w, const int32_t* indptr,
                                 int32_t n_reqs, const int32_t* row_ctx, const int32_t* block_table, int32_t bt_stride,
                                 const uint8_t* payload, const uint8_t* scale, int64_t num_pages, int32_t k,
                                 int32_t* out_idx, int32_t max_rows_per_req, int32_t n_rows, hipStream_t stream) {
  return launch(mqa_logits_topk_kernel<NMT, J>, dim3((unsigned)max_rows_per_req, (unsigned)n_reqs),
                dim3(kFusedThreads), 0, stream, block_table, indptr, row_ctx, payload, scale, num_pages, bt_stride,
                q_fp4, q_scale, w, k, out_idx, n_rows);
}

template <int NMT>
static hipError_t launch_fused_nmt(const uint8_t* q_fp4, const uint8_t* q_scale, const float* w,
                                   const int32_t* indptr, int32_t n_reqs, const int32_t* row_ctx,
                                   const int32_t* block_table, int32_t bt_stride, const uint8_t* payload,
                                   const uint8_t* scale, int64_t num_pages, int32_t k, int32_t* out_idx,
                                   int32_t max_rows_per_req, int64_t max_ctx, int32_t n_rows, hipStream_t stream) {
  // J slots per thread cover the longest row (J * 1024 >= max_ctx)
  if (max_ctx <= 1024)
    return launch_fused_j<NMT, 1>(q_fp4, q_scale, w, indptr, n_reqs, row_ctx, block_table, bt_stride, payload, scale,
                                  num_pages, k, out_idx, max_rows_per_req, n_rows, stream);
  if (max_ctx <= 4096)
    return launch_fused_j<NMT, 4>(q_fp4, q_scale, w, indptr, n_reqs, row_ctx, block_table, bt_stride, payload, scale,
                                  num_pages, k, out_idx, max_rows_per_req, n_rows, stream);
  if (max_ctx <= 8192)
    return launch_fused_j<NMT, 8>(q_fp4, q_scale, w, indptr, n_reqs, row_ctx, block_table, bt_stride, payload, scale,
                                  num_pages, k, out_idx, max_rows_per_req, n_rows, stream);
  if (max_ctx <= 16384)
    return launch_fused_j<NMT, 16>(q_fp4, q_scale, w, indptr, n_reqs, row_ctx, block_table, bt_stride, payload,
                                   scale, num_pages, k, out_idx, max_rows_per_req, n_rows, stream);
  return launch_fused_j<NMT, 32>(q_fp4, q_scale, w, indptr, n_reqs, row_ctx, block_table, bt_stride, payload, scale,
                                 num_pages, k, out_idx, max_rows_per_req, n_rows, stream);
}

hipError_t launch_mqa_logits_topk(const uint8_t* q_fp4, const uint8_t* q_scale, const float* w, int64_t n_rows, int n_heads,
                                  const int32_t* indptr, int32_t n_reqs, const int32_t* row_ctx,
                                  const int32_t* block_table, int32_t bt_stride, const uint8_t* payload,
                                  const uint8_t* scale, int64_t num_pages, int32_t k, int32_t* out_idx,
                                  int32_t max_rows_per_req, int64_t max_ctx, hipStream_t stream) {
  if (max_ctx > kFusedMaxCtx || n_rows > 0x7FFFFFFFLL || n_reqs > 65535) return hipErrorInvalidConfiguration;
  return with_head_tiles<4>(n_heads, [&](auto nmt) {
    return launch_fused_nmt<decltype(nmt)::value>(q_fp4, q_scale, w, indptr, n_reqs, row_ctx, block_table, bt_stride,
                                                 payload, scale, num_pages, k, out_idx, max_rows_per_req, max_ctx,
                                                 (int32_t)n_rows, stream);
  });
}

}  // namespace fp4idx
