// Host-side launchers of the gfx950 kernels (called by the C ABI layer after
// argument validation).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "schedule.hpp"

namespace fp4idx {

// Events armed by fp4idx_time_next_call() for the calling thread's next entry
// point call (cleared when that call returns).
struct TimingEvents {
  hipEvent_t start;
  hipEvent_t stop;
};
extern thread_local TimingEvents t_timing;

// Every kernel of the library is launched through here.  With armed events the
// launch goes through hipExtLaunchKernel, which stamps the events with the
// dispatch's own start and end times.
template <typename... KArgs, typename... Args>
inline hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t lds_bytes, hipStream_t stream,
                         Args... args) {
  if (t_timing.start != nullptr || t_timing.stop != nullptr) {
    hipExtLaunchKernelGGL(kernel, grid, block, lds_bytes, stream, t_timing.start, t_timing.stop, 0,
                          static_cast<KArgs>(args)...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds_bytes, stream, static_cast<KArgs>(args)...);
  }
  return hipGetLastError();
}

// f(std::integral_constant<int, NMT>{}) for the head count's 16-head M tiles,
// NMT = n_heads / 16 (head counts 16, 32, ..., 16 * MAX_NMT); any other count
// is hipErrorInvalidValue.
template <int N, int MAX_NMT, typename F>
inline hipError_t call_head_tiles(F& f) {
  if constexpr (N <= MAX_NMT)
    return f(std::integral_constant<int, N>{});
  else
    return hipErrorInvalidValue;
}
template <int MAX_NMT = 8, typename F>
inline hipError_t with_head_tiles(int n_heads, F&& f) {
  if (n_heads <= 0 || n_heads % 16 != 0) return hipErrorInvalidValue;
  switch (n_heads / 16) {
    case 1: return call_head_tiles<1, MAX_NMT>(f);
    case 2: return call_head_tiles<2, MAX_NMT>(f);
    case 3: return call_head_tiles<3, MAX_NMT>(f);
    case 4: return call_head_tiles<4, MAX_NMT>(f);
    case 5: return call_head_tiles<5, MAX_NMT>(f);
    case 6: return call_head_tiles<6, MAX_NMT>(f);
    case 7: return call_head_tiles<7, MAX_NMT>(f);
    case 8: return call_head_tiles<8, MAX_NMT>(f);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_write_k(const uint16_t* k, int64_t n_tokens, int64_t k_row_stride, const int32_t* pos,
                          const int32_t* slot, const uint16_t* norm_w, float eps, const uint16_t* cos_sin,
                          int32_t max_pos, uint8_t* payload, uint8_t* scale, int64_t num_pages, hipStream_t stream);

hipError_t launch_pack_q(const uint16_t* q, int64_t n_rows, int n_heads, int64_t q_row_stride, const int32_t* pos,
                         const uint16_t* cos_sin, int32_t max_pos, const float* w_in, float w_scale, uint8_t* q_fp4,
                         uint8_t* q_scale, float* w_out, hipStream_t stream);

hipError_t launch_write_k_pack_q(const uint16_t* k, int64_t n_tokens, int64_t k_row_stride, const int32_t* pos_k,
                                 const int32_t* slot, const uint16_t* norm_w, float eps, const uint16_t* cos_sin,
                                 int32_t max_pos, uint8_t* payload, uint8_t* scale, int64_t num_pages,
                                 const uint16_t* q, int64_t n_rows, int n_heads, int64_t q_row_stride,
                                 const int32_t* pos_q, const float* w_in, float w_scale, uint8_t* q_fp4,
                                 uint8_t* q_scale, float* w_out, hipStream_t stream);

hipError_t launch_write_k_fp8(const uint16_t* k, int64_t n_tokens, int64_t k_row_stride, const int32_t* pos,
                              const int32_t* slot, const uint16_t* norm_w, float eps, const uint16_t* cos_sin,
                              int32_t max_pos, uint8_t* pool, int64_t num_pages, hipStream_t stream);

hipError_t launch_pack_q_fp8(const uint16_t* q, int64_t n_rows, int n_heads, int64_t q_row_stride,
                             const int32_t* pos, const uint16_t* cos_sin, int32_t max_pos, const float* w_in,
                             float w_scale, uint8_t* q_fp8, float* q_scale, float* w_out, hipStream_t stream);

hipError_t launch_write_k_pack_q_fp8(const uint16_t* k, int64_t n_tokens, int64_t k_row_stride,
                                     const int32_t* pos_k, const int32_t* slot, const uint16_t* norm_w, float eps,
                                     const uint16_t* cos_sin, int32_t max_pos, uint8_t* pool, int64_t num_pages,
                                     const uint16_t* q, int64_t n_rows, int n_heads, int64_t q_row_stride,
                                     const int32_t* pos_q, const float* w_in, float w_scale, uint8_t* q_fp8,
                                     float* q_scale, float* w_out, hipStream_t stream);

hipError_t launch_mqa_logits_bounded(const uint8_t* q_fp4, const uint8_t* q_scale, const float* w, int64_t n_rows,
                                     int n_heads, const int32_t* indptr, int32_t n_reqs, const int32_t* row_ctx,
                                     const int32_t* block_table, int32_t bt_stride, const uint8_t* payload,
                                     const uint8_t* scale, int64_t num_pages, float* logits, int64_t logits_stride,
                                     int32_t max_rows_per_req, int64_t max_ctx, hipStream_t stream);

// The scheduled logits: the plan kernel (the batch's items into the
// workspace) and the persistent kernel that walks them.
hipError_t launch_plan(const int32_t* indptr, int32_t n_reqs, int64_t n_rows, const int32_t* row_ctx,
                       int64_t max_ctx, int32_t* ws, int64_t cap_items, const PlanSizes& sz, const PlanShape& sh,
                       int fixed, int target, int resident, hipStream_t stream);
PlanShape plan_shape(int64_t n_rows, int32_t n_reqs, int n_heads);
int64_t plan_workspace_bytes(int64_t n_rows, int32_t n_reqs, int64_t max_ctx);
hipError_t launch_mqa_logits_plan(int64_t n_rows, int n_heads, const int32_t* indptr, int32_t n_reqs,
                                  const int32_t* row_ctx, int64_t max_ctx, void* workspace, int64_t workspace_bytes,
                                  hipStream_t stream);
hipError_t launch_mqa_logits_run(const uint8_t* q_fp4, const uint8_t* q_scale, const float* w, int64_t n_rows,
                                 int n_heads, const int32_t* indptr, int32_t n_reqs, const int32_t* row_ctx,
                                 const int32_t* block_table, int32_t bt_stride, const uint8_t* payload,
                                 const uint8_t* scale, int64_t num_pages, float* logits, int64_t logits_stride,
                                 void* workspace, int64_t workspace_bytes, hipStream_t stream);

hipError_t launch_mqa_logits_fp8(const uint8_t* q_fp8, const float* q_scale, const float* w, int64_t n_rows, int n_heads,
                                 const int32_t* indptr, int32_t n_reqs, const int32_t* row_ctx,
                                 const int32_t* block_table, int32_t bt_stride, const uint8_t* pool,
                                 int64_t num_pages, float* logits, int64_t logits_stride, int32_t max_rows_per_req,
                                 int64_t max_ctx, hipStream_t stream);

// Longest row the fused logits + top-k kernel holds (its LDS row).
constexpr int64_t kFusedMaxCtx = 32768;

hipError_t launch_mqa_logits_topk(const uint8_t* q_fp4, const uint8_t* q_scale, const float* w, int64_t n_rows, int n_heads,
                                  const int32_t* indptr, int32_t n_reqs, const int32_t* row_ctx,
                                  const int32_t* block_table, int32_t bt_stride, const uint8_t* payload,
                                  const uint8_t* scale, int64_t num_pages, int32_t k, int32_t* out_idx,
                                  int32_t max_rows_per_req, int64_t max_ctx, hipStream_t stream);

hipError_t launch_peak_mfma_fp4(int32_t iters, float* sink, hipStream_t stream);
hipError_t launch_peak_valu_fp32(int32_t iters, float* sink, hipStream_t stream);
hipError_t launch_peak_mix(int32_t mode, int32_t iters, float* sink, hipStream_t stream);
hipError_t launch_peak_read(const uint8_t* buf, int64_t bytes, uint32_t* sink, hipStream_t stream);

hipError_t launch_read_k(const uint8_t* payload, const uint8_t* scale, int64_t num_pages, const int32_t* slot,
                         int64_t n_tokens, float* out, int64_t out_stride, hipStream_t stream);

hipError_t launch_topk(const float* logits, int64_t n_rows, int64_t logits_stride, const int32_t* row_ctx, int32_t k,
                       int32_t* out_idx, int64_t max_ctx, hipStream_t stream);

}  // namespace fp4idx
