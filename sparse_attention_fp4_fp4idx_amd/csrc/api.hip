// C ABI of the FP4 lightning-indexer library (declared in include/fp4idx.h).
//
// Validation looks at host scalars and pointer values only (never at device
// memory), so every entry point can be captured in a HIP graph.  On any
// negative status nothing has been launched.
#include <algorithm>
#include <atomic>
#include <cstring>
#include <mutex>

#include "fp4idx.h"
#include "launch.hpp"

namespace fp4idx {
thread_local TimingEvents t_timing = {nullptr, nullptr};
}

// Scratch of fp4idx_mqa_logits_noalloc: a fixed array in every device's
// copy of the code object, holding the work schedule of that call.  Host
// code never passes the array's name to a kernel (on the host it is a
// stand-in, not a device address): it uses the address hipGetSymbolAddress
// gives for the current device, looked up once per device.
static __device__ __align__(256) uint8_t scratch[FP4IDX_SCRATCH_BYTES];

namespace {

// Disarms the timing events when an entry point returns, launched or not.
struct TimingScope {
  ~TimingScope() { fp4idx::t_timing = {nullptr, nullptr}; }
};

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other architecture
std::atomic<int> g_arch[kMaxDevices];

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FP4IDX_E_LAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return FP4IDX_E_UNSUPPORTED;
  int a = g_arch[dev].load(std::memory_order_relaxed);
  if (a == 0) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return FP4IDX_E_LAUNCH;
    a = (std::strncmp(p.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch[dev].store(a, std::memory_order_relaxed);
  }
  return a == 1 ? FP4IDX_OK : FP4IDX_E_UNSUPPORTED;
}

// Index head counts: a multiple of 16 (one MFMA M tile) up to 128.
inline bool valid_heads(int32_t n_heads) { return n_heads >= 16 && n_heads <= 128 && n_heads % 16 == 0; }

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

inline int launched(hipError_t e) { return e == hipSuccess ? FP4IDX_OK : FP4IDX_E_LAUNCH; }

}  // namespace

extern "C" {

int fp4idx_version(void) { return 100; }

int fp4idx_time_next_call(void* start_event, void* stop_event) {
  fp4idx::t_timing = {static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event)};
  return FP4IDX_OK;
}

const char* fp4idx_status_string(int status) {
  switch (status) {
    case FP4IDX_OK: return "ok";
    case FP4IDX_E_INVALID: return "invalid argument";
    case FP4IDX_E_UNSUPPORTED: return "unsupported device (gfx950 required)";
    case FP4IDX_E_LAUNCH: return "HIP launch or runtime error";
    case FP4IDX_E_WORKSPACE: return "workspace missing or too small";
    case FP4IDX_E_SCRATCH:
      return "the batch's work schedule needs more than the library's built-in scratch "
             "(FP4IDX_SCRATCH_BYTES); use fp4idx_mqa_logits with a workspace";
    default: return "unknown status";
  }
}

}  // extern "C"

namespace {

// Host checks of the K writer's arguments (an empty batch checks no pointer).
int check_write_k(const uint16_t* k_bf16, int64_t n_tokens, int64_t k_row_stride, const int32_t* pos,
                  const int32_t* slot, const uint16_t* norm_w_bf16, float eps, const uint16_t* cos_sin_bf16,
                  int32_t max_pos, const uint8_t* payload, const uint8_t* scale, int64_t num_pages) {
  if (n_tokens < 0 || num_pages < 0 || max_pos <= 0) return FP4IDX_E_INVALID;
  if (k_row_stride < FP4IDX_HEAD_DIM || (k_row_stride % 8) != 0) return FP4IDX_E_INVALID;
  if (n_tokens == 0) return FP4IDX_OK;
  if (!k_bf16 || !pos || !slot || !norm_w_bf16 || !cos_sin_bf16 || !payload || !scale) return FP4IDX_E_INVALID;
  if (!aligned(k_bf16, 16) || !aligned(cos_sin_bf16, 16) || !aligned(payload, 16)) return FP4IDX_E_INVALID;
  if (!(eps >= 0.0f)) return FP4IDX_E_INVALID;
  if (n_tokens > ((int64_t)0x7FFFFFFF) * 64) return FP4IDX_E_INVALID;  // 4 lanes per token, grid x < 2^31
  return FP4IDX_OK;
}

// Host checks of the Q pack's arguments (an empty batch checks no pointer).
int check_pack_q(const uint16_t* q_bf16, int64_t n_rows, int32_t n_heads, int64_t q_row_stride, const int32_t* pos,
                 const uint16_t* cos_sin_bf16, int32_t max_pos, const float* w_in, const uint8_t* q_fp4,
                 const uint8_t* q_scale, const float* w_out) {
  if (n_rows < 0 || max_pos <= 0) return FP4IDX_E_INVALID;
  if (!valid_heads(n_heads)) return FP4IDX_E_INVALID;
  if (q_row_stride < (int64_t)n_heads * FP4IDX_HEAD_DIM || (q_row_stride % 8) != 0) return FP4IDX_E_INVALID;
  if (n_rows == 0) return FP4IDX_OK;
  if (!q_bf16 || !pos || !cos_sin_bf16 || !w_in || !q_fp4 || !q_scale || !w_out) return FP4IDX_E_INVALID;
  if (!aligned(q_bf16, 16) || !aligned(cos_sin_bf16, 16) || !aligned(q_fp4, 16) || !aligned(q_scale, 4))
    return FP4IDX_E_INVALID;
  if (n_rows * n_heads > ((int64_t)0x7FFFFFFF) * 64) return FP4IDX_E_INVALID;  // 4 lanes per vector
  return FP4IDX_OK;
}

// Host checks of the logits calls' scalars shared by both caches.
int check_logits(int64_t n_rows, int32_t n_heads, int32_t n_reqs, int32_t bt_stride, int64_t num_pages,
                 int64_t logits_stride, int32_t max_rows_per_req, int64_t max_ctx) {
  if (n_rows < 0 || n_reqs < 0 || num_pages < 0 || bt_stride < 0 || logits_stride < 0 || max_rows_per_req < 0 ||
      max_ctx < 0)
    return FP4IDX_E_INVALID;
  if (!valid_heads(n_heads)) return FP4IDX_E_INVALID;
  if (max_ctx > (int64_t)bt_stride * FP4IDX_PAGE_TOKENS || max_ctx > logits_stride) return FP4IDX_E_INVALID;
  if (max_rows_per_req > n_rows || n_reqs > 65535 || n_rows > 0x7FFFFFFF) return FP4IDX_E_INVALID;
  if (n_rows == 0 || n_reqs == 0 || max_ctx == 0 || max_rows_per_req == 0) return FP4IDX_OK;
  if (num_pages == 0) return FP4IDX_E_INVALID;
  return FP4IDX_OK;
}

// Host checks of a plan's arguments.
int check_plan(int64_t n_rows, int32_t n_heads, const int32_t* indptr, int32_t n_reqs, const int32_t* row_ctx,
               int64_t max_ctx, const void* workspace, size_t workspace_bytes) {
  if (n_rows < 0 || n_reqs < 0 || max_ctx < 0 || n_rows > 0x7FFFFFFF) return FP4IDX_E_INVALID;
  if (!valid_heads(n_heads)) return FP4IDX_E_INVALID;
  if (n_rows == 0 || n_reqs == 0) return FP4IDX_OK;
  if (!indptr || !row_ctx) return FP4IDX_E_INVALID;
  if (!workspace || !aligned(workspace, 16) || workspace_bytes > (size_t)INT64_MAX) return FP4IDX_E_WORKSPACE;
  const fp4idx::PlanShape sh = fp4idx::plan_shape(n_rows, n_reqs, n_heads);
  const fp4idx::PlanSizes sz = fp4idx::plan_sizes(n_rows, n_reqs, sh.rows);
  const int64_t cap = fp4idx::plan_capacity(sz, (int64_t)workspace_bytes);
  if (cap < sz.blocks || cap > 0x7FFFFFFF) return FP4IDX_E_WORKSPACE;
  return FP4IDX_OK;
}

// Host checks of a scheduled logits call's buffers and scalars, apart from
// its workspace.
int check_planned_args(const uint8_t* q_fp4, const uint8_t* q_scale, const float* w, int64_t n_rows,
                       int32_t n_heads, const int32_t* indptr, int32_t n_reqs, const int32_t* row_ctx,
                       const int32_t* block_table, int32_t bt_stride, const uint8_t* payload, const uint8_t* scale,
                       int64_t num_pages, const float* logits, int64_t logits_stride) {
  if (bt_stride < 0 || num_pages < 0 || logits_stride < 0) return FP4IDX_E_INVALID;
  if (n_rows < 0 || n_reqs < 0 || n_rows > 0x7FFFFFFF) return FP4IDX_E_INVALID;
  if (!valid_heads(n_heads)) return FP4IDX_E_INVALID;
  if (n_rows == 0 || n_reqs == 0) return FP4IDX_OK;
  if (!indptr || !row_ctx) return FP4IDX_E_INVALID;
  if (num_pages == 0 || !q_fp4 || !q_scale || !w || !block_table || !payload || !scale || !logits)
    return FP4IDX_E_INVALID;
  if (!aligned(q_fp4, 16) || !aligned(w, 16) || !aligned(payload, 16) || !aligned(scale, 4)) return FP4IDX_E_INVALID;
  return FP4IDX_OK;
}

// Host checks of a scheduled logits call (its plan's checks, then the rest).
int check_planned(const uint8_t* q_fp4, const uint8_t* q_scale, const float* w, int64_t n_rows, int32_t n_heads,
                  const int32_t* indptr, int32_t n_reqs, const int32_t* row_ctx, const int32_t* block_table,
                  int32_t bt_stride, const uint8_t* payload, const uint8_t* scale, int64_t num_pages,
                  const float* logits, int64_t logits_stride, const void* workspace, size_t workspace_bytes) {
  if (bt_stride < 0 || num_pages < 0 || logits_stride < 0) return FP4IDX_E_INVALID;
  const int rc = check_plan(n_rows, n_heads, indptr, n_reqs, row_ctx, 0, workspace, workspace_bytes);
  if (rc != FP4IDX_OK || n_rows == 0 || n_reqs == 0) return rc;
  return check_planned_args(q_fp4, q_scale, w, n_rows, n_heads, indptr, n_reqs, row_ctx, block_table, bt_stride,
                            payload, scale, num_pages, logits, logits_stride);
}

// Plan and run in sequence on one stream.  Armed timing events stamp the
// plan's start and the run's end.
hipError_t planned_logits(const uint8_t* q_fp4, const uint8_t* q_scale, const float* w, int64_t n_rows,
                          int32_t n_heads, const int32_t* indptr, int32_t n_reqs, const int32_t* row_ctx,
                          const int32_t* block_table, int32_t bt_stride, const uint8_t* payload, const uint8_t* scale,
                          int64_t num_pages, float* logits, int64_t logits_stride, void* workspace,
                          int64_t workspace_bytes, hipStream_t stream) {
  const fp4idx::TimingEvents armed = fp4idx::t_timing;
  // contexts are cut to the logits row and the block table in any case
  const int64_t ctx_bound = std::min<int64_t>(logits_stride, (int64_t)bt_stride * FP4IDX_PAGE_TOKENS);
  fp4idx::t_timing = {armed.start, nullptr};
  hipError_t e = fp4idx::launch_mqa_logits_plan(n_rows, n_heads, indptr, n_reqs, row_ctx, ctx_bound, workspace,
                                                workspace_bytes, stream);
  fp4idx::t_timing = {nullptr, armed.stop};
  if (e == hipSuccess)
    e = fp4idx::launch_mqa_logits_run(q_fp4, q_scale, w, n_rows, n_heads, indptr, n_reqs, row_ctx, block_table,
                                      bt_stride, payload, scale, num_pages, logits, logits_stride, workspace,
                                      workspace_bytes, stream);
  return e;
}

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch[kMaxDevices];

// The current device's scratch address (FP4IDX_E_LAUNCH when the lookup fails).
int scratch_of_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FP4IDX_E_LAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return FP4IDX_E_UNSUPPORTED;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    const std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FP4IDX_E_LAUNCH;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return FP4IDX_OK;
}

}  // namespace

extern "C" {

int fp4idx_write_k(const uint16_t* k_bf16, int64_t n_tokens, int64_t k_row_stride, const int32_t* pos,
                   const int32_t* slot, const uint16_t* norm_w_bf16, float eps, const uint16_t* cos_sin_bf16,
                   int32_t max_pos, uint8_t* payload, uint8_t* scale, int64_t num_pages, void* stream) {
  const TimingScope timing_scope;
  const int rc = check_write_k(k_bf16, n_tokens, k_row_stride, pos, slot, norm_w_bf16, eps, cos_sin_bf16, max_pos,
                               payload, scale, num_pages);
  if (rc != FP4IDX_OK || n_tokens == 0) return rc;
  const int dev = check_device();
  if (dev != FP4IDX_OK) return dev;
  return launched(fp4idx::launch_write_k(k_bf16, n_tokens, k_row_stride, pos, slot, norm_w_bf16, eps, cos_sin_bf16,
                                         max_pos, payload, scale, num_pages, static_cast<hipStream_t>(stream)));
}

int fp4idx_pack_q(const uint16_t* q_bf16, int64_t n_rows, int32_t n_heads, int64_t q_row_stride,
                  const int32_t* pos, const uint16_t* cos_sin_bf16, int32_t max_pos, const float* w_in,
                  float w_scale, uint8_t* q_fp4, uint8_t* q_scale, float* w_out, void* stream) {
  const TimingScope timing_scope;
  const int rc = check_pack_q(q_bf16, n_rows, n_heads, q_row_stride, pos, cos_sin_bf16, max_pos, w_in, q_fp4,
                              q_scale, w_out);
  if (rc != FP4IDX_OK || n_rows == 0) return rc;
  const int dev = check_device();
  if (dev != FP4IDX_OK) return dev;
  return launched(fp4idx::launch_pack_q(q_bf16, n_rows, n_heads, q_row_stride, pos, cos_sin_bf16, max_pos, w_in,
                                        w_scale, q_fp4, q_scale, w_out, static_cast<hipStream_t>(stream)));
}

int fp4idx_write_k_pack_q(const uint16_t* k_bf16, int64_t n_tokens, int64_t k_row_stride, const int32_t* pos_k,
                          const int32_t* slot, const uint16_t* norm_w_bf16, float eps, const uint16_t* cos_sin_bf16,
                          int32_t max_pos, uint8_t* payload, uint8_t* scale, int64_t num_pages,
                          const uint16_t* q_bf16, int64_t n_rows, int32_t n_heads, int64_t q_row_stride,
                          const int32_t* pos_q, const float* w_in, float w_scale, uint8_t* q_fp4, uint8_t* q_scale,
                          float* w_out, void* stream) {
  const TimingScope timing_scope;
  int rc = check_write_k(k_bf16, n_tokens, k_row_stride, pos_k, slot, norm_w_bf16, eps, cos_sin_bf16, max_pos,
                         payload, scale, num_pages);
  if (rc != FP4IDX_OK) return rc;
  rc = check_pack_q(q_bf16, n_rows, n_heads, q_row_stride, pos_q, cos_sin_bf16, max_pos, w_in, q_fp4, q_scale,
                    w_out);
  if (rc != FP4IDX_OK) return rc;
  if (n_tokens == 0 && n_rows == 0) return FP4IDX_OK;
  const int dev = check_device();
  if (dev != FP4IDX_OK) return dev;
  return launched(fp4idx::launch_write_k_pack_q(k_bf16, n_tokens, k_row_stride, pos_k, slot, norm_w_bf16, eps,
                                                cos_sin_bf16, max_pos, payload, scale, num_pages, q_bf16, n_rows,
                                                n_heads, q_row_stride, pos_q, w_in, w_scale, q_fp4, q_scale, w_out,
                                                static_cast<hipStream_t>(stream)));
}

int fp4idx_mqa_logits_bounded(const uint8_t* q_fp4, const uint8_t* q_scale, const float* w, int64_t n_rows,
                              int32_t n_heads, const int32_t* req_row_indptr, int32_t n_reqs,
                              const int32_t* row_ctx_len, const int32_t* block_table, int32_t bt_stride,
                              const uint8_t* payload, const uint8_t* scale, int64_t num_pages, float* logits,
                              int64_t logits_stride, int32_t max_rows_per_req, int64_t max_ctx, void* stream) {
  const TimingScope timing_scope;
  int rc = check_logits(n_rows, n_heads, n_reqs, bt_stride, num_pages, logits_stride, max_rows_per_req, max_ctx);
  if (rc != FP4IDX_OK || n_rows == 0 || n_reqs == 0 || max_ctx == 0 || max_rows_per_req == 0) return rc;
  if (!q_fp4 || !q_scale || !w || !req_row_indptr || !row_ctx_len || !block_table || !payload || !scale || !logits)
    return FP4IDX_E_INVALID;
  if (!aligned(q_fp4, 16) || !aligned(w, 16) || !aligned(payload, 16) || !aligned(scale, 4)) return FP4IDX_E_INVALID;
  const int dev = check_device();
  if (dev != FP4IDX_OK) return dev;
  return launched(fp4idx::launch_mqa_logits_bounded(q_fp4, q_scale, w, n_rows, n_heads, req_row_indptr, n_reqs,
                                                    row_ctx_len, block_table, bt_stride, payload, scale, num_pages,
                                                    logits, logits_stride, max_rows_per_req, max_ctx,
                                                    static_cast<hipStream_t>(stream)));
}

size_t fp4idx_mqa_logits_workspace_bytes(int64_t n_rows, int32_t n_reqs, int64_t max_ctx) {
  if (n_rows <= 0 || n_reqs <= 0 || max_ctx < 0 || n_rows > 0x7FFFFFFF) return 0;
  return (size_t)fp4idx::plan_workspace_bytes(n_rows, n_reqs, max_ctx);
}

int fp4idx_mqa_logits_plan(int64_t n_rows, int32_t n_heads, const int32_t* req_row_indptr, int32_t n_reqs,
                           const int32_t* row_ctx_len, int64_t max_ctx, void* workspace, size_t workspace_bytes,
                           void* stream) {
  const TimingScope timing_scope;
  int rc = check_plan(n_rows, n_heads, req_row_indptr, n_reqs, row_ctx_len, max_ctx, workspace, workspace_bytes);
  if (rc != FP4IDX_OK || n_rows == 0 || n_reqs == 0) return rc;
  const int dev = check_device();
  if (dev != FP4IDX_OK) return dev;
  return launched(fp4idx::launch_mqa_logits_plan(n_rows, n_heads, req_row_indptr, n_reqs, row_ctx_len, max_ctx,
                                                 workspace, (int64_t)workspace_bytes,
                                                 static_cast<hipStream_t>(stream)));
}

int fp4idx_mqa_logits_run(const uint8_t* q_fp4, const uint8_t* q_scale, const float* w, int64_t n_rows,
                          int32_t n_heads, const int32_t* req_row_indptr, int32_t n_reqs, const int32_t* row_ctx_len,
                          const int32_t* block_table, int32_t bt_stride, const uint8_t* payload, const uint8_t* scale,
                          int64_t num_pages, float* logits, int64_t logits_stride, void* workspace,
                          size_t workspace_bytes, void* stream) {
  const TimingScope timing_scope;
  int rc = check_planned(q_fp4, q_scale, w, n_rows, n_heads, req_row_indptr, n_reqs, row_ctx_len, block_table,
                         bt_stride, payload, scale, num_pages, logits, logits_stride, workspace, workspace_bytes);
  if (rc != FP4IDX_OK || n_rows == 0 || n_reqs == 0) return rc;
  const int dev = check_device();
  if (dev != FP4IDX_OK) return dev;
  return launched(fp4idx::launch_mqa_logits_run(q_fp4, q_scale, w, n_rows, n_heads, req_row_indptr, n_reqs,
                                                row_ctx_len, block_table, bt_stride, payload, scale, num_pages,
                                                logits, logits_stride, workspace, (int64_t)workspace_bytes,
                                                static_cast<hipStream_t>(stream)));
}

int fp4idx_mqa_logits(const uint8_t* q_fp4, const uint8_t* q_scale, const float* w, int64_t n_rows, int32_t n_heads,
                      const int32_t* req_row_indptr, int32_t n_reqs, const int32_t* row_ctx_len,
                      const int32_t* block_table, int32_t bt_stride, const uint8_t* payload, const uint8_t* scale,
                      int64_t num_pages, float* logits, int64_t logits_stride, void* workspace, size_t workspace_bytes,
                      void* stream) {
  const TimingScope timing_scope;
  int rc = check_planned(q_fp4, q_scale, w, n_rows, n_heads, req_row_indptr, n_reqs, row_ctx_len, block_table,
                         bt_stride, payload, scale, num_pages, logits, logits_stride, workspace, workspace_bytes);
  if (rc != FP4IDX_OK || n_rows == 0 || n_reqs == 0) return rc;
  const int dev = check_device();
  if (dev != FP4IDX_OK) return dev;
  return launched(planned_logits(q_fp4, q_scale, w, n_rows, n_heads, req_row_indptr, n_reqs, row_ctx_len, block_table,
                                 bt_stride, payload, scale, num_pages, logits, logits_stride, workspace,
                                 (int64_t)workspace_bytes, static_cast<hipStream_t>(stream)));
}

int fp4idx_mqa_logits_noalloc(const uint8_t* q_fp4, const uint8_t* q_scale, const float* w, int64_t n_rows,
                              int32_t n_heads, const int32_t* req_row_indptr, int32_t n_reqs,
                              const int32_t* row_ctx_len, const int32_t* block_table, int32_t bt_stride,
                              const uint8_t* payload, const uint8_t* scale, int64_t num_pages, float* logits,
                              int64_t logits_stride, void* stream) {
  const TimingScope timing_scope;
  const int rc = check_planned_args(q_fp4, q_scale, w, n_rows, n_heads, req_row_indptr, n_reqs, row_ctx_len,
                                    block_table, bt_stride, payload, scale, num_pages, logits, logits_stride);
  if (rc != FP4IDX_OK || n_rows == 0 || n_reqs == 0) return rc;
  // the workspace fp4idx_mqa_logits would be given for this batch
  const int64_t ctx_bound = std::min<int64_t>(logits_stride, (int64_t)bt_stride * FP4IDX_PAGE_TOKENS);
  const int64_t need = fp4idx::plan_workspace_bytes(n_rows, n_reqs, ctx_bound);
  if (need > (int64_t)FP4IDX_SCRATCH_BYTES) return FP4IDX_E_SCRATCH;
  const int dev = check_device();
  if (dev != FP4IDX_OK) return dev;
  void* ws = nullptr;
  const int sc = scratch_of_current_device(&ws);
  if (sc != FP4IDX_OK) return sc;
  return launched(planned_logits(q_fp4, q_scale, w, n_rows, n_heads, req_row_indptr, n_reqs, row_ctx_len, block_table,
                                 bt_stride, payload, scale, num_pages, logits, logits_stride, ws, need,
                                 static_cast<hipStream_t>(stream)));
}

int fp4idx_mqa_logits_topk(const uint8_t* q_fp4, const uint8_t* q_scale, const float* w, int64_t n_rows,
                           int32_t n_heads, const int32_t* req_row_indptr, int32_t n_reqs,
                           const int32_t* row_ctx_len, const int32_t* block_table, int32_t bt_stride,
                           const uint8_t* payload, const uint8_t* scale, int64_t num_pages, int32_t k,
                           int32_t* out_idx, int32_t max_rows_per_req, int64_t max_ctx, void* stream) {
  const TimingScope timing_scope;
  if (n_rows < 0 || n_reqs < 0 || num_pages < 0 || bt_stride < 0 || max_rows_per_req < 0 || max_ctx < 0)
    return FP4IDX_E_INVALID;
  if (!valid_heads(n_heads) || n_heads > 64) return FP4IDX_E_INVALID;
  if (k < 1 || k > FP4IDX_MAX_TOPK) return FP4IDX_E_INVALID;
  if (max_ctx > (int64_t)bt_stride * FP4IDX_PAGE_TOKENS || max_ctx > FP4IDX_FUSED_MAX_CTX) return FP4IDX_E_INVALID;
  if (max_rows_per_req > n_rows || n_reqs > 65535 || n_rows > 0x7FFFFFFF) return FP4IDX_E_INVALID;
  if (n_rows == 0 || n_reqs == 0) return FP4IDX_OK;
  if (max_rows_per_req < 1) return FP4IDX_E_INVALID;  // every row's k outputs are written
  if (max_ctx > 0 && num_pages == 0) return FP4IDX_E_INVALID;
  if (!q_fp4 || !q_scale || !w || !req_row_indptr || !row_ctx_len || !block_table || !out_idx ||
      (max_ctx > 0 && (!payload || !scale)))
    return FP4IDX_E_INVALID;
  if (!aligned(q_fp4, 16) || !aligned(w, 16) || !aligned(payload, 16)) return FP4IDX_E_INVALID;
  const int dev = check_device();
  if (dev != FP4IDX_OK) return dev;
  return launched(fp4idx::launch_mqa_logits_topk(q_fp4, q_scale, w, n_rows, n_heads, req_row_indptr, n_reqs, row_ctx_len,
                                                 block_table, bt_stride, payload, scale, num_pages, k, out_idx,
                                                 max_rows_per_req, max_ctx, static_cast<hipStream_t>(stream)));
}

int fp4idx_read_k(const uint8_t* payload, const uint8_t* scale, int64_t num_pages, const int32_t* slot,
                  int64_t n_tokens, float* out, int64_t out_row_stride, void* stream) {
  const TimingScope timing_scope;
  if (n_tokens < 0 || num_pages < 0) return FP4IDX_E_INVALID;
  if (out_row_stride < FP4IDX_HEAD_DIM || (out_row_stride % 4) != 0) return FP4IDX_E_INVALID;
  if (n_tokens == 0) return FP4IDX_OK;
  if (!payload || !scale || !slot || !out) return FP4IDX_E_INVALID;
  if (!aligned(payload, 4) || !aligned(out, 16)) return FP4IDX_E_INVALID;
  if (n_tokens > ((int64_t)0x7FFFFFFF) * 16) return FP4IDX_E_INVALID;  // 16 lanes per token, grid x < 2^31
  const int dev = check_device();
  if (dev != FP4IDX_OK) return dev;
  return launched(fp4idx::launch_read_k(payload, scale, num_pages, slot, n_tokens, out, out_row_stride,
                                        static_cast<hipStream_t>(stream)));
}

int fp4idx_peak_mfma_fp4(int32_t iterations, float* sink, void* stream) {
  const TimingScope timing_scope;
  if (iterations < 1 || !sink) return FP4IDX_E_INVALID;
  const int dev = check_device();
  if (dev != FP4IDX_OK) return dev;
  return launched(fp4idx::launch_peak_mfma_fp4(iterations, sink, static_cast<hipStream_t>(stream)));
}

int fp4idx_peak_valu_fp32(int32_t iterations, float* sink, void* stream) {
  const TimingScope timing_scope;
  if (iterations < 1 || !sink) return FP4IDX_E_INVALID;
  const int dev = check_device();
  if (dev != FP4IDX_OK) return dev;
  return launched(fp4idx::launch_peak_valu_fp32(iterations, sink, static_cast<hipStream_t>(stream)));
}

int fp4idx_peak_mfma_valu(int32_t mode, int32_t iterations, float* sink, void* stream) {
  const TimingScope timing_scope;
  if (mode < 0 || mode > 2 || iterations < 1 || !sink) return FP4IDX_E_INVALID;
  const int dev = check_device();
  if (dev != FP4IDX_OK) return dev;
  return launched(fp4idx::launch_peak_mix(mode, iterations, sink, static_cast<hipStream_t>(stream)));
}

int fp4idx_peak_read(const uint8_t* buf, int64_t bytes, uint32_t* sink, void* stream) {
  const TimingScope timing_scope;
  if (bytes <= 0 || (bytes % 16) != 0 || !buf || !sink || !aligned(buf, 16)) return FP4IDX_E_INVALID;
  const int dev = check_device();
  if (dev != FP4IDX_OK) return dev;
  return launched(fp4idx::launch_peak_read(buf, bytes, sink, static_cast<hipStream_t>(stream)));
}

int fp4idx_topk(const float* logits, int64_t n_rows, int64_t logits_stride, const int32_t* row_ctx_len, int32_t k,
                int32_t* out_idx, void* stream) {
  return fp4idx_topk_bounded(logits, n_rows, logits_stride, row_ctx_len, k, out_idx, logits_stride, stream);
}

int fp4idx_topk_bounded(const float* logits, int64_t n_rows, int64_t logits_stride, const int32_t* row_ctx_len,
                        int32_t k, int32_t* out_idx, int64_t max_ctx, void* stream) {
  const TimingScope timing_scope;
  if (n_rows < 0 || logits_stride < 0 || max_ctx < 0 || max_ctx > logits_stride) return FP4IDX_E_INVALID;
  if (k < 1 || k > FP4IDX_MAX_TOPK) return FP4IDX_E_INVALID;
  if (max_ctx > 0x7FFFFFFF) return FP4IDX_E_INVALID;
  if (n_rows == 0) return FP4IDX_OK;
  if (!logits || !row_ctx_len || !out_idx) return FP4IDX_E_INVALID;
  if (n_rows > 0x7FFFFFFF) return FP4IDX_E_INVALID;
  const int dev = check_device();
  if (dev != FP4IDX_OK) return dev;
  return launched(fp4idx::launch_topk(logits, n_rows, logits_stride, row_ctx_len, k, out_idx, max_ctx,
                                      static_cast<hipStream_t>(stream)));
}

/* ---- FP8 cache ---------------------------------------------------------- */

int fp4idx_write_k_fp8(const uint16_t* k_bf16, int64_t n_tokens, int64_t k_row_stride, const int32_t* pos,
                       const int32_t* slot, const uint16_t* norm_w_bf16, float eps, const uint16_t* cos_sin_bf16,
                       int32_t max_pos, uint8_t* pool, int64_t num_pages, void* stream) {
  const TimingScope timing_scope;
  const int rc = check_write_k(k_bf16, n_tokens, k_row_stride, pos, slot, norm_w_bf16, eps, cos_sin_bf16, max_pos,
                               pool, pool, num_pages);
  if (rc != FP4IDX_OK || n_tokens == 0) return rc;
  const int dev = check_device();
  if (dev != FP4IDX_OK) return dev;
  return launched(fp4idx::launch_write_k_fp8(k_bf16, n_tokens, k_row_stride, pos, slot, norm_w_bf16, eps,
                                             cos_sin_bf16, max_pos, pool, num_pages,
                                             static_cast<hipStream_t>(stream)));
}

int fp4idx_pack_q_fp8(const uint16_t* q_bf16, int64_t n_rows, int32_t n_heads, int64_t q_row_stride,
                      const int32_t* pos, const uint16_t* cos_sin_bf16, int32_t max_pos, const float* w_in,
                      float w_scale, uint8_t* q_fp8, float* q_scale, float* w_out, void* stream) {
  const TimingScope timing_scope;
  const int rc = check_pack_q(q_bf16, n_rows, n_heads, q_row_stride, pos, cos_sin_bf16, max_pos, w_in, q_fp8,
                              reinterpret_cast<const uint8_t*>(q_scale), w_out);
  if (rc != FP4IDX_OK || n_rows == 0) return rc;
  const int dev = check_device();
  if (dev != FP4IDX_OK) return dev;
  return launched(fp4idx::launch_pack_q_fp8(q_bf16, n_rows, n_heads, q_row_stride, pos, cos_sin_bf16, max_pos, w_in,
                                            w_scale, q_fp8, q_scale, w_out, static_cast<hipStream_t>(stream)));
}

int fp4idx_write_k_pack_q_fp8(const uint16_t* k_bf16, int64_t n_tokens, int64_t k_row_stride, const int32_t* pos_k,
                              const int32_t* slot, const uint16_t* norm_w_bf16, float eps,
                              const uint16_t* cos_sin_bf16, int32_t max_pos, uint8_t* pool, int64_t num_pages,
                              const uint16_t* q_bf16, int64_t n_rows, int32_t n_heads, int64_t q_row_stride,
                              const int32_t* pos_q, const float* w_in, float w_scale, uint8_t* q_fp8,
                              float* q_scale, float* w_out, void* stream) {
  const TimingScope timing_scope;
  int rc = check_write_k(k_bf16, n_tokens, k_row_stride, pos_k, slot, norm_w_bf16, eps, cos_sin_bf16, max_pos, pool,
                         pool, num_pages);
  if (rc != FP4IDX_OK) return rc;
  rc = check_pack_q(q_bf16, n_rows, n_heads, q_row_stride, pos_q, cos_sin_bf16, max_pos, w_in, q_fp8,
                    reinterpret_cast<const uint8_t*>(q_scale), w_out);
  if (rc != FP4IDX_OK) return rc;
  if (n_tokens == 0 && n_rows == 0) return FP4IDX_OK;
  const int dev = check_device();
  if (dev != FP4IDX_OK) return dev;
  return launched(fp4idx::launch_write_k_pack_q_fp8(k_bf16, n_tokens, k_row_stride, pos_k, slot, norm_w_bf16, eps,
                                                    cos_sin_bf16, max_pos, pool, num_pages, q_bf16, n_rows, n_heads,
                                                    q_row_stride, pos_q, w_in, w_scale, q_fp8, q_scale, w_out,
                                                    static_cast<hipStream_t>(stream)));
}

int fp4idx_mqa_logits_fp8(const uint8_t* q_fp8, const float* q_scale, const float* w, int64_t n_rows,
                          int32_t n_heads, const int32_t* req_row_indptr, int32_t n_reqs, const int32_t* row_ctx_len,
                          const int32_t* block_table, int32_t bt_stride, const uint8_t* pool, int64_t num_pages,
                          float* logits, int64_t logits_stride, int32_t max_rows_per_req, int64_t max_ctx,
                          void* stream) {
  const TimingScope timing_scope;
  int rc = check_logits(n_rows, n_heads, n_reqs, bt_stride, num_pages, logits_stride, max_rows_per_req, max_ctx);
  if (rc != FP4IDX_OK || n_rows == 0 || n_reqs == 0 || max_ctx == 0 || max_rows_per_req == 0) return rc;
  if (!q_fp8 || !q_scale || !w || !req_row_indptr || !row_ctx_len || !block_table || !pool || !logits)
    return FP4IDX_E_INVALID;
  if (!aligned(q_fp8, 16) || !aligned(q_scale, 4) || !aligned(w, 16) || !aligned(pool, 16)) return FP4IDX_E_INVALID;
  const int dev = check_device();
  if (dev != FP4IDX_OK) return dev;
  return launched(fp4idx::launch_mqa_logits_fp8(q_fp8, q_scale, w, n_rows, n_heads, req_row_indptr, n_reqs, row_ctx_len,
                                                block_table, bt_stride, pool, num_pages, logits, logits_stride,
                                                max_rows_per_req, max_ctx, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
