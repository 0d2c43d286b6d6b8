// The device-built work schedule of the multi-row logits (FP4 cache).
//
// "dsv4.1-amd: KV cache layouts, FP4 indexer, compressor and router kernels"
// (Summary) builds the indexer's decode schedule on the device, in two
// dispatches whose registers do not grow with the row count; "[AMD] Enable
// FP4 indexer for Deepseek V4" (Modifications / Attention runtime) builds
// decode schedules during graph capture and reuses page tables and schedules
// across every compressed-attention layer of a step.  Here: one plan kernel
// (a single work-group, its working set in the caller's workspace, so its
// registers and LDS do not depend on the batch) turns the batch's row split
// and context lengths into a list of work items, and the logits kernels run
// one item per work-group (work-groups past the list's length exit at once).  The plan depends on nothing but
// the batch (indptr, context lengths, head count), so one plan serves every
// layer of a step and every replay of a captured step.
//
// Workspace layout (int32 words, 16-byte aligned):
//   header  [kHdrWords]: n_items, 0, 0, capacity, rows per block, waves
//           per block (0: per-wave items), pages of a per-wave item
//   per request: its first row block            [n_reqs + 1, padded to 4]
//   per block: kBlkWords words (request, first row, rows, pages, large and
//              short chunk lengths and counts, the first large and the first
//              short item)                       [most blocks x 10, padded]
//   items: int4 {request, first row, first page, rows | pages << 8}, as many
//          as the rest of the workspace holds; in per-XCD order (item x + 8k
//          is the k-th of XCD x's list), empty items (all zero) evening out
//          the lists
// Item: rows [row0, row0 + rows) of one request (rows <= the kernel's rows
// per work-group) and pages [page0, page0 + pages) of its block table
// (pages <= kMaxItemPages).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4idx {

constexpr int kHdrWords = 16;       // 64-byte header
constexpr int kMaxItemPages = 512;  // page ids one work-group stages in LDS
constexpr int kMinItemPages = 4;    // the shortest chunk the plan makes

// Items a plan may add to a batch's chunks: the empty items that even out
// the eight per-XCD lists (two per XCD at most).
constexpr int kXcdSlack = 16;

enum HdrWord { kHdrItems = 0, kHdrCap = 3, kHdrRows = 4, kHdrWaves = 5, kHdrFixed = 6 };
constexpr int kBlkWords = 10;

// Work units of the plan's cost model: scoring one page for one row, and
// staging one page in LDS (shared-page kernel).
constexpr int kRowPageCost = 8, kStagePageCost = 2;

// Large chunk of a shared-page block whose busiest wave scores `busiest`
// rows: about `target` units of work.
inline __host__ __device__ int plan_big_pages(int target, int busiest) {
  const int per_page = kStagePageCost + busiest * kRowPageCost;
  const int L = (target + per_page - 1) / per_page;
  return L < kMinItemPages ? kMinItemPages : (L > kMaxItemPages ? kMaxItemPages : L);
}

// The schedule's tuning constants (compile-time; overridable with -D for
// measurement builds): the work of a large shared-page item, the work of
// the short items at the end of the list in rounds of the device's resident
// work-groups (x 100), and the large-to-short chunk ratio.
#ifndef FP4IDX_ITEM_TARGET
#define FP4IDX_ITEM_TARGET 576
#endif
#ifndef FP4IDX_SHORT_ROUNDS_X100
#define FP4IDX_SHORT_ROUNDS_X100 100
#endif
#ifndef FP4IDX_SHORT_DIVISOR
#define FP4IDX_SHORT_DIVISOR 4
#endif
constexpr int kItemTarget = FP4IDX_ITEM_TARGET;
constexpr int kShortRoundsX100 = FP4IDX_SHORT_ROUNDS_X100;
constexpr int kShortDivisor = FP4IDX_SHORT_DIVISOR;

// Short chunk: a fraction of the large one.
inline __host__ __device__ int plan_small_pages(int big) {
  const int L = big / kShortDivisor;
  return L < kMinItemPages ? kMinItemPages : L;
}

// Sizes for a batch of n_rows rows in n_reqs requests when the kernel takes
// `rows` rows per work-group.
struct PlanSizes {
  int64_t blocks;     // most row blocks any such batch has
  int64_t req_off;    // word offset of the per-request list
  int64_t blk_off;    // word offset of the per-block list
  int64_t items_off;  // word offset of the items
};

inline PlanSizes plan_sizes(int64_t n_rows, int64_t n_reqs, int rows) {
  PlanSizes s{};
  // sum_b ceil(R_b / rows) with sum_b R_b = n_rows: at most one partial
  // block per request that has rows
  const int64_t nonempty = n_reqs < n_rows ? n_reqs : n_rows;
  int64_t blocks = nonempty > 0 ? (n_rows + nonempty * (rows - 1)) / rows : 0;
  if (blocks > n_rows) blocks = n_rows;
  s.blocks = blocks;
  s.req_off = kHdrWords;
  s.blk_off = s.req_off + ((n_reqs + 1 + 3) & ~int64_t(3));
  s.items_off = s.blk_off + ((kBlkWords * blocks + 3) & ~int64_t(3));
  return s;
}

// The kernel a plan is made for: the shared-page kernel with `waves` waves
// and `rows` rows per work-group, or (waves 0) the per-wave kernel with
// `rows` rows per wave.
struct PlanShape {
  int waves;
  int rows;
};

// Items a workspace of `bytes` holds (negative: not even the lists fit).
inline int64_t plan_capacity(const PlanSizes& s, int64_t bytes) { return (bytes / 4 - s.items_off) / 4; }

// Items per block a plan of this shape makes at most for contexts of
// `pages` pages (`fixed`: the pages of a per-wave item; `target`: the
// shared-page item work).
inline int64_t plan_items_per_block(const PlanShape& sh, int64_t pages, int fixed, int target) {
  if (pages <= 0) return 1;
  if (sh.waves == 0) return (pages + fixed - 1) / fixed;
  const int small = plan_small_pages(plan_big_pages(target, (sh.rows + sh.waves - 1) / sh.waves));
  return (pages + small - 1) / small + 1;
}

// Workspace bytes a plan of this shape needs for contexts of at most max_ctx.
inline int64_t plan_bytes(const PlanShape& sh, int64_t n_rows, int64_t n_reqs, int64_t max_ctx, int fixed,
                          int target) {
  const PlanSizes s = plan_sizes(n_rows, n_reqs, sh.rows);
  return 4 * (s.items_off + 4 * (s.blocks * plan_items_per_block(sh, (max_ctx + 63) / 64, fixed, target) + kXcdSlack));
}

}  // namespace fp4idx
