// The plan kernel: the batch's work items for the scheduled logits kernels.
//
// One work-group of 1,024 threads (its registers and LDS do not depend on
// the batch: the per-request list lives in the workspace, and so does the
// per-block list beyond the first 1,024 blocks; the first 1,024 blocks'
// working set stays in registers):
//  1. blocks per request: a request of R rows (its indptr range, clamped
//     into [0, n_rows]) becomes ceil(R / rows) row blocks, its rows spread
//     evenly over them; a block scan gives each request its first block.
//  2. per block: the longest context among its rows (cut to the plan's
//     bound) gives its pages P, and the block's work is P times the work of
//     a page (for the shared-page kernel: staging it plus scoring the
//     busiest wave's rows); the batch's work W is their sum.
//  3. per block, its chunks.  Per-wave items have a fixed length (the work-
//     group's four waves' pages).  Shared-page items: large chunks of about
//     `target` units of work first, then the rest of the block in chunks a
//     quarter as long; the share of pages in short chunks is the work of one
//     round of the device's resident work-groups over W (at least the
//     remainder of the large chunks).  Block scans of the two counts place
//     every block's large items in one list and its short items in a second
//     list that follows the first.
//  4. the items: for the shared-page kernel each list cut into eight
//     contiguous ranges, one per XCD, stored interleaved (item x + 8k is
//     the k-th of XCD x's list; see below), for per-wave items in plain
//     order; written coalesced (thread t builds items t, t + 1,024, ...)
//     for up to 128 row blocks, else by one thread per block.
// The logits kernel's work-groups take the items in list order, so the
// hardware's dispatch keeps every CU busy while large items remain and the
// list ends with short ones that fill the tail.  Context lengths of up to
// 4,096 rows and the row ranges of up to 4,096 requests are staged in LDS.  The item count never
// exceeds the workspace's capacity: a block gets at most capacity / blocks
// items (its chunks grow instead, and a per-wave block's pages past them are
// not scored), which contexts within the workspace's bound never need.
#include <algorithm>

#include "launch.hpp"
#include "schedule.hpp"
#include "topk_core.hpp"

namespace fp4idx {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kPlanLdsReqs = 4096;  // request offsets searched in LDS up to this many requests
constexpr int kPlanTiles = 1;       // tiles of blocks whose working set stays in registers
constexpr int kPlanBlockRows = 8;   // most rows of a row block (the kernels' shapes)
constexpr int kPlanCoalescedBlocks = 128;  // batches of up to this many blocks write items coalesced
constexpr int kPlanLdsRows = 4096;         // context lengths staged in LDS up to this many rows

// A block's plan: its request, first row and rows, its pages, and its large
// and short chunks (length, count, first item of each kind).
struct BlockPlan {
  int b, r0, nr, P, Lb, nbig, Ls, nsmall, fb, fs;
};

// Exclusive prefix of v over the work-group; total gets the sum.  Ends with
// the work-group in step (its scratch may be reused right away).
__device__ __forceinline__ int plan_scan(int v, int lane, int wave, uint32_t* part, int& total) {
  const int excl = (int)block_excl_scan<kPlanWaves>((uint32_t)v, lane, wave, part);
  int t = 0;
#pragma unroll
  for (int i = 0; i < kPlanWaves; ++i) t += (int)part[i];
  total = t;
  __syncthreads();
  return excl;
}

// Sum of v over the 64 lanes in a fixed order (result uniform): DPP within
// each 16-lane row, then the four rows' sums in turn.
__device__ __forceinline__ float plan_wave_sum(float v) {
  v += __uint_as_float(dppu<kQpXor1>(__float_as_uint(v)));
  v += __uint_as_float(dppu<kQpXor2>(__float_as_uint(v)));
  v += __uint_as_float(dppu<kRowHalfMirror>(__float_as_uint(v)));
  v += __uint_as_float(dppu<kRowMirror>(__float_as_uint(v)));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return ((r0 + r1) + r2) + r3;
}

struct PlanParams {
  const int32_t* indptr;
  int32_t n_reqs;
  int32_t n_rows;
  const int32_t* row_ctx;
  int32_t ctx_cap;
  int32_t* ws;
  int32_t cap_items;
  int64_t req_off, blk_off, items_off;
  int32_t max_blocks;
  int32_t rows_per_block;
  int32_t waves;      // 0: per-wave items
  int32_t fixed;      // pages of a per-wave item
  int32_t target;     // work of a large shared-page item
  int32_t resident;   // work-groups the device holds at once
};

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanParams p) {
  __shared__ uint32_t part[kPlanWaves];
  __shared__ int32_t first_lds[kPlanLdsReqs + 1];
  __shared__ int32_t ip0_lds[kPlanLdsReqs], ip1_lds[kPlanLdsReqs];  // each request's clamped row range
  __shared__ float s_wsum[kPlanWaves];  // the waves' sums of their blocks' work
  __shared__ int32_t ctx_lds[kPlanLdsRows];  // the rows' context lengths (batches of up to kPlanLdsRows rows)
  // per-block plans for the coalesced item writer (batches of up to
  // kPlanCoalescedBlocks row blocks): first large and short item, request,
  // first row, rows, pages, large and short chunk lengths
  __shared__ int32_t s_blk[8][kPlanCoalescedBlocks];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t* req_first = p.ws + p.req_off;
  int32_t* blk = p.ws + p.blk_off;
  int4* items = reinterpret_cast<int4*>(p.ws + p.items_off);
  const int rows_pb = p.rows_per_block;
  auto rows_of = [&](int b, int& ip0, int& ip1) {
    ip0 = min(max(p.indptr[b], 0), p.n_rows);
    ip1 = min(max(p.indptr[b + 1], ip0), p.n_rows);
  };
  // Every row's context length (cut to the plan's bound), loaded in the
  // same round trip as indptr when the batch has at most kPlanLdsRows rows
  // (the blocks then read them from LDS); stored after pass 1's barriers.
  const bool ctx_in_lds = p.n_rows <= kPlanLdsRows;
  int32_t ctx_pre[kPlanLdsRows / kPlanThreads];
  if (ctx_in_lds) {
#pragma unroll
    for (int k = 0; k < kPlanLdsRows / kPlanThreads; ++k) {
      const int r = tid + k * kPlanThreads;
      ctx_pre[k] = r < p.n_rows ? p.row_ctx[r] : 0;
    }
  }

  // 1. row blocks per request, and each request's first block
  int nb = 0;
  for (int base = 0; base < p.n_reqs; base += kPlanThreads) {
    const int b = base + tid;
    int cnt = 0, ip0 = 0, ip1 = 0;
    if (b < p.n_reqs) {
      rows_of(b, ip0, ip1);
      cnt = (ip1 - ip0 + rows_pb - 1) / rows_pb;
    }
    int tile = 0;
    const int first = nb + plan_scan(cnt, lane, wave, part, tile);
    if (b < p.n_reqs) {
      req_first[b] = first;
      if (b < kPlanLdsReqs) {
        first_lds[b] = first;
        ip0_lds[b] = ip0;
        ip1_lds[b] = ip1;
      }
    }
    nb += tile;
  }
  if (ctx_in_lds) {
#pragma unroll
    for (int k = 0; k < kPlanLdsRows / kPlanThreads; ++k) {
      const int r = tid + k * kPlanThreads;
      if (r < p.n_rows) ctx_lds[r] = min(max(ctx_pre[k], 0), p.ctx_cap);
    }
  }
  // more blocks than rows make only overlapping request ranges (a broken
  // indptr): the blocks past the bound are not scheduled
  nb = min(nb, p.max_blocks);
  if (tid == 0) {
    req_first[p.n_reqs] = nb;
    if (p.n_reqs < kPlanLdsReqs) first_lds[p.n_reqs] = nb;
  }
  __syncthreads();
  const bool in_lds = p.n_reqs < kPlanLdsReqs;
  // the request holding block g: the last b with first[b] <= g (requests
  // without rows share their successor's first block and are skipped)
  auto request_of = [&](int g) {
    int lo = 0, hi = p.n_reqs;  // first[lo] <= g < first[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      const int f = in_lds ? first_lds[mid] : req_first[mid];
      if (f <= g) lo = mid;
      else hi = mid;
    }
    return lo;
  };
  auto busiest_rows = [&](int nr) { return p.waves > 0 ? (nr + p.waves - 1) / p.waves : nr; };

  // Per-block working set: in registers for the first kPlanTiles tiles of
  // kPlanThreads blocks, in the workspace's per-block list beyond them.
  BlockPlan reg[kPlanTiles];
  // f(g, e) for every block g (g >= nb: a thread without a block, which
  // still takes part in the scans); tiles in order, work-group uniform
  auto visit = [&](auto&& f) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < kPlanTiles; ++k)
      if (k * kPlanThreads < nb) f(k * kPlanThreads + tid, reg[k]);
    for (int base = kPlanTiles * kPlanThreads; base < nb; base += kPlanThreads) {
      const int g = base + tid;
      int32_t* ep = blk + (int64_t)kBlkWords * g;
      BlockPlan e{};
      if (g < nb) e = BlockPlan{ep[0], ep[1], ep[2], ep[3], ep[4], ep[5], ep[6], ep[7], ep[8], ep[9]};
      f(g, e);
      if (g < nb) {
        ep[0] = e.b; ep[1] = e.r0; ep[2] = e.nr; ep[3] = e.P; ep[4] = e.Lb;
        ep[5] = e.nbig; ep[6] = e.Ls; ep[7] = e.nsmall; ep[8] = e.fb; ep[9] = e.fs;
      }
    }
  };

  // 2. per block: request, rows, pages; the batch's work
  float work = 0.0f;
  visit([&](int g, BlockPlan& e) __attribute__((always_inline)) {
    if (g >= nb) return;
    const int b = request_of(g);
    int ip0, ip1;
    if (in_lds) {
      ip0 = ip0_lds[b];
      ip1 = ip1_lds[b];
    } else {
      rows_of(b, ip0, ip1);
    }
    const int R = ip1 - ip0;
    const int nblk = (R + rows_pb - 1) / rows_pb;
    const int i = g - (in_lds ? first_lds[b] : req_first[b]);
    int r0 = ip0, nr = 0, cmax = 0;
    if (i >= 0 && i < nblk) {  // always, for the request the search finds
      r0 = ip0 + (int)((int64_t)i * R / nblk);
      const int r1 = ip0 + (int)((int64_t)(i + 1) * R / nblk);
      nr = r1 - r0;
      // the block's context lengths, all in flight together (a block has at
      // most kPlanBlockRows rows; the loop after it only guards the bound)
      if (ctx_in_lds) {
        for (int r = r0; r < r1; ++r) cmax = max(cmax, ctx_lds[r]);
      } else {
        int c[kPlanBlockRows];
#pragma unroll
        for (int k = 0; k < kPlanBlockRows; ++k) c[k] = k < nr ? p.row_ctx[r0 + k] : 0;
#pragma unroll
        for (int k = 0; k < kPlanBlockRows; ++k) cmax = max(cmax, min(max(c[k], 0), p.ctx_cap));
        for (int r = r0 + kPlanBlockRows; r < r1; ++r) cmax = max(cmax, min(max(p.row_ctx[r], 0), p.ctx_cap));
      }
    }
    e.b = b;
    e.r0 = r0;
    e.nr = nr;
    e.P = (cmax + 63) >> 6;
    work += (float)e.P * (float)(kStagePageCost + busiest_rows(nr) * kRowPageCost);
  });
  // share of each shared-page block's pages in short chunks, from the
  // batch's work summed in a fixed order (within each wave, then the waves
  // in turn), so that one batch always gets the same plan; per-wave items
  // (work-group uniform) have no short ones
  float short_share = 0.0f;
  if (p.waves > 0) {
    const float wsum = plan_wave_sum(work);
    if (lane == 0) s_wsum[wave] = wsum;
    __syncthreads();
    float total = 0.0f;
#pragma unroll
    for (int i = 0; i < kPlanWaves; ++i) total += s_wsum[i];
    short_share = fminf(1.0f, 0.01f * (float)kShortRoundsX100 * (float)p.resident * (float)p.target /
                                  fmaxf(total, 1.0f));
  }

  // 3. chunks per block; large items first, then the short ones
  const int chunk_cap = nb > 0 ? max(1, p.cap_items / nb) : 1;
  int n_big = 0, n_small = 0;
  visit([&](int g, BlockPlan& e) __attribute__((always_inline)) {
    int nbig = 0, nsmall = 0;
    if (g < nb) {
      int P = e.P;
      int Lb = 1, Ls = 1;
      if (P > 0) {
        if (p.waves == 0) {
          Lb = p.fixed;
          nbig = min((P + Lb - 1) / Lb, chunk_cap);
          P = min(P, nbig * Lb);  // pages past the workspace's bound are not scored
        } else {
          Lb = plan_big_pages(p.target, busiest_rows(e.nr));
          Ls = plan_small_pages(Lb);
          const int short_pages = min(P, (int)ceilf(short_share * (float)P));
          nbig = (P - short_pages) / Lb;
          const int rest = P - nbig * Lb;
          nsmall = (rest + Ls - 1) / Ls;
          if (nsmall > 0) Ls = (rest + nsmall - 1) / nsmall;  // even short chunks
          if (nbig + nsmall > chunk_cap) {  // a workspace below the contexts' size: fewer, longer chunks
            const int nch = min(chunk_cap, (P + Lb - 1) / Lb);
            Lb = (P + nch - 1) / nch;
            if (Lb > kMaxItemPages) {
              Lb = kMaxItemPages;
              P = nch * Lb;
            }
            nbig = (P + Lb - 1) / Lb;
            nsmall = 0;
          }
        }
      }
      e.P = P;
      e.Lb = Lb;
      e.nbig = nbig;
      e.Ls = Ls;
      e.nsmall = nsmall;
    }
    int tb = 0, ts = 0;
    e.fb = n_big + plan_scan(nbig, lane, wave, part, tb);
    e.fs = n_small + (p.waves > 0 ? plan_scan(nsmall, lane, wave, part, ts) : 0);  // per-wave items: no short ones
    n_big += tb;
    n_small += ts;
  });

  // 4. the items.  Work-group i of the run goes to XCD i mod 8 (the
  // hardware's round-robin dispatch), and each XCD has its own L2: so the
  // large list is cut into eight contiguous ranges, one per XCD, and so is
  // the short list, and XCD x's large items, then its short ones, go to
  // indices x, x + 8, x + 16, ...  A row block's chunks are consecutive in
  // the lists, so they share an XCD (and its cached Q rows and pages) except
  // at a range boundary, and every XCD still gets large items first and
  // short ones last.  Indices no XCD fills (the ranges differ by one item at
  // most) get empty items.  A workspace without room for those (at most 16)
  // keeps the lists in plain order, and so do per-wave items (each reads its
  // own pages once; the shared Q row is a few KiB).
  const bool spread = p.waves > 0 && (int64_t)n_big + n_small + kXcdSlack <= p.cap_items &&
                      n_big + n_small < (1 << 27);  // so n * 8 + 7 fits in 32 bits
  auto first_of = [](int n, int x) { return (n * x + 7) >> 3; };  // XCD x's first of n
  // writes a block's `cnt` chunks, the list's items gi0 .. gi0 + cnt - 1 (of
  // n, after `before` items of the XCD's earlier list): the XCD of the first
  // from the list position, then stepping to the next XCD at each range end
  auto put = [&](int gi0, int cnt, int n, bool small, auto&& item_of) __attribute__((always_inline)) {
    if (cnt <= 0) return;
    if (!spread) {
      for (int c = 0; c < cnt; ++c) items[(small ? n_big : 0) + gi0 + c] = item_of(c);
      return;
    }
    int x = 0;
    while (x < 7 && first_of(n, x + 1) <= gi0) ++x;
    int next = first_of(n, x + 1);
    int base = first_of(n, x) - (small ? first_of(n_big, x + 1) - first_of(n_big, x) : 0);
    for (int c = 0; c < cnt; ++c) {
      const int gi = gi0 + c;
      while (gi >= next) {  // the next XCD's range
        ++x;
        next = first_of(n, x + 1);
        base = first_of(n, x) - (small ? first_of(n_big, x + 1) - first_of(n_big, x) : 0);
      }
      items[x + 8 * (gi - base)] = item_of(c);
    }
  };
  if (nb <= kPlanCoalescedBlocks) {
    // Coalesced writer: the blocks' plans go to LDS, then thread t builds
    // items t, t + 1,024, ... of the final order, finding each item's
    // block by a binary search over the blocks' first items.  For few
    // blocks it beats one thread per block writing its chunks in turn
    // (mixed batch, 70 blocks of about 42 items: plan 13.4 -> 10.9 us); for
    // hundreds of blocks the searches cost more than the short per-block
    // chains (prefill, 512 blocks: 14.6 -> 18.9 us), so those keep the
    // per-block writer.
    if (tid < nb) {
      const BlockPlan& e = reg[0];
      s_blk[0][tid] = e.fb;
      s_blk[1][tid] = e.fs;
      s_blk[2][tid] = e.b;
      s_blk[3][tid] = e.r0;
      s_blk[4][tid] = e.nr;
      s_blk[5][tid] = e.P;
      s_blk[6][tid] = e.Lb;
      s_blk[7][tid] = e.Ls;
    }
    __syncthreads();
    // the block holding item gi of the large (k = 0) or short (k = 1) list:
    // the last block whose first item is <= gi (blocks without items of
    // that kind share their successor's first item)
    auto block_of = [&](int k, int gi) {
      int lo = 0, hi = nb;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_blk[k][mid] <= gi) lo = mid;
        else hi = mid;
      }
      return lo;
    };
    int total = n_big + n_small;
    if (spread) {
      int longest = 0;
      for (int x = 0; x < 8; ++x)
        longest = max(longest, first_of(n_big, x + 1) - first_of(n_big, x) + first_of(n_small, x + 1) -
                                   first_of(n_small, x));
      total = 8 * longest;
    }
    for (int i = tid; i < total; i += kPlanThreads) {
      int gi = i;  // index in the plain order: large list, then short list
      if (spread) {
        const int x = i & 7, pos = i >> 3;
        const int nbx = first_of(n_big, x + 1) - first_of(n_big, x);
        const int nsx = first_of(n_small, x + 1) - first_of(n_small, x);
        gi = pos < nbx ? first_of(n_big, x) + pos : pos < nbx + nsx ? n_big + first_of(n_small, x) + pos - nbx : -1;
      }
      int4 it = make_int4(0, 0, 0, 0);  // an empty item
      if (gi >= 0) {
        const bool small = gi >= n_big;
        const int li = small ? gi - n_big : gi;
        const int g = block_of(small ? 1 : 0, li);
        const int c = li - s_blk[small ? 1 : 0][g];
        const int L = s_blk[small ? 7 : 6][g], P = s_blk[5][g];
        // a short chunk follows the block's large ones
        const int nbig_g = (g + 1 < nb ? s_blk[0][g + 1] : n_big) - s_blk[0][g];
        const int p0 = small ? nbig_g * s_blk[6][g] + c * L : c * L;
        it = make_int4(s_blk[2][g], s_blk[3][g], p0, s_blk[4][g] | (min(L, P - p0) << 8));
      }
      items[i] = it;
    }
  } else {
  visit([&](int g, BlockPlan& e) __attribute__((always_inline)) {
    if (g >= nb) return;
    put(e.fb, e.nbig, n_big, false, [&](int c) {
      const int p0 = c * e.Lb;
      return make_int4(e.b, e.r0, p0, e.nr | (min(e.Lb, e.P - p0) << 8));
    });
    const int s0 = e.nbig * e.Lb;
    put(e.fs, e.nsmall, n_small, true, [&](int c) {
      const int p0 = s0 + c * e.Ls;
      return make_int4(e.b, e.r0, p0, e.nr | (min(e.Ls, e.P - p0) << 8));
    });
  });
  }
  int n_items = n_big + n_small;
  if (spread) {
    int longest = 0;
    for (int x = 0; x < 8; ++x)
      longest = max(longest, first_of(n_big, x + 1) - first_of(n_big, x) + first_of(n_small, x + 1) -
                                 first_of(n_small, x));
    n_items = 8 * longest;
    if (nb > kPlanCoalescedBlocks && tid < 8) {  // the empty items of XCD tid
      const int len = first_of(n_big, tid + 1) - first_of(n_big, tid) + first_of(n_small, tid + 1) -
                      first_of(n_small, tid);
      for (int pos = len; pos < longest; ++pos) items[tid + 8 * pos] = make_int4(0, 0, 0, 0);
    }
  }
  if (tid == 0) {
    p.ws[kHdrItems] = min(n_items, p.cap_items);
    p.ws[1] = 0;
    p.ws[2] = 0;
    p.ws[kHdrCap] = p.cap_items;
    p.ws[kHdrRows] = rows_pb;
    p.ws[kHdrWaves] = p.waves;
    p.ws[kHdrFixed] = p.fixed;
  }
}

hipError_t launch_plan(const int32_t* indptr, int32_t n_reqs, int64_t n_rows, const int32_t* row_ctx,
                       int64_t max_ctx, int32_t* ws, int64_t cap_items, const PlanSizes& sz, const PlanShape& sh,
                       int fixed, int target, int resident, hipStream_t stream) {
  if (n_rows > 0x7FFFFFFFLL || cap_items > 0x7FFFFFFFLL || cap_items < sz.blocks) return hipErrorInvalidConfiguration;
  const PlanParams p{indptr, n_reqs, (int32_t)n_rows, row_ctx, (int32_t)std::min<int64_t>(max_ctx, 0x7FFFFFFFLL),
                     ws, (int32_t)cap_items, sz.req_off, sz.blk_off, sz.items_off, (int32_t)sz.blocks, sh.rows,
                     sh.waves, fixed, target, resident};
  return launch(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, p);
}

}  // namespace fp4idx
