// Paged-MQA indexer logits on gfx950 block-scaled MFMA, for the FP4 cache
// (split payload/scale pools) and the FP8 cache (one fused pool).
//
// Score (DeepSeek lightning indexer, as the FP4 indexer of "[AMD] Enable FP4
// indexer for Deepseek V4" computes it over the split payload/scale cache,
// and the FP8 indexer it replaces over its fused 132-byte tokens):
//   logits[t][s] = sum_h w[t][h] * ReLU( qhat[t][h] . khat[s] )
//
// One kernel template serves both caches; a format type (Fp4Split, Fp8Fused
// below) supplies the page loads, the Q operand and the MFMA form, and
// everything else (work split, prefetch, epilogue) is shared.
//
// Work decomposition
//   work-group (256 threads = 4 waves) = (request, group of up to RW rows,
//   chunk of 4*PPW pages), a 3-D grid with each request's chunks rotated
//   across the XCDs; wave w takes PPW consecutive pages of the chunk.
//   Every wave keeps its rows' packed Q (the MFMA A operand) and head weights
//   in registers and streams K pages: per 16-token tile each lane loads 16
//   payload bytes (one 128-bit load; the 64 lanes read 4 runs of 256 B) and
//   one scale byte (Fp8Fused: 32 code bytes in two 128-bit loads, and a
//   scale word), straight into the B operand.  D pages are in flight per
//   wave; the page ids and Q are requested before the context lengths
//   arrive so the prologue costs one memory latency less.
//   Batches with three or more rows per request on average (either cache)
//   use mqa_logits_shared_kernel instead: its waves split a block of rows
//   and share each page through LDS (see that kernel); FP8 batches of one or
//   two rows per request use it too, with one-wave work-groups, because an
//   FP8 token's code bytes are one 128-byte row and direct operand loads
//   would read half lines.
//
// MFMA mapping for FP4 (V_MFMA_SCALE_F32_16X16X128_F8F6F4, both operands
// e2m1; FP8 in Fp8Fused below):
//   A (16 x 128) = 16 heads of one query row; lane l holds head l%16, K
//   elements 32*(l/16)..+31 and that block's UE8M0 scale (byte mt of a packed
//   scale register, picked by op_sel).  B (128 x 16) = 16 tokens; lane l holds
//   token l%16, block l/16, i.e. exactly the 16-byte payload chunk at
//   [page][block l/16][token][0..15] and the scale byte [page][block][token]:
//   the page layout feeds the MFMA without any shuffle.
//   D (16 x 16, fp32): lane l holds token l%16, heads 4*(l/16)+i, i = 0..3.
// Epilogue per lane and row: for each of the page's 4 tiles, p_t = sum over
// the row's M-tiles and i of w * ReLU(d) (one fixed-order FMA chain), then
// the four lane groups of the four tiles are summed
// together with two permlane swap steps that leave tile t's total for token
// l%16 in lane 16*t + l%16, i.e. the page's 64 logits in lane order, stored
// as one 256-byte row segment.
// Each (row, token) is computed by exactly one lane in a fixed order, so the
// result does not depend on batch composition, page placement or grid shape.
#include <algorithm>

#include "launch.hpp"
#include "logits_core.hpp"
#include "store.hpp"
#include "schedule.hpp"

namespace fp4idx {

// A logits store: written once, read only by the next kernel (store.hpp).
__device__ __forceinline__ void store_logit(float* p, float v) { store_through(p, v); }

// RW rows per wave, NMT = heads/16, PPW pages per wave, D pages in flight.
// Few rows per wave (decode) means little work per wave: keep several waves
// per SIMD resident so memory latency overlaps (four for FP4; two for FP8,
// whose 36-register pages need the larger register budget for four pages in
// flight, the same bytes in flight per SIMD); more rows keep their register
// budget.
template <typename FMT, int RW, int NMT>
constexpr int kMinWavesPerSimd = NMT > 4 ? 1 : RW == 1 ? FMT::kWaves1 : RW == 2 ? FMT::kWaves2 : 1;

// The arguments every per-wave item needs.
struct WaveArgs {
  const int32_t* block_table;
  const int32_t* indptr;
  const int32_t* row_ctx;
  const uint8_t* payload;
  const uint8_t* scale;
  int64_t num_pages;
  int32_t bt_stride;
  const uint8_t* q_fp4;
  const uint8_t* q_scale;
  const float* w;
  float* logits;
  int64_t logits_stride;
  int32_t n_rows;
};

// One wave's share of a per-wave item: request req, pages [page_begin,
// page_end) of its block table (page_end - page_begin <= PPW), and the rows
// rows(row0, nrows) names once the wave's page ids are on their way (0 <=
// nrows <= RW, rows inside [0, n_rows); nrows 0 leaves).  Wave-uniform.
// EARLY_Q: rows() needs no memory read (the scheduled kernel), so the Q
// operands join round trip 1; otherwise (rows() reads indptr) they follow
// the first pages, which keeps their registers free while the row range is
// on its way.
template <typename FMT, int RW, int NMT, int PPW, int D, bool EARLY_Q, typename Rows>
__device__ __forceinline__ void wave_item(const WaveArgs& a, int req, int page_begin, int page_end, Rows rows) {
  static_assert(RW >= 1 && RW <= 4, "rows per wave");
  static_assert(PPW % D == 0 && PPW <= 64, "pages per wave: a multiple of the prefetch depth, one id per lane");
  constexpr int H = NMT * 16;
  constexpr int NSC = (NMT + 3) / 4;  // packed A-scale registers per row
  // one row per wave means one row group per request, so every page is read
  // once (non-temporal); with more rows, other row groups re-read the pages
  constexpr bool kPageNT = RW == 1;
  const int lane = threadIdx.x & 63;
  const int li = lane & 15;  // token within tile (B, D) / head within M-tile (A)
  const int lg = lane >> 4;  // K block (A, B) / head quad (D)
  const uint32_t lane_pay = FMT::lane_pay(li, lg);
  const uint32_t lane_sc = FMT::lane_sc(li, lg);
  const int bt_stride = a.bt_stride;
  const int64_t num_pages = a.num_pages;

  // Memory round trip 1: the wave's page ids (one vector load, lane i reads
  // entry i, clamped into the table), then, once rows() has the row range,
  // the context lengths (lane r reads row r) and the stationary Q operands
  // and weights, all in flight together.  No branch depends on them before
  // the pages are requested: an empty row group loads in-range rows and
  // leaves afterwards.
  const int32_t* bt = a.block_table + (int64_t)req * bt_stride;
  const int32_t my_pid = bt[min(page_begin + (lane % PPW), bt_stride - 1)];
  __builtin_amdgcn_sched_barrier(0);  // keep the load issued ahead of the row range
  int row0 = 0, nrows = 0;
  rows(row0, nrows);
  const int row_hi = max(0, min(row0 + nrows, a.n_rows) - 1);  // a valid row index to clamp to
  const int32_t my_ctx = a.row_ctx[min(row0 + (lane & 3), row_hi)];
  typename FMT::QOp aq[RW][NMT];
  uint32_t asc[RW][NSC];
  float wv[RW][NMT][4];
  auto load_rows = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int row = min(row0 + (r < nrows ? r : 0), row_hi);
#pragma unroll
      for (int c = 0; c < NSC; ++c) asc[r][c] = 0;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        const int64_t hrow = (int64_t)row * H + mt * 16 + li;
        aq[r][mt] = FMT::load_q(a.q_fp4, hrow, lg);
        asc[r][mt >> 2] |= FMT::q_scale_byte(a.q_scale, hrow, lg) << (8 * (mt & 3));
        const float4 w4 = *reinterpret_cast<const float4*>(a.w + (int64_t)row * H + mt * 16 + lg * 4);
        const bool live = r < nrows;
        wv[r][mt][0] = live ? w4.x : 0.f;
        wv[r][mt][1] = live ? w4.y : 0.f;
        wv[r][mt][2] = live ? w4.z : 0.f;
        wv[r][mt][3] = live ? w4.w : 0.f;
      }
    }
  };
  if constexpr (EARLY_Q) load_rows();
  __builtin_amdgcn_sched_barrier(0);  // all of round trip 1 issued before waiting for the page ids

  // Round trip 2: the first D pages (fetched before the context lengths say
  // whether they are needed).
  int32_t pid[D];  // the first D page ids; later ones are read from my_pid when they are loaded
#pragma unroll
  for (int i = 0; i < D; ++i)
    pid[i] = (nrows > 0 && page_begin + i < bt_stride) ? __builtin_amdgcn_readlane(my_pid, i) : -1;
  // A wave whose first page id is outside [0, num_pages) has nothing to
  // store: the table only promises valid ids for pages some row needs, and
  // the wave's pages start past them (an empty row group has no ids at all).
  // It leaves before loading any page, so it neither holds a slot nor
  // queues page traffic ahead of the waves that have work.
  if (!(pid[0] >= 0 && pid[0] < num_pages)) return;
  // Branch-free from here, so all loads issue back to back: another id
  // outside the pool (past the request's pages) re-reads the first page and
  // its tile is never stored.
  // D page buffers; page p is scored from buf[p % D], which then loads page
  // p + D (a rolling prefetch: D pages in flight, D pages of registers)
  typename FMT::Page buf[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    const int64_t pg = (pid[i] >= 0 && pid[i] < num_pages) ? pid[i] : pid[0];
    FMT::template load_page<kPageNT>(buf[i], a.payload, a.scale, pg, lane_pay, lane_sc);
  }
  if constexpr (!EARLY_Q) load_rows();

  // a context length beyond the row or the table (a broken contract) is cut
  // to what both hold, so no store leaves the row
  const int ctx_cap = (int)min(min((int64_t)bt_stride * 64, a.logits_stride), (int64_t)0x7FFFFFFF);
  int ctx_r[4] = {0, 0, 0, 0};
  int gmax = 0;
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    ctx_r[r] = r < nrows ? min(__builtin_amdgcn_readlane(my_ctx, r), ctx_cap) : 0;
    gmax = max(gmax, ctx_r[r]);
  }
  const int pages_needed = min((gmax + 63) >> 6, page_end);
  if (nrows == 0 || page_begin >= pages_needed) return;
  const int n_pages = min(PPW, pages_needed - page_begin);

  // per row: the (wave-uniform) logits address of token page_begin*64 and
  // the in-row limit relative to it; a page's 64 logits are then stored at
  // base + lane + an immediate offset
  float* rowp[RW];
  int lim[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    rowp[r] = a.logits + (int64_t)(row0 + (r < nrows ? r : 0)) * a.logits_stride + (int64_t)page_begin * 64;
    lim[r] = r < nrows ? ctx_r[r] - page_begin * 64 : 0;
  }
  // groups of D pages (a runtime loop; within a group the buffer index is a
  // compile-time constant, so the pages stay in registers)
  for (int g0 = 0; g0 < n_pages; g0 += D) {
    static_for<D>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      const int p = g0 + i;
      if (p >= n_pages) return;
      static_for<RW>([&](auto rc) __attribute__((always_inline)) {
        constexpr int r = decltype(rc)::value;
        if (r < nrows) {
          const float tot = row_page_logits<FMT, NMT, RW == 1>(aq[r], asc[r], wv[r], buf[i]);
          if (lane + p * 64 < lim[r]) store_logit(rowp[r] + lane + p * 64, tot);
        }
      });
      const int pn = p + D;  // < PPW <= 64: lane pn of my_pid holds its id
      if (pn < n_pages) {
        const int32_t id = __builtin_amdgcn_readlane(my_pid, pn);
        if (id >= 0 && id < num_pages)
          FMT::template load_page<kPageNT>(buf[i], a.payload, a.scale, id, lane_pay, lane_sc);
      }
    });
  }
}

// Host-bounded grid: x = page chunk, y = row group, z = request.  Work-
// groups go to the eight XCDs round robin by linear id, so with the chunk
// count a multiple of 8 a fixed chunk index would always land on the same
// XCD; early chunks exist for every request, late ones only for long
// requests, which would load the first XCDs most.  Rotating each request's
// chunks by its index spreads every request over all XCDs (a bijection per
// request).  Wave w takes PPW consecutive pages of the chunk.
template <typename FMT, int RW, int NMT, int PPW, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kMinWavesPerSimd<FMT, RW, NMT>))) void
mqa_logits_kernel(WaveArgs a) {
  const int n_chunks = gridDim.x;
  const int grp = blockIdx.y;
  const int req = blockIdx.z;
  int rot = req & 7;
  if (rot >= n_chunks) rot %= n_chunks;
  int chunk = (int)blockIdx.x + rot;
  if (chunk >= n_chunks) chunk -= n_chunks;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int page_begin = (chunk * 4 + wave) * PPW;
  if (page_begin >= a.bt_stride) return;
  wave_item<FMT, RW, NMT, PPW, D, false>(a, req, page_begin, page_begin + PPW, [&](int& row0, int& nrows) {
    // the request's rows, kept inside [0, n_rows) whatever indptr holds
    const int ip0 = min(max(a.indptr[req], 0), a.n_rows), ip1 = min(max(a.indptr[req + 1], ip0), a.n_rows);
    row0 = ip0 + grp * RW;
    nrows = max(0, min(RW, ip1 - row0));
  });
}

// Scheduled: work-group i takes item i of the plan (request, RW rows,
// 4 * PPW pages; wave w its w-th PPW pages), or leaves when the plan has
// fewer items.  The item is checked against the call's requests and rows.
template <typename FMT, int RW, int NMT, int PPW, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kMinWavesPerSimd<FMT, RW, NMT>))) void
mqa_logits_wave_planned_kernel(WaveArgs a, const int32_t* __restrict__ hdr, const int4* __restrict__ items,
                               int32_t n_reqs, int32_t cap_items) {
  const int item = blockIdx.x;
  // the item is read with the header (the grid never exceeds the capacity)
  const int4 iv = items[min(item, cap_items - 1)];  // the same for the whole work-group: scalar registers
  const int n_items = (hdr[kHdrRows] == RW && hdr[kHdrWaves] == 0) ? min(max(hdr[kHdrItems], 0), cap_items) : 0;
  if (item >= n_items) return;
  const int4 it = make_int4(__builtin_amdgcn_readfirstlane(iv.x), __builtin_amdgcn_readfirstlane(iv.y),
                            __builtin_amdgcn_readfirstlane(iv.z), __builtin_amdgcn_readfirstlane(iv.w));
  const int req = it.x, pb = it.z, nr = it.w & 0xFF, npg = it.w >> 8;
  if (req < 0 || req >= n_reqs || nr <= 0 || nr > RW || pb < 0 || npg <= 0 || npg > 4 * PPW) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int page_begin = pb + wave * PPW;
  const int page_end = min(page_begin + PPW, pb + npg);
  if (page_begin >= page_end || page_begin >= a.bt_stride) return;
  wave_item<FMT, RW, NMT, PPW, D, true>(a, req, page_begin, page_end, [&](int& row0, int& nrows) {
    row0 = it.y;
    nrows = (it.y >= 0 && it.y + nr <= a.n_rows) ? nr : 0;  // rows inside the call's rows
  });
}

// Page ids one shared-page work-group stages in LDS (its chunk of pages),
// and the bytes of one FP4 page in the payload and scale pools.
constexpr int kSharedMaxChunk = kMaxItemPages;
constexpr int kPayBytes = 4096, kScBytes = 256;
// Pages x rows one wave of a shared-page work-group scores at most.
constexpr int kSharedPageRows = 64;

// Requests with several rows: a work-group of NW waves takes a block of
// NW*RW rows of one request and a chunk of that request's pages; each page
// is read from memory once per work-group, in whole contiguous 16-byte
// pieces, and shared by its waves through LDS, and each wave scores its RW
// rows.  Page i's bytes are loaded into registers two pages ahead, written
// to LDS slot i&1 just before page i is scored, and one barrier per page
// publishes the slot (the barrier also proves every wave has finished page
// i-2, the slot's previous page).  The slot layout is the cache format's
// (Fp4Staged, Fp8Staged): a lane's B operand per tile is one (FP4) or two
// (FP8) 16-byte LDS reads and its four tiles' scales one word.  Each (row,
// token) goes through row_page_logits with the same operands as in
// mqa_logits_kernel, so the logits are the same bits whichever kernel
// computes them.
// How a cache's pages travel through a shared-page work-group of NT threads:
// Regs<NT> holds one page in flight (fetch: coalesced 16-byte loads, thread
// t taking pieces t, t + NT, ...), stage() writes it to an LDS slot of
// kSlotBytes, and read<SLOT>() gives a lane its B operands and scale word
// for the page's four tiles from slot SLOT (a compile-time offset on top of
// the lane's address registers).  Q and QSc load a row's A operands and
// scale bytes as the per-wave kernel does; Op is the operand format that
// row_page_logits scores with.
//
// FP4 (split pools): the slot holds the payload in pool order, so lane
// (token li, block lg) finds its 16 bytes at lg*1024 + li*16 + t*256, and
// the page's scale bytes transposed, so that one word gives a lane its four
// tiles' scales (block j, token l, tile t at payload end + 64 j + 4 l + t).
struct Fp4Staged {
  static constexpr int kSlotBytes = kPayBytes + kScBytes;
  typedef Fp4Split Q;
  typedef Fp4Lds Op;
  template <int NT>
  struct Regs {
    typedef uint32_t Vec __attribute__((ext_vector_type(4 * (kPayBytes / 16 / NT))));
    Vec p;  // one native vector, so the pieces stay in registers
    uint32_t s;
  };
  struct Lane {
    uint32_t pay, sc;
  };
  static __device__ __forceinline__ Lane lane(int li, int lg) {
    return Lane{(uint32_t)(lg * 1024 + li * 16), (uint32_t)(kPayBytes + lg * 64 + li * 4)};
  }
  template <int NT>
  static __device__ __forceinline__ void fetch(Regs<NT>& r, const uint8_t* __restrict__ payload,
                                               const uint8_t* __restrict__ scale, int64_t pid, int tid) {
    const uint8_t* pp = payload + pid * kPayBytes;
    static_for<kPayBytes / 16 / NT>([&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value;
      const uint4 v = *reinterpret_cast<const uint4*>(pp + 16 * (tid + NT * m));
      r.p[4 * m + 0] = v.x;
      r.p[4 * m + 1] = v.y;
      r.p[4 * m + 2] = v.z;
      r.p[4 * m + 3] = v.w;
    });
    if (tid < 64) r.s = *reinterpret_cast<const uint32_t*>(scale + pid * kScBytes + 4 * tid);
  }
  // Scale word t holds block j = t/16, tokens 4*(t%16) + b; token 16*tile + l's
  // byte goes to [j][l][tile].
  template <int NT>
  static __device__ __forceinline__ void stage(const Regs<NT>& r, uint8_t* slot, int tid) {
    static_for<kPayBytes / 16 / NT>([&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value;
      *reinterpret_cast<uint4*>(slot + 16 * (tid + NT * m)) =
          make_uint4(r.p[4 * m + 0], r.p[4 * m + 1], r.p[4 * m + 2], r.p[4 * m + 3]);
    });
    if (tid < 64) {
      uint8_t* d = slot + kPayBytes + (tid >> 4) * 64 + ((tid & 15) >> 2);
#pragma unroll
      for (int b = 0; b < 4; ++b) d[(4 * (tid & 3) + b) * 4] = (uint8_t)(r.s >> (8 * b));
    }
  }
  template <int SLOT>
  static __device__ __forceinline__ Fp4Lds::Page read(const uint8_t* ring, const Lane& l) {
    Fp4Lds::Page pg;
#pragma unroll
    for (int t = 0; t < 4; ++t) pg.b[t] = *reinterpret_cast<const uint4*>(ring + l.pay + SLOT + 256 * t);
    pg.s = *reinterpret_cast<const uint32_t*>(ring + l.sc + SLOT);
    return pg;
  }
};

// An FP8 page staged in LDS: Fp8Fused's operands (lane (token li, K group lg)
// holds code bytes 32 lg .. 32 lg + 31 of token 16 t + li in tile t) with
// the same bytes in the same K slots, so every logit is computed by the same
// operations.
struct Fp8Lds {
  struct Page {
    v8i b[4];
    uint32_t s;  // byte t: tile t's scale byte for the lane's token
  };
  typedef v8i QOp;
  template <int OPA>
  static __device__ __forceinline__ v4f mfma(const QOp& a, const Page& p, int t, uint32_t sa) {
    const v4f z = {0.f, 0.f, 0.f, 0.f};
    switch (t) {  // t is a compile-time constant at every call
      case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, p.b[0], z, 0, 0, OPA, (int)sa, 0, (int)p.s);
      case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, p.b[1], z, 0, 0, OPA, (int)sa, 1, (int)p.s);
      case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, p.b[2], z, 0, 0, OPA, (int)sa, 2, (int)p.s);
      default: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, p.b[3], z, 0, 0, OPA, (int)sa, 3, (int)p.s);
    }
  }
};

// FP8 (fused pool): the page's 8,192 code bytes (64 token rows of 128) are
// fetched in pool order, 16 bytes per piece, and each piece is written to
// where a lane reads it: piece c is token c/8, bytes 16 (c%8) .., i.e. half
// h = c%2 of group lg = (c%8)/2 of token li = (c/8)%16 in tile t = c/128,
// stored at t*2048 + h*1024 + 16 (16 lg + (li ^ (4 lg + 2 h))).  Within one
// 16-byte column the 16 lanes of a group lg read one contiguous 256-byte
// row (the xor permutes it), and the 16 consecutive pieces of two tokens
// land in 16 different 16-byte bank groups (li ^ (4 lg + 2 h) runs over all
// 16 values for li in {2i, 2i+1}), so neither the writes nor the reads
// collide on a bank.  After the codes, word li byte t = the exponent byte of
// token 16 t + li's fp32 scale (a power of two: the MFMA's E8M0 scale).
struct Fp8Staged {
  static constexpr int kCodeBytes = 8192, kPageBytes = 8448;
  static constexpr int kSlotBytes = kCodeBytes + 64;
  typedef Fp8Fused Q;
  typedef Fp8Lds Op;
  template <int NT>
  struct Regs {
    typedef uint32_t Vec __attribute__((ext_vector_type(4 * (kCodeBytes / 16 / NT))));
    Vec c;  // one native vector, so the pieces stay in registers
    uint32_t s;
  };
  struct Lane {
    uint32_t h0, h1, sc;
  };
  static __device__ __forceinline__ Lane lane(int li, int lg) {
    return Lane{(uint32_t)(16 * (16 * lg + (li ^ (4 * lg)))), (uint32_t)(1024 + 16 * (16 * lg + (li ^ (4 * lg + 2)))),
                (uint32_t)(kCodeBytes + 4 * li)};
  }
  template <int NT>
  static __device__ __forceinline__ void fetch(Regs<NT>& r, const uint8_t* __restrict__ pool, const uint8_t*,
                                               int64_t pid, int tid) {
    const uint8_t* pp = pool + pid * kPageBytes;
    static_for<kCodeBytes / 16 / NT>([&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value;
      const uint4 v = *reinterpret_cast<const uint4*>(pp + 16 * (tid + NT * m));
      r.c[4 * m + 0] = v.x;
      r.c[4 * m + 1] = v.y;
      r.c[4 * m + 2] = v.z;
      r.c[4 * m + 3] = v.w;
    });
    if (tid < 64) r.s = *reinterpret_cast<const uint32_t*>(pp + kCodeBytes + 4 * tid);
  }
  template <int NT>
  static __device__ __forceinline__ void stage(const Regs<NT>& r, uint8_t* slot, int tid) {
    static_for<kCodeBytes / 16 / NT>([&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value;
      const int c = tid + NT * m;
      const int li = (c >> 3) & 15, lg = (c >> 1) & 3, h = c & 1, t = c >> 7;
      *reinterpret_cast<uint4*>(slot + t * 2048 + h * 1024 + 16 * (16 * lg + (li ^ (4 * lg + 2 * h)))) =
          make_uint4(r.c[4 * m + 0], r.c[4 * m + 1], r.c[4 * m + 2], r.c[4 * m + 3]);
    });
    if (tid < 64) slot[kCodeBytes + 4 * (tid & 15) + (tid >> 4)] = (uint8_t)((r.s >> 23) & 0xFFu);
  }
  template <int SLOT>
  static __device__ __forceinline__ Fp8Lds::Page read(const uint8_t* ring, const Lane& l) {
    Fp8Lds::Page pg;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      pg.b[t] = Fp8Fused::join(*reinterpret_cast<const uint4*>(ring + l.h0 + SLOT + 2048 * t),
                               *reinterpret_cast<const uint4*>(ring + l.h1 + SLOT + 2048 * t));
    pg.s = *reinterpret_cast<const uint32_t*>(ring + l.sc + SLOT);
    return pg;
  }
};

// LDS of a shared-page work-group: two page slots, the chunk's page ids and
// the block's context lengths.
template <typename SF, int ROWS>
struct SharedLds {
  __attribute__((aligned(16))) uint8_t ring[2][SF::kSlotBytes];
  int32_t pid[kSharedMaxChunk];
  int32_t ctx[ROWS];
};

// The scalar arguments every shared-page item needs.
struct SharedArgs {
  const int32_t* block_table;
  const int32_t* row_ctx;
  const uint8_t* payload;
  const uint8_t* scale;
  int64_t num_pages;
  int32_t bt_stride;
  const uint8_t* q;        // packed Q (FP4 codes or FP8 codes)
  const uint8_t* q_scale;  // its scales (FP4: UE8M0 bytes; FP8: fp32 powers of two)
  const float* w;
  float* logits;
  int64_t logits_stride;
};

// One shared-page item: rows [row0, row0 + nrows) of request req (0 <
// nrows <= NW*RW, rows inside the call's rows) and the pages [pb, pb +
// n_max) of its block table (n_max <= kSharedMaxChunk), cut to the pages
// the rows' contexts reach.  Work-group uniform; starts and ends with the
// work-group in step (the caller's barriers order it against the previous
// item's LDS use).
// tid is the thread's index in the work-group; rot picks which waves take a
// block's extra rows.
template <typename SF, int NW, int RW, int NMT>
__device__ __forceinline__ void shared_item(SharedLds<SF, NW * RW>& L, const SharedArgs& a, int req, int row0,
                                            int nrows, int pb, int n_max, int tid, int rot) {
  constexpr int NT = NW * 64;
  constexpr int H = NMT * 16;
  constexpr int NSC = (NMT + 3) / 4;
  constexpr int ROWS = NW * RW;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int li = lane & 15, lg = lane >> 4;

  // Round trip 1, all in flight together: the block's context lengths, the
  // chunk's page ids (none past the table row) and the wave's Q operands and
  // weights (its rows: the block's rows spread evenly over the waves, so a
  // block short of ROWS rows leaves no wave with more than ceil(nrows / NW)).
  // A context length beyond the row or the table (a broken contract) is cut
  // to what both hold, so no store leaves the row; a page id outside the pool
  // (a broken table) reads page 0, so every load stays in the pool.
  const int ctx_cap = (int)min(min((int64_t)a.bt_stride * 64, a.logits_stride), (int64_t)0x7FFFFFFF);
  const int32_t my_ctx = tid < nrows ? a.row_ctx[row0 + tid] : 0;
  const int32_t* bt = a.block_table + (int64_t)req * a.bt_stride + pb;
  const int n_ids = max(0, min(n_max, a.bt_stride - pb));
  constexpr int NID = (kSharedMaxChunk + NT - 1) / NT;
  int32_t ids[NID];
#pragma unroll
  for (int m = 0; m < NID; ++m) ids[m] = tid + NT * m < n_ids ? bt[tid + NT * m] : 0;
  // The block's rows over the waves: every wave floor(nrows / NW) rows and
  // the remainder one more each (at most RW), consecutive rows per wave.
  // Which waves take the extra rows rotates with `rot`, so that across the
  // work-groups of a launch no SIMD (a work-group's wave w runs on the same
  // SIMD in every work-group) gets the busier waves more often than the
  // others.  Results do not depend on which wave scores a row.
  const int slot = (wave + rot) % NW;  // wave-uniform
  const int base = nrows / NW, extra = nrows - base * NW;
  const int nr = base + (slot < extra ? 1 : 0);  // wave-uniform, <= RW
  const int first = slot * base + min(slot, extra);  // the wave's first row within the block
  const int wrow0 = row0 + first;
  typename SF::Op::QOp aq[RW][NMT];
  uint32_t asc[RW][NSC];
  float wv[RW][NMT][4];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int row = r < nr ? wrow0 + r : row0;
#pragma unroll
    for (int c = 0; c < NSC; ++c) asc[r][c] = 0;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const int64_t hrow = (int64_t)row * H + mt * 16 + li;
      aq[r][mt] = SF::Q::load_q(a.q, hrow, lg);
      asc[r][mt >> 2] |= SF::Q::q_scale_byte(a.q_scale, hrow, lg) << (8 * (mt & 3));
      const float4 w4 = *reinterpret_cast<const float4*>(a.w + (int64_t)row * H + mt * 16 + lg * 4);
      wv[r][mt][0] = w4.x;
      wv[r][mt][1] = w4.y;
      wv[r][mt][2] = w4.z;
      wv[r][mt][3] = w4.w;
    }
  }
  if (tid < ROWS) L.ctx[tid] = min(max(my_ctx, 0), ctx_cap);
#pragma unroll
  for (int m = 0; m < NID; ++m) {
    const int k = tid + NT * m;
    if (k < n_ids) L.pid[k] = (ids[m] >= 0 && ids[m] < a.num_pages) ? ids[m] : 0;
  }
  __syncthreads();  // context lengths and page ids staged
  int gmax = 0;
#pragma unroll
  for (int r = 0; r < ROWS; ++r) gmax = max(gmax, L.ctx[r]);
  const int n = min(n_ids, ((gmax + 63) >> 6) - pb);
  if (n <= 0) return;  // the whole work-group: no row needs these pages
  float* rowp[RW];
  int lim[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int row = r < nr ? wrow0 + r : row0;
    rowp[r] = a.logits + (int64_t)row * a.logits_stride + (int64_t)pb * 64;
    lim[r] = r < nr ? L.ctx[first + r] - pb * 64 : 0;
  }

  // page bytes in flight: two register sets, used in turn
  typename SF::template Regs<NT> set0, set1;
  // a lane's B operand bytes and scale word within an LDS slot; the slot and
  // the tile are compile-time offsets on top (immediate offsets of the LDS
  // reads, so both slots share the lane's address registers)
  const uint8_t* ring = &L.ring[0][0];
  const typename SF::Lane lo = SF::lane(li, lg);
  auto score = [&](auto sc, int i) __attribute__((always_inline)) {
    constexpr int slot = decltype(sc)::value * SF::kSlotBytes;
    if (nr == 0) return;  // wave-uniform: a wave past the block's rows only loads
    const typename SF::Op::Page pg = SF::template read<slot>(ring, lo);
    static_for<RW>([&](auto rc) __attribute__((always_inline)) {
      constexpr int r = decltype(rc)::value;
      if (r < nr) {
        const float tot = row_page_logits<typename SF::Op, NMT, false>(aq[r], asc[r], wv[r], pg);
        if (lane + i * 64 < lim[r]) store_logit(rowp[r] + lane + i * 64, tot);
      }
    });
  };
  SF::template fetch<NT>(set0, a.payload, a.scale, L.pid[0], tid);
  if (n > 1) SF::template fetch<NT>(set1, a.payload, a.scale, L.pid[1], tid);
  for (int i = 0; i < n; i += 2) {
    SF::template stage<NT>(set0, L.ring[0], tid);
    __syncthreads();
    if (i + 2 < n) SF::template fetch<NT>(set0, a.payload, a.scale, L.pid[i + 2], tid);
    score(std::integral_constant<int, 0>{}, i);
    if (i + 1 < n) {
      SF::template stage<NT>(set1, L.ring[1], tid);
      __syncthreads();
      if (i + 3 < n) SF::template fetch<NT>(set1, a.payload, a.scale, L.pid[i + 3], tid);
      score(std::integral_constant<int, 1>{}, i + 1);
    }
  }
}

// Host-bounded grid: (page chunk, row block, request), each request's chunks
// rotated across the XCDs as in mqa_logits_kernel.
template <typename SF, int NW, int RW, int NMT>
__global__ __launch_bounds__(NW * 64) void mqa_logits_shared_kernel(SharedArgs a, const int32_t* __restrict__ indptr,
                                                                    int32_t chunk_pages, int32_t n_rows) {
  constexpr int ROWS = NW * RW;
  __shared__ SharedLds<SF, ROWS> L;
  const int n_chunks = gridDim.x;
  const int req = blockIdx.z;
  int rot = req & 7;
  if (rot >= n_chunks) rot %= n_chunks;
  int chunk = (int)blockIdx.x + rot;
  if (chunk >= n_chunks) chunk -= n_chunks;
  // the request's rows, kept inside [0, n_rows) whatever indptr holds
  const int ip0 = min(max(indptr[req], 0), n_rows), ip1 = min(max(indptr[req + 1], ip0), n_rows);
  const int row0 = ip0 + (int)blockIdx.y * ROWS;
  const int nrows = max(0, min(ROWS, ip1 - row0));
  if (nrows == 0) return;  // the whole work-group
  shared_item<SF, NW, RW, NMT>(L, a, req, row0, nrows, chunk * chunk_pages, chunk_pages, threadIdx.x,
                           (int)(blockIdx.x + blockIdx.y));
}

// Scheduled: work-group i takes item i of the plan (request, up to NW*RW
// rows, a page chunk), or leaves when the plan has fewer items.  The item
// is checked against the call's requests and rows (a plan of another batch
// never takes the kernel outside the buffers).
template <int NW, int RW, int NMT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW == 4 && NMT <= 4 ? 4 : 1))) void
mqa_logits_planned_kernel(SharedArgs a, int32_t n_reqs, int32_t n_rows,
                                                                     const int32_t* __restrict__ hdr,
                                                                     const int4* __restrict__ items,
                                                                     int32_t cap_items) {
  constexpr int ROWS = NW * RW;
  __shared__ SharedLds<Fp4Staged, ROWS> L;
  const int item = blockIdx.x;
  // the item is read with the header (the grid never exceeds the capacity)
  const int4 iv = items[min(item, cap_items - 1)];  // the same for the whole work-group: scalar registers
  const int n_items =
      (hdr[kHdrRows] == ROWS && hdr[kHdrWaves] == NW) ? min(max(hdr[kHdrItems], 0), cap_items) : 0;
  if (item >= n_items) return;
  const int4 it = make_int4(__builtin_amdgcn_readfirstlane(iv.x), __builtin_amdgcn_readfirstlane(iv.y),
                            __builtin_amdgcn_readfirstlane(iv.z), __builtin_amdgcn_readfirstlane(iv.w));
  const int req = it.x, pb = it.z, nrows = it.w & 0xFF, n_max = it.w >> 8;
  if (req < 0 || req >= n_reqs || nrows <= 0 || nrows > ROWS || pb < 0 || n_max <= 0 || n_max > kSharedMaxChunk ||
      (int64_t)pb + n_max > a.bt_stride)
    return;
  if (it.y < 0 || it.y + nrows > n_rows) return;  // rows inside the call's rows
  shared_item<Fp4Staged, NW, RW, NMT>(L, a, req, it.y, nrows, pb, n_max, threadIdx.x, item);
}

// The arguments of one logits call, as the launchers pass them down.
struct LogitsCall {
  const uint8_t* q;
  const uint8_t* q_scale;
  const float* w;
  const int32_t* indptr;
  int32_t n_reqs;
  int32_t n_rows;
  const int32_t* row_ctx;
  const int32_t* block_table;
  int32_t bt_stride;
  const uint8_t* payload;
  const uint8_t* scale;
  int64_t num_pages;
  float* logits;
  int64_t logits_stride;
  int32_t max_rows_per_req;
  int64_t max_ctx;
  hipStream_t stream;
};

template <typename SF, int NW, int RW, int NMT>
static hipError_t launch_shared(const LogitsCall& c, int page_rows) {
  constexpr int ROWS = NW * RW;
  const int64_t pages = (c.max_ctx + 63) / 64;
  const int64_t blocks = (c.max_rows_per_req + ROWS - 1) / ROWS;
  if (pages == 0 || blocks == 0 || c.n_reqs == 0) return hipSuccess;
  if (blocks > 65535 || c.n_reqs > 65535) return hipErrorInvalidConfiguration;
  // Page chunks: at least about two waves for each of the 1,024 SIMDs, and
  // no work-group longer than about page_rows page-rows per wave (a
  // request's block whose rows are long must not become the critical path:
  // the hardware balances many short work-groups across the CUs), and not
  // shorter than 8 pages (a work-group's set-up is paid per chunk).
  const int64_t want = 2048 / NW;
  int64_t chunks = (want + c.n_reqs * blocks - 1) / (c.n_reqs * blocks);
  chunks = std::max<int64_t>(chunks, (pages * RW + page_rows - 1) / page_rows);
  chunks = std::max<int64_t>(1, std::min<int64_t>(chunks, (pages + 7) / 8));
  int64_t chunk_pages = std::min<int64_t>((pages + chunks - 1) / chunks, kSharedMaxChunk);
  chunks = (pages + chunk_pages - 1) / chunk_pages;
  if (chunks > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  const SharedArgs a{c.block_table, c.row_ctx, c.payload, c.scale, c.num_pages, c.bt_stride,
                     c.q, c.q_scale, c.w, c.logits, c.logits_stride};
  return launch(mqa_logits_shared_kernel<SF, NW, RW, NMT>, dim3((unsigned)chunks, (unsigned)blocks, (unsigned)c.n_reqs),
                dim3(NW * 64), 0, c.stream, a, c.indptr, (int32_t)chunk_pages, c.n_rows);
}

template <typename FMT, int RW, int NMT, int PPW, int D>
static hipError_t launch_rw(const LogitsCall& c) {
  const int64_t pages = (c.max_ctx + 63) / 64;
  const int64_t n_chunks = (pages + 4 * PPW - 1) / (4 * PPW);
  const int64_t n_groups = (c.max_rows_per_req + RW - 1) / RW;
  if (n_chunks == 0 || n_groups == 0 || c.n_reqs == 0) return hipSuccess;
  if (n_chunks > 0x7FFFFFFFLL || n_groups > 65535 || c.n_reqs > 65535) return hipErrorInvalidConfiguration;
  const WaveArgs a{c.block_table, c.indptr, c.row_ctx, c.payload, c.scale, c.num_pages, c.bt_stride,
                   c.q, c.q_scale, c.w, c.logits, c.logits_stride, c.n_rows};
  return launch(mqa_logits_kernel<FMT, RW, NMT, PPW, D>,
                dim3((unsigned)n_chunks, (unsigned)n_groups, (unsigned)c.n_reqs), dim3(256), 0, c.stream, a);
}

template <typename FMT, int NMT>
static hipError_t launch_nmt(const LogitsCall& c) {
  constexpr int cap = NMT > 4 ? FMT::kRowsCapWide : FMT::kRowsCap;
  const int r = c.max_rows_per_req;
  if (r <= 1) return launch_rw<FMT, 1, NMT, FMT::kPpw1, FMT::kD1>(c);
  if constexpr (cap <= 2) {
    return launch_rw<FMT, 2, NMT, FMT::kPpw2, FMT::kD2>(c);
  } else {
    if (r == 2) return launch_rw<FMT, 2, NMT, FMT::kPpw2, FMT::kD2>(c);
    if (r == 3 || r == 6) return launch_rw<FMT, 3, NMT, FMT::kPpwMany, FMT::kDMany>(c);
    return launch_rw<FMT, 4, NMT, FMT::kPpwMany, FMT::kDMany>(c);
  }
}

template <typename FMT>
static hipError_t launch_heads(const LogitsCall& c, int n_heads) {
  return with_head_tiles(n_heads, [&](auto nmt) { return launch_nmt<FMT, decltype(nmt)::value>(c); });
}

// FP4 batches of requests with three or more rows each on average: the
// shared-page kernel, NW waves of RW rows per work-group.  Two rows per wave
// at most past six rows: a third or fourth row's Q operands and weights take
// enough registers to cut the waves per SIMD from four to two, which costs
// more than the extra page staging saves (prefill, 4,096 rows: 365 us with
// 4 x 2 against 386 us with 4 x 4; 6-row decode: 2 x 3 and 4 x 2 alike).  A
// batch whose row counts are far from uniform (the average below 3/4 of the
// largest) takes two waves of two rows and page chunks of at most 16
// page-rows per wave: its work-groups' lengths vary with their requests' rows
// and contexts, and the last ones to finish set the kernel's time (48
// requests of 1-16 rows over 8k-32k tokens: 76 us, against 85 us with 4 x 3
// and 32 page-rows and 111 us with the near-uniform shape and chunks).
template <int NMT>
static hipError_t launch_fp4_shared(const LogitsCall& c, bool uniform) {
  const int page_rows = uniform ? kSharedPageRows : kSharedPageRows / 4;
  const int r = c.max_rows_per_req;
  if (!uniform || r <= 4) return launch_shared<Fp4Staged, 2, 2, NMT>(c, page_rows);
  if constexpr (NMT <= 4) {
    if (r <= 6) return launch_shared<Fp4Staged, 2, 3, NMT>(c, page_rows);
  }
  return launch_shared<Fp4Staged, 4, 2, NMT>(c, page_rows);
}

// FP8 batches of requests with three or more rows each on average: the
// shared-page kernel with the FP8 pages staged in LDS (Fp8Staged).  The
// shapes follow the FP4 rule with the FP8 operands' register cost: NW waves
// of RW rows (FP4IDX_FP8_SHARED_SHAPE = NW * 10 + RW in measurement builds).
#ifndef FP4IDX_FP8_SHARED_SHAPE
#define FP4IDX_FP8_SHARED_SHAPE 41
#endif
template <int NMT>
static hipError_t launch_fp8_shared(const LogitsCall& c, bool uniform) {
  const int page_rows = uniform ? kSharedPageRows : kSharedPageRows / 4;
  constexpr int NW = FP4IDX_FP8_SHARED_SHAPE / 10, RW = NMT > 4 ? 1 : FP4IDX_FP8_SHARED_SHAPE % 10;
  if (!uniform) return launch_shared<Fp8Staged, 2, 2 < RW ? 2 : RW, NMT>(c, page_rows);
  return launch_shared<Fp8Staged, NW, RW, NMT>(c, page_rows);
}

hipError_t launch_mqa_logits_bounded(const uint8_t* q_fp4, const uint8_t* q_scale, const float* w, int64_t n_rows,
                                     int n_heads, const int32_t* indptr, int32_t n_reqs, const int32_t* row_ctx,
                                     const int32_t* block_table, int32_t bt_stride, const uint8_t* payload,
                                     const uint8_t* scale, int64_t num_pages, float* logits, int64_t logits_stride,
                                     int32_t max_rows_per_req, int64_t max_ctx, hipStream_t stream) {
  if (n_rows > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  const LogitsCall c{q_fp4,       q_scale,   w,       indptr,    n_reqs,    (int32_t)n_rows, row_ctx,
                     block_table, bt_stride, payload, scale,     num_pages, logits,          logits_stride,
                     max_rows_per_req, max_ctx, stream};
  // The shared-page kernel splits a request's rows among a work-group's
  // waves and stages each page once for all of them; the per-wave kernel
  // splits pages instead and reads each page once per wave.  Shared pages
  // pay from three rows per request on average (about 5 % on the prefill and
  // 256 x 6 decode batches, 20 % on a batch of 1-16 rows per request).
  // Near-uniform: the requests' average row count is at least 3/4 of the
  // largest.  Both kernels give the same bits.
  const bool uniform = 4 * n_rows >= 3 * (int64_t)max_rows_per_req * n_reqs;
  const int64_t avg_rows = n_reqs > 0 ? (n_rows + n_reqs - 1) / n_reqs : 0;
  if (max_rows_per_req <= 2 || avg_rows < 3) return launch_heads<Fp4Split>(c, n_heads);
  return with_head_tiles(n_heads, [&](auto nmt) { return launch_fp4_shared<decltype(nmt)::value>(c, uniform); });
}

// ---- the scheduled path: the plan (schedule.hip), then one work-group per item


// The kernel and shape for a batch, from what the host knows: the average
// rows per request and the head count (the same rule for the plan and the
// run).  Under about three rows per request the per-wave kernel (rows per
// wave = 1 or 2, each wave its own pages), else the shared-page kernel.
PlanShape plan_shape(int64_t n_rows, int32_t n_reqs, int n_heads) {
  const int64_t avg10 = n_reqs > 0 ? 10 * n_rows / n_reqs : 0;  // rows per request x 10
#ifdef FP4IDX_PLAN_SHAPE  // measurement builds: waves * 10 + rows per work-group (per wave when waves is 0)
  if (avg10 >= 15) return PlanShape{FP4IDX_PLAN_SHAPE / 10, FP4IDX_PLAN_SHAPE % 10};
#endif
  if (avg10 < 15) return PlanShape{0, 1};
  if (avg10 < 30) return PlanShape{0, 2};
  if (n_heads > 64) return avg10 >= 60 ? PlanShape{4, 8} : PlanShape{2, 4};
  if (avg10 >= 70) return PlanShape{4, 8};
  if (avg10 >= 45) return PlanShape{2, 6};
  return PlanShape{2, 4};
}

// Pages of one per-wave item: the work-group's four waves, PPW pages each.
template <typename FMT, int RW>
constexpr int kWaveItemPages = 4 * (RW == 1 ? FMT::kPpw1 : FMT::kPpw2);

static int wave_item_pages(const PlanShape& sh) {
  return sh.rows == 1 ? kWaveItemPages<Fp4Split, 1> : kWaveItemPages<Fp4Split, 2>;
}

// The most items a plan of this shape makes for the batch sizes and the
// context bound (the run's grid; work-groups past the plan's items leave).
static int64_t plan_item_bound(const PlanShape& sh, int64_t n_rows, int32_t n_reqs, int64_t max_ctx) {
  const PlanSizes sz = plan_sizes(n_rows, n_reqs, sh.rows);
  return sz.blocks * plan_items_per_block(sh, (max_ctx + 63) / 64, wave_item_pages(sh), kItemTarget) + kXcdSlack;
}

int64_t plan_workspace_bytes(int64_t n_rows, int32_t n_reqs, int64_t max_ctx) {
  int64_t bytes = 0;
  for (int heads : {64, 128}) {  // the shapes a batch of these sizes can get
    const PlanShape sh = plan_shape(n_rows, n_reqs, heads);
    bytes = std::max(bytes, plan_bytes(sh, n_rows, n_reqs, max_ctx, wave_item_pages(sh), kItemTarget));
  }
  return bytes;
}

// Work-groups of a kernel the device holds at once.
template <typename K>
static int resident_groups(K kernel, int threads) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1024;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 1024;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kernel), threads, 0) !=
      hipSuccess)
    return 1024;
  return cus * std::max(per_cu, 1);
}

// The work-groups a plan's kernel keeps resident (the plan sizes its short
// chunks from it).
template <int NMT>
static int planned_resident(const PlanShape& sh) {
  if (sh.waves == 0) return 0;
  if (sh.waves == 4) return resident_groups(mqa_logits_planned_kernel<4, 2, NMT>, 256);
  if constexpr (NMT <= 4) {
    if (sh.rows == 6) return resident_groups(mqa_logits_planned_kernel<2, 3, NMT>, 128);
  }
  return resident_groups(mqa_logits_planned_kernel<2, 2, NMT>, 128);
}

template <int NW, int RW, int NMT>
static hipError_t launch_planned(const LogitsCall& c, const int32_t* ws, int64_t grid, int64_t cap_items,
                                 const PlanSizes& sz) {
  const SharedArgs a{c.block_table, c.row_ctx, c.payload, c.scale, c.num_pages, c.bt_stride,
                     c.q, c.q_scale, c.w, c.logits, c.logits_stride};
  return launch(mqa_logits_planned_kernel<NW, RW, NMT>, dim3((unsigned)grid), dim3(NW * 64), 0, c.stream, a,
                c.n_reqs, c.n_rows, ws, reinterpret_cast<const int4*>(ws + sz.items_off),
                (int32_t)cap_items);
}

template <int RW, int NMT>
static hipError_t launch_wave_planned(const LogitsCall& c, const int32_t* ws, int64_t grid, int64_t cap_items,
                                      const PlanSizes& sz) {
  const WaveArgs a{c.block_table, c.indptr, c.row_ctx, c.payload, c.scale, c.num_pages, c.bt_stride,
                   c.q, c.q_scale, c.w, c.logits, c.logits_stride, c.n_rows};
  constexpr int PPW = RW == 1 ? Fp4Split::kPpw1 : Fp4Split::kPpw2;
  constexpr int D = RW == 1 ? Fp4Split::kD1 : Fp4Split::kD2;
  return launch(mqa_logits_wave_planned_kernel<Fp4Split, RW, NMT, PPW, D>, dim3((unsigned)grid), dim3(256), 0,
                c.stream, a, ws, reinterpret_cast<const int4*>(ws + sz.items_off), c.n_reqs, (int32_t)cap_items);
}

template <int NMT>
static hipError_t launch_planned_nmt(const LogitsCall& c, PlanShape sh, const int32_t* ws, int64_t grid,
                                     int64_t cap_items, const PlanSizes& sz) {
  if (sh.waves == 0) {
    if (sh.rows == 1) return launch_wave_planned<1, NMT>(c, ws, grid, cap_items, sz);
    return launch_wave_planned<2, NMT>(c, ws, grid, cap_items, sz);
  }
  if (sh.waves == 4) return launch_planned<4, 2, NMT>(c, ws, grid, cap_items, sz);
  if constexpr (NMT <= 4) {
    if (sh.rows == 6) return launch_planned<2, 3, NMT>(c, ws, grid, cap_items, sz);
  }
  return launch_planned<2, 2, NMT>(c, ws, grid, cap_items, sz);
}

hipError_t launch_mqa_logits_plan(int64_t n_rows, int n_heads, const int32_t* indptr, int32_t n_reqs,
                                  const int32_t* row_ctx, int64_t max_ctx, void* workspace, int64_t workspace_bytes,
                                  hipStream_t stream) {
  const PlanShape sh = plan_shape(n_rows, n_reqs, n_heads);
  const PlanSizes sz = plan_sizes(n_rows, n_reqs, sh.rows);
  const int64_t cap = plan_capacity(sz, workspace_bytes);
  int resident = 0;
  const hipError_t e = with_head_tiles(n_heads, [&](auto nmt) {
    resident = planned_resident<decltype(nmt)::value>(sh);
    return hipSuccess;
  });
  if (e != hipSuccess) return e;
  return launch_plan(indptr, n_reqs, n_rows, row_ctx, max_ctx, static_cast<int32_t*>(workspace), cap, sz, sh,
                     sh.waves == 0 ? wave_item_pages(sh) : 0, kItemTarget, resident, stream);
}

hipError_t launch_mqa_logits_run(const uint8_t* q_fp4, const uint8_t* q_scale, const float* w, int64_t n_rows,
                                 int n_heads, const int32_t* indptr, int32_t n_reqs, const int32_t* row_ctx,
                                 const int32_t* block_table, int32_t bt_stride, const uint8_t* payload,
                                 const uint8_t* scale, int64_t num_pages, float* logits, int64_t logits_stride,
                                 void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  if (n_rows > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  const PlanShape sh = plan_shape(n_rows, n_reqs, n_heads);
  const PlanSizes sz = plan_sizes(n_rows, n_reqs, sh.rows);
  const int64_t cap = plan_capacity(sz, workspace_bytes);
  if (cap < sz.blocks || cap > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  // contexts are cut to the logits row and the block table in any case
  const int64_t ctx_bound = std::min<int64_t>(logits_stride, (int64_t)bt_stride * 64);
  const int64_t grid = std::min<int64_t>(plan_item_bound(sh, n_rows, n_reqs, ctx_bound), cap);
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  const LogitsCall c{q_fp4,       q_scale,   w,       indptr,    n_reqs,    (int32_t)n_rows, row_ctx,
                     block_table, bt_stride, payload, scale,     num_pages, logits,          logits_stride,
                     0,           0,         stream};
  const int32_t* ws = static_cast<const int32_t*>(workspace);
  return with_head_tiles(n_heads, [&](auto nmt) {
    return launch_planned_nmt<decltype(nmt)::value>(c, sh, ws, grid, cap, sz);
  });
}

hipError_t launch_mqa_logits_fp8(const uint8_t* q_fp8, const float* q_scale, const float* w, int64_t n_rows,
                                 int n_heads, const int32_t* indptr, int32_t n_reqs, const int32_t* row_ctx,
                                 const int32_t* block_table, int32_t bt_stride, const uint8_t* pool,
                                 int64_t num_pages, float* logits, int64_t logits_stride, int32_t max_rows_per_req,
                                 int64_t max_ctx, hipStream_t stream) {
  if (n_rows > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  const LogitsCall c{q_fp8,       reinterpret_cast<const uint8_t*>(q_scale), w, indptr, n_reqs, (int32_t)n_rows,
                     row_ctx,     block_table, bt_stride, pool, pool, num_pages, logits, logits_stride,
                     max_rows_per_req, max_ctx, stream};
  // Pages are staged through LDS whenever the batch allows: an FP8 token's
  // 128 code bytes are one row of the page, so a lane's direct operand loads
  // (Fp8Fused) read half lines of sixteen rows per instruction, while staging
  // reads the page in whole lines (decode batch 64: 32.4 -> 23.0 us).  One or
  // two rows per request: one-wave work-groups, each staging its own pages;
  // three or more on average: the shared-page shapes above; in between (a few
  // long requests among one-row ones) the per-wave kernel, several rows per
  // wave.  Every kernel gives the same bits.
  const bool uniform = 4 * n_rows >= 3 * (int64_t)max_rows_per_req * n_reqs;
  const int64_t avg_rows = n_reqs > 0 ? (n_rows + n_reqs - 1) / n_reqs : 0;
#ifndef FP4IDX_FP8_WAVE_STAGED  // 0 in measurement builds: the per-wave kernel for one or two rows
#define FP4IDX_FP8_WAVE_STAGED 1
#endif
  if (FP4IDX_FP8_WAVE_STAGED && max_rows_per_req <= 2)
    return with_head_tiles(n_heads, [&](auto nmt) {
      constexpr int NMT = decltype(nmt)::value;
      if (max_rows_per_req <= 1) return launch_shared<Fp8Staged, 1, 1, NMT>(c, kSharedPageRows);
      return launch_shared<Fp8Staged, 1, 2, NMT>(c, kSharedPageRows);
    });
  if (max_rows_per_req <= 2 || avg_rows < 3) return launch_heads<Fp8Fused>(c, n_heads);
  return with_head_tiles(n_heads, [&](auto nmt) { return launch_fp8_shared<decltype(nmt)::value>(c, uniform); });
}

}  // namespace fp4idx
