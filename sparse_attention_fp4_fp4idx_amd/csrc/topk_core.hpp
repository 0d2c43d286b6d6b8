// Top-k selection over one row held in registers (gfx950), shared by the
// top-k kernels and the fused logits + top-k kernel.  See topk.hip for the
// method.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4idx {

constexpr int kBins = 2048;
// First-cut bins in LDS: bin b (b >= -64; b < 0 are the lanes' spare
// counters) at word bin_word(b) = b + floor(b / 32) past kHistBase: one pad
// word per 32 bins, so the 32 bins a lane sums start 33 words after the
// previous lane's and a wave's reads fall in different banks.
constexpr int kHistBase = 66;
constexpr int kHistWords = kHistBase + kBins + kBins / 32;
__device__ __forceinline__ int bin_word(int b) { return b + (b >> 5); }

__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;  // -0 and +0 are the same value
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Value of an order-preserving key (inverse of order_key; -0 comes back as +0).
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

constexpr int64_t kRegMaxCtx = 32768;  // longest row held in registers
constexpr int kCandMax = 256;          // threshold-bin values ranked directly

// DPP controls (gfx9): quad_perm xor 1 / xor 2, row_half_mirror, row_mirror,
// row_shr:n.
constexpr int kQpXor1 = 0xB1, kQpXor2 = 0x4E, kRowHalfMirror = 0x141, kRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dppu(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

// max / min over the 64 lanes (result uniform): DPP within each 16-lane row,
// then the four row results through scalar reads.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dppu<kQpXor1>(v));
  v = max(v, dppu<kQpXor2>(v));
  v = max(v, dppu<kRowHalfMirror>(v));
  v = max(v, dppu<kRowMirror>(v));
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dppu<kQpXor1>(v));
  v = min(v, dppu<kQpXor2>(v));
  v = min(v, dppu<kRowHalfMirror>(v));
  v = min(v, dppu<kRowMirror>(v));
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return min(min(a, b), min(c, d));
}

// Inclusive prefix sum over the 64 lanes: Hillis-Steele inside each 16-lane
// row (row_shr 1, 2, 4, 8; lanes shifted past the row start read 0), then the
// totals of the rows below are added.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
  v += dppu<0x111>(v);
  v += dppu<0x112>(v);
  v += dppu<0x114>(v);
  v += dppu<0x118>(v);
  const uint32_t t0 = __builtin_amdgcn_readlane(v, 15), t1 = __builtin_amdgcn_readlane(v, 31);
  const uint32_t t2 = __builtin_amdgcn_readlane(v, 47);
  const int row = lane >> 4;
  return v + (row == 0 ? 0u : row == 1 ? t0 : row == 2 ? t0 + t1 : t0 + t1 + t2);
}

// Exclusive prefix over the block (NW waves) of per-thread values; `part`
// holds the wave totals.  Includes the barrier that publishes them.
template <int NW>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, int lane, int wave, uint32_t* part) {
  const uint32_t incl = wave_incl_scan(v, lane);
  if (lane == 63) part[wave] = incl;
  __syncthreads();
  // the waves below this one: lane w holds wave w's total, one wave scan
  const uint32_t pw = lane < NW ? part[lane] : 0u;
  const uint32_t below = wave_incl_scan(pw, lane) - pw;
  return incl - v + (uint32_t)__builtin_amdgcn_readlane((int)below, wave);
}

// Picks the bin holding the K-th largest key given counts hist[0, nb) and
// cnt_above keys above them: thread t of NT owns the reversed bins
// nb-1 - (BPT t .. BPT t + BPT-1), BPT = 2048 / NT.  Returns the bin; s_cnt
// gets the count of keys above it.  Ends with a barrier.
template <int NT>
__device__ __forceinline__ int select_bin(const uint32_t* hist, int nb, int K, int cnt_above, int tid, int lane,
                                          int wave, uint32_t* part, int32_t& s_bin, int32_t& s_cnt) {
  constexpr int BPT = kBins / NT;
  uint32_t c[BPT];
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    const int b = nb - 1 - (BPT * tid + i);
    c[i] = b >= 0 ? hist[b] : 0u;
    local += c[i];
  }
  int acc = cnt_above + (int)block_excl_scan<NT / 64>(local, lane, wave, part);
  if (acc < K && acc + (int)local >= K) {
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      if (acc < K && acc + (int)c[i] >= K) {
        s_bin = nb - 1 - (BPT * tid + i);
        s_cnt = acc;
      }
      acc += (int)c[i];
    }
  }
  __syncthreads();
  return s_bin;
}

// The need-th largest of the m candidate values (1 <= need <= m <= kCandMax):
// *s_T, and *s_gt = how many candidates exceed it.  IEEE comparisons, so -0
// and +0 are one value.
__device__ __forceinline__ void rank_candidates(const float* cand, int m, int need, int tid, float& s_T,
                                                int32_t& s_gt) {
  if (tid < m) {
    const float vt = cand[tid];
    int gt = 0, ge = 0;
    for (int c0 = 0; c0 < m; c0 += 8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = c0 + u;
        const float vc = cand[min(c, m - 1)];
        gt += (c < m && vc > vt) ? 1 : 0;
        ge += (c < m && vc >= vt) ? 1 : 0;
      }
    }
    if (gt < need && need <= ge) {
      s_T = vt;
      s_gt = gt;
    }
  }
}

// Rows of up to NT*J positions, one work-group of NT threads per row: slot j
// of thread t is position t + NT j.  Every pass runs over all J slots with no
// per-slot branches on the common path (so the loads issue back to back and
// independent slots overlap); the launch picks J for the longest row.  Slots
// past the row end load a copy of the row's last value (clamped offset), which
// cannot move the row's minimum or maximum, and are then set to -inf, which no
// (finite) logit equals.  Values stay fp32: IEEE comparisons already treat -0
// and +0 as one value.
// LDS of one row's selection (NT threads, J slots per thread).
template <int NT, int J>
struct TopkRegShared {
  static constexpr int NW = NT / 64;       // waves
  static constexpr int NWD = NT * J / 32;  // 32-position mask words of a row
  uint32_t hist[kHistWords];               // first-cut bins, padded (bin_word), and 64 spare counters
  uint32_t gtmask[NWD], eqmask[NWD];       // one bit per position
  float cand[kCandMax];
  int32_t cand_pos[kCandMax];
  uint32_t part[NW];
  uint32_t wmin[NW], wmax[NW];
  int32_t s_bin, s_cnt, s_ncand, s_gt;
  float s_T;
};

// Ordered compaction of a row's bit masks (word wd holds positions 32 wd ..
// 32 wd + 31): the positions set in gtmask, then (EQ) the first need_eq set
// in eqmask, in position order; written ascending to o[0, K), -1 after.
// Thread t owns the J positions J t .. J t + J - 1 (every thread has a share,
// so no lane walks more than J bits): one scan of both counts (packed in
// 16-bit halves; a row has at most 32768 positions), then ties are taken in
// position order.
template <int NT, int J, bool EQ>
__device__ __forceinline__ void compact_masks(TopkRegShared<NT, J>& sh, int need_eq, int K, int k,
                                              int32_t* __restrict__ o) {
  constexpr int NW = NT / 64;
  constexpr int NWD = NT * J / 32;
  constexpr int NCH = (J + 31) / 32;  // the thread's bits in 32-bit chunks
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int p0 = J * tid;
  auto chunk = [&](const uint32_t* m, int q) {
    const int pos = p0 + 32 * q, nb = J - 32 * q < 32 ? J - 32 * q : 32;
    const int wd = pos >> 5;
    const uint64_t two = (uint64_t)m[wd] | ((uint64_t)m[min(wd + 1, NWD - 1)] << 32);
    const uint32_t bits = (uint32_t)(two >> (pos & 31));
    return nb < 32 ? bits & ((1u << nb) - 1u) : bits;
  };
  uint32_t gw[NCH], ew[NCH];
  uint32_t packed = 0;
#pragma unroll
  for (int q = 0; q < NCH; ++q) {
    gw[q] = chunk(sh.gtmask, q);
    ew[q] = EQ ? chunk(sh.eqmask, q) : 0u;
    packed += (uint32_t)__popc(gw[q]) | ((uint32_t)__popc(ew[q]) << 16);
  }
  const uint32_t before = block_excl_scan<NW>(packed, lane, wave, sh.part);
  const int gt_before = (int)(before & 0xFFFFu);
  int eq_seen = (int)(before >> 16);
  int out = gt_before + min(eq_seen, need_eq);
#pragma unroll
  for (int q = 0; q < NCH; ++q) {
    uint32_t sel = gw[q];
    if constexpr (EQ) {
      int take = min(max(need_eq - eq_seen, 0), __popc(ew[q]));
      eq_seen += __popc(ew[q]);
      uint32_t e = ew[q];
      for (; take > 0; --take) {
        sel |= e & (~e + 1u);  // lowest remaining tie
        e &= e - 1u;
      }
    }
    while (sel) {
      const int b = __ffs(sel) - 1;
      if (out < K) o[out] = p0 + 32 * q + b;
      ++out;
      sel &= sel - 1u;
    }
  }
  for (int i = K + tid; i < k; i += NT) o[i] = -1;
}

// The rare paths of topk_select.  They keep no copy of the row: every use of
// slot j's value is a fresh reload(j) (the value of slot j, -inf past the row
// end), and their slot loops go eight slots at a time, so they need few
// registers and the common path holds nothing for them.  crowded: the first
// cut's bin c_bin (bins of (v - c_vmin) * c_vscale) holds more than kCandMax
// values; otherwise [lo, hi] is the key interval left to search.  cnt_above
// values lie above the interval.
template <int NT, int J, typename Reload>
__device__ __forceinline__ void topk_select_exact(Reload reload, int ctx, int K, int k, int32_t* __restrict__ o,
                                                  TopkRegShared<NT, J>* shp, bool crowded, int c_bin,
                                                  float c_vmin, float c_vscale, uint32_t lo, uint32_t hi,
                                                  int cnt_above) {
  constexpr int NW = NT / 64;               // waves
  constexpr int NWD = NT * J / 32;          // 32-position mask words of a row
  TopkRegShared<NT, J>& sh = *shp;
  uint32_t* bins = sh.hist + kHistBase;  // the rounds' bins: plain, [0, nb)
  uint32_t* gtmask = sh.gtmask;
  uint32_t* eqmask = sh.eqmask;
  float* cand = sh.cand;
  uint32_t* part = sh.part;
  uint32_t* wmin = sh.wmin;
  uint32_t* wmax = sh.wmax;
  int32_t& s_bin = sh.s_bin;
  int32_t& s_cnt = sh.s_cnt;
  int32_t& s_ncand = sh.s_ncand;
  int32_t& s_gt = sh.s_gt;
  float& s_T = sh.s_T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // eight slots at a time: their loads are in flight together
  auto slots = [&](auto&& f) {
#pragma unroll 8
    for (int j = 0; j < J; ++j) f(j);
  };
  bool found = false;
  float T = key_value(lo);
  if (crowded) {
    uint32_t cmin = 0xFFFFFFFFu, cmax = 0u;
    const float spare = -1.0f - (float)lane;
    slots([&](int j) {
      const float x = reload(j);
      const int bj = (int)__builtin_amdgcn_fmed3f((x - c_vmin) * c_vscale, spare, (float)(kBins - 1));
      const bool in = bj == c_bin;
      const uint32_t kj = order_key(x);
      cmin = min(cmin, in ? kj : 0xFFFFFFFFu);
      cmax = max(cmax, in ? kj : 0u);
    });
    cmin = wave_min_u32(cmin);
    cmax = wave_max_u32(cmax);
    if (lane == 0) {
      wmin[wave] = cmin;
      wmax[wave] = cmax;
    }
    __syncthreads();
    lo = 0xFFFFFFFFu;
    hi = 0u;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      lo = min(lo, wmin[w]);
      hi = max(hi, wmax[w]);
    }
    lo = __builtin_amdgcn_readfirstlane(lo);
    hi = __builtin_amdgcn_readfirstlane(hi);
    __syncthreads();
  }
  // Exact rounds over the order keys in [lo, hi]: cut into at most 2048
  //     bins (a shift of the key offset), keep the bin holding the K-th
  //     largest; when it holds <= kCandMax values they are ranked directly.
  //     (Keys are recomputed from fresh reloads each round.  -inf maps below
  //     every finite key.)
  auto key_of = [&](int j) {
    return order_key(reload(j));
  };
  for (int round = 0; round < 4 && !found && lo < hi; ++round) {
    const uint32_t range = hi - lo;
    const int width = 32 - __clz(range);
    const int shift = width > 11 ? width - 11 : 0;
    const int nb = (int)(range >> shift) + 1;
    for (int b = tid; b < nb; b += NT) bins[b] = 0;
    if (tid == 0) s_ncand = 0;
    __syncthreads();
    slots([&](int j) {
      const uint32_t kj = key_of(j);
      if (kj >= lo && kj <= hi) atomicAdd(&bins[(kj - lo) >> shift], 1u);
    });
    __syncthreads();
    const int b = select_bin<NT>(bins, nb, K, cnt_above, tid, lane, wave, part, s_bin, s_cnt);
    const int m = (int)bins[b];
    cnt_above = s_cnt;
    const uint64_t nlo = (uint64_t)lo + ((uint64_t)b << shift);
    const uint64_t nhi = nlo + ((1ull << shift) - 1ull);
    lo = (uint32_t)nlo;
    hi = (uint32_t)min<uint64_t>(nhi, (uint64_t)hi);
    if (lo < hi && m <= kCandMax) {
      slots([&](int j) {
        const float x = reload(j);
        const uint32_t kj = order_key(x);
        const bool in = (kj >= lo) & (kj <= hi);
        const uint64_t mask = __ballot(in);
        if (mask) {
          const int leader = __ffsll((unsigned long long)mask) - 1;
          int base = 0;
          if (lane == leader) base = atomicAdd(&s_ncand, __popcll(mask));
          base = __shfl(base, leader);
          if (in) cand[base + __popcll(mask & ((1ull << lane) - 1ull))] = x;
        }
      });
      __syncthreads();
      rank_candidates(cand, m, K - cnt_above, tid, s_T, s_gt);
      __syncthreads();
      cnt_above += s_gt;
      T = s_T;
      found = true;
    }
    __syncthreads();  // everyone has read s_bin / hist before the next clear
  }
  if (!found) T = key_value(lo);
  const int need_eq = K - cnt_above;

  // 3. ordered compaction.  Bit masks of the positions with value > T and
  //    value == T (-inf is neither), one ballot per slot: slot j of wave w
  //    covers positions NT j + 64 w .. +63, mask words NT j / 32 + 2 w, + 1.
  slots([&](int j) {
    const float x = reload(j);
    const uint64_t g = __ballot(x > T);
    const uint64_t e = __ballot(x == T);
    if (lane == 0) {
      const int wd = NT / 32 * j + 2 * wave;
      gtmask[wd] = (uint32_t)g;
      gtmask[wd + 1] = (uint32_t)(g >> 32);
      eqmask[wd] = (uint32_t)e;
      eqmask[wd + 1] = (uint32_t)(e >> 32);
    }
  });
  __syncthreads();
  compact_masks<NT, J, true>(sh, need_eq, K, k, o);
}

// The first-cut bin holding the K-th largest value, picked by one wave (the
// caller's wave 0) in two scans: lane l first sums the 32 bins of group
// g = 63 - l (bins 32 g .. 32 g + 31, at words 33 g .. 33 g + 31), lanes in
// descending bin order, so a wave scan counts the values above each group;
// then lanes 0..31 take the 32 bins of the group that holds the K-th largest,
// again in descending order.  Lane 0 writes the bin to s_bin and the count
// of values above it to s_cnt.  (K is at most the number of binned values,
// so each scan has exactly one lane where the count crosses K.)
__device__ __forceinline__ void select_bin_wave(const uint32_t* bins, int K, int lane, int32_t& s_bin,
                                                int32_t& s_cnt) {
  const uint32_t* src = bins + 33 * (63 - lane);
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) local += src[i];
  const uint32_t incl = wave_incl_scan(local, lane);
  const uint64_t hit = __builtin_amdgcn_ballot_w64((int)(incl - local) < K && (int)incl >= K);
  const int l1 = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
  const int g = 63 - l1;
  const uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)(incl - local), l1);
  const uint32_t c = lane < 32 ? bins[33 * g + 31 - lane] : 0u;
  const uint32_t incl2 = wave_incl_scan(c, lane) + above;
  const uint64_t hit2 = __builtin_amdgcn_ballot_w64(lane < 32 && (int)(incl2 - c) < K && (int)incl2 >= K);
  const int l2 = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit2));
  const int cnt = __builtin_amdgcn_readlane((int)(incl2 - c), l2);
  if (lane == 0) {
    s_bin = 32 * g + 31 - l2;
    s_cnt = cnt;
  }
}

// The selection for one row of ctx positions (K = min(k, ctx) < ctx): slot j
// of thread t holds position t + NT j; slots at or past ctx hold a copy of a
// value of the row (they are set to -inf here, after the range).  at(p) reads
// the value of position p < ctx again.  Writes the row's k outputs to o.
//
// Common path (the threshold bin of the first histogram holds at most
// kCandMax values): one pass writes bit masks of the positions in bins above
// the threshold bin and gathers the threshold bin's positions; each
// candidate's rank in (value descending, position ascending) order decides
// whether it is one of the K - above selected from that bin, whose bits join
// the masks; the masks are compacted in position order.  Otherwise exact key
// rounds find the K-th largest value T and positions are compacted from bit
// masks of value > T and value == T.
template <int NT, int J, typename At>
__device__ __forceinline__ void topk_select(float (&v)[J], int ctx, int K, int k, int32_t* __restrict__ o,
                                            TopkRegShared<NT, J>& sh, At&& at) {
  static_assert(NT >= kCandMax && NT <= 1024 && kBins % NT == 0, "threads per row");
  constexpr int NW = NT / 64;       // waves
  constexpr int NWD = NT * J / 32;  // 32-position mask words of a row
  // Rows of up to 32 slots keep their values beside the bins (J more
  // registers fit), so the threshold bin's values are gathered from
  // registers; longer rows keep only the bins and read those values again.
  constexpr bool KEEP = J <= 32;
  uint32_t* bins = sh.hist + kHistBase;  // first-cut bin b counts at bins[bin_word(b)]
  uint32_t* gtmask = sh.gtmask;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  auto slots = [&](auto&& f) {
#pragma unroll
    for (int j = 0; j < J; ++j) f(j);
  };
  // a slot's position, recomputed where it is used (an opaque copy of the
  // thread index), not kept in J registers
  auto pos_of = [&](int j) {
    int t = tid;
    asm volatile("" : "+v"(t));
    return t + j * NT;
  };

  for (int b = tid; b < kHistWords; b += NT) sh.hist[b] = 0;
  if (tid == 0) sh.s_ncand = 0;
  float mn = v[0], mx = v[0];
  slots([&](int j) {
    if (j > 0) {
      mn = fminf(mn, v[j]);
      mx = fmaxf(mx, v[j]);
    }
  });
  {
    const uint32_t kmn = wave_min_u32(order_key(mn)), kmx = wave_max_u32(order_key(mx));
    if (lane == 0) {
      sh.wmin[wave] = kmn;
      sh.wmax[wave] = kmx;
    }
  }
  slots([&](int j) {
    if (tid >= ctx - j * NT) v[j] = -__builtin_inff();  // position tid + NT j past the row end
  });
  __syncthreads();
  // order keys of the row's min and max: lane w holds wave w's, one wave
  // reduction (its result is uniform: the branches on it are scalar)
  uint32_t lo = wave_min_u32(lane < NW ? sh.wmin[lane] : 0xFFFFFFFFu);
  uint32_t hi = wave_max_u32(lane < NW ? sh.wmax[lane] : 0u);
  int cnt_above = 0;     // values above the current search interval
  bool crowded = false;  // first-cut bin c_bin holds more than kCandMax values
  int c_bin = 0;
  float c_vmin = 0.0f, c_vscale = 0.0f;

  // 2. threshold search.
  // 2a. First cut, linear in value: bin(v) = min(2047, (v - vmin) * (2048 /
  //     (vmax - vmin))), each step correctly rounded, is monotone in v, so the
  //     bin holding the K-th largest value holds a contiguous value interval,
  //     and ties share a bin.  (Bins linear in the bit pattern would be
  //     logarithmic in value and pile a row onto a few bins.)  v - vmin >= 0
  //     for every value of the row, and -inf (past the row end) gives
  //     -1 - lane: the lane's spare counter, never a bin, so no per-slot test
  //     and no pile-up of atomics on one bin.  Skipped when the value range is
  //     not a finite positive float.
  if (lo < hi) {
    const float vmin = key_value(lo), vmax = key_value(hi);
    const float vrange = vmax - vmin;
    const float vscale = (float)kBins / vrange;
    if (vrange > 0.0f && vrange <= 3.4028234664e38f && vscale <= 3.4028234664e38f) {
      const float spare = -1.0f - (float)lane;
      int bn[KEEP ? J : 1];  // the slots' bins (KEEP), else held in v
      slots([&](int j) {
        const int b = (int)__builtin_amdgcn_fmed3f((v[j] - vmin) * vscale, spare, (float)(kBins - 1));
        atomicAdd(&bins[bin_word(b)], 1u);
        if constexpr (KEEP) bn[j] = b;
        else v[j] = __int_as_float(b);  // the slot's bin from here on
      });
      auto bin_of = [&](int j) {
        if constexpr (KEEP) return bn[j];
        else return __float_as_int(v[j]);
      };
      __syncthreads();
      if (wave == 0) select_bin_wave(bins, K, lane, sh.s_bin, sh.s_cnt);
      __syncthreads();
      const int bsel = __builtin_amdgcn_readfirstlane(sh.s_bin);
      const int m = __builtin_amdgcn_readfirstlane((int)bins[bin_word(bsel)]);
      cnt_above = __builtin_amdgcn_readfirstlane(sh.s_cnt);
      if (m <= kCandMax) {
        // 2b. Bit masks of the positions in bins above bsel (lane 2 j + h of
        //     each wave collects half h of slot j's ballot, then every lane
        //     writes its word: slot j of wave w covers positions NT j + 64 w
        //     .. + 63, mask words NT j / 32 + 2 w, + 1), and the positions
        //     (and values, KEEP) of bin bsel.
        const int need = K - cnt_above;  // 1 <= need <= m
        constexpr int NMV = (2 * J + 63) / 64;
        uint32_t gw[NMV];
#pragma unroll
        for (int r = 0; r < NMV; ++r) gw[r] = 0;
        int bselv = bsel;
        slots([&](int j) {
          const int b = bin_of(j);
          const uint64_t gm = __builtin_amdgcn_ballot_w64(b > bselv);
          if (__builtin_amdgcn_ballot_w64(b == bselv)) {  // wave-uniform, rare
            if (b == bselv) {
              const int idx = atomicAdd(&sh.s_ncand, 1);
              sh.cand_pos[idx] = pos_of(j);
              if constexpr (KEEP) sh.cand[idx] = v[j];
            }
          }
          const uint32_t glo = (uint32_t)gm, ghi = (uint32_t)(gm >> 32);
          asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(gw[(2 * j) / 64]) : "s"(glo), "n"((2 * j) % 64));
          asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(gw[(2 * j + 1) / 64]) : "s"(ghi), "n"((2 * j + 1) % 64));
          // one slot at a time: the next slot's compares take bselv through
          // this opaque copy, so the compiler does not compute every slot's
          // ballots up front
          asm volatile("" : "+s"(bselv) : "v"(gw[(2 * j) / 64]));
        });
#pragma unroll
        for (int r = 0; r < NMV; ++r) {
          const int e = 64 * r + lane;  // 2 j + h
          if (e < 2 * J) gtmask[NT / 32 * (e >> 1) + 2 * wave + (e & 1)] = gw[r];
        }
        __syncthreads();
        // 2c. A candidate is selected when fewer than need candidates come
        //     before it in (value descending, position ascending) order; its
        //     bit joins gtmask.
        if (m <= 64) {
          // one wave: candidate c in lane c, compared through lane reads
          if (wave == 0) {
            const int pt = lane < m ? sh.cand_pos[lane] : 0;
            float vt = 0.0f;
            if constexpr (KEEP) vt = lane < m ? sh.cand[lane] : 0.0f;
            else vt = lane < m ? at(pt) : 0.0f;
            int before = 0;
            for (int c = 0; c < m; ++c) {
              const float vc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vt), c));
              const int pc = __builtin_amdgcn_readlane(pt, c);
              before += (vc > vt || (vc == vt && pc < pt)) ? 1 : 0;
            }
            if (lane < m && before < need) atomicOr(&gtmask[pt >> 5], 1u << (pt & 31));
          }
        } else {
          if constexpr (!KEEP) {
            if (tid < m) sh.cand[tid] = at(sh.cand_pos[tid]);
            __syncthreads();
          }
          if (tid < m) {
            const float vt = sh.cand[tid];
            const int pt = sh.cand_pos[tid];
            int before = 0;
            for (int c0 = 0; c0 < m; c0 += 4) {
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                const int c = min(c0 + u, m - 1);
                const float vc = sh.cand[c];
                const int pc = sh.cand_pos[c];
                before += (c0 + u < m && (vc > vt || (vc == vt && pc < pt))) ? 1 : 0;
              }
            }
            if (before < need) atomicOr(&gtmask[pt >> 5], 1u << (pt & 31));
          }
        }
        __syncthreads();
        // 2d. The selected positions, ascending.
        compact_masks<NT, J, false>(sh, 0, K, k, o);
        return;
      }
      crowded = true;  // the bin needs exact key rounds, over its key interval
      c_bin = bsel;
      c_vmin = vmin;
      c_vscale = vscale;
    }
  }
  topk_select_exact<NT, J>(
      [&](int j) {
        const int p = pos_of(j);  // a fresh read: not merged with the first one
        const float x = at(min(p, ctx - 1));
        return p < ctx ? x : -__builtin_inff();
      },
      ctx, K, k, o, &sh, crowded, c_bin, c_vmin, c_vscale, lo, hi, cnt_above);
}

}  // namespace fp4idx
