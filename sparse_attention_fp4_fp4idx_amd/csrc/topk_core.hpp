// Top-k selection over one row held in registers (gfx950), shared by the
// top-k kernels and the fused logits + top-k kernel.  See topk.hip for the
// method.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4idx {

constexpr int kBins = 2048;

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
  uint32_t before = incl - v;
#pragma unroll
  for (int w = 0; w < NW; ++w) before += w < wave ? part[w] : 0u;
  return before;
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
// branches (so the loads issue back to back and independent slots overlap);
// the launch picks J for the longest row.  Slots past the row end load a copy
// of the row's last value (clamped offset), which cannot move the row's
// minimum or maximum, and are then set to -inf, which no (finite) logit
// equals.  Values stay fp32: IEEE comparisons already treat -0 and +0 as one
// value.
// LDS of one row's selection (NT threads, J slots per thread).
template <int NT, int J>
struct TopkRegShared {
  static constexpr int NW = NT / 64;       // waves
  static constexpr int NWD = NT * J / 32;  // 32-position mask words of a row
  uint32_t hist[kBins + 64];               // + 64 spare counters (one per lane)
  uint32_t gtmask[NWD], eqmask[NWD];       // one bit per position
  float cand[kCandMax];
  uint32_t part[NW];
  uint32_t wmin[NW], wmax[NW];
  int32_t s_bin, s_cnt, s_ncand, s_gt;
  float s_T;
};

// The selection for one row of ctx positions (K = min(k, ctx) < ctx): slot j
// of thread t holds position t + NT j; slots at or past ctx hold a copy of a
// value of the row (they are set to -inf here, after the range).  Writes the
// row's k outputs to o.
template <int NT, int J>
__device__ __forceinline__ void topk_select(float (&v)[J], int ctx, int K, int k, int32_t* __restrict__ o,
                                            TopkRegShared<NT, J>& sh) {
  static_assert(NT >= kCandMax && NT <= 1024 && kBins % NT == 0, "threads per row");
  constexpr int NW = NT / 64;               // waves
  constexpr int NWD = NT * J / 32;          // 32-position mask words of a row
  constexpr int WPT = (NWD + NT - 1) / NT;  // mask words owned by a thread
  uint32_t* hist = sh.hist;
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
  const int nj = (ctx + NT - 1) / NT;  // 1 <= nj <= J
  auto slots = [&](auto&& f) {
#pragma unroll
    for (int j = 0; j < J; ++j) f(j);
  };

  for (int b = tid; b < kBins; b += NT) hist[b] = 0;
  if (tid == 0) s_ncand = 0;
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
      wmin[wave] = kmn;
      wmax[wave] = kmx;
    }
  }
  slots([&](int j) {
    if (tid + j * NT >= ctx) v[j] = -__builtin_inff();
  });
  __syncthreads();
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;  // order keys of the row's min and max
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    lo = min(lo, wmin[w]);
    hi = max(hi, wmax[w]);
  }
  int cnt_above = 0;  // values above the current search interval
  bool found = false;
  float T = key_value(lo);

  // 2. threshold search: the K-th largest value T.
  // 2a. First cut, linear in value: bin(v) = min(2047, (v - vmin) * 2048 /
  //     (vmax - vmin)) is monotone in v, so the bin holding the K-th largest
  //     value holds a contiguous value interval, and ties share a bin.  (Bins
  //     linear in the bit pattern would be logarithmic in value and pile a
  //     row onto a few bins.)  Skipped when the value range is not a finite
  //     positive float.
  if (lo < hi) {
    const float vmin = key_value(lo), vmax = key_value(hi);
    const float vrange = vmax - vmin;
    const float vscale = (float)kBins / vrange;
    if (vrange > 0.0f && vrange <= 3.4028234664e38f && vscale <= 3.4028234664e38f) {
      // bin of a value: one correctly rounded fma is monotone in x, and the
      // clamp before the conversion keeps it defined for -inf (bin 0)
      const float voff = -vmin * vscale;
      auto bin_of = [&](float x) {
        return (int)__builtin_amdgcn_fmed3f(__builtin_fmaf(x, vscale, voff), 0.0f, (float)(kBins - 1));
      };
      // slots past the row end count into a per-lane spare counter that is
      // never read: no branch, and no pile-up of atomics on one bin
      slots([&](int j) { atomicAdd(&hist[v[j] >= vmin ? bin_of(v[j]) : kBins + lane], 1u); });
      __syncthreads();
      const int bsel = select_bin<NT>(hist, kBins, K, cnt_above, tid, lane, wave, part, s_bin, s_cnt);
      const int m = (int)hist[bsel];
      cnt_above = s_cnt;
      // The bins (and the row-end tests) are recomputed below rather than
      // kept from the histogram pass (J more registers); the opaque copies
      // stop the compiler from keeping them.  Same operands, same bins.
      float vscale2 = vscale, vmin2 = vmin;
      asm volatile("" : "+v"(vscale2), "+v"(vmin2));
      auto in_bin = [&](int j) {
        const int bj = (int)__builtin_amdgcn_fmed3f(__builtin_fmaf(v[j], vscale2, voff), 0.0f, (float)(kBins - 1));
        return (bj == bsel) & (v[j] >= vmin2);
      };
      if (m <= kCandMax) {
        // gather the bin's values and rank them
        slots([&](int j) {
          const bool in = in_bin(j);
          const uint64_t mask = __ballot(in);
          if (mask) {
            const int leader = __ffsll((unsigned long long)mask) - 1;
            int base = 0;
            if (lane == leader) base = atomicAdd(&s_ncand, __popcll(mask));
            base = __shfl(base, leader);
            if (in) cand[base + __popcll(mask & ((1ull << lane) - 1ull))] = v[j];
          }
        });
        __syncthreads();
        rank_candidates(cand, m, K - cnt_above, tid, s_T, s_gt);
        __syncthreads();
        cnt_above += s_gt;
        T = s_T;
        found = true;
      } else {
        // a crowded bin: exact key rounds below, over its key interval
        uint32_t cmin = 0xFFFFFFFFu, cmax = 0u;
        slots([&](int j) {
          const bool in = in_bin(j);
          const uint32_t kj = order_key(v[j]);
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
      }
      __syncthreads();
    }
  }
  // 2b. Exact rounds over the order keys in [lo, hi]: cut into at most 2048
  //     bins (a shift of the key offset), keep the bin holding the K-th
  //     largest; when it holds <= kCandMax values they are ranked directly.
  //     (Keys are recomputed each round; the opaque copy keeps the compiler
  //     from hoisting J of them out of the loop.  -inf maps below every
  //     finite key.)
  auto key_of = [&](int j) {
    float x = v[j];
    asm volatile("" : "+v"(x));
    return order_key(x);
  };
  for (int round = 0; round < 4 && !found && lo < hi; ++round) {
    const uint32_t range = hi - lo;
    const int width = 32 - __clz(range);
    const int shift = width > 11 ? width - 11 : 0;
    const int nb = (int)(range >> shift) + 1;
    for (int b = tid; b < nb; b += NT) hist[b] = 0;
    if (tid == 0) s_ncand = 0;
    __syncthreads();
    slots([&](int j) {
      const uint32_t kj = key_of(j);
      if (kj >= lo && kj <= hi) atomicAdd(&hist[(kj - lo) >> shift], 1u);
    });
    __syncthreads();
    const int b = select_bin<NT>(hist, nb, K, cnt_above, tid, lane, wave, part, s_bin, s_cnt);
    const int m = (int)hist[b];
    cnt_above = s_cnt;
    const uint64_t nlo = (uint64_t)lo + ((uint64_t)b << shift);
    const uint64_t nhi = nlo + ((1ull << shift) - 1ull);
    lo = (uint32_t)nlo;
    hi = (uint32_t)min<uint64_t>(nhi, (uint64_t)hi);
    if (lo < hi && m <= kCandMax) {
      slots([&](int j) {
        const uint32_t kj = key_of(j);
        const bool in = (kj >= lo) & (kj <= hi);
        const uint64_t mask = __ballot(in);
        if (mask) {
          const int leader = __ffsll((unsigned long long)mask) - 1;
          int base = 0;
          if (lane == leader) base = atomicAdd(&s_ncand, __popcll(mask));
          base = __shfl(base, leader);
          if (in) cand[base + __popcll(mask & ((1ull << lane) - 1ull))] = v[j];
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
    const uint64_t g = __ballot(v[j] > T);
    const uint64_t e = __ballot(v[j] == T);
    if (lane == 0) {
      const int wd = NT / 32 * j + 2 * wave;
      gtmask[wd] = (uint32_t)g;
      gtmask[wd + 1] = (uint32_t)(g >> 32);
      eqmask[wd] = (uint32_t)e;
      eqmask[wd + 1] = (uint32_t)(e >> 32);
    }
  });
  __syncthreads();
  //    Thread t owns the 32*WPT consecutive positions of words WPT t ..: one
  //    scan of both counts (packed in 16-bit halves; a row has at most 32768
  //    positions), then ties are taken in position order.
  const int nwd = nj * (NT / 32);  // words past the last slot holding positions are all zero
  uint32_t gw[WPT], ew[WPT];
  uint32_t packed = 0;
#pragma unroll
  for (int u = 0; u < WPT; ++u) {
    const int wd = WPT * tid + u;
    gw[u] = wd < nwd ? gtmask[wd] : 0u;
    ew[u] = wd < nwd ? eqmask[wd] : 0u;
    packed += (uint32_t)__popc(gw[u]) | ((uint32_t)__popc(ew[u]) << 16);
  }
  const uint32_t before = block_excl_scan<NW>(packed, lane, wave, part);
  const int gt_before = (int)(before & 0xFFFFu);
  int eq_seen = (int)(before >> 16);
  int out = gt_before + min(eq_seen, need_eq);
#pragma unroll
  for (int u = 0; u < WPT; ++u) {
    int take = min(max(need_eq - eq_seen, 0), __popc(ew[u]));
    eq_seen += __popc(ew[u]);
    uint32_t sel = gw[u];
    uint32_t e = ew[u];
    for (; take > 0; --take) {
      sel |= e & (~e + 1u);  // lowest remaining tie
      e &= e - 1u;
    }
    while (sel) {
      const int b = __ffs(sel) - 1;
      if (out < K) o[out] = 32 * (WPT * tid + u) + b;
      ++out;
      sel &= sel - 1u;
    }
  }
  for (int i = K + tid; i < k; i += NT) o[i] = -1;
}

}  // namespace fp4idx
