// Position-ordered top-k over logits rows on gfx950.
//
// "[AMD] DeepSeek-V4.1-Flash on MI350X (gfx950)", Changes (sorted top-k
// selection) and Historical results (decode selections come back in
// token-position order rather than pool-slot order).  Result for a row: the
// K = min(k, ctx) positions with the largest values, ties resolved toward the
// lower position, written in ascending position order and padded with -1.
//
// Rows up to 32768 positions (topk_reg_kernel), one 1024-thread work-group
// per row, everything in registers and a few KiB of LDS:
//  1. Coalesced load of the row; slot j of thread t is position t + 1024 j
//     (16 or 32 slots), mapped to an order-preserving 32-bit key (-0 folded
//     onto +0; slots past the row end hold key 0, which no finite value has).
//  2. Threshold search for the K-th largest key T: one histogram of 2048 bins
//     linear in value between the row's min and max, then the chosen bin's
//     keys (typically a handful) are ranked directly; exact key-space rounds
//     (bins of the key offset) cover bins with more than 256 keys.
//  3. Ordered compaction: wave ballots write bit masks of the positions with
//     key > T and key == T; thread t owns the 32 positions of mask word t, one
//     block scan of the two popcounts gives its output offset, and ties are
//     taken in position order until K.
// Longer rows (topk_long_kernel) re-read the logits in each pass, with four
// waves per row and ballot-based compaction.
#include "launch.hpp"

namespace fp4idx {

constexpr int kTopkThreads = 256;
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

struct TopkShared {
  uint32_t lo, hi;
  int32_t cnt_above;
  int32_t bin;
  int32_t wave_part[4];
  int32_t wave_gt[4];
  int32_t wave_eq[4];
  uint32_t kmin[4], kmax[4];
};

template <bool KEYS_IN_LDS>
__global__ __launch_bounds__(kTopkThreads) void topk_long_kernel(const float* __restrict__ logits, int64_t stride,
                                                            const int32_t* __restrict__ row_ctx, int k,
                                                            int32_t* __restrict__ out_idx) {
  // Loads are issued in batches (kLoadBatch per thread, kPassBatch per lane in
  // the ordered passes) so that memory latency is paid once per batch, not once
  // per element.
  constexpr int kLoadBatch = 32;
  constexpr int kPassBatch = 8;
  extern __shared__ uint32_t smem[];
  __shared__ TopkShared sh;
  uint32_t* hist = smem;            // [kBins]
  uint32_t* keys = smem + kBins;    // [ctx] when KEYS_IN_LDS
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ctx = (int)min<int64_t>(max(row_ctx[row], 0), stride);  // in-row reads whatever the value
  const float* src = logits + row * stride;
  int32_t* o = out_idx + row * (int64_t)k;
  const int K = min(k, ctx);

  if (K == ctx) {  // everything is selected (includes ctx == 0)
    for (int i = tid; i < k; i += kTopkThreads) o[i] = i < ctx ? i : -1;
    return;
  }

  auto key_at = [&](int i) -> uint32_t { return KEYS_IN_LDS ? keys[i] : order_key(src[i]); };

  // 1. load keys, key range
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  for (int base = 0; base < ctx; base += kTopkThreads * kLoadBatch) {
    float v[kLoadBatch];
#pragma unroll
    for (int j = 0; j < kLoadBatch; ++j) {
      const int i = base + j * kTopkThreads + tid;
      v[j] = i < ctx ? __builtin_nontemporal_load(src + i) : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < kLoadBatch; ++j) {
      const int i = base + j * kTopkThreads + tid;
      if (i < ctx) {
        const uint32_t kk = order_key(v[j]);
        if (KEYS_IN_LDS) keys[i] = kk;
        kmin = min(kmin, kk);
        kmax = max(kmax, kk);
      }
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
  }
  if (lane == 0) {
    sh.kmin[wave] = kmin;
    sh.kmax[wave] = kmax;
  }
  __syncthreads();
  uint32_t lo = min(min(sh.kmin[0], sh.kmin[1]), min(sh.kmin[2], sh.kmin[3]));
  uint32_t hi = max(max(sh.kmax[0], sh.kmax[1]), max(sh.kmax[2], sh.kmax[3]));
  int cnt_above = 0;  // keys > hi

  // 2. threshold search (each round shrinks the key range by 2^11 or ends it;
  //    32-bit keys need at most 3 rounds, the cap only bounds the loop)
  for (int round = 0; round < 4 && lo < hi; ++round) {
    const uint32_t range = hi - lo;
    const int width = 32 - __clz(range);
    const int shift = width > 11 ? width - 11 : 0;
    const int nb = (int)(range >> shift) + 1;
    for (int b = tid; b < nb; b += kTopkThreads) hist[b] = 0;
    if (tid == 0) {
      sh.bin = nb - 1;
      sh.cnt_above = cnt_above;
    }
    __syncthreads();
    for (int base = 0; base < ctx; base += kTopkThreads * kPassBatch) {
      uint32_t kv[kPassBatch];
#pragma unroll
      for (int j = 0; j < kPassBatch; ++j) {
        const int i = base + j * kTopkThreads + tid;
        kv[j] = i < ctx ? key_at(i) : 0u;
      }
#pragma unroll
      for (int j = 0; j < kPassBatch; ++j) {
        const int i = base + j * kTopkThreads + tid;
        if (i < ctx && kv[j] >= lo && kv[j] <= hi) atomicAdd(&hist[(kv[j] - lo) >> shift], 1u);
      }
    }
    __syncthreads();
    // suffix counts from the top bin down: thread t owns reversed bins [8t, 8t+8)
    int local = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int b = nb - 1 - (tid * 8 + j);
      if (b >= 0) local += (int)hist[b];
    }
    int incl = local;  // inclusive prefix over threads within the wave
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    if (lane == 63) sh.wave_part[wave] = incl;
    __syncthreads();
    int before = cnt_above + incl - local;
    for (int w2 = 0; w2 < wave; ++w2) before += sh.wave_part[w2];
    if (before < K && before + local >= K) {
      int acc = before;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int b = nb - 1 - (tid * 8 + j);
        if (b < 0) break;
        const int c = (int)hist[b];
        if (acc + c >= K) {
          sh.bin = b;
          sh.cnt_above = acc;
          break;
        }
        acc += c;
      }
    }
    __syncthreads();
    const uint32_t b = (uint32_t)sh.bin;
    cnt_above = sh.cnt_above;
    const uint64_t nlo = (uint64_t)lo + ((uint64_t)b << shift);
    const uint64_t nhi = nlo + ((1ull << shift) - 1ull);
    lo = (uint32_t)nlo;
    hi = (uint32_t)min<uint64_t>(nhi, (uint64_t)hi);
    __syncthreads();  // hist is cleared again next round
  }
  const uint32_t T = lo;
  const int need_eq = K - cnt_above;

  // 3. ordered compaction: wave w owns positions [q0, q1), walked in batches
  //    of kPassBatch x 64 consecutive positions.
  const int per = (ctx + 3) / 4;
  const int q0 = min(ctx, wave * per), q1 = min(ctx, q0 + per);
  int n_gt = 0, n_eq = 0;
  for (int base = q0; base < q1; base += 64 * kPassBatch) {
    uint32_t kv[kPassBatch];
#pragma unroll
    for (int u = 0; u < kPassBatch; ++u) {
      const int i = base + u * 64 + lane;
      kv[u] = i < q1 ? key_at(i) : 0u;
    }
#pragma unroll
    for (int u = 0; u < kPassBatch; ++u) {
      const bool in = base + u * 64 + lane < q1;
      n_gt += __popcll(__ballot(in && kv[u] > T));
      n_eq += __popcll(__ballot(in && kv[u] == T));
    }
  }
  if (lane == 0) {
    sh.wave_gt[wave] = n_gt;
    sh.wave_eq[wave] = n_eq;
  }
  __syncthreads();
  int eq_before = 0, sel_before = 0;
  for (int w2 = 0; w2 < wave; ++w2) {
    const int e = sh.wave_eq[w2];
    const int take = max(0, min(e, need_eq - eq_before));
    sel_before += sh.wave_gt[w2] + take;
    eq_before += e;
  }
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  for (int base = q0; base < q1; base += 64 * kPassBatch) {
    uint32_t kv[kPassBatch];
#pragma unroll
    for (int u = 0; u < kPassBatch; ++u) {
      const int i = base + u * 64 + lane;
      kv[u] = i < q1 ? key_at(i) : 0u;
    }
#pragma unroll
    for (int u = 0; u < kPassBatch; ++u) {
      const int i = base + u * 64 + lane;
      const bool in = i < q1;
      const bool gt = in && kv[u] > T;
      const bool eq = in && kv[u] == T;
      const uint64_t eq_mask = __ballot(eq);
      const int eq_rank = eq_before + __popcll(eq_mask & lt_mask);
      const bool sel = gt || (eq && eq_rank < need_eq);
      const uint64_t sel_mask = __ballot(sel);
      const int slot = sel_before + __popcll(sel_mask & lt_mask);
      if (sel && slot < K) o[slot] = i;
      sel_before += __popcll(sel_mask);
      eq_before += __popcll(eq_mask);
    }
  }
  for (int i = K + tid; i < k; i += kTopkThreads) o[i] = -1;
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
template <int NT, int J>
__global__ __launch_bounds__(NT) void topk_reg_kernel(const float* __restrict__ logits, int64_t stride,
                                                      const int32_t* __restrict__ row_ctx, int k,
                                                      int32_t* __restrict__ out_idx) {
  static_assert(NT >= kCandMax && NT <= 1024 && kBins % NT == 0, "threads per row");
  constexpr int NW = NT / 64;               // waves
  constexpr int NWD = NT * J / 32;          // 32-position mask words of a row
  constexpr int WPT = (NWD + NT - 1) / NT;  // mask words owned by a thread
  __shared__ uint32_t hist[kBins + 64];     // + 64 spare counters (one per lane)
  __shared__ uint32_t gtmask[NWD], eqmask[NWD];  // one bit per position
  __shared__ float cand[kCandMax];
  __shared__ uint32_t part[NW];
  __shared__ uint32_t wmin[NW], wmax[NW];
  __shared__ int32_t s_bin, s_cnt, s_ncand, s_gt;
  __shared__ float s_T;
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // (device values beyond the documented bounds are clamped so that every
  // access stays inside the row and the registers)
  const int ctx = min(max(row_ctx[row], 0), (int)min<int64_t>(stride, (int64_t)J * NT));
  const int K = min(k, ctx);
  int32_t* o = out_idx + row * (int64_t)k;
  if (K == ctx) {  // everything is selected (includes ctx == 0)
    for (int i = tid; i < k; i += NT) o[i] = i < ctx ? i : -1;
    return;
  }
  const int nj = (ctx + NT - 1) / NT;  // 1 <= nj <= J
  auto slots = [&](auto&& f) {
#pragma unroll
    for (int j = 0; j < J; ++j) f(j);
  };

  // 1. load (uniform row base, one 32-bit offset register per load), range
  const char* srcb = reinterpret_cast<const char*>(logits + row * stride);
  const uint32_t off0 = 4u * (uint32_t)tid, off_last = 4u * (uint32_t)(ctx - 1);
  float v[J];
  slots([&](int j) {
    const uint32_t off = min(off0 + 4u * (uint32_t)(j * NT), off_last);
    v[j] = __builtin_nontemporal_load(reinterpret_cast<const float*>(srcb + off));
  });
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

template <int NT, int J>
static hipError_t launch_reg(const float* logits, int64_t n_rows, int64_t logits_stride, const int32_t* row_ctx,
                             int32_t k, int32_t* out_idx, hipStream_t stream) {
  return launch(topk_reg_kernel<NT, J>, dim3((unsigned)n_rows), dim3(NT), 0, stream, logits, logits_stride, row_ctx, k,
                out_idx);
}

// Rows in registers: a few rows (at most one per CU) take 1024 threads each,
// the shortest path for one row; more rows take 512 threads each, so that two
// rows share a CU and one row's barriers overlap the other's work (up to
// 24,576 positions; longer rows need too many registers for two).  J covers
// the longest row with little slack (every slot is processed).
constexpr int64_t kRowsPerCuSwitch = 256;

hipError_t launch_topk(const float* logits, int64_t n_rows, int64_t logits_stride, const int32_t* row_ctx, int32_t k,
                       int32_t* out_idx, int64_t max_ctx, hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  if (n_rows > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  if (max_ctx <= kRegMaxCtx && (n_rows <= kRowsPerCuSwitch || max_ctx > 24576)) {
    if (max_ctx <= 8192) return launch_reg<1024, 8>(logits, n_rows, logits_stride, row_ctx, k, out_idx, stream);
    if (max_ctx <= 16384) return launch_reg<1024, 16>(logits, n_rows, logits_stride, row_ctx, k, out_idx, stream);
    if (max_ctx <= 24576) return launch_reg<1024, 24>(logits, n_rows, logits_stride, row_ctx, k, out_idx, stream);
    return launch_reg<1024, 32>(logits, n_rows, logits_stride, row_ctx, k, out_idx, stream);
  }
  if (max_ctx <= 24576) {  // two 512-thread rows per CU fit the registers up to here
    if (max_ctx <= 8192) return launch_reg<512, 16>(logits, n_rows, logits_stride, row_ctx, k, out_idx, stream);
    if (max_ctx <= 12288) return launch_reg<512, 24>(logits, n_rows, logits_stride, row_ctx, k, out_idx, stream);
    if (max_ctx <= 16384) return launch_reg<512, 32>(logits, n_rows, logits_stride, row_ctx, k, out_idx, stream);
    if (max_ctx <= 18432) return launch_reg<512, 36>(logits, n_rows, logits_stride, row_ctx, k, out_idx, stream);
    return launch_reg<512, 48>(logits, n_rows, logits_stride, row_ctx, k, out_idx, stream);
  }
  return launch(topk_long_kernel<false>, dim3((unsigned)n_rows), dim3(kTopkThreads), kBins * sizeof(uint32_t), stream,
                logits, logits_stride, row_ctx, k, out_idx);
}

}  // namespace fp4idx
