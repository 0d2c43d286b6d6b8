// Position-ordered top-k over logits rows on gfx950.
//
// "[AMD] DeepSeek-V4.1-Flash on MI350X (gfx950)", Changes (sorted top-k
// selection) and Historical results (decode top-k is ordered by position, not
// by KV slot).  Result for a row: the K = min(k, ctx) positions with the
// largest values, ties resolved toward the lower position, written in
// ascending position order and padded with -1.
//
// Rows up to 32768 positions (topk_reg_kernel), one 1024-thread work-group
// per row:
//  1. Coalesced load of the row (32 loads in flight per thread), each value
//     mapped to an order-preserving 32-bit key (-0 folded onto +0).  Every
//     thread keeps its 32 keys (positions tid + 1024*j) in registers and also
//     writes them to LDS at padded addresses for step 3.
//  2. Exact threshold search on the register keys: the key range [lo, hi]
//     holding the K-th largest key is cut into at most 2048 equal bins (a
//     shift of the key offset), an LDS histogram of the in-range keys picks
//     the bin holding the K-th largest, and the range shrinks to that bin.  At
//     most three rounds reach a single key T; the count above T is tracked.
//  3. Ordered compaction: thread t reads a contiguous segment of ceil(ctx/1024)
//     positions back from LDS (one pad word per 32 spreads the reads over the
//     banks), counts keys > T and == T, one block-wide scan of both counts gives
//     every thread its output offset, and keys == T are taken in position order
//     until K.
// Longer rows (topk_long_kernel) keep the keys in LDS or re-read them from
// memory, with four waves per row and ballot-based compaction.
#include "launch.hpp"

namespace fp4idx {

constexpr int kTopkThreads = 256;
constexpr int kBins = 2048;

__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;  // -0 and +0 are the same value
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
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
  const int ctx = row_ctx[row];
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


constexpr int kRegThreads = 1024;
constexpr int kRegKeys = 32;
constexpr int kRegWaves = kRegThreads / 64;
constexpr int64_t kRegMaxCtx = (int64_t)kRegThreads * kRegKeys;

__device__ __forceinline__ int lds_pad(int p) { return p + (p >> 5); }

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t u = (uint32_t)__shfl_up((int)v, off);
    if (lane >= off) v += u;
  }
  return v;
}

__global__ __launch_bounds__(kRegThreads) void topk_reg_kernel(const float* __restrict__ logits, int64_t stride,
                                                               const int32_t* __restrict__ row_ctx, int k,
                                                               int32_t* __restrict__ out_idx) {
  extern __shared__ uint32_t lkeys[];  // padded copy of the row's keys
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t wpart[kRegWaves];
  __shared__ uint32_t wmin[kRegWaves], wmax[kRegWaves];
  __shared__ int32_t s_bin, s_cnt;
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ctx = row_ctx[row];
  const int K = min(k, ctx);
  int32_t* o = out_idx + row * (int64_t)k;
  if (K == ctx) {  // everything is selected (includes ctx == 0)
    for (int i = tid; i < k; i += kRegThreads) o[i] = i < ctx ? i : -1;
    return;
  }
  const float* src = logits + row * stride;

  // 1. load.  Slot j of this thread is position tid + 1024 j; slots past the
  //    row's end are skipped wave by wave (jw = slots any lane of the wave uses).
  const int jw = min(kRegKeys, max(0, (ctx - wave * 64 + kRegThreads - 1) / kRegThreads));
  float v[kRegKeys];
#pragma unroll
  for (int j = 0; j < kRegKeys; ++j) {
    const int p = tid + j * kRegThreads;
    v[j] = 0.0f;
    if (j < jw) v[j] = p < ctx ? __builtin_nontemporal_load(src + p) : 0.0f;
  }
  uint32_t key[kRegKeys];
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < kRegKeys; ++j) {
    const int p = tid + j * kRegThreads;
    key[j] = order_key(v[j]);
    if (j < jw && p < ctx) {
      lkeys[lds_pad(p)] = key[j];
      kmin = min(kmin, key[j]);
      kmax = max(kmax, key[j]);
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
  }
  if (lane == 0) {
    wmin[wave] = kmin;
    wmax[wave] = kmax;
  }
  __syncthreads();
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int w = 0; w < kRegWaves; ++w) {
    lo = min(lo, wmin[w]);
    hi = max(hi, wmax[w]);
  }
  int cnt_above = 0;  // keys > hi

  // 2. threshold search (at most 3 rounds for 32-bit keys; the cap bounds it)
  for (int round = 0; round < 4 && lo < hi; ++round) {
    const uint32_t range = hi - lo;
    const int width = 32 - __clz(range);
    const int shift = width > 11 ? width - 11 : 0;
    const int nb = (int)(range >> shift) + 1;
    for (int b = tid; b < nb; b += kRegThreads) hist[b] = 0;
    if (tid == 0) {
      s_bin = nb - 1;
      s_cnt = cnt_above;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kRegKeys; ++j) {
      if (j < jw) {
        const int p = tid + j * kRegThreads;
        if (p < ctx && key[j] >= lo && key[j] <= hi) atomicAdd(&hist[(key[j] - lo) >> shift], 1u);
      }
    }
    __syncthreads();
    // counts from the top bin down; thread t owns reversed bins 2t, 2t+1
    const int b0 = nb - 1 - 2 * tid, b1 = b0 - 1;
    const uint32_t c0 = b0 >= 0 ? hist[b0] : 0u, c1 = b1 >= 0 ? hist[b1] : 0u;
    const uint32_t local = c0 + c1;
    const uint32_t incl = wave_incl_scan(local, lane);
    if (lane == 63) wpart[wave] = incl;
    __syncthreads();
    int before = cnt_above + (int)(incl - local);
    for (int w = 0; w < wave; ++w) before += (int)wpart[w];
    if (before < K && before + (int)local >= K) {
      if (before + (int)c0 >= K) {
        s_bin = b0;
        s_cnt = before;
      } else {
        s_bin = b1;
        s_cnt = before + (int)c0;
      }
    }
    __syncthreads();
    const uint32_t b = (uint32_t)s_bin;
    cnt_above = s_cnt;
    const uint64_t nlo = (uint64_t)lo + ((uint64_t)b << shift);
    const uint64_t nhi = nlo + ((1ull << shift) - 1ull);
    lo = (uint32_t)nlo;
    hi = (uint32_t)min<uint64_t>(nhi, (uint64_t)hi);
    __syncthreads();  // everyone has read s_bin / hist before the next clear
  }
  const uint32_t T = lo;
  const int need_eq = K - cnt_above;

  // 3. ordered compaction: thread t owns the contiguous segment
  //    [seg t, seg t + seg), seg = ceil(ctx / 1024) <= 32.
  const int seg = (ctx + kRegThreads - 1) / kRegThreads;
  const int p0 = tid * seg;
  uint32_t sk[kRegKeys];
  uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
  for (int j = 0; j < kRegKeys; ++j) {
    const int p = p0 + j;
    sk[j] = 0u;
    if (j < seg && p < ctx) {
      sk[j] = lkeys[lds_pad(p)];
      n_gt += sk[j] > T ? 1u : 0u;
      n_eq += sk[j] == T ? 1u : 0u;
    }
  }
  // one scan of both counts packed in 16-bit halves (each total <= 32768)
  const uint32_t packed = n_gt | (n_eq << 16);
  const uint32_t pincl = wave_incl_scan(packed, lane);
  if (lane == 63) wpart[wave] = pincl;
  __syncthreads();
  uint32_t pbefore = pincl - packed;
  for (int w = 0; w < wave; ++w) pbefore += wpart[w];
  const int gt_before = (int)(pbefore & 0xFFFFu);
  int eq_seen = (int)(pbefore >> 16);
  int out = gt_before + min(eq_seen, need_eq);
#pragma unroll
  for (int j = 0; j < kRegKeys; ++j) {
    const int p = p0 + j;
    if (j < seg && p < ctx) {
      bool sel = sk[j] > T;
      if (sk[j] == T) {
        sel = eq_seen < need_eq;
        ++eq_seen;
      }
      if (sel && out < K) o[out++] = p;
    }
  }
  for (int i = K + tid; i < k; i += kRegThreads) o[i] = -1;
}

hipError_t launch_topk(const float* logits, int64_t n_rows, int64_t logits_stride, const int32_t* row_ctx, int32_t k,
                       int32_t* out_idx, int64_t max_ctx, hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  if (n_rows > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  if (max_ctx <= kRegMaxCtx) {
    const size_t lds = (size_t)(max_ctx + max_ctx / 32 + 1) * sizeof(uint32_t);
    hipLaunchKernelGGL(topk_reg_kernel, dim3((unsigned)n_rows), dim3(kRegThreads), lds, stream, logits,
                       logits_stride, row_ctx, k, out_idx);
  } else {
    hipLaunchKernelGGL(topk_long_kernel<false>, dim3((unsigned)n_rows), dim3(kTopkThreads),
                       (size_t)kBins * sizeof(uint32_t), stream, logits, logits_stride, row_ctx, k, out_idx);
  }
  return hipGetLastError();
}

}  // namespace fp4idx
