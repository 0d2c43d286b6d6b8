/*
 * fp4idx: FP4 lightning-indexer hot path for AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels.  Sources, cited by page title and
 * section:
 *   [P1] "dsv4.1-amd: KV cache layouts, FP4 indexer, compressor and router
 *        kernels" (sglang PR 41019)
 *   [P2] "[AMD] Enable FP4 indexer for Deepseek V4" (sglang PR 37353)
 *   [P3] "[AMD] DeepSeek-V4.1-Flash on MI350X (gfx950)" (sglang PR 39186)
 *
 * Common conventions
 *   - Every pointer argument is a DEVICE pointer owned by the caller (device
 *     memory of the current HIP device).  The library allocates nothing and
 *     keeps no state between calls apart from a per-device architecture check
 *     and, for fp4idx_mqa_logits_noalloc alone, a fixed scratch array of
 *     FP4IDX_SCRATCH_BYTES in each device's copy of its code object.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Every call
 *     is asynchronous on that stream: no host synchronisation, no device reads
 *     on the host, so calls can be captured in a HIP graph.
 *   - Argument validation checks host scalars and pointer non-nullness only.
 *     Values held in device memory (positions, slots, block-table entries,
 *     context lengths) are the caller's contract; a value outside its stated
 *     range never makes a kernel access memory outside the buffers described
 *     here, and each call states what it does with such values.
 *   - Return value: FP4IDX_OK (0), or a negative status; on a negative status
 *     nothing was launched.  fp4idx_status_string() names the status.
 *   - Sizes and offsets are 64-bit; pools larger than 2 GiB are supported.
 *   - Fixed geometry: head dim 128, rotary dims = the first 64, 64 tokens per
 *     page, one UE8M0 scale per 32 elements, e2m1 FP4 codes.  The *_fp8 calls
 *     serve the FP8 indexer cache instead (see "FP8 cache" below).
 *   - Numerics: the two encoders (write_k, pack_q) are bit-exact encodings
 *     whose fp32 operation order is fixed (see each call); logits are fp32
 *     with fp32 accumulation; top-k is exact on the logits it is given.
 */
#ifndef FP4IDX_H
#define FP4IDX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP4IDX_OK 0
#define FP4IDX_E_INVALID (-1)     /* null pointer, bad size, stride or count  */
#define FP4IDX_E_UNSUPPORTED (-2) /* current device is not gfx950            */
#define FP4IDX_E_LAUNCH (-3)      /* a HIP runtime call or launch failed      */
#define FP4IDX_E_WORKSPACE (-4)   /* workspace missing or too small           */
#define FP4IDX_E_SCRATCH (-5)     /* batch too large for the built-in scratch */

#define FP4IDX_HEAD_DIM 128
#define FP4IDX_ROPE_DIM 64
#define FP4IDX_PAGE_TOKENS 64
#define FP4IDX_PAYLOAD_PAGE_BYTES 4096 /* [1, 4, 64, 16] */
#define FP4IDX_SCALE_PAGE_BYTES 256    /* [1, 4, 64]     */
#define FP4IDX_FP8_PAGE_BYTES 8448     /* [64][128] codes + [64] fp32 scales */
#define FP4IDX_MAX_TOPK 2048
#define FP4IDX_FUSED_MAX_CTX 32768     /* longest row of fp4idx_mqa_logits_topk */
#define FP4IDX_SCRATCH_BYTES (16u << 20) /* per-device scratch of fp4idx_mqa_logits_noalloc */

/*
 * Fused K writer.  [P2] Modifications / fp4_indexer_hip.py and compress.py:
 * RMSNorm -> RoPE -> Hadamard -> FP4 quantisation -> paged write, fed with
 * per-forward positions and cache slots, the BF16 RMSNorm weight and the
 * model's BF16 RoPE cos/sin table; [P2] Motivation: split payload/scale pool.
 *
 *   k_bf16       [n_tokens, k_row_stride] bf16 bits; the first 128 of each row
 *   pos          [n_tokens] int32 RoPE position, 0 <= pos < max_pos
 *   slot         [n_tokens] int32 pool slot = page*64 + in-page index; a
 *                negative slot skips the token (padding).  Slots must be
 *                unique within one call and < num_pages*64.  A token whose
 *                slot is >= num_pages*64 or whose pos is outside
 *                [0, max_pos) is skipped as well.
 *   norm_w_bf16  [128] bf16 RMSNorm weight g (plain g, not 1+g)
 *   eps          RMSNorm epsilon (>= 0).  Inputs must keep every intermediate
 *                finite: with eps = 0 an all-zero (or fully underflowing)
 *                row divides by zero and its bytes are unspecified.
 *   cos_sin_bf16 [max_pos, 64] bf16: cos(p*theta_j) in columns 0..31, sin in 32..63
 *   payload      [num_pages, 1, 4, 64, 16] u8: byte b of block j of in-page
 *                token t holds elements 32j+2b (low nibble) and 32j+2b+1
 *   scale        [num_pages, 1, 4, 64] u8: UE8M0 byte of block j of token t
 *
 * Per token with slot >= 0, in fp32, exactly this order (no FMA contraction,
 * correctly rounded sqrt and division, denormals kept):
 *   x = bf16 row; S = balanced pairwise tree sum of x_i*x_i (T[a,b) =
 *   T[a,mid) + T[mid,b)); r = 1 / sqrt(S*(1/128) + eps); y_i = (x_i*r)*g_i;
 *   RoPE on dims 0..63, pairs (j, j+32): y_j = a*c - b*s, y_{j+32} = b*c + a*s;
 *   fast Walsh-Hadamard, stages h = 1,2,...,64, (u,v) -> (u+v, u-v); times
 *   C = fp32(128^-1/2); per 32-block: e = smallest integer with 6*2^e >= amax,
 *   clamped to [-127,127], scale byte e+127; code = nearest e2m1 value to
 *   z/2^e, ties to even, sign bit kept.
 * Writes exactly 64 payload bytes + 4 scale bytes per written token and
 * touches nothing else.
 */
int fp4idx_write_k(const uint16_t* k_bf16, int64_t n_tokens, int64_t k_row_stride, const int32_t* pos,
                   const int32_t* slot, const uint16_t* norm_w_bf16, float eps, const uint16_t* cos_sin_bf16,
                   int32_t max_pos, uint8_t* payload, uint8_t* scale, int64_t num_pages, void* stream);

/*
 * Index-Q pack + head weights in one launch.  [P1] Summary (one-launch
 * index-Q pack + head weights); [P2] Attention runtime (indexer Q rotated and
 * FP4-quantised).
 *
 *   q_bf16   [n_rows, q_row_stride] bf16 bits; head h of row t is the 128
 *            elements at t*q_row_stride + h*128
 *   n_heads  a multiple of 16, from 16 to 128
 *   pos      [n_rows] int32 RoPE position of each query row, 0 <= pos < max_pos;
 *            a row with pos outside that range is encoded as the zero vector
 *   w_in     [n_rows, n_heads] fp32 head weights
 *   q_fp4    [n_rows, n_heads, 64] u8 (out): same nibble order as K
 *   q_scale  [n_rows, n_heads, 4] u8 (out): UE8M0 per 32-block
 *   w_out    [n_rows, n_heads] fp32 (out): w_in * w_scale (one rounding)
 * Per (row, head): the K steps without RMSNorm (RoPE, Hadamard, FP4).
 */
int fp4idx_pack_q(const uint16_t* q_bf16, int64_t n_rows, int32_t n_heads, int64_t q_row_stride,
                  const int32_t* pos, const uint16_t* cos_sin_bf16, int32_t max_pos, const float* w_in,
                  float w_scale, uint8_t* q_fp4, uint8_t* q_scale, float* w_out, void* stream);

/*
 * A decode step's K write and Q pack in one launch.  The two are independent
 * ([P2] FP4 kernel adapters: the writer is fed the step's positions and
 * slots; the Q adapter packs the step's query rows), so one grid does both:
 * its first work-groups run fp4idx_write_k's kernel, the rest
 * fp4idx_pack_q's.  Arguments, layouts, results and errors are exactly those
 * of the two calls (the cos/sin table and max_pos are shared; pos_k is the
 * K tokens' positions, pos_q the query rows'); either batch may be empty.
 * Equivalent to fp4idx_write_k followed by fp4idx_pack_q on the same stream,
 * with one launch less.
 */
int fp4idx_write_k_pack_q(const uint16_t* k_bf16, int64_t n_tokens, int64_t k_row_stride, const int32_t* pos_k,
                          const int32_t* slot, const uint16_t* norm_w_bf16, float eps, const uint16_t* cos_sin_bf16,
                          int32_t max_pos, uint8_t* payload, uint8_t* scale, int64_t num_pages,
                          const uint16_t* q_bf16, int64_t n_rows, int32_t n_heads, int64_t q_row_stride,
                          const int32_t* pos_q, const float* w_in, float w_scale, uint8_t* q_fp4, uint8_t* q_scale,
                          float* w_out, void* stream);

/*
 * Paged-MQA FP4 logits.  [P2] Attention runtime (FP4 paged-MQA logits over
 * the split payload/scale cache, padded rows at zero context; schedules built
 * once and reused by every compressed-attention layer of a step, decode
 * schedules built during graph capture); [P1] Summary (the schedule built
 * on the device in two dispatches whose registers do not grow with the row
 * count).  The score is the lightning-indexer score
 *     logits[t][s] = sum_h w[t][h] * ReLU( qhat[t][h] . khat[s] )
 * with qhat, khat the dequantised FP4 vectors (e2m1 * 2^(byte-127)).
 *
 *   q_fp4, q_scale, w   as produced by fp4idx_pack_q ([n_rows, n_heads, ...]);
 *                       n_heads a multiple of 16, from 16 to 128
 *   req_row_indptr      [n_reqs+1] int32: rows of request b are
 *                       [indptr[b], indptr[b+1]); indptr[0] = 0, indptr[n_reqs] = n_rows,
 *                       non-decreasing (each bound is clamped into [0, n_rows] and
 *                       indptr[b+1] to at least indptr[b], so broken values only
 *                       ever touch rows 0..n_rows-1; their results are then unspecified)
 *   row_ctx_len         [n_rows] int32: row t scores tokens [0, ctx[t]); a value
 *                       above min(logits_stride, bt_stride*64) is cut to it
 *   block_table         [n_reqs, bt_stride] int32: token s of request b is in
 *                       page block_table[b*bt_stride + s/64], slot s%64.  Entries
 *                       for s/64 < ceil(max ctx of b's rows / 64) must be valid
 *                       page ids < num_pages (an invalid one never addresses
 *                       the pool: a valid page is read in its place, and its
 *                       tokens' logits are unspecified); later entries of
 *                       the row may be read but are never used.
 *   logits              [n_rows, logits_stride] fp32 (out); only [0, ctx[t]) of
 *                       each row is written, the rest is left untouched.
 *   workspace           device memory of workspace_bytes bytes, 16-byte aligned,
 *                       owned by the caller; fp4idx_mqa_logits_workspace_bytes()
 *                       gives the size.  It holds the work schedule; its
 *                       contents between calls belong to the library.  Calls
 *                       that overlap in time must not share a workspace.
 * Arithmetic: per 16 heads x 16 tokens, one block-scaled FP4 MFMA
 * (16x16x128) with fp32 accumulation; ReLU and the head weight in fp32; the
 * head sum in a fixed order.  The result for (t, s) does not depend on the
 * batch composition, the physical pages, the schedule or the launch shape,
 * and equals fp4idx_mqa_logits_bounded's bit for bit.
 *
 * Two launches on `stream`: the plan (fp4idx_mqa_logits_plan with max_ctx =
 * min(logits_stride, bt_stride*64)) and the run (fp4idx_mqa_logits_run).
 * Returns FP4IDX_E_WORKSPACE when workspace is NULL, unaligned or smaller
 * than the lists of the batch's row blocks need; a workspace smaller than
 * fp4idx_mqa_logits_workspace_bytes() for the batch's longest context makes
 * longer (fewer) work items and stays correct.  With armed timing events
 * (fp4idx_time_next_call) the start is the plan's and the stop the run's.
 */
int fp4idx_mqa_logits(const uint8_t* q_fp4, const uint8_t* q_scale, const float* w, int64_t n_rows, int32_t n_heads,
                      const int32_t* req_row_indptr, int32_t n_reqs, const int32_t* row_ctx_len,
                      const int32_t* block_table, int32_t bt_stride, const uint8_t* payload, const uint8_t* scale,
                      int64_t num_pages, float* logits, int64_t logits_stride, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * Workspace bytes of fp4idx_mqa_logits and fp4idx_mqa_logits_plan for a
 * batch of n_rows rows in n_reqs requests whose rows have at most max_ctx
 * tokens of context (any head count).  0 for an empty batch.
 */
size_t fp4idx_mqa_logits_workspace_bytes(int64_t n_rows, int32_t n_reqs, int64_t max_ctx);

/*
 * The work schedule of a batch, built on the device into workspace (one
 * launch of one work-group; its registers and LDS do not depend on the
 * batch).  The kernel follows from n_rows / n_reqs and n_heads: under about
 * three rows per request the per-wave kernel (1 or 2 rows per wave, each
 * wave streaming its own pages), else the shared-page kernel (4, 6 or 8
 * rows per work-group, each page staged once in LDS for all of them).  Each
 * request's rows are split evenly into row blocks of at most that many
 * rows, and each block's pages into chunks: for the per-wave kernel of the
 * work-group's pages; for the shared-page kernel of about equal work (the
 * busier a block's waves, the shorter its chunks), large ones first and
 * the last share of every block in chunks a quarter as long, so that the
 * item list, taken in order, ends with short items.  The items are
 * (request, row block, page chunk).  The list is cut into eight contiguous
 * ranges, one per XCD, stored interleaved (the run's work-group i executes
 * on XCD i mod 8), so a block's chunks share one XCD's L2; at most 16 empty
 * items even out the ranges.  Context lengths are read here (cut to
 * max_ctx) and by the run.
 *
 * The schedule depends only on n_rows, n_heads, req_row_indptr, n_reqs and
 * row_ctx_len, so one plan serves any number of fp4idx_mqa_logits_run calls
 * for that batch (every compressed-attention layer of a step: other Q,
 * weights, pools and block tables), including replays of a captured graph.
 * Rebuild it when the batch changes.  Arguments as fp4idx_mqa_logits;
 * max_ctx >= 0 bounds the contexts the schedule covers.
 */
int fp4idx_mqa_logits_plan(int64_t n_rows, int32_t n_heads, const int32_t* req_row_indptr, int32_t n_reqs,
                           const int32_t* row_ctx_len, int64_t max_ctx, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * The logits of a batch from a schedule fp4idx_mqa_logits_plan built in
 * workspace for the same n_rows, n_heads, req_row_indptr, n_reqs and
 * row_ctx_len (one launch: work-group i scores item i of the schedule; the
 * grid is an upper bound on the item count from the host's sizes, and
 * work-groups past the schedule's items leave at once).  Arguments as
 * fp4idx_mqa_logits.  The run only reads the workspace, so runs that share
 * one plan may overlap.  A workspace holding another batch's schedule, or
 * none, never makes the kernel touch memory outside the buffers described
 * here (each item is checked against the call's requests and rows); the
 * logits are then unspecified.
 */
int fp4idx_mqa_logits_run(const uint8_t* q_fp4, const uint8_t* q_scale, const float* w, int64_t n_rows,
                          int32_t n_heads, const int32_t* req_row_indptr, int32_t n_reqs, const int32_t* row_ctx_len,
                          const int32_t* block_table, int32_t bt_stride, const uint8_t* payload, const uint8_t* scale,
                          int64_t num_pages, float* logits, int64_t logits_stride, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * fp4idx_mqa_logits for callers that cannot allocate device memory or pass
 * a workspace (code under graph capture, tight serving loops, harnesses that
 * forbid allocation): the work schedule goes into the library's own scratch
 * array of FP4IDX_SCRATCH_BYTES on the current device instead of a caller
 * workspace.  Arguments, arithmetic and results as fp4idx_mqa_logits (bit
 * for bit); no allocation, no hipMalloc or hipFree.
 *
 * Limit: the batch's schedule, fp4idx_mqa_logits_workspace_bytes(n_rows,
 * n_reqs, min(logits_stride, bt_stride*64)) bytes, must fit in
 * FP4IDX_SCRATCH_BYTES (e.g. 16,384 rows in 64 requests at 131,072 tokens
 * need 8.3 MiB); a larger batch returns FP4IDX_E_SCRATCH and launches
 * nothing.  Every call on one device shares that device's array, which keeps
 * the last call's schedule (the plan writes every word the run reads, so
 * nothing needs clearing): calls that overlap in time on one device (on
 * different streams, or from several host threads without ordering) race
 * and their logits are unspecified.  The first call on a device looks the
 * array's address up (hipGetSymbolAddress); FP4IDX_E_LAUNCH if that fails.
 */
int fp4idx_mqa_logits_noalloc(const uint8_t* q_fp4, const uint8_t* q_scale, const float* w, int64_t n_rows,
                              int32_t n_heads, const int32_t* req_row_indptr, int32_t n_reqs,
                              const int32_t* row_ctx_len, const int32_t* block_table, int32_t bt_stride,
                              const uint8_t* payload, const uint8_t* scale, int64_t num_pages, float* logits,
                              int64_t logits_stride, void* stream);

/*
 * The same logits without a workspace: the launch grid covers (request, row
 * group, token chunk) from two host bounds and idle work-groups exit at
 * once.  Arguments as fp4idx_mqa_logits, plus
 *   max_rows_per_req    host bound >= max_b (indptr[b+1]-indptr[b])
 *   max_ctx             host bound >= max_t ctx[t]; max_ctx <= bt_stride*64 and
 *                       max_ctx <= logits_stride (a larger ctx[t] is cut to
 *                       min(logits_stride, bt_stride*64))
 *   n_reqs              at most 65535
 * Results equal fp4idx_mqa_logits's bit for bit.
 */
int fp4idx_mqa_logits_bounded(const uint8_t* q_fp4, const uint8_t* q_scale, const float* w, int64_t n_rows,
                              int32_t n_heads, const int32_t* req_row_indptr, int32_t n_reqs,
                              const int32_t* row_ctx_len, const int32_t* block_table, int32_t bt_stride,
                              const uint8_t* payload, const uint8_t* scale, int64_t num_pages, float* logits,
                              int64_t logits_stride, int32_t max_rows_per_req, int64_t max_ctx, void* stream);

/*
 * Top-k over each logits row.  [P3] Changes (sorted top-k selection) and
 * Historical results (the decode selection is returned in token-position order,
 * not in pool-slot order).
 *
 *   logits      [n_rows, logits_stride] fp32; row t uses [0, ctx[t]); finite values
 *   row_ctx_len [n_rows] int32, 0 <= ctx[t] <= logits_stride (a value
 *               outside that range is cut into it; that row's result is then
 *               unspecified)
 *   k           1 <= k <= FP4IDX_MAX_TOPK
 *   out_idx     [n_rows, k] int32 (out): the min(k, ctx[t]) positions with the
 *               largest values (ties: lower position first), ascending by
 *               position, then -1.  -0.0 and +0.0 compare equal.
 * The kernel variant (register band, rows per work-group) is picked for rows
 * of up to logits_stride values; fp4idx_topk_bounded takes a tighter bound.
 */
int fp4idx_topk(const float* logits, int64_t n_rows, int64_t logits_stride, const int32_t* row_ctx_len, int32_t k,
                int32_t* out_idx, void* stream);

/*
 * fp4idx_topk with a host bound on the contexts: 0 <= ctx[t] <= max_ctx <=
 * logits_stride (a larger ctx[t] is cut to max_ctx), so that logits rows
 * wider than their contexts still get the variant sized for max_ctx.
 * Results equal fp4idx_topk's whenever every ctx[t] <= max_ctx.
 */
int fp4idx_topk_bounded(const float* logits, int64_t n_rows, int64_t logits_stride, const int32_t* row_ctx_len,
                        int32_t k, int32_t* out_idx, int64_t max_ctx, void* stream);

/*
 * Fused logits + top-k: the top-k positions of every row without writing the
 * logits to memory.  [P3] Changes (sorted top-k selection) over the FP4
 * paged-MQA logits of [P2] Modifications (decode logits dispatch).
 *
 * Arguments as fp4idx_mqa_logits (without the logits buffer) plus k and
 * out_idx as fp4idx_topk; n_heads 16, 32, 48 or 64; max_ctx <=
 * FP4IDX_FUSED_MAX_CTX (the row is held in LDS); max_rows_per_req >= 1 when
 * n_rows > 0.  out_idx [n_rows, k] int32 receives exactly what
 * fp4idx_mqa_logits followed by fp4idx_topk would write (same logits bit
 * for bit, same selection and order), including the -1 padding and rows of
 * context 0.  One work-group per row scores every page of its row, so the
 * call suits batches of single-row requests (decode); rows of one request
 * each read the request's pages, where the two-call path shares them.
 */
int fp4idx_mqa_logits_topk(const uint8_t* q_fp4, const uint8_t* q_scale, const float* w, int64_t n_rows,
                           int32_t n_heads, const int32_t* req_row_indptr, int32_t n_reqs,
                           const int32_t* row_ctx_len, const int32_t* block_table, int32_t bt_stride,
                           const uint8_t* payload, const uint8_t* scale, int64_t num_pages, int32_t k,
                           int32_t* out_idx, int32_t max_rows_per_req, int64_t max_ctx, void* stream);

/*
 * Split-pool reader: pool tokens back to their values.  [P1] Summary (split
 * writer and reader for the FP4 pool); [P2] Device memory.
 *
 *   payload, scale  the pool as fp4idx_write_k fills it (num_pages pages)
 *   slot            [n_tokens] int32 pool slots (page = slot/64, in-page
 *                   index = slot%64); a slot outside [0, num_pages*64)
 *                   (e.g. -1 padding) reads as a zero row
 *   out             [n_tokens, out_row_stride] fp32 (out), 16-byte aligned,
 *                   out_row_stride >= 128 and a multiple of 4: row i gets the
 *                   128 values e2m1(code) * 2^(scale byte - 127), exactly
 *                   (+-inf where the value exceeds fp32; the writer never
 *                   stores scale byte 255, whose result is unspecified)
 */
int fp4idx_read_k(const uint8_t* payload, const uint8_t* scale, int64_t num_pages, const int32_t* slot,
                  int64_t n_tokens, float* out, int64_t out_row_stride, void* stream);

/*
 * ---- FP8 cache --------------------------------------------------------------
 * The FP8 indexer that the FP4 one replaces.  [P2] Device memory and sizing:
 * 132 bytes per compressed token (128 FP8 codes + a 4-byte scale) in one
 * fused region, against 68 split bytes for FP4.  The pages give no
 * byte-level layout; the one here:
 *   pool  [num_pages][8448] u8: per page, token t's 128 codes at t*128, then
 *         the 64 tokens' fp32 scales at 8192 + 4t.  Code i of a token is
 *         element i, an OCP FP8 E4M3 value (bias 7, largest finite 448,
 *         0x7F/0xFF NaN, never written).
 * Encoding: the K (or Q) steps of the FP4 calls up to and including the
 * Hadamard, identical fp32 operations; then one power-of-two scale per
 * vector: e = smallest integer with 448*2^e >= amax over its 128 values,
 * clamped to [-127, 127] (a zero vector gives -127), scale = 2^e stored as
 * fp32 (2^-127 as the subnormal); code = the E4M3 value nearest to z/2^e,
 * ties to even, sign bit kept.  Scales other than powers of two are read
 * by their exponent field alone.
 */

/* K writer into the FP8 pool; arguments and skip rules as fp4idx_write_k
 * (pool 16-byte aligned).  Writes exactly the token's 128 code bytes and its
 * 4 scale bytes and touches nothing else. */
int fp4idx_write_k_fp8(const uint16_t* k_bf16, int64_t n_tokens, int64_t k_row_stride, const int32_t* pos,
                       const int32_t* slot, const uint16_t* norm_w_bf16, float eps, const uint16_t* cos_sin_bf16,
                       int32_t max_pos, uint8_t* pool, int64_t num_pages, void* stream);

/* Q pack for the FP8 cache; arguments as fp4idx_pack_q except the outputs:
 *   q_fp8    [n_rows, n_heads, 128] u8 (out), 16-byte aligned: E4M3 codes
 *   q_scale  [n_rows, n_heads] fp32 (out): the power-of-two scale
 *   w_out    [n_rows, n_heads] fp32 (out): w_in * w_scale */
int fp4idx_pack_q_fp8(const uint16_t* q_bf16, int64_t n_rows, int32_t n_heads, int64_t q_row_stride,
                      const int32_t* pos, const uint16_t* cos_sin_bf16, int32_t max_pos, const float* w_in,
                      float w_scale, uint8_t* q_fp8, float* q_scale, float* w_out, void* stream);

/* fp4idx_write_k_fp8 and fp4idx_pack_q_fp8 in one launch, as
 * fp4idx_write_k_pack_q is for the FP4 pair. */
int fp4idx_write_k_pack_q_fp8(const uint16_t* k_bf16, int64_t n_tokens, int64_t k_row_stride, const int32_t* pos_k,
                              const int32_t* slot, const uint16_t* norm_w_bf16, float eps,
                              const uint16_t* cos_sin_bf16, int32_t max_pos, uint8_t* pool, int64_t num_pages,
                              const uint16_t* q_bf16, int64_t n_rows, int32_t n_heads, int64_t q_row_stride,
                              const int32_t* pos_q, const float* w_in, float w_scale, uint8_t* q_fp8,
                              float* q_scale, float* w_out, void* stream);

/* Paged-MQA logits over the FP8 pool: the same score, rows, block table and
 * bounds as fp4idx_mqa_logits, with qhat, khat the dequantised FP8 vectors
 * (e4m3 * scale).  Arithmetic: per 16 heads x 16 tokens one block-scaled FP8
 * MFMA (16x16x128) whose four block scales all carry the vector's exponent.
 * That MFMA forms each dot product from groups of 8 products whose low bits
 * (below 2^-13 of the group's largest product) are dropped before the group
 * sums are added and rounded to fp32, so |error| <= 7*2^-13 * sum_i |q_i k_i|
 * per head (plus that rounding) before the fp32 ReLU / weight / head sum; the result for (t, s) again does not
 * depend on batch composition, pages or launch shape.
 *   q_fp8, q_scale, w   as produced by fp4idx_pack_q_fp8 (q_fp8 16-byte
 *                       aligned, q_scale 4-byte aligned)
 *   pool                the FP8 pool (16-byte aligned, num_pages pages) */
int fp4idx_mqa_logits_fp8(const uint8_t* q_fp8, const float* q_scale, const float* w, int64_t n_rows,
                          int32_t n_heads, const int32_t* req_row_indptr, int32_t n_reqs, const int32_t* row_ctx_len,
                          const int32_t* block_table, int32_t bt_stride, const uint8_t* pool, int64_t num_pages,
                          float* logits, int64_t logits_stride, int32_t max_rows_per_req, int64_t max_ctx,
                          void* stream);

/*
 * Kernel timing (measurement support, not part of the method).  Arms two HIP
 * events for the calling thread's next call of fp4idx_write_k, fp4idx_pack_q,
 * fp4idx_write_k_pack_q, fp4idx_mqa_logits, fp4idx_topk, fp4idx_mqa_logits_topk,
 * fp4idx_read_k, one of the *_fp8 calls or a peak microbenchmark; each of
 * these launches exactly one kernel.
 * That kernel is then dispatched with hipExtLaunchKernel, which stamps the
 * events with the dispatch's own start and end times, so
 * hipEventElapsedTime(start, stop) is the kernel's execution time with no
 * marker packets in between.
 *
 *   start_event, stop_event  hipEvent_t created by the caller with timing
 *                            enabled, on the device of the next call; either
 *                            may be NULL.  Ownership stays with the caller.
 *
 * The arming belongs to the calling thread and is used up by its next call
 * whatever that call returns; a call that launches nothing (empty sizes or a
 * negative status) leaves the events as they were.  Not meant for use under
 * graph capture.  Returns FP4IDX_OK.
 */
int fp4idx_time_next_call(void* start_event, void* stop_event);

/*
 * Peak microbenchmarks (measurement support, not part of the method): the
 * roofline fractions are stated against vendor peaks and against these
 * measured ones.  Time a call with fp4idx_time_next_call.
 *
 * fp4idx_peak_mfma_fp4: 4,096 waves (four per SIMD of a 256-CU device) each
 *   run 4 * iterations V_MFMA_SCALE_F32_16X16X128_F8F6F4 instructions with
 *   e2m1 operands (the logits kernel's instruction), 65,536 flop each:
 *   flop = 4096 * 4 * iterations * 65536.  sink: one device float (never
 *   written in practice).
 * fp4idx_peak_valu_fp32: 4,096 waves each run 16 * iterations fp32 FMAs per
 *   lane on 16 independent chains: FMA lane-ops = 4096 * 64 * 16 * iterations
 *   (two flop each).  sink: one device float (never written in practice).
 * fp4idx_peak_mfma_valu: whether a SIMD's matrix and vector pipes overlap.
 *   4,096 waves each run `iterations` rounds of, by mode, 8 FP4 MFMAs (mode
 *   0), 32 fp32 FMAs (mode 1) or both interleaved one MFMA : four FMAs (mode
 *   2), every chain carried across rounds.  Compare the three durations:
 *   mode 2 near the longer of modes 0 and 1 means the pipes overlap, near
 *   their sum that they take turns.  mode outside 0..2 is FP4IDX_E_INVALID.
 *   sink: one device float (never written in practice).
 * fp4idx_peak_read: reads every byte of buf[0, bytes) once with 16-byte
 *   non-temporal loads; bytes a positive multiple of 16, buf 16-byte
 *   aligned; sink: one device uint32 (never written in practice).  Use a
 *   buffer well above the 256 MB last-level cache.
 */
int fp4idx_peak_mfma_fp4(int32_t iterations, float* sink, void* stream);
int fp4idx_peak_valu_fp32(int32_t iterations, float* sink, void* stream);
int fp4idx_peak_mfma_valu(int32_t mode, int32_t iterations, float* sink, void* stream);
int fp4idx_peak_read(const uint8_t* buf, int64_t bytes, uint32_t* sink, void* stream);

/* Human-readable name of a status code (static storage). */
const char* fp4idx_status_string(int status);

/* Library version: major*10000 + minor*100 + patch. */
int fp4idx_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP4IDX_H */
