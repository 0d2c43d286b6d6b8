/*
 * CPU oracle for the FP4 lightning-indexer hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may load, call or
 * link this file; only the tests, the package's smoke check and the bench's
 * CPU-baseline leg do.  It shares no code, header, table or constant with the
 * HIP library: every step below is written out from the definitions.
 *
 * Sources (web pages, cited by title and section):
 *   [P1] "dsv4.1-amd: KV cache layouts, FP4 indexer, compressor and router
 *        kernels" (sglang PR 41019)
 *   [P2] "[AMD] Enable FP4 indexer for Deepseek V4" (sglang PR 37353)
 *   [P3] "[AMD] DeepSeek-V4.1-Flash on MI350X (gfx950)" (sglang PR 39186)
 *
 * What each part is:
 *   - K encoding and Q encoding are ENCODINGS: the result is whatever the
 *     steps below produce in IEEE fp32 (round-to-nearest-even, no fused
 *     multiply-add, no flush of denormals) in exactly this order.  The GPU
 *     must reproduce every byte.  Where the pages leave the order open the
 *     reading taken is stated at the step.
 *   - The FP4 code of a value and the block exponent are exact decisions,
 *     taken here in exact (real) arithmetic on the fp32 value.
 *   - Logits are a plain definition on exactly dequantised values, evaluated
 *     in fp64 and rounded once to fp32.
 *   - Top-k is a plain definition (the k largest, lower position on ties).
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC.
 * All pointers are host pointers.  Functions return 0 on success and a
 * negative value on a rejected argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define D 128          /* index head dimension */
#define ROPE 64        /* rotary dims: the first 64 of the 128 */
#define PAGE 64        /* tokens per page */
#define BLK 32         /* elements per UE8M0 scale block */
#define NBLK (D / BLK) /* 4 scale blocks per token / per head */

/* ---- threads ----------------------------------------------------------- */

void orc_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int orc_get_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---- scalar helpers ---------------------------------------------------- */

/* bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 bits. */
static float f32_of_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Balanced pairwise sum: T[a,b) = T[a,m) + T[m,b), m = a + (b-a)/2.
 * Reading (the pages give no reduction order): this tree. */
static float tree_sum(const float *v, int n) {
  if (n == 1) return v[0];
  int m = n / 2;
  float lo = tree_sum(v, m);
  float hi = tree_sum(v + m, n - m);
  return lo + hi;
}

/* ---- a2: RMSNorm -------------------------------------------------------- */
/* [P2] Modifications / compressor.py + FP4 kernel adapters: the K writer
 * applies RMSNorm with a BF16 weight before RoPE.
 *   S  = tree-sum of x_i*x_i
 *   ms = S * (1/128)            (exact power-of-two scaling)
 *   r  = 1 / sqrt(ms + eps)     (three correctly rounded fp32 ops)
 *   y_i = (x_i * r) * g_i
 * Reading: plain weight g (not 1+g); eps passed in. */
void orc_rmsnorm128(const float *x, const float *g, float eps, float *y) {
  float sq[D];
  for (int i = 0; i < D; ++i) sq[i] = x[i] * x[i];
  float S = tree_sum(sq, D);
  float ms = S * 0.0078125f;
  float t = ms + eps;
  float s = sqrtf(t);
  float r = 1.0f / s;
  for (int i = 0; i < D; ++i) {
    float xr = x[i] * r;
    y[i] = xr * g[i];
  }
}

/* ---- a3: partial RoPE --------------------------------------------------- */
/* [P2] Modifications / deepseek_v4.py: Q and K use the model's BF16 RoPE
 * cos/sin cache; the rotary part is 64 of the 128 dims.
 * Reading: the FIRST 64 dims, rotate-half pairs (j, j+32) for j < 32, table
 * row = [cos_0..cos_31, sin_0..sin_31].  Dims 64..127 are unchanged.
 *   y_j      = a*c - b*s
 *   y_{j+32} = b*c + a*s       (each product rounded, then the sum) */
void orc_rope64(float *y, const float *cs) {
  for (int j = 0; j < ROPE / 2; ++j) {
    float c = cs[j];
    float s = cs[ROPE / 2 + j];
    float a = y[j];
    float b = y[j + ROPE / 2];
    float ac = a * c, bs = b * s, bc = b * c, as = a * s;
    y[j] = ac - bs;
    y[j + ROPE / 2] = bc + as;
  }
}

/* ---- a4: Hadamard-128 --------------------------------------------------- */
/* [P2] Modifications / fp4_indexer_hip.py: Hadamard rotation before FP4.
 * Normalised Sylvester Hadamard, H[i][j] = (-1)^popcount(i&j) / sqrt(128).
 * Fast transform, stages h = 1,2,4,...,64 in that order; at each stage every
 * pair (i, i+h) with (i & h) == 0 becomes (u+v, u-v).  Then every element is
 * multiplied by C = fp32 nearest to 128^-1/2.
 * Reading: this stage order, normalisation last as one fp32 multiply. */
float orc_hadamard_scale(void) { return (float)(1.0 / sqrt(128.0)); }

void orc_fwht128(float *z) {
  for (int h = 1; h < D; h <<= 1) {
    for (int i = 0; i < D; ++i) {
      if (i & h) continue;
      float u = z[i], v = z[i + h];
      z[i] = u + v;
      z[i + h] = u - v;
    }
  }
  float C = orc_hadamard_scale();
  for (int i = 0; i < D; ++i) z[i] = z[i] * C;
}

/* ---- a5: MXFP4 encoding ------------------------------------------------- */
/* [P2] Motivation: e2m1 FP4 codes with one UE8M0 scale per 32 elements;
 * [P1] Summary: round-to-nearest-even.
 * Block exponent: the smallest integer e with 6 * 2^e >= amax, i.e.
 * ceil(log2(amax/6)) in real arithmetic, clamped to [-127, 127] so the scale
 * byte e+127 is never the E8M0 NaN 0xFF.  amax = 0 gives e = -127 (byte 0).
 * Evaluated exactly: ldexp(6, e) and amax are exact doubles. */
int orc_block_exponent(float amax) {
  double a = (double)amax;
  int e;
  if (a == 0.0) return -127;
  (void)frexp(a, &e); /* start near the answer, then walk to the definition */
  e -= 3;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  while (e < 127 && ldexp(6.0, e) < a) ++e;
  while (e > -127 && ldexp(6.0, e - 1) >= a) --e;
  return e;
}

/* The e2m1 magnitudes, indexed by the 3-bit magnitude code. */
static const double E2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* 4-bit code of z at block exponent e: magnitude = the grid value nearest to
 * |z| * 2^-e (exact), ties to the even code; bit 3 = sign bit of z (a
 * negative value that rounds to zero keeps its sign, as an IEEE conversion
 * does). */
int orc_e2m1_code(float z, int e) {
  double v = ldexp(fabs((double)z), -e);
  int best = 0;
  double bd = fabs(v - E2M1[0]);
  for (int c = 1; c < 8; ++c) {
    double d = fabs(v - E2M1[c]);
    if (d < bd || (d == bd && (c & 1) == 0)) {
      best = c;
      bd = d;
    }
  }
  return best | (signbit(z) ? 8 : 0);
}

/* Quantise one 128-vector: codes[64] (element 2i in the low nibble of byte
 * i, element 2i+1 in the high nibble) and sc[4] (one E8M0 byte per 32). */
void orc_quant128(const float *z, uint8_t *codes, uint8_t *sc) {
  for (int j = 0; j < NBLK; ++j) {
    float amax = 0.0f;
    for (int i = 0; i < BLK; ++i) {
      float m = fabsf(z[j * BLK + i]);
      if (m > amax) amax = m;
    }
    int e = orc_block_exponent(amax);
    sc[j] = (uint8_t)(e + 127);
    for (int b = 0; b < BLK / 2; ++b) {
      int lo = orc_e2m1_code(z[j * BLK + 2 * b], e);
      int hi = orc_e2m1_code(z[j * BLK + 2 * b + 1], e);
      codes[j * (BLK / 2) + b] = (uint8_t)(lo | (hi << 4));
    }
  }
}

/* Exact dequantisation of one 128-vector (codes + scales) into doubles. */
void orc_dequant128(const uint8_t *codes, const uint8_t *sc, double *out) {
  for (int i = 0; i < D; ++i) {
    int j = i / BLK;
    uint8_t byte = codes[i / 2];
    int c = (i & 1) ? (byte >> 4) : (byte & 15);
    double m = E2M1[c & 7];
    if (c & 8) m = -m;
    out[i] = ldexp(m, (int)sc[j] - 127);
  }
}

/* ---- a1..a5 for one K token -------------------------------------------- */
/* [P2] FP4 kernel adapters: the fused writer runs RMSNorm -> RoPE ->
 * Hadamard -> FP4 quantisation -> paged write.  Intermediates stay fp32
 * (reading: no bf16 rounding between the fused steps). */
void orc_encode_k_token(const uint16_t *k_row, const uint16_t *norm_w, float eps,
                        const uint16_t *cs_row, uint8_t *codes, uint8_t *sc) {
  float x[D], g[D], y[D], cs[ROPE];
  for (int i = 0; i < D; ++i) {
    x[i] = f32_of_bf16(k_row[i]);
    g[i] = f32_of_bf16(norm_w[i]);
  }
  for (int i = 0; i < ROPE; ++i) cs[i] = f32_of_bf16(cs_row[i]);
  orc_rmsnorm128(x, g, eps, y);
  orc_rope64(y, cs);
  orc_fwht128(y);
  orc_quant128(y, codes, sc);
}

/* One Q head: RoPE -> Hadamard -> FP4 (no RMSNorm). */
void orc_encode_q_head(const uint16_t *q_row, const uint16_t *cs_row, uint8_t *codes, uint8_t *sc) {
  float y[D], cs[ROPE];
  for (int i = 0; i < D; ++i) y[i] = f32_of_bf16(q_row[i]);
  for (int i = 0; i < ROPE; ++i) cs[i] = f32_of_bf16(cs_row[i]);
  orc_rope64(y, cs);
  orc_fwht128(y);
  orc_quant128(y, codes, sc);
}

/* ---- a6: split paged store ---------------------------------------------- */
/* [P2] Motivation: payload [num_pages, 1, 4, 64, 16] bytes and scale
 * [num_pages, 1, 4, 64] bytes, 64 tokens per page, 68 B per token.
 * Reading of "preshuffled": the index order of those shapes,
 *   payload[page][0][block j][token t][byte b]  (b holds elements 32j+2b, 32j+2b+1)
 *   scale  [page][0][block j][token t]
 * slot = page*64 + t; slot < 0 means "skip this token". */
int orc_write_k(const uint16_t *k, int64_t n_tokens, int64_t k_row_stride, const int32_t *pos,
                const int32_t *slot, const uint16_t *norm_w, float eps, const uint16_t *cos_sin,
                int32_t max_pos, uint8_t *payload, uint8_t *scale, int64_t num_pages) {
  if (n_tokens < 0 || k_row_stride < D || max_pos <= 0 || num_pages < 0) return -1;
  for (int64_t n = 0; n < n_tokens; ++n) {
    if (slot[n] >= 0 && (int64_t)slot[n] >= num_pages * PAGE) return -2;
    if (slot[n] >= 0 && (pos[n] < 0 || pos[n] >= max_pos)) return -3;
  }
  /* duplicate slots within one call have no defined result: reject them */
  if (n_tokens > 0 && num_pages > 0) {
    uint8_t *seen = (uint8_t *)calloc((size_t)(num_pages * PAGE), 1);
    if (!seen) return -4;
    int dup = 0;
    for (int64_t n = 0; n < n_tokens; ++n) {
      if (slot[n] < 0) continue;
      if (seen[slot[n]]) dup = 1;
      seen[slot[n]] = 1;
    }
    free(seen);
    if (dup) return -5;
  }
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < n_tokens; ++n) {
    if (slot[n] < 0) continue;
    uint8_t codes[D / 2], sc[NBLK];
    orc_encode_k_token(k + n * k_row_stride, norm_w, eps, cos_sin + (int64_t)pos[n] * ROPE, codes, sc);
    int64_t page = slot[n] / PAGE, t = slot[n] % PAGE;
    for (int j = 0; j < NBLK; ++j) {
      memcpy(payload + page * (PAGE * D / 2) + j * (PAGE * BLK / 2) + t * (BLK / 2), codes + j * (BLK / 2), BLK / 2);
      scale[page * (PAGE * NBLK) + j * PAGE + t] = sc[j];
    }
  }
  return 0;
}

/* ---- a7: Q pack + head weights ----------------------------------------- */
/* [P1] Summary: one launch packs index-Q and the head weights;
 * [P2] Attention runtime: indexer Q is rotated and FP4-quantised like K.
 * Output in natural order: q_fp4[t][h][64], q_scale[t][h][4];
 * w_out[t][h] = w_in[t][h] * w_scale (one fp32 rounding). */
int orc_pack_q(const uint16_t *q, int64_t n_rows, int32_t n_heads, int64_t q_row_stride,
               const int32_t *pos, const uint16_t *cos_sin, int32_t max_pos, const float *w_in,
               float w_scale, uint8_t *q_fp4, uint8_t *q_scale, float *w_out) {
  if (n_rows < 0 || n_heads <= 0 || q_row_stride < (int64_t)n_heads * D || max_pos <= 0) return -1;
  for (int64_t t = 0; t < n_rows; ++t)
    if (pos[t] < 0 || pos[t] >= max_pos) return -3;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n_rows; ++t) {
    for (int h = 0; h < n_heads; ++h) {
      int64_t o = t * n_heads + h;
      orc_encode_q_head(q + t * q_row_stride + (int64_t)h * D, cos_sin + (int64_t)pos[t] * ROPE,
                        q_fp4 + o * (D / 2), q_scale + o * NBLK);
      w_out[o] = w_in[o] * w_scale;
    }
  }
  return 0;
}

/* ---- a9..a11: paged MQA logits ----------------------------------------- */
/* Lightning-indexer score (DeepSeek sparse attention indexer):
 *   logit[t][s] = sum_h w[t][h] * ReLU( qhat[t][h] . khat[s] )
 * over every cached token s < ctx[t] of the row's request, read through the
 * block table: token s sits in page block_table[b][s/64], in-page slot s%64
 * ([P2] Attention runtime: paged-MQA logits over the split cache; padded
 * rows keep ctx 0 and get no scores).
 * qhat, khat are the exact dequantised FP4 values; the dot products and the
 * weighted sum are evaluated in fp64 (each product of two FP4 values is
 * exact in fp64) and rounded once to fp32.  tol_ref (optional) receives
 * sum_h |w| * max(d_h, 0), the quantity the fp32 tolerance is relative to. */
static void dequant_token(const uint8_t *payload, const uint8_t *scale, int64_t page, int t, double *out) {
  uint8_t codes[D / 2], sc[NBLK];
  for (int j = 0; j < NBLK; ++j) {
    memcpy(codes + j * (BLK / 2), payload + page * (PAGE * D / 2) + j * (PAGE * BLK / 2) + t * (BLK / 2), BLK / 2);
    sc[j] = scale[page * (PAGE * NBLK) + j * PAGE + t];
  }
  orc_dequant128(codes, sc, out);
}

/* ---- the split-pool reader ------------------------------------------------ */
/* [P1] Summary and [P2] Device memory (a split writer and reader for the
 * FP4 pool): token `slot` of the pool back to its 128 values, exactly, in
 * fp64.  A slot outside [0, num_pages*64) (padding) reads as zeros. */
int orc_read_k(const uint8_t *payload, const uint8_t *scale, int64_t num_pages, const int32_t *slot,
               int64_t n_tokens, double *out) {
  if (n_tokens < 0 || num_pages < 0) return -1;
  for (int64_t i = 0; i < n_tokens; ++i) {
    const int64_t s = slot[i];
    if (s < 0 || s >= num_pages * PAGE) {
      for (int e = 0; e < D; ++e) out[i * D + e] = 0.0;
      continue;
    }
    dequant_token(payload, scale, s / PAGE, (int)(s % PAGE), out + i * D);
  }
  return 0;
}

/* Also returns T = sum_h |w_h| max(d_h, 0) and A = sum_h |w_h| sum_i |q_hi k_i|,
 * the two scales an fp32 evaluation's error is measured against. */
static double score_one(const double *qd /* [H][D] */, const float *w /* [H] */, int32_t n_heads,
                        const double *kd, double *tol_ref, double *abs_ref) {
  double L = 0.0, T = 0.0, A = 0.0;
  for (int h = 0; h < n_heads; ++h) {
    double d = 0.0, a = 0.0;
    for (int i = 0; i < D; ++i) {
      d += qd[h * D + i] * kd[i];
      a += fabs(qd[h * D + i] * kd[i]);
    }
    double r = d > 0.0 ? d : 0.0;
    L += (double)w[h] * r;
    T += fabs((double)w[h]) * r;
    A += fabs((double)w[h]) * a;
  }
  if (tol_ref) *tol_ref = T;
  if (abs_ref) *abs_ref = A;
  return L;
}

static int row_request(const int32_t *indptr, int32_t n_reqs, int64_t t) {
  for (int b = 0; b < n_reqs; ++b)
    if (t >= indptr[b] && t < indptr[b + 1]) return b;
  return -1;
}

static int check_logits_args(int64_t n_rows, int32_t n_heads, const int32_t *indptr, int32_t n_reqs,
                             const int32_t *row_ctx, const int32_t *block_table, int32_t bt_stride,
                             int64_t num_pages, int64_t logits_stride) {
  if (n_rows < 0 || n_heads <= 0 || n_reqs < 0 || bt_stride < 0) return -1;
  if (indptr[0] != 0 || indptr[n_reqs] != n_rows) return -1;
  for (int b = 0; b < n_reqs; ++b)
    if (indptr[b + 1] < indptr[b]) return -1;
  for (int b = 0; b < n_reqs; ++b) {
    for (int64_t t = indptr[b]; t < indptr[b + 1]; ++t) {
      int64_t c = row_ctx[t];
      if (c < 0 || c > logits_stride || c > (int64_t)bt_stride * PAGE) return -1;
      for (int64_t p = 0; p < (c + PAGE - 1) / PAGE; ++p) {
        int32_t pg = block_table[(int64_t)b * bt_stride + p];
        if (pg < 0 || pg >= num_pages) return -2;
      }
    }
  }
  return 0;
}

int orc_logits(const uint8_t *q_fp4, const uint8_t *q_scale, const float *w, int64_t n_rows,
               int32_t n_heads, const int32_t *indptr, int32_t n_reqs, const int32_t *row_ctx,
               const int32_t *block_table, int32_t bt_stride, const uint8_t *payload,
               const uint8_t *scale, int64_t num_pages, float *logits, int64_t logits_stride,
               double *logits_f64 /* optional, same layout */, double *tol_ref /* optional */,
               double *abs_ref /* optional */) {
  int rc = check_logits_args(n_rows, n_heads, indptr, n_reqs, row_ctx, block_table, bt_stride, num_pages,
                             logits_stride);
  if (rc) return rc;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < n_rows; ++t) {
    int b = row_request(indptr, n_reqs, t);
    double *qd = (double *)malloc(sizeof(double) * (size_t)n_heads * D);
    double kd[D];
    for (int h = 0; h < n_heads; ++h)
      orc_dequant128(q_fp4 + (t * n_heads + h) * (D / 2), q_scale + (t * n_heads + h) * NBLK, qd + h * D);
    for (int64_t s = 0; s < row_ctx[t]; ++s) {
      int64_t page = block_table[(int64_t)b * bt_stride + s / PAGE];
      dequant_token(payload, scale, page, (int)(s % PAGE), kd);
      double T, A;
      double L = score_one(qd, w + t * n_heads, n_heads, kd, &T, &A);
      logits[t * logits_stride + s] = (float)L;
      if (logits_f64) logits_f64[t * logits_stride + s] = L;
      if (tol_ref) tol_ref[t * logits_stride + s] = T;
      if (abs_ref) abs_ref[t * logits_stride + s] = A;
    }
    free(qd);
  }
  return 0;
}

/* Scores for an explicit list of (row, token) pairs, for sampled checks of
 * large problems.  out[i] = fp64 logit, tol_ref[i] = sum |w| max(d,0),
 * abs_ref[i] = sum |w| sum |q k|. */
int orc_logits_sampled(const uint8_t *q_fp4, const uint8_t *q_scale, const float *w, int32_t n_heads,
                       const int32_t *indptr, int32_t n_reqs, const int32_t *block_table, int32_t bt_stride,
                       const uint8_t *payload, const uint8_t *scale, int64_t num_pages, int64_t n_samples,
                       const int64_t *rows, const int64_t *toks, double *out, double *tol_ref,
                       double *abs_ref) {
  if (n_heads <= 0 || n_samples < 0) return -1;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : bad)
  for (int64_t i = 0; i < n_samples; ++i) {
    int64_t t = rows[i], s = toks[i];
    int b = row_request(indptr, n_reqs, t);
    if (b < 0 || s < 0 || s / PAGE >= bt_stride) { bad = 1; continue; }
    int64_t page = block_table[(int64_t)b * bt_stride + s / PAGE];
    if (page < 0 || page >= num_pages) { bad = 1; continue; }
    double *qd = (double *)malloc(sizeof(double) * (size_t)n_heads * D);
    double kd[D];
    for (int h = 0; h < n_heads; ++h)
      orc_dequant128(q_fp4 + (t * n_heads + h) * (D / 2), q_scale + (t * n_heads + h) * NBLK, qd + h * D);
    dequant_token(payload, scale, page, (int)(s % PAGE), kd);
    out[i] = score_one(qd, w + t * n_heads, n_heads, kd, &tol_ref[i], &abs_ref[i]);
    free(qd);
  }
  return bad ? -2 : 0;
}

/* ==== FP8 indexer variant ================================================== */
/* [P2] Device memory and sizing: the FP8 indexer keeps 132 bytes per
 * compressed token in one fused region, where the FP4 indexer splits a
 * 64-byte payload and 4 scale bytes.  The pages give no byte-level layout;
 * the readings taken here:
 *   - 128 e4m3 codes (OCP FP8 E4M3: bias 7, 3 mantissa bits, largest finite
 *     448, subnormal step 2^-9, 0x7F/0xFF NaN) + one fp32 scale per token;
 *   - the scale is the power of two 2^e with e the smallest integer such
 *     that 448 * 2^e >= amax over the token's 128 values, clamped to
 *     [-127, 127] (amax = 0 gives -127), so z / 2^e is exact and the only
 *     rounding is onto the e4m3 grid: nearest, ties to the even code, the
 *     sign of zero kept;
 *   - the same steps as the FP4 writer up to the Hadamard (RMSNorm, RoPE,
 *     Hadamard in the canonical fp32 order), and Q per (row, head) likewise
 *     without RMSNorm;
 *   - page layout: [64 tokens][128 code bytes] then [64][fp32 scale], 8448
 *     bytes per page, code byte i of a token = element i. */
#define FP8_MAX 448.0
#define PAGE8_BYTES (PAGE * (D + 4))

int orc_fp8_exponent(float amax) {
  double a = (double)amax;
  int e;
  if (a == 0.0) return -127;
  (void)frexp(a, &e); /* start near the answer, then walk to the definition */
  e -= 9;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  while (e < 127 && ldexp(FP8_MAX, e) < a) ++e;
  while (e > -127 && ldexp(FP8_MAX, e - 1) >= a) --e;
  return e;
}

/* Value of an e4m3 magnitude code 0..126 (bit 7 is the sign). */
double orc_e4m3_value(int code) {
  int ex = (code >> 3) & 15, m = code & 7;
  double v = ex == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, ex - 7);
  return (code & 0x80) ? -v : v;
}

/* Code of z at token exponent e: the e4m3 magnitude nearest to |z| 2^-e
 * (exact), ties to the even code, sign bit of z kept. */
int orc_e4m3_code(float z, int e) {
  double v = ldexp(fabs((double)z), -e);
  int best = 0;
  double bd = v;
  for (int c = 1; c <= 126; ++c) {
    double d = fabs(v - orc_e4m3_value(c));
    if (d < bd || (d == bd && (c & 1) == 0)) {
      best = c;
      bd = d;
    }
  }
  return best | (signbit(z) ? 0x80 : 0);
}

/* One 128-vector: codes[128] and its fp32 scale 2^e. */
void orc_quant_fp8_128(const float *z, uint8_t *codes, float *scale) {
  float amax = 0.0f;
  for (int i = 0; i < D; ++i) {
    float m = fabsf(z[i]);
    if (m > amax) amax = m;
  }
  int e = orc_fp8_exponent(amax);
  *scale = (float)ldexp(1.0, e); /* exact: 2^-127 .. 2^127 are fp32 values (2^-127 subnormal) */
  for (int i = 0; i < D; ++i) codes[i] = (uint8_t)orc_e4m3_code(z[i], e);
}

void orc_encode_k_token_fp8(const uint16_t *k_row, const uint16_t *norm_w, float eps, const uint16_t *cs_row,
                            uint8_t *codes, float *scale) {
  float x[D], g[D], y[D], cs[ROPE];
  for (int i = 0; i < D; ++i) {
    x[i] = f32_of_bf16(k_row[i]);
    g[i] = f32_of_bf16(norm_w[i]);
  }
  for (int i = 0; i < ROPE; ++i) cs[i] = f32_of_bf16(cs_row[i]);
  orc_rmsnorm128(x, g, eps, y);
  orc_rope64(y, cs);
  orc_fwht128(y);
  orc_quant_fp8_128(y, codes, scale);
}

void orc_encode_q_head_fp8(const uint16_t *q_row, const uint16_t *cs_row, uint8_t *codes, float *scale) {
  float y[D], cs[ROPE];
  for (int i = 0; i < D; ++i) y[i] = f32_of_bf16(q_row[i]);
  for (int i = 0; i < ROPE; ++i) cs[i] = f32_of_bf16(cs_row[i]);
  orc_rope64(y, cs);
  orc_fwht128(y);
  orc_quant_fp8_128(y, codes, scale);
}

/* K tokens into the fused FP8 pool (num_pages * 8448 bytes); slot < 0 skips,
 * duplicate slots are rejected as in orc_write_k. */
int orc_write_k_fp8(const uint16_t *k, int64_t n_tokens, int64_t k_row_stride, const int32_t *pos,
                    const int32_t *slot, const uint16_t *norm_w, float eps, const uint16_t *cos_sin,
                    int32_t max_pos, uint8_t *pool, int64_t num_pages) {
  if (n_tokens < 0 || k_row_stride < D || max_pos <= 0 || num_pages < 0) return -1;
  for (int64_t n = 0; n < n_tokens; ++n) {
    if (slot[n] >= 0 && (int64_t)slot[n] >= num_pages * PAGE) return -2;
    if (slot[n] >= 0 && (pos[n] < 0 || pos[n] >= max_pos)) return -3;
  }
  if (n_tokens > 0 && num_pages > 0) {
    uint8_t *seen = (uint8_t *)calloc((size_t)(num_pages * PAGE), 1);
    if (!seen) return -4;
    int dup = 0;
    for (int64_t n = 0; n < n_tokens; ++n) {
      if (slot[n] < 0) continue;
      if (seen[slot[n]]) dup = 1;
      seen[slot[n]] = 1;
    }
    free(seen);
    if (dup) return -5;
  }
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < n_tokens; ++n) {
    if (slot[n] < 0) continue;
    uint8_t codes[D];
    float sc;
    orc_encode_k_token_fp8(k + n * k_row_stride, norm_w, eps, cos_sin + (int64_t)pos[n] * ROPE, codes, &sc);
    int64_t page = slot[n] / PAGE, t = slot[n] % PAGE;
    memcpy(pool + page * PAGE8_BYTES + t * D, codes, D);
    memcpy(pool + page * PAGE8_BYTES + PAGE * D + t * 4, &sc, 4);
  }
  return 0;
}

/* Q rows: q_fp8[t][h][128] codes, q_scale[t][h] fp32, w_out = w_in * w_scale. */
int orc_pack_q_fp8(const uint16_t *q, int64_t n_rows, int32_t n_heads, int64_t q_row_stride, const int32_t *pos,
                   const uint16_t *cos_sin, int32_t max_pos, const float *w_in, float w_scale, uint8_t *q_fp8,
                   float *q_scale, float *w_out) {
  if (n_rows < 0 || n_heads <= 0 || q_row_stride < (int64_t)n_heads * D || max_pos <= 0) return -1;
  for (int64_t t = 0; t < n_rows; ++t)
    if (pos[t] < 0 || pos[t] >= max_pos) return -3;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n_rows; ++t) {
    for (int h = 0; h < n_heads; ++h) {
      int64_t o = t * n_heads + h;
      orc_encode_q_head_fp8(q + t * q_row_stride + (int64_t)h * D, cos_sin + (int64_t)pos[t] * ROPE, q_fp8 + o * D,
                            q_scale + o);
      w_out[o] = w_in[o] * w_scale;
    }
  }
  return 0;
}

/* Exact values of one 128-vector of e4m3 codes with its fp32 scale. */
void orc_dequant_fp8_128(const uint8_t *codes, float scale, double *out) {
  for (int i = 0; i < D; ++i) out[i] = orc_e4m3_value(codes[i]) * (double)scale;
}

static void dequant_token_fp8(const uint8_t *pool, int64_t page, int t, double *out) {
  float sc;
  memcpy(&sc, pool + page * PAGE8_BYTES + PAGE * D + t * 4, 4);
  orc_dequant_fp8_128(pool + page * PAGE8_BYTES + t * D, sc, out);
}

/* B16 = sum_h |w_h| * (the sum of the 16 largest |q_hi k_i| of head h): the
 * scale of what an evaluation loses when it forms each dot product from 16
 * groups of 8 products and cuts every product below a fixed fraction of its
 * group's largest (the 16 group maxima are 16 distinct products, so their
 * sum is at most this).  A checker's scale, not part of the score. */
static double top16_scale(const double *qd, const float *w, int32_t n_heads, const double *kd) {
  double B = 0.0;
  for (int h = 0; h < n_heads; ++h) {
    double top[16];
    int n = 0;
    for (int i = 0; i < D; ++i) {
      double a = fabs(qd[h * D + i] * kd[i]);
      if (n < 16) {
        int j = n++;
        while (j > 0 && top[j - 1] < a) { top[j] = top[j - 1]; --j; }
        top[j] = a;
      } else if (a > top[15]) {
        int j = 15;
        while (j > 0 && top[j - 1] < a) { top[j] = top[j - 1]; --j; }
        top[j] = a;
      }
    }
    double sum = 0.0;
    for (int j = 0; j < n; ++j) sum += top[j];
    B += fabs((double)w[h]) * sum;
  }
  return B;
}

/* The same score on the FP8 variant's exact values (fp64, rounded once). */
int orc_logits_fp8(const uint8_t *q_fp8, const float *q_scale, const float *w, int64_t n_rows, int32_t n_heads,
                   const int32_t *indptr, int32_t n_reqs, const int32_t *row_ctx, const int32_t *block_table,
                   int32_t bt_stride, const uint8_t *pool, int64_t num_pages, float *logits, int64_t logits_stride,
                   double *logits_f64, double *tol_ref, double *abs_ref, double *top16_ref /* optional */) {
  int rc = check_logits_args(n_rows, n_heads, indptr, n_reqs, row_ctx, block_table, bt_stride, num_pages,
                             logits_stride);
  if (rc) return rc;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < n_rows; ++t) {
    int b = row_request(indptr, n_reqs, t);
    double *qd = (double *)malloc(sizeof(double) * (size_t)n_heads * D);
    double kd[D];
    for (int h = 0; h < n_heads; ++h) orc_dequant_fp8_128(q_fp8 + (t * n_heads + h) * D, q_scale[t * n_heads + h], qd + h * D);
    for (int64_t s = 0; s < row_ctx[t]; ++s) {
      int64_t page = block_table[(int64_t)b * bt_stride + s / PAGE];
      dequant_token_fp8(pool, page, (int)(s % PAGE), kd);
      double T, A;
      double L = score_one(qd, w + t * n_heads, n_heads, kd, &T, &A);
      logits[t * logits_stride + s] = (float)L;
      if (logits_f64) logits_f64[t * logits_stride + s] = L;
      if (tol_ref) tol_ref[t * logits_stride + s] = T;
      if (abs_ref) abs_ref[t * logits_stride + s] = A;
      if (top16_ref) top16_ref[t * logits_stride + s] = top16_scale(qd, w + t * n_heads, n_heads, kd);
    }
    free(qd);
  }
  return 0;
}

int orc_logits_fp8_sampled(const uint8_t *q_fp8, const float *q_scale, const float *w, int32_t n_heads,
                           const int32_t *indptr, int32_t n_reqs, const int32_t *block_table, int32_t bt_stride,
                           const uint8_t *pool, int64_t num_pages, int64_t n_samples, const int64_t *rows,
                           const int64_t *toks, double *out, double *tol_ref, double *abs_ref,
                           double *top16_ref /* optional */) {
  if (n_heads <= 0 || n_samples < 0) return -1;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : bad)
  for (int64_t i = 0; i < n_samples; ++i) {
    int64_t t = rows[i], s = toks[i];
    int b = row_request(indptr, n_reqs, t);
    if (b < 0 || s < 0 || s / PAGE >= bt_stride) { bad = 1; continue; }
    int64_t page = block_table[(int64_t)b * bt_stride + s / PAGE];
    if (page < 0 || page >= num_pages) { bad = 1; continue; }
    double *qd = (double *)malloc(sizeof(double) * (size_t)n_heads * D);
    double kd[D];
    for (int h = 0; h < n_heads; ++h) orc_dequant_fp8_128(q_fp8 + (t * n_heads + h) * D, q_scale[t * n_heads + h], qd + h * D);
    dequant_token_fp8(pool, page, (int)(s % PAGE), kd);
    out[i] = score_one(qd, w + t * n_heads, n_heads, kd, &tol_ref[i], &abs_ref[i]);
    if (top16_ref) top16_ref[i] = top16_scale(qd, w + t * n_heads, n_heads, kd);
    free(qd);
  }
  return bad ? -2 : 0;
}

/* ---- a12: top-k ---------------------------------------------------------- */
/* [P3] Changes: sorted top-k selection; Historical results: the decode
 * selection comes back in token-position order rather than pool-slot order.
 * Row t: among positions s < ctx[t], the K* = min(k, ctx[t]) positions with
 * the largest values, ties broken toward the lower position (reading: the
 * pages give no tie rule); written ascending by position, then -1 padding.
 * Values compare as IEEE numbers (-0 == +0).  ctx 0 gives all -1. */
typedef struct {
  float v;
  int32_t s;
} vs_t;

static int by_value_desc_pos_asc(const void *pa, const void *pb) {
  const vs_t *a = (const vs_t *)pa, *b = (const vs_t *)pb;
  if (a->v > b->v) return -1;
  if (a->v < b->v) return 1;
  return (a->s > b->s) - (a->s < b->s);
}

static int by_pos(const void *pa, const void *pb) {
  int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
  return (a > b) - (a < b);
}

int orc_topk(const float *logits, int64_t n_rows, int64_t logits_stride, const int32_t *row_ctx, int32_t k,
             int32_t *out_idx) {
  if (n_rows < 0 || k <= 0) return -1;
  for (int64_t t = 0; t < n_rows; ++t)
    if (row_ctx[t] < 0 || row_ctx[t] > logits_stride) return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < n_rows; ++t) {
    int32_t c = row_ctx[t];
    int32_t *o = out_idx + t * k;
    vs_t *a = (vs_t *)malloc(sizeof(vs_t) * (size_t)(c > 0 ? c : 1));
    for (int32_t s = 0; s < c; ++s) {
      float v = logits[t * logits_stride + s];
      a[s].v = (v == 0.0f) ? 0.0f : v; /* -0 and +0 are one value */
      a[s].s = s;
    }
    qsort(a, (size_t)c, sizeof(vs_t), by_value_desc_pos_asc);
    int32_t kk = c < k ? c : k;
    for (int32_t i = 0; i < kk; ++i) o[i] = a[i].s;
    qsort(o, (size_t)kk, sizeof(int32_t), by_pos);
    for (int32_t i = kk; i < k; ++i) o[i] = -1;
    free(a);
  }
  return 0;
}

/* Vector form of orc_e2m1_code, for exhaustive checks of the rounding rule. */
void orc_e2m1_codes(const float *z, int64_t n, int e, uint8_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_e2m1_code(z[i], e);
}
