/*
 * kvoracle.c -- plain fp64 CPU oracle for one autoregressive decode step of
 * grouped-query attention with RoPE and a KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library: it is written from the pages
 * alone, as plain loops, so a reader can check it against them by eye.
 *
 * Pages cited (by title):
 *   [KVGR] "Transformer推理核心：KV Cache、GQA与RoPE原理与工程实践"
 *   [SA4]  "4. 自注意力机制推理：单步计算、KV Cache的引入与原理"
 *   [OPT]  "Transformer架构优化实战2026：注意力机制、KV Cache与推理加速完整指南"
 *
 * What is computed, step by step (all arithmetic in fp64):
 *   1. theta_i = base^(-2i/D), i = 0..D/2-1               [KVGR] §3 (the
 *      per-pair frequency formula and its arange(0, dim, 2)/dim code form;
 *      the prose counts i from 1, the code from 0 -- same values).
 *   2. angle = position * theta_i; rotate each pair (a, b) by multiplying
 *      a + i*b with cos(angle) + i*sin(angle)                [KVGR] §3.
 *      Pairs are (2i, 2i+1) ("interleaved", the pages' real/imag reading) or
 *      (i, i + D/2) ("half"), selected by the caller.  V is never rotated.
 *   3. The new k (rotated) and v are written into the preallocated cache at
 *      slot `position`, every other slot untouched             [SA4] §4.5;
 *      [OPT] §四 (KVCache.update).  Stored k is rounded ONCE from the fp64
 *      rotated value to the cache dtype, round-to-nearest-even.
 *      Paged caches map position p of sequence b to physical block
 *      table[b][p / block_size], offset p % block_size         [OPT] §四
 *      (PagedKVCache), [KVGR] §4.1.
 *   4. For query head h the cache head is g = h / n_rep (repeat_interleave
 *      on the head axis)                          [KVGR] §2.2; [OPT] §六.
 *   5. s_j = scale * <q_rot, K_j> for j < L (the causal bound of one query at
 *      the last position), textbook two-pass softmax, o = sum_j p_j V_j,
 *      lse = m + ln(sum_j e_j)         [KVGR] §2.1; [SA4] §4.1, §4.5.
 *   6. Several new tokens per step (the *_mq functions, T = n_query): the
 *      verification pass of speculative decoding, where the target model
 *      processes the gamma draft tokens in one forward ([OPT] §五).  The T
 *      new tokens of sequence b sit at positions P_b .. P_b + T - 1 and are
 *      all appended; query t attends the tokens j <= P_b + t, i.e. j < L_b -
 *      T + 1 + t with L_b = P_b + T (the causal mask inside the window,
 *      [KVGR] §5.1 b.v).  T = 1 is the single-token step above.
 *
 * Storage dtypes: KVO_F64 (used by the pins' exact decode loop), KVO_F32 and
 * KVO_BF16 (raw 16-bit patterns; value = bits << 16 read as an IEEE float).
 *
 * KVO_I8: the INT8 cache of [KVGR] §4.3 (K and V held as 8-bit integers,
 * quantisation parameters calibrated per attention head).  q, k_new and
 * v_new are then bf16; each cache element is a code n in [-127, 127] whose
 * value is scale[g] * n, with one fp32 scale per KV head for K and one for
 * V.  A new element x is stored as the code nearest to x / scale (ties to
 * even; x is the exact rotated key, or v_new as given).  Layout: tokens are
 * grouped by 16 (contiguous: group r = b * S_max/16 + pos/16; paged: group
 * (block * block_size + pos % block_size) / 16 of the pool, a block being
 * block_size / 16 consecutive groups), and each group holds, per KV head,
 * the 16 K rows
 * ([G][16][D]: element (pos, g, d) at ((r * G + g) * 16 + pos % 16) * D + d)
 * and the V block transposed ([G][D][16]: at ((r * G + g) * D + d) * 16 +
 * pos % 16).
 *
 * Mixed precision (the *_mixed functions): [KVGR] §4.3 also names caches that
 * keep the most recent tokens at high precision and quantise the older
 * history.  Here the W newest tokens of each sequence sit in a bf16 ring
 * [B, W, G, D] (token p in row p mod W) and every older token in an INT8
 * cache as above, at its own position.  Appending the token at position P
 * (one per sequence): when P >= W, token P - W leaves the ring -- its stored
 * bf16 K and V values become codes (nearest to value / scale, as for a new
 * INT8 element) at position P - W of the INT8 cache -- and then the rotated k
 * (one rounding to bf16) and v_new take ring row P mod W.  Attention over L
 * tokens reads token j from the ring when j >= L - W, else from the INT8
 * cache.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { KVO_F64 = 0, KVO_F32 = 1, KVO_BF16 = 2, KVO_I8 = 3 };
enum { KVO_INTERLEAVED = 0, KVO_HALF = 1 };

typedef struct {
  int32_t batch, n_heads, n_kv_heads, head_dim;
  int32_t dtype;              /* storage dtype of q, k_new, v_new and caches */
  int32_t block_size;         /* 0: contiguous [B, S_max, G, D]; >0: paged pool */
  int32_t max_seq_len;        /* contiguous S_max (paged: row capacity per seq) */
  int32_t num_blocks;         /* paged pool size */
  int32_t max_blocks_per_seq; /* paged block-table row stride */
} kvo_shape;

/* ---------------------------------------------------------------- scalars */

static double bf16_bits_to_double(uint16_t bits) {
  uint32_t w = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

/* Nearest bf16 value of x (ties to even), computed directly from x so there
 * is exactly one rounding.  bf16 keeps 8 significant bits; its normal range
 * starts at 2^-126 and its subnormals are multiples of 2^-133. */
double kvo_round_to_bf16(double x) {
  if (isnan(x) || isinf(x) || x == 0.0) return x;
  int e;
  (void)frexp(fabs(x), &e);          /* |x| = f * 2^e, f in [0.5, 1) */
  int qexp = e - 8;                  /* spacing of 8-bit significands there */
  if (qexp < -133) qexp = -133;      /* subnormal spacing */
  double r = ldexp(nearbyint(ldexp(fabs(x), -qexp)), qexp);
  const double bf16_max = ldexp(255.0, 120);  /* (2 - 2^-7) * 2^127 */
  if (r > bf16_max) r = INFINITY;
  return copysign(r, x);
}

uint16_t kvo_bf16_bits(double x) {
  float f = (float)kvo_round_to_bf16(x);  /* exact: the value is a bf16 */
  uint32_t w;
  memcpy(&w, &f, sizeof w);
  if (isnan(x)) w = (w & 0x80000000u) | 0x7fc00000u;
  return (uint16_t)(w >> 16);
}

/* INT8 code of x under scale s ([KVGR] §4.3): the integer in [-127, 127]
 * nearest to x / s, ties to even, the quotient taken in fp64.  A NaN quotient
 * gives 0; quotients beyond the range saturate at +-127. */
int kvo_quantize_i8(double x, double s) {
  double q = x / s;
  if (isnan(q)) return 0;
  if (q >= 127.0) return 127;
  if (q <= -127.0) return -127;
  return (int)nearbyint(q);   /* default rounding mode: nearest, ties to even */
}

static double load_elem(const void* p, int dtype, int64_t i) {
  switch (dtype) {
    case KVO_F64: return ((const double*)p)[i];
    case KVO_F32: return (double)((const float*)p)[i];
    default:      return bf16_bits_to_double(((const uint16_t*)p)[i]);
  }
}

static void store_elem(void* p, int dtype, int64_t i, double v) {
  switch (dtype) {
    case KVO_F64: ((double*)p)[i] = v; break;
    case KVO_F32: ((float*)p)[i] = (float)v; break;  /* one RNE rounding */
    default:      ((uint16_t*)p)[i] = kvo_bf16_bits(v); break;
  }
}

/* dtype of q, k_new and v_new: bf16 in front of an INT8 cache */
static int input_dtype(int dtype) { return dtype == KVO_I8 ? KVO_BF16 : dtype; }

/* Copy one stored element without any arithmetic (the append of v). */
static void copy_elem(void* dst, int64_t di, const void* src, int64_t si, int dtype) {
  switch (dtype) {
    case KVO_F64: ((double*)dst)[di] = ((const double*)src)[si]; break;
    case KVO_F32: ((float*)dst)[di] = ((const float*)src)[si]; break;
    default:      ((uint16_t*)dst)[di] = ((const uint16_t*)src)[si]; break;
  }
}

/* ------------------------------------------------------------------ RoPE */

double kvo_theta(int i, int head_dim, double base) {
  return pow(base, -2.0 * (double)i / (double)head_dim);
}

/* y = R_pos x for one head vector of length D (x and y may not alias). */
void kvo_rope_rotate(const double* x, double* y, int head_dim, double pos,
                     double base, int style) {
  int half = head_dim / 2;
  for (int i = 0; i < half; ++i) {
    double angle = pos * kvo_theta(i, head_dim, base);
    double c = cos(angle), s = sin(angle);
    int ia = (style == KVO_HALF) ? i : 2 * i;
    int ib = (style == KVO_HALF) ? i + half : 2 * i + 1;
    double a = x[ia], b = x[ib];
    y[ia] = a * c - b * s;   /* real part of (a + ib)(c + is) */
    y[ib] = a * s + b * c;   /* imaginary part */
  }
}

/* ------------------------------------------------------- cache addressing */

/* Row index (in units of D elements) of token `pos` of sequence b, KV head g;
 * -1 when the slot does not exist. */
static int64_t cache_row(const kvo_shape* sh, const int32_t* table, int b, int64_t pos, int g) {
  if (pos < 0 || pos >= sh->max_seq_len) return -1;
  if (sh->block_size == 0) {
    return ((int64_t)b * sh->max_seq_len + pos) * sh->n_kv_heads + g;
  }
  int64_t logical = pos / sh->block_size;
  if (logical >= sh->max_blocks_per_seq) return -1;
  int32_t phys = table[(int64_t)b * sh->max_blocks_per_seq + logical];
  if (phys < 0 || phys >= sh->num_blocks) return -1;
  int64_t off = pos % sh->block_size;
  return ((int64_t)phys * sh->block_size + off) * sh->n_kv_heads + g;
}

/* INT8 caches: the 16-token group of slot (b, pos) whose row is `row`
 * (cache_row's result, which carries the block-table lookup); -1 when the
 * slot does not exist. */
static int64_t i8_group(const kvo_shape* sh, int b, int64_t pos, int64_t row) {
  if (row < 0) return -1;
  if (sh->block_size == 0) return (int64_t)b * (sh->max_seq_len / 16) + pos / 16;
  /* a physical block of block_size tokens is block_size / 16 groups */
  return (row / sh->n_kv_heads) / 16;
}

/* INT8 K element (pos, g, d): group-major, the head's 16 rows together */
static int64_t kq_index(const kvo_shape* sh, int b, int64_t pos, int g, int d, int64_t row) {
  int64_t r = i8_group(sh, b, pos, row);
  if (r < 0) return -1;
  return ((r * sh->n_kv_heads + g) * 16 + pos % 16) * sh->head_dim + d;
}

/* INT8 V element (pos, g, d): group-major, the head's block transposed */
static int64_t vt_index(const kvo_shape* sh, int b, int64_t pos, int g, int d, int64_t row) {
  int64_t r = i8_group(sh, b, pos, row);
  if (r < 0) return -1;
  return ((r * sh->n_kv_heads + g) * sh->head_dim + d) * 16 + pos % 16;
}

/* ----------------------------------------------------- rope + cache append */

/* q: [B,H,D], k_new/v_new: [B,G,D] in the input dtype (q may be NULL).
 * q_rot: [B,H,D] fp64 out.  Caches are modified in place at slot positions[b].
 * k_scale/v_scale: [G] per-head scales of an INT8 cache (NULL otherwise).
 * Returns 0, or -1 when a position or block id is out of range (that
 * sequence's append is then skipped). */
static int rope_append_impl(const kvo_shape* sh, int T, const void* q, const void* k_new,
                            const void* v_new, double* q_rot, void* k_cache,
                            void* v_cache, const float* k_scale, const float* v_scale,
                            const int32_t* positions, const int32_t* block_table,
                            double base, int style) {
  const int H = sh->n_heads, G = sh->n_kv_heads, D = sh->head_dim;
  const int in_dt = input_dtype(sh->dtype);
  int rc = 0;
  double* x = (double*)malloc(sizeof(double) * D);
  double* y = (double*)malloc(sizeof(double) * D);
  /* row bt = b * T + t holds new token t of sequence b, at position P_b + t */
  for (int bt = 0; bt < sh->batch * T; ++bt) {
    const int b = bt / T;
    const int64_t slot = (int64_t)positions[b] + bt % T;
    double pos = (double)slot;
    if (q != NULL) {
      for (int h = 0; h < H; ++h) {
        int64_t base_i = ((int64_t)bt * H + h) * D;
        for (int d = 0; d < D; ++d) x[d] = load_elem(q, in_dt, base_i + d);
        kvo_rope_rotate(x, y, D, pos, base, style);
        for (int d = 0; d < D; ++d) q_rot[base_i + d] = y[d];
      }
    }
    for (int g = 0; g < G; ++g) {
      int64_t row = cache_row(sh, block_table, b, slot, g);
      if (row < 0) { rc = -1; continue; }
      int64_t src = ((int64_t)bt * G + g) * D;
      for (int d = 0; d < D; ++d) x[d] = load_elem(k_new, in_dt, src + d);
      kvo_rope_rotate(x, y, D, pos, base, style);
      for (int d = 0; d < D; ++d) {
        if (sh->dtype == KVO_I8) {
          /* codes of the exact rotated key and of v_new ([KVGR] §4.3) */
          ((int8_t*)k_cache)[kq_index(sh, b, slot, g, d, row)] =
              (int8_t)kvo_quantize_i8(y[d], k_scale[g]);
          ((int8_t*)v_cache)[vt_index(sh, b, slot, g, d, row)] =
              (int8_t)kvo_quantize_i8(load_elem(v_new, in_dt, src + d), v_scale[g]);
        } else {
          store_elem(k_cache, sh->dtype, row * D + d, y[d]);
          copy_elem(v_cache, row * D + d, v_new, src + d, sh->dtype);
        }
      }
    }
  }
  free(x);
  free(y);
  return rc;
}

int kvo_rope_append(const kvo_shape* sh, const void* q, const void* k_new,
                    const void* v_new, double* q_rot, void* k_cache,
                    void* v_cache, const int32_t* positions,
                    const int32_t* block_table, double base, int style) {
  if (sh->dtype == KVO_I8) return -2;   /* needs the scales */
  return rope_append_impl(sh, 1, q, k_new, v_new, q_rot, k_cache, v_cache, NULL, NULL,
                          positions, block_table, base, style);
}

/* The append into an INT8 cache (sh->dtype == KVO_I8). */
int kvo_rope_append_i8(const kvo_shape* sh, const void* q, const void* k_new,
                       const void* v_new, double* q_rot, int8_t* k_cache,
                       int8_t* v_cache, const float* k_scale, const float* v_scale,
                       const int32_t* positions, const int32_t* block_table,
                       double base, int style) {
  if (sh->dtype != KVO_I8) return -2;
  return rope_append_impl(sh, 1, q, k_new, v_new, q_rot, k_cache, v_cache, k_scale, v_scale,
                          positions, block_table, base, style);
}

/* T new tokens per sequence (q [B,T,H,D], k_new/v_new [B,T,G,D], q_rot
 * [B,T,H,D]); token t of sequence b goes to slot positions[b] + t.  Scales
 * only for an INT8 cache. */
int kvo_rope_append_mq(const kvo_shape* sh, int T, const void* q, const void* k_new,
                       const void* v_new, double* q_rot, void* k_cache, void* v_cache,
                       const float* k_scale, const float* v_scale, const int32_t* positions,
                       const int32_t* block_table, double base, int style) {
  if (T < 1 || (sh->dtype == KVO_I8) != (k_scale != NULL && v_scale != NULL)) return -2;
  return rope_append_impl(sh, T, q, k_new, v_new, q_rot, k_cache, v_cache, k_scale, v_scale,
                          positions, block_table, base, style);
}

/* The mixed-precision append (file header): sh describes the INT8 cache,
 * k_recent / v_recent the bf16 rings [B, window, G, D] (bit patterns).
 * Returns 0, or -1 when a position is outside [0, max_seq_len) (that
 * sequence's cache update is skipped) or the INT8 slot of a leaving token
 * does not exist (that token's codes are not written; the ring row is still
 * overwritten). */
int kvo_rope_append_mixed(const kvo_shape* sh, int window, const void* q, const void* k_new,
                          const void* v_new, double* q_rot, int8_t* k_cache, int8_t* v_cache,
                          const float* k_scale, const float* v_scale, uint16_t* k_recent,
                          uint16_t* v_recent, const int32_t* positions,
                          const int32_t* block_table, double base, int style) {
  if (sh->dtype != KVO_I8 || window < 1) return -2;
  const int H = sh->n_heads, G = sh->n_kv_heads, D = sh->head_dim;
  int rc = 0;
  double* x = (double*)malloc(sizeof(double) * D);
  double* y = (double*)malloc(sizeof(double) * D);
  for (int b = 0; b < sh->batch; ++b) {
    const int64_t P = positions[b];
    if (q != NULL) {
      for (int h = 0; h < H; ++h) {
        int64_t base_i = ((int64_t)b * H + h) * D;
        for (int d = 0; d < D; ++d) x[d] = load_elem(q, KVO_BF16, base_i + d);
        kvo_rope_rotate(x, y, D, (double)P, base, style);
        for (int d = 0; d < D; ++d) q_rot[base_i + d] = y[d];
      }
    }
    if (P < 0 || P >= sh->max_seq_len) { rc = -1; continue; }
    for (int g = 0; g < G; ++g) {
      const int64_t ring = (((int64_t)b * window + P % window) * G + g) * D;
      if (P >= window) {
        /* token P - window leaves the ring for the INT8 cache */
        const int64_t old = P - window;
        int64_t row = cache_row(sh, block_table, b, old, g);
        if (row < 0) {
          rc = -1;
        } else {
          for (int d = 0; d < D; ++d) {
            k_cache[kq_index(sh, b, old, g, d, row)] =
                (int8_t)kvo_quantize_i8(bf16_bits_to_double(k_recent[ring + d]), k_scale[g]);
            v_cache[vt_index(sh, b, old, g, d, row)] =
                (int8_t)kvo_quantize_i8(bf16_bits_to_double(v_recent[ring + d]), v_scale[g]);
          }
        }
      }
      int64_t src = ((int64_t)b * G + g) * D;
      for (int d = 0; d < D; ++d) x[d] = load_elem(k_new, KVO_BF16, src + d);
      kvo_rope_rotate(x, y, D, (double)P, base, style);
      for (int d = 0; d < D; ++d) {
        k_recent[ring + d] = kvo_bf16_bits(y[d]);
        v_recent[ring + d] = ((const uint16_t*)v_new)[src + d];
      }
    }
  }
  free(x);
  free(y);
  return rc;
}

/* ------------------------------------------------------------- attention */

typedef struct {
  const kvo_shape* sh;
  const double* q_rot;
  const void* k_cache;
  const void* v_cache;
  const int32_t* seq_lens;
  const int32_t* table;
  double scale;
  const float* k_scale;    /* INT8 caches: [G] per-head scales */
  const float* v_scale;
  int n_query;             /* T new tokens (queries) per sequence */
  int window;              /* mixed precision: W > 0, the bf16 rings below */
  const uint16_t* k_recent;
  const uint16_t* v_recent;
  const int32_t* unit_b;   /* NULL: unit u is (u / (T H), u % (T H)) */
  const int32_t* unit_h;   /* query row t * H + h of its sequence */
  int64_t n_units;
  double* out;             /* [n_units, D] */
  double* lse;             /* [n_units] or NULL */
  double* probs;           /* [n_units, max_seq_len] or NULL */
  int64_t next;            /* work counter, guarded by mu */
  pthread_mutex_t mu;
  int bad;                 /* set when a referenced slot does not exist */
} attn_job;

/* Value of cached K / V element d of slot (b, j, g) whose row is `row`.
 * INT8 caches dequantise exactly: scale[g] * code ([KVGR] §4.3). */
static double key_at(const attn_job* job, int b, int64_t j, int64_t row, int g, int d) {
  const kvo_shape* sh = job->sh;
  if (sh->dtype == KVO_I8)
    return (double)job->k_scale[g] *
           (double)((const int8_t*)job->k_cache)[kq_index(sh, b, j, g, d, row)];
  return load_elem(job->k_cache, sh->dtype, row * sh->head_dim + d);
}

static double value_at(const attn_job* job, int b, int64_t j, int64_t row, int g, int d) {
  const kvo_shape* sh = job->sh;
  if (sh->dtype == KVO_I8)
    return (double)job->v_scale[g] *
           (double)((const int8_t*)job->v_cache)[vt_index(sh, b, j, g, d, row)];
  return load_elem(job->v_cache, sh->dtype, row * sh->head_dim + d);
}

/* Mixed precision: token j of sequence b is in the ring when it is among the
 * W newest of the L attended (j >= L - W). */
static int in_ring(const attn_job* job, int64_t L, int64_t j) {
  return job->window > 0 && j >= L - job->window;
}

static double ring_at(const attn_job* job, const uint16_t* ring, int b, int64_t j, int g, int d) {
  const kvo_shape* sh = job->sh;
  return bf16_bits_to_double(
      ring[(((int64_t)b * job->window + j % job->window) * sh->n_kv_heads + g) * sh->head_dim + d]);
}

static void attn_unit(attn_job* job, int64_t u, double* s) {
  const kvo_shape* sh = job->sh;
  const int H = sh->n_heads, G = sh->n_kv_heads, D = sh->head_dim;
  const int n_rep = H / G;
  const int T = job->n_query, TH = T * H;
  int b = job->unit_b ? job->unit_b[u] : (int)(u / TH);
  int th = job->unit_h ? job->unit_h[u] : (int)(u % TH);
  int t = th / H, h = th % H;
  int g = h / n_rep;
  int64_t L = job->seq_lens[b];
  const double* q = job->q_rot + ((int64_t)b * TH + th) * D;
  double* o = job->out + u * D;
  for (int d = 0; d < D; ++d) o[d] = 0.0;
  if (L > sh->max_seq_len) { job->bad = 1; L = sh->max_seq_len; }
  L = L - T + 1 + t;                 /* query t sees the tokens up to its own */
  if (L <= 0) {
    if (job->lse) job->lse[u] = -INFINITY;
    return;
  }
  /* pass 1: scores and their maximum */
  double m = -INFINITY;
  for (int64_t j = 0; j < L; ++j) {
    double dot = 0.0;
    if (in_ring(job, L, j)) {
      for (int d = 0; d < D; ++d) dot += q[d] * ring_at(job, job->k_recent, b, j, g, d);
      s[j] = job->scale * dot;
      if (s[j] > m) m = s[j];
      continue;
    }
    int64_t row = cache_row(sh, job->table, b, j, g);
    if (row < 0) { job->bad = 1; s[j] = -INFINITY; continue; }
    for (int d = 0; d < D; ++d) dot += q[d] * key_at(job, b, j, row, g, d);
    s[j] = job->scale * dot;
    if (s[j] > m) m = s[j];
  }
  /* pass 2: exponentials and their sum */
  double l = 0.0;
  for (int64_t j = 0; j < L; ++j) {
    s[j] = exp(s[j] - m);
    l += s[j];
  }
  /* pass 3: normalised weights times V */
  for (int64_t j = 0; j < L; ++j) {
    double p = s[j] / l;
    if (job->probs) job->probs[u * sh->max_seq_len + j] = p;
    if (in_ring(job, L, j)) {
      for (int d = 0; d < D; ++d) o[d] += p * ring_at(job, job->v_recent, b, j, g, d);
      continue;
    }
    int64_t row = cache_row(sh, job->table, b, j, g);
    if (row < 0) continue;
    for (int d = 0; d < D; ++d) o[d] += p * value_at(job, b, j, row, g, d);
  }
  if (job->lse) job->lse[u] = m + log(l);
}

static void* attn_worker(void* arg) {
  attn_job* job = (attn_job*)arg;
  int64_t cap = job->sh->max_seq_len > 0 ? job->sh->max_seq_len : 1;
  double* s = (double*)malloc(sizeof(double) * cap);
  for (;;) {
    pthread_mutex_lock(&job->mu);
    int64_t u = job->next++;
    pthread_mutex_unlock(&job->mu);
    if (u >= job->n_units) break;
    attn_unit(job, u, s);
  }
  free(s);
  return NULL;
}

static int run_attn(attn_job* job, int n_threads) {
  if (n_threads < 1) n_threads = 1;
  if (n_threads > 256) n_threads = 256;
  pthread_mutex_init(&job->mu, NULL);
  job->next = 0;
  job->bad = 0;
  pthread_t tid[256];
  int started = 0;
  for (int t = 1; t < n_threads; ++t)
    if (pthread_create(&tid[started], NULL, attn_worker, job) == 0) ++started;
  attn_worker(job);
  for (int t = 0; t < started; ++t) pthread_join(tid[t], NULL);
  pthread_mutex_destroy(&job->mu);
  return job->bad ? -1 : 0;
}

/* Every (b, h): out [B,H,D], lse [B,H] (may be NULL), probs [B,H,max_seq_len]
 * (may be NULL).  seq_lens[b] tokens are attended.  k_scale/v_scale: the
 * per-head scales of an INT8 cache (NULL for the other dtypes). */
int kvo_decode_attn_mq(const kvo_shape* sh, int T, const double* q_rot, const void* k_cache,
                       const void* v_cache, const float* k_scale, const float* v_scale,
                       const int32_t* seq_lens, const int32_t* block_table, double scale,
                       double* out, double* lse, double* probs, int n_threads) {
  if (T < 1 || (sh->dtype == KVO_I8) != (k_scale != NULL && v_scale != NULL)) return -2;
  attn_job job;
  memset(&job, 0, sizeof job);
  job.sh = sh; job.q_rot = q_rot; job.k_cache = k_cache; job.v_cache = v_cache;
  job.k_scale = k_scale; job.v_scale = v_scale; job.n_query = T;
  job.seq_lens = seq_lens; job.table = block_table; job.scale = scale;
  job.n_units = (int64_t)sh->batch * T * sh->n_heads;
  job.out = out; job.lse = lse; job.probs = probs;
  return run_attn(&job, n_threads);
}

int kvo_decode_attn_i8(const kvo_shape* sh, const double* q_rot, const void* k_cache,
                       const void* v_cache, const float* k_scale, const float* v_scale,
                       const int32_t* seq_lens, const int32_t* block_table, double scale,
                       double* out, double* lse, double* probs, int n_threads) {
  return kvo_decode_attn_mq(sh, 1, q_rot, k_cache, v_cache, k_scale, v_scale, seq_lens,
                            block_table, scale, out, lse, probs, n_threads);
}

int kvo_decode_attn(const kvo_shape* sh, const double* q_rot, const void* k_cache,
                    const void* v_cache, const int32_t* seq_lens,
                    const int32_t* block_table, double scale, double* out,
                    double* lse, double* probs, int n_threads) {
  return kvo_decode_attn_i8(sh, q_rot, k_cache, v_cache, NULL, NULL, seq_lens, block_table,
                            scale, out, lse, probs, n_threads);
}

/* Only the listed (unit_b[u], unit_h[u]) pairs: out [n, D], lse [n]. */
int kvo_decode_attn_units_mq(const kvo_shape* sh, int T, const double* q_rot,
                             const void* k_cache, const void* v_cache,
                             const float* k_scale, const float* v_scale,
                             const int32_t* seq_lens, const int32_t* block_table,
                             double scale, const int32_t* unit_b,
                             const int32_t* unit_h, int64_t n_units, double* out,
                             double* lse, int n_threads) {
  if (T < 1 || (sh->dtype == KVO_I8) != (k_scale != NULL && v_scale != NULL)) return -2;
  attn_job job;
  memset(&job, 0, sizeof job);
  job.sh = sh; job.q_rot = q_rot; job.k_cache = k_cache; job.v_cache = v_cache;
  job.k_scale = k_scale; job.v_scale = v_scale; job.n_query = T;
  job.seq_lens = seq_lens; job.table = block_table; job.scale = scale;
  job.unit_b = unit_b; job.unit_h = unit_h; job.n_units = n_units;
  job.out = out; job.lse = lse;
  return run_attn(&job, n_threads);
}

int kvo_decode_attn_units_i8(const kvo_shape* sh, const double* q_rot,
                             const void* k_cache, const void* v_cache,
                             const float* k_scale, const float* v_scale,
                             const int32_t* seq_lens, const int32_t* block_table,
                             double scale, const int32_t* unit_b,
                             const int32_t* unit_h, int64_t n_units, double* out,
                             double* lse, int n_threads) {
  return kvo_decode_attn_units_mq(sh, 1, q_rot, k_cache, v_cache, k_scale, v_scale, seq_lens,
                                  block_table, scale, unit_b, unit_h, n_units, out, lse,
                                  n_threads);
}

int kvo_decode_attn_units(const kvo_shape* sh, const double* q_rot,
                          const void* k_cache, const void* v_cache,
                          const int32_t* seq_lens, const int32_t* block_table,
                          double scale, const int32_t* unit_b,
                          const int32_t* unit_h, int64_t n_units, double* out,
                          double* lse, int n_threads) {
  return kvo_decode_attn_units_i8(sh, q_rot, k_cache, v_cache, NULL, NULL, seq_lens,
                                  block_table, scale, unit_b, unit_h, n_units, out, lse,
                                  n_threads);
}

/* Attention over a mixed-precision cache (file header): every (b, h), or
 * only the listed units when unit_b is not NULL; one new token per
 * sequence. */
int kvo_decode_attn_mixed(const kvo_shape* sh, int window, const double* q_rot,
                          const void* k_cache, const void* v_cache, const float* k_scale,
                          const float* v_scale, const uint16_t* k_recent,
                          const uint16_t* v_recent, const int32_t* seq_lens,
                          const int32_t* block_table, double scale, const int32_t* unit_b,
                          const int32_t* unit_h, int64_t n_units, double* out, double* lse,
                          int n_threads) {
  if (sh->dtype != KVO_I8 || window < 1 || !k_scale || !v_scale) return -2;
  attn_job job;
  memset(&job, 0, sizeof job);
  job.sh = sh; job.q_rot = q_rot; job.k_cache = k_cache; job.v_cache = v_cache;
  job.k_scale = k_scale; job.v_scale = v_scale; job.n_query = 1;
  job.window = window; job.k_recent = k_recent; job.v_recent = v_recent;
  job.seq_lens = seq_lens; job.table = block_table; job.scale = scale;
  job.unit_b = unit_b; job.unit_h = unit_h;
  job.n_units = unit_b ? n_units : (int64_t)sh->batch * sh->n_heads;
  job.out = out; job.lse = lse;
  return run_attn(&job, n_threads);
}
