/*
 * kvdecode.h -- C ABI of libkvdecode.so: one autoregressive decode step of
 * grouped-query attention on an AMD Instinct MI355X (gfx950).
 *
 * The step is the one the pages below describe for inference with a KV cache:
 *   1. rope_append_kv: rotate the new query and key with RoPE at the token's
 *      position and write the rotated key and the value into a preallocated
 *      KV cache at that position;
 *   2. gqa_decode_attn: softmax(q K^T * scale) V of that single query over all
 *      cached tokens, each KV head shared by n_heads / n_kv_heads query heads.
 *
 * Pages (cited by title and section):
 *   [KVGR] "Transformer推理核心：KV Cache、GQA与RoPE原理与工程实践"
 *   [SA4]  "4. 自注意力机制推理：单步计算、KV Cache的引入与原理"
 *   [OPT]  "Transformer架构优化实战2026：注意力机制、KV Cache与推理加速完整指南"
 *
 * Conventions shared by every call
 * --------------------------------
 * - All pointers to tensors are DEVICE pointers (hipMalloc'd or torch CUDA
 *   tensors) unless stated otherwise; `shape` is a HOST pointer.
 * - Every tensor is dense and row-major in the layout given per argument.
 * - The caller owns every buffer.  The library never allocates, frees or
 *   synchronises inside these calls; work is enqueued on `stream` (a
 *   hipStream_t; NULL = the legacy default stream) and KVD_OK means
 *   "validated and enqueued".
 * - Host-checkable argument errors return a status and enqueue nothing.
 *   Launch failures return KVD_EHIP.
 * - Values that live on the device (positions, seq_lens, block-table
 *   entries) cannot be checked on the host.  The kernels never read or write
 *   outside the buffers the shape describes: an out-of-range position or
 *   block id skips that append; a length above max_seq_len_host is clamped
 *   to it; a block id outside [0, num_blocks) contributes nothing.  Outputs
 *   for such inputs are unspecified.
 * - The library holds no state between calls apart from a per-device cache
 *   of the compute-unit count: plan overrides and timing events travel with
 *   the call (kvd_options).  Calls on different streams are independent as
 *   long as they do not share a workspace or an output buffer.
 */
#ifndef KVDECODE_H
#define KVDECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVD_OK = 0,
  KVD_EINVAL = 1,        /* null pointer, inconsistent shape, aliasing */
  KVD_EUNSUPPORTED = 2,  /* head_dim, dtype or block_size not supported */
  KVD_ERANGE = 3,        /* max_seq_len_host outside [0, max_seq_len] */
  KVD_EWORKSPACE = 4,    /* workspace missing or smaller than required */
  KVD_EHIP = 5           /* a HIP runtime call or launch failed */
} kvd_status;

typedef enum {
  KVD_FP32 = 0,          /* IEEE binary32 */
  KVD_BF16 = 1,          /* bfloat16 (upper half of a binary32) */
  /* INT8 cache ([KVGR] §4.3): K and V held as signed 8-bit codes with one
   * fp32 scale per KV head for each; q, k_new and v_new are bfloat16.  Only
   * the *_int8 calls below accept it.  Layout: tokens grouped by 16, each
   * group holding per KV head its K rows and its V block transposed (see
   * rope_append_kv_int8). */
  KVD_INT8 = 2
} kvd_dtype;

typedef enum {
  /* Pair (2i, 2i+1) is (real, imag) of the i-th complex number: the pages'
   * reading of RoPE as interleaved real/imaginary parts ([KVGR] §3). */
  KVD_ROPE_INTERLEAVED = 0,
  /* Pair (i, i + D/2): the "rotate half" arrangement. */
  KVD_ROPE_HALF = 1
} kvd_rope_style;

/*
 * Geometry of the decode problem.
 *   batch       B >= 0 sequences (B == 0: the calls validate and do nothing)
 *   n_heads     H >= 1 query heads
 *   n_kv_heads  G >= 1 KV heads; H % G == 0 ([OPT] §六 asserts it); query head
 *               h reads KV head h / (H / G) ([KVGR] §2.2, repeat_interleave)
 *   head_dim    D in {64, 128}
 *   kv_dtype    kvd_dtype of q, k_new, v_new, k_cache and v_cache (KVD_INT8:
 *               caches only, the rest bfloat16)
 *   block_size  0  = contiguous cache  [B, max_seq_len, G, D]
 *                    ([OPT] §四 KVCache: (batch, seq, heads, head_dim));
 *               16 or 32 = paged pool [num_blocks, block_size, G, D] with an
 *                    int32 block table [B, max_blocks_per_seq]: token p of
 *                    sequence b is row p % block_size of block
 *                    table[b][p / block_size] ([OPT] §四 PagedKVCache;
 *                    [KVGR] §4.1, 16-token blocks; [OPT] §九 recommends 32
 *                    for long sequences).  Several rows may name the same
 *                    block (a shared prompt prefix, [OPT] §九 prefix
 *                    caching), read only: a block that receives an append
 *                    must belong to that sequence alone (copying a shared
 *                    block before writing it is the caller's)
 *   max_seq_len contiguous: S_max, the row capacity per sequence (a multiple
 *               of 16 for KVD_INT8); paged: must equal
 *               max_blocks_per_seq * block_size
 *   num_blocks  paged: pool size (>= 1); contiguous: ignored
 *   max_blocks_per_seq  paged: table row stride (>= 1); contiguous: ignored
 */
typedef struct kvd_shape {
  int32_t batch;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t kv_dtype;
  int32_t block_size;
  int32_t max_seq_len;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
} kvd_shape;

/* Kernels of the split-K attention (kvd_options.kernel, kvd_get_plan). */
typedef enum {
  KVD_KERNEL_AUTO = 0,   /* the planner's choice */
  KVD_KERNEL_VALU = 1,   /* vector-ALU dot products: fp32 and bf16 caches, one new token */
  KVD_KERNEL_MFMA = 2,   /* matrix cores: bf16 caches, up to 32 query rows per KV head */
  KVD_KERNEL_INT8 = 3    /* matrix cores on INT8 codes: INT8 caches (their only kernel) */
} kvd_kernel;

/* Order in which the (sequence, KV head, split) units of the matrix-core
 * decode kernels, or the (sequence, KV head, query tile) workgroups of the
 * prefill kernel, are dispatched (kvd_options.dispatch_order).  Results do
 * not depend on it: each unit writes its own partial and the merge reads
 * them in split order; each prefill workgroup writes its own rows.  Values
 * 1-5 apply to the decode calls, 6-8 to gqa_prefill_attn; the other kind
 * gives EINVAL. */
typedef enum {
  KVD_ORDER_AUTO = 0,            /* the planner's choice */
  KVD_ORDER_SPLIT_HEAD_SEQ = 1,  /* split fastest, then KV head, then sequence */
  KVD_ORDER_HEAD_SEQ_SPLIT = 2,  /* KV head fastest, then sequence, then split */
  KVD_ORDER_HEAD_SPLIT_SEQ = 3,  /* KV head fastest, then split, then sequence */
  /* a work list of the (sequence, split) units that hold tokens, built on
   * the device from seq_lens by a kernel before the split kernel: full
   * splits sequence by sequence, then the partial last splits longest
   * first (ignored with a single split) */
  KVD_ORDER_DEVICE_LIST = 4,
  /* the same list derived inside the split kernel without the extra launch
   * (batches of at most 64 sequences; ignored otherwise) */
  KVD_ORDER_WAVE_LIST = 5,
  /* prefill: (sequence, KV head) pair fastest, the query tiles with the
   * most keys first */
  KVD_ORDER_PREFILL_PAIRS_FASTEST = 6,
  /* prefill: the query tiles of one pair consecutive (most keys first),
   * pairs in order */
  KVD_ORDER_PREFILL_TILES_FASTEST = 7,
  /* prefill: the order of 7, but each XCD (the device hands consecutive
   * workgroups to its XCDs in turn) takes a contiguous run of it, so the
   * query tiles that read one pair's keys share that XCD's L2 */
  KVD_ORDER_PREFILL_XCD_RUNS = 8
} kvd_dispatch_order;

/*
 * Per-call options of the attention calls that take them.  A NULL pointer,
 * or a zero-initialised struct, means "automatic" for every field.
 *   kernel           kvd_kernel; a kernel that cannot run this call gives
 *                    EUNSUPPORTED
 *   split_tokens     tokens per split: 0 automatic, else a multiple of 16 in
 *                    [16, 8192]
 *   tail_split_tokens, tail_span_tokens
 *                    the last tail_span_tokens positions of the length bound
 *                    (0: those after the last whole split) are cut into
 *                    splits of tail_split_tokens (a multiple of 16, at most
 *                    the split size; 0: none), so that the units dispatched
 *                    last are short
 *   dispatch_order   kvd_dispatch_order
 *   reserved         must be 0
 *   event_start, event_stop
 *                    hipEvent_t handles (both or neither, created by the
 *                    caller with timing enabled) tied to the dispatch of the
 *                    call's main kernel -- the split-K kernel, the prefill
 *                    kernel -- through hipExtLaunchKernel: they take that
 *                    kernel's own start and end times, so their interval is
 *                    its execution; NULL: none
 * Errors: EINVAL for values outside these ranges.
 */
typedef struct kvd_options {
  int32_t kernel;
  int32_t split_tokens;
  int32_t tail_split_tokens;
  int32_t tail_span_tokens;
  int32_t dispatch_order;
  int32_t reserved;
  void* event_start;
  void* event_stop;
} kvd_options;

/*
 * rope_append_kv -- RoPE on q and the new k, then the cache append.
 *
 * For every sequence b with P = positions[b]:
 *   theta_i = rope_base^(-2i/D), angle_i = P * theta_i  ([KVGR] §3);
 *   every pair (a, c) of q[b,h,:] and k_new[b,g,:] becomes
 *   (a cos - c sin, a sin + c cos), i.e. multiplication by cos + i sin;
 *   q_rot[b,h,:] = rotated q (fp32);
 *   K cache slot (b, P, g) = rotated k_new, rounded once (nearest-even) from
 *   the exact rotation to kv_dtype; V slot (b, P, g) = v_new, bit copy
 *   ([SA4] §4.5: preallocated cache written at index `step`; [OPT] §四
 *   KVCache.update).  The cache stores rotated keys, so history is never
 *   rotated again ([KVGR] §3).  V is not rotated.
 *
 *   q          [B, H, D] kv_dtype, or NULL to rotate and append k/v only
 *   k_new      [B, G, D] kv_dtype, not yet rotated
 *   v_new      [B, G, D] kv_dtype
 *   q_rot      [B, H, D] fp32 output (ignored when q == NULL); must not
 *              overlap q, k_new, v_new or the caches
 *   k_cache, v_cache   cache tensors as described by `shape`; modified in
 *              place at the B appended slots only
 *   positions  [B] int32, 0 <= positions[b] < max_seq_len (the number of
 *              tokens already cached for sequence b)
 *   block_table  [B, max_blocks_per_seq] int32 when paged, NULL otherwise;
 *              the block that receives an append must belong to that
 *              sequence alone
 *   rope_base  > 0 (10000 in the pages; some models use 1e6)
 *   rope_style kvd_rope_style
 * Buffers need only their element alignment.  When q, k_new, v_new, q_rot
 * and the caches are all 16-byte aligned and the call appends 128 tokens or
 * more, a vector form of the kernel runs; it writes the same bits.
 * Errors: EINVAL (null pointer, H % G != 0, B < 0, table given for a
 * contiguous cache or missing for a paged one, q_rot == q, base <= 0),
 * EUNSUPPORTED (head_dim, kv_dtype, block_size, rope_style), EHIP.
 */
kvd_status rope_append_kv(const kvd_shape* shape, const void* q, const void* k_new,
                          const void* v_new, float* q_rot, void* k_cache, void* v_cache,
                          const int32_t* positions, const int32_t* block_table,
                          double rope_base, int32_t rope_style, void* stream);

/*
 * gqa_decode_attn -- one query per (b, h) attending over its sequence.
 *
 *   s_j = scale * <q_rot[b,h,:], K[b, j, h / (H/G), :]>   for j < L_b,
 *   out[b,h,:] = sum_j softmax(s)_j * V[b, j, h / (H/G), :],
 *   lse[b,h]   = ln(sum_j exp(s_j))
 * with L_b = seq_lens[b] ([KVGR] §2.1 and §4.2; [SA4] §4.1, §4.5: attend
 * over cache[:step+1]).  Tokens j >= L_b are never read (the causal bound
 * of the last position, [KVGR] §5.1).  The work is split along the sequence
 * in chunks that are multiples of 16 tokens; partial results are merged by
 * log-sum-exp in a second kernel when more than one chunk is needed.
 *
 *   q_rot      [B, H, D] fp32 (already rotated, e.g. by rope_append_kv)
 *   k_cache, v_cache   as described by `shape` (read only)
 *   seq_lens   [B] int32, 0 <= seq_lens[b] <= max_seq_len_host
 *              (seq_lens[b] == 0 gives out = 0 and lse = -inf)
 *   block_table  as in rope_append_kv
 *   max_seq_len_host  host-side upper bound of seq_lens, used to plan the
 *              grid; 0 <= max_seq_len_host <= shape->max_seq_len
 *   scale      softmax scale, finite; 0 selects the default 1/sqrt(D)
 *              ([KVGR] §2.1: d_k is the per-head dimension; [OPT] §三: the
 *              default 1/sqrt(d_k)), computed by the library in double
 *              precision
 *   out        [B, H, D] fp32 output
 *   lse        [B, H] fp32 output (natural log), or NULL
 *   workspace  device scratch of at least gqa_decode_workspace_size(shape,
 *              max_seq_len_host) bytes, 256-byte aligned, or NULL when that
 *              size is 0; contents on entry are ignored.  Calls that may
 *              run at the same time (other streams) need separate
 *              workspaces.
 * Errors: EINVAL (null pointers, inconsistent shape, out overlapping q_rot),
 * EUNSUPPORTED, ERANGE (max_seq_len_host), EWORKSPACE, EHIP.
 */
kvd_status gqa_decode_attn(const kvd_shape* shape, const float* q_rot, const void* k_cache,
                           const void* v_cache, const int32_t* seq_lens,
                           const int32_t* block_table, int32_t max_seq_len_host,
                           float scale, float* out, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * rope_append_kv_int8 -- rope_append_kv for an INT8 cache
 * (shape->kv_dtype == KVD_INT8).
 *
 * [KVGR] §4.3 stores the cached K and V as 8-bit integers instead of
 * 16-bit floats, with quantisation parameters calibrated per attention
 * head.  Here: a code n in [-127, 127] stands for scale[g] * n, with
 * k_scale[g] for K and v_scale[g] for V (calibrated by the caller).  The
 * rotation is as in rope_append_kv; the stored K code is the integer nearest
 * to (exact rotated key) / k_scale[g] and the V code the one nearest to
 * v_new / v_scale[g], the quotient taken in fp64, ties to even, saturating at
 * +-127 (a NaN quotient stores 0).
 *
 *   q, k_new, v_new   bfloat16, shapes as in rope_append_kv
 *   q_rot      [B, H, D] fp32 output (ignored when q == NULL)
 *   k_cache    int8, tokens grouped by 16 and each group by head:
 *              contiguous [B, max_seq_len / 16, G, 16, D], paged
 *              [num_blocks, block_size / 16, G, 16, D]; element (token p,
 *              head g, dim d) is [b, p / 16, g, p % 16, d] (contiguous) or
 *              [table[b][p / block_size], (p % block_size) / 16, g, p % 16, d]
 *   v_cache    int8, the same grouping with each head's block transposed:
 *              [B, max_seq_len / 16, G, D, 16] or [num_blocks,
 *              block_size / 16, G, D, 16]; element (p, g, d) is [.., group,
 *              g, d, p % 16]
 *   k_scale, v_scale  [G] fp32 device arrays, finite and > 0
 *   positions, block_table, rope_base, rope_style   as in rope_append_kv
 * Errors: as rope_append_kv; EUNSUPPORTED when kv_dtype is not KVD_INT8 (and
 * rope_append_kv itself rejects KVD_INT8); EINVAL for null scales.
 */
kvd_status rope_append_kv_int8(const kvd_shape* shape, const void* q, const void* k_new,
                               const void* v_new, float* q_rot, int8_t* k_cache,
                               int8_t* v_cache, const float* k_scale, const float* v_scale,
                               const int32_t* positions, const int32_t* block_table,
                               double rope_base, int32_t rope_style, void* stream);

/*
 * gqa_decode_attn_int8 -- gqa_decode_attn over an INT8 cache
 * (shape->kv_dtype == KVD_INT8): the same result with K[.., g, :] =
 * k_scale[g] * codes and V[.., g, :] = v_scale[g] * codes, layouts as in
 * rope_append_kv_int8.  Up to 32 query heads per KV head.  Arguments,
 * workspace and errors as gqa_decode_attn (workspace size from
 * gqa_decode_workspace_size with the same shape); EUNSUPPORTED for more
 * than 32 query heads per KV head or a non-INT8 shape (gqa_decode_attn
 * itself rejects KVD_INT8); EINVAL for null scales.
 */
kvd_status gqa_decode_attn_int8(const kvd_shape* shape, const float* q_rot,
                                const int8_t* k_cache, const int8_t* v_cache,
                                const float* k_scale, const float* v_scale,
                                const int32_t* seq_lens, const int32_t* block_table,
                                int32_t max_seq_len_host, float scale, float* out, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace gqa_decode_attn needs for this shape and length bound
 * on the current device with the automatic plan (0 when no split merge is
 * needed).  Returns 0 for an invalid shape as well; gqa_decode_attn then
 * reports the shape error. */
size_t gqa_decode_workspace_size(const kvd_shape* shape, int32_t max_seq_len_host);

/*
 * Several new tokens per sequence in one step: the verification pass of
 * speculative decoding, in which the target model scores all gamma draft
 * tokens in a single forward ("Transformer架构优化实战2026" §五), i.e.
 * n_query = gamma + 1 queries per sequence under the causal mask of [KVGR]
 * §5.1 inside the window.  With n_query = 1 these are the calls above.
 *
 * rope_append_kv_multi: token t (0 <= t < n_query) of sequence b is at
 * position P + t with P = positions[b]; it is rotated at that position and
 * appended at slot P + t, exactly as rope_append_kv does for one token.
 *   q          [B, n_query, H, D], or NULL (k/v only)
 *   k_new, v_new   [B, n_query, G, D]
 *   q_rot      [B, n_query, H, D] fp32 output
 *   k_scale, v_scale  [G] fp32 for an INT8 cache (as rope_append_kv_int8),
 *              NULL for the other dtypes
 *   input dtypes, caches, block_table, rope_base, rope_style as in
 *   rope_append_kv (bf16 inputs for INT8 caches); every slot P + t must be
 *   below max_seq_len and, when paged, in a block of sequence b's own
 *
 * gqa_decode_attn_multi (the general form of the attention calls: any
 * cache dtype, T new tokens, per-call options): with L_b = seq_lens[b]
 * counting the new tokens
 * (L_b = P + n_query after the append), query t of sequence b attends the
 * tokens j < L_b - n_query + 1 + t, its own and those before it:
 *   out[b, t, h, :], lse[b, t, h] as gqa_decode_attn over those tokens
 *   (a query that sees no token gets out = 0, lse = -inf)
 *   q_rot      [B, n_query, H, D] fp32; out [B, n_query, H, D]; lse
 *              [B, n_query, H] or NULL
 *   k_scale, v_scale  as in rope_append_kv_multi
 *   workspace  gqa_decode_workspace_size_multi(shape, n_query, .., options)
 *              bytes (the options change the plan, hence the size)
 *   options    kvd_options or NULL
 * The matrix-core kernels take the n_query * H / G query rows of a KV head
 * together: at most 32 of them (bf16 and INT8 caches).  fp32 caches take
 * n_query = 1 only.
 * Errors: as the single-token calls; EUNSUPPORTED for n_query outside
 * [1, max_seq_len] (rope_append_kv_multi) or [1, 32] (gqa_decode_attn_multi),
 * more than 32 query rows per KV head, or fp32 with n_query > 1; EINVAL when
 * scales are given for a non-INT8 cache or missing for an INT8 one.  Longer
 * windows (prompts, chunks of prompts) go through gqa_prefill_attn.
 */
kvd_status rope_append_kv_multi(const kvd_shape* shape, int32_t n_query, const void* q,
                                const void* k_new, const void* v_new, float* q_rot,
                                void* k_cache, void* v_cache, const float* k_scale,
                                const float* v_scale, const int32_t* positions,
                                const int32_t* block_table, double rope_base, int32_t rope_style,
                                void* stream);
kvd_status gqa_decode_attn_multi(const kvd_shape* shape, int32_t n_query, const float* q_rot,
                                 const void* k_cache, const void* v_cache, const float* k_scale,
                                 const float* v_scale, const int32_t* seq_lens,
                                 const int32_t* block_table, int32_t max_seq_len_host,
                                 float scale, float* out, float* lse, void* workspace,
                                 size_t workspace_bytes, const kvd_options* options,
                                 void* stream);
/*
 * gqa_prefill_attn -- causal attention of a prompt, or of one chunk of a
 * prompt appended after a cached history: n_query = T new tokens per
 * sequence, already rotated and appended by rope_append_kv_multi, over a
 * bf16 cache (contiguous or paged).  The result is that of
 * gqa_decode_attn_multi for any T: with L_b = seq_lens[b] (the new tokens
 * included), query t of sequence b attends the tokens j < L_b - T + 1 + t
 * ([KVGR] §5.1 b.v causal mask; the tiled online-softmax attention of
 * [KVGR] §4.2, here on the matrix cores).
 *
 * Arithmetic: q * scale and the softmax probabilities are rounded once to
 * bf16 for the matrix cores, accumulation is fp32, and each row is
 * normalised by the fp32 sum of its probabilities (the precision of
 * FlashAttention-2 in bf16: about 1e-3 relative per output element, where
 * gqa_decode_attn_multi keeps q and P to ~2^-17).
 *
 * Key splits: a workgroup owns 128 query rows of one (sequence, KV head)
 * pair.  When those workgroups are too few to fill the device (a short
 * chunk after a long history), each row's keys [0, bound) are cut into
 * splits of split_tokens (whole 32-token tiles); every split writes its
 * normalised output and log2-sum-exp to the workspace, and the splits are
 * merged by their log-sum-exp weights as in gqa_decode_attn (the same
 * blockwise softmax algebra, [KVGR] §4.2).
 *
 *   q_rot      [B, T, H, D] fp32; out [B, T, H, D] fp32; lse [B, T, H] fp32
 *              (natural log) or NULL
 *   k_cache, v_cache, seq_lens, block_table, max_seq_len_host, scale
 *              as in gqa_decode_attn
 *   workspace  NULL (no key split unless options ask for one), or device
 *              memory of gqa_prefill_workspace_size(shape, n_query,
 *              max_seq_len_host, options) bytes, 256-byte aligned, owned by
 *              the caller and not read before it is written; one workspace
 *              per call in flight
 *   options    NULL, or kvd_options with split_tokens (0 automatic, else a
 *              multiple of 32; one split when it covers max_seq_len_host),
 *              a prefill dispatch_order (6-8) and timing events; kernel and
 *              the tail fields must be 0
 * Errors: EINVAL, ERANGE as gqa_decode_attn (EINVAL also for decode plan
 * fields in options); EWORKSPACE when the plan needs a workspace that is
 * missing, smaller than the size above or misaligned; EUNSUPPORTED for a
 * cache dtype other than bf16 or n_query outside [1, max_seq_len]; EHIP.
 */
kvd_status gqa_prefill_attn(const kvd_shape* shape, int32_t n_query, const float* q_rot,
                            const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                            const int32_t* block_table, int32_t max_seq_len_host, float scale,
                            float* out, float* lse, void* workspace, size_t workspace_bytes,
                            const kvd_options* options, void* stream);

/*
 * gqa_prefill_attn_int8 -- gqa_prefill_attn over an INT8 cache (layout and
 * per-head scales as in gqa_decode_attn_int8; [KVGR] §4.3).  Each key tile's
 * codes are converted once per workgroup to exact fp16 values; q * scale and
 * the probabilities are rounded once to fp16 for the matrix cores, fp32
 * accumulation; the scores are q . code times k_scale[g], the output is
 * scaled by v_scale[g].  Key splits, options and workspace as in
 * gqa_prefill_attn (gqa_prefill_workspace_size takes INT8 shapes too).
 * Errors: as gqa_prefill_attn; EINVAL also for missing scales; EUNSUPPORTED
 * for a cache dtype other than INT8.
 */
kvd_status gqa_prefill_attn_int8(const kvd_shape* shape, int32_t n_query, const float* q_rot,
                                 const void* k_cache, const void* v_cache, const float* k_scale,
                                 const float* v_scale, const int32_t* seq_lens,
                                 const int32_t* block_table, int32_t max_seq_len_host,
                                 float scale, float* out, float* lse, void* workspace,
                                 size_t workspace_bytes, const kvd_options* options,
                                 void* stream);

/*
 * gqa_prefill_workspace_size -- bytes of workspace gqa_prefill_attn (bf16
 * shapes) or gqa_prefill_attn_int8 (INT8 shapes) needs for these arguments
 * with a non-NULL workspace: 0 when the plan has no key split, or when an
 * argument is invalid (the call itself says which).
 */
size_t gqa_prefill_workspace_size(const kvd_shape* shape, int32_t n_query,
                                  int32_t max_seq_len_host, const kvd_options* options);

/*
 * Mixed-precision cache ([KVGR] §4.3 names caches that keep the most recent
 * tokens at high precision and quantise the older history): the `window`
 * (W) newest tokens of each sequence are kept in bf16 rings k_recent /
 * v_recent [B, W, G, D] (token p in row p mod W, the bf16 cache's row
 * layout), every older token in an INT8 cache described by `shape`
 * (kv_dtype KVD_INT8, contiguous or paged, layout and scales as for
 * rope_append_kv_int8), at its own position.  One new token per sequence.
 *
 * rope_append_kv_mixed -- RoPE of q and k as in rope_append_kv; then for
 * every sequence b with P = positions[b] in [0, max_seq_len):
 *   if P >= W, token P - W leaves the ring: its stored bf16 K and V values
 *   are quantised (the code nearest to value / scale[g], ties to even,
 *   saturating at +-127) into the INT8 cache at position P - W (skipped if
 *   that slot's block id is outside the pool);
 *   ring row P mod W then receives the rotated k, rounded once to bf16, and
 *   v_new (bits).
 * A position outside [0, max_seq_len) changes nothing for its sequence.
 *   window     W, 1 <= W <= max_seq_len; k_recent / v_recent bf16
 *              [B, W, G, D], modified in place at row P mod W only
 *   other arguments as rope_append_kv_int8 (q, k_new, v_new bf16)
 * Errors: EINVAL, EUNSUPPORTED (shape not INT8, bad style), ERANGE (window),
 * EHIP.
 */
kvd_status rope_append_kv_mixed(const kvd_shape* shape, int32_t window, const void* q,
                                const void* k_new, const void* v_new, float* q_rot,
                                void* k_cache, void* v_cache, const float* k_scale,
                                const float* v_scale, void* k_recent, void* v_recent,
                                const int32_t* positions, const int32_t* block_table,
                                double rope_base, int32_t rope_style, void* stream);

/*
 * gqa_decode_attn_mixed -- gqa_decode_attn over a mixed-precision cache:
 * with L = seq_lens[b] (clamped to [0, max_seq_len_host]), query (b, h)
 * attends its L tokens, token j read from the rings when j >= L - W and
 * dequantised (scale[g] * code) from the INT8 cache otherwise.  The history
 * runs on the INT8 kernel and the ring on the bf16 kernels (the ring's
 * rows read in ring order: a softmax does not depend on the order of its
 * keys); both write split partials to the workspace and one log-sum-exp
 * merge combines them.  Options: split_tokens and dispatch_order apply to
 * both parts; kernel and the tail fields must be 0 (EINVAL); the timing
 * events bracket both split kernels.
 *   workspace  gqa_decode_workspace_size_mixed(shape, window,
 *              max_seq_len_host, options) bytes, 256-byte aligned
 *   other arguments as gqa_decode_attn_int8; k_recent / v_recent as above
 * Errors: as gqa_decode_attn_multi, and ERANGE for the window.
 */
kvd_status gqa_decode_attn_mixed(const kvd_shape* shape, int32_t window, const float* q_rot,
                                 const void* k_cache, const void* v_cache, const float* k_scale,
                                 const float* v_scale, const void* k_recent,
                                 const void* v_recent, const int32_t* seq_lens,
                                 const int32_t* block_table, int32_t max_seq_len_host,
                                 float scale, float* out, float* lse, void* workspace,
                                 size_t workspace_bytes, const kvd_options* options,
                                 void* stream);

/* Workspace bytes of gqa_decode_attn_mixed (0 for invalid arguments). */
size_t gqa_decode_workspace_size_mixed(const kvd_shape* shape, int32_t window,
                                       int32_t max_seq_len_host, const kvd_options* options);

/*
 * gqa_decode_attn_multi_noalloc -- gqa_decode_attn_multi without a
 * workspace argument, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The split partials and the work list go to a library-owned
 * device array of KVD_NOALLOC_SCRATCH_BYTES (32 MiB), one per device, held
 * until the process ends (looked up with hipGetSymbolAddress on the first
 * call on each device).  The call allocates and frees nothing.
 *   Arguments, results and errors as gqa_decode_attn_multi, and in
 *   addition EWORKSPACE when gqa_decode_workspace_size_multi(shape,
 *   n_query, max_seq_len_host, options) exceeds KVD_NOALLOC_SCRATCH_BYTES
 *   (nothing enqueued).
 *   Calls that may run at the same time on one device (other streams,
 *   other host threads) share the array and race: serialise them.  No
 *   part of the array needs clearing between calls.
 */
#define KVD_NOALLOC_SCRATCH_BYTES (32u << 20)
kvd_status gqa_decode_attn_multi_noalloc(const kvd_shape* shape, int32_t n_query,
                                         const float* q_rot, const void* k_cache,
                                         const void* v_cache, const float* k_scale,
                                         const float* v_scale, const int32_t* seq_lens,
                                         const int32_t* block_table, int32_t max_seq_len_host,
                                         float scale, float* out, float* lse,
                                         const kvd_options* options, void* stream);

/*
 * gqa_decode_step -- the whole decode step in one launch (plus the merge):
 * rope_append_kv followed by gqa_decode_attn_multi with n_query = 1 and
 * seq_lens[b] = positions[b] + 1 ([KVGR] §3 and §5.1 b.ii-vi; [SA4] §4.5),
 * for bf16 caches with up to 32 query heads per KV head (and, below, INT8
 * caches with up to 16).  The split kernel
 * rotates q itself, and for each (sequence, KV head) the workgroup of the
 * last split writes the rotated key and the value into the cache slot
 * before it reads any tile; the results are those of the two calls.
 *   q, k_new, v_new, k_cache, v_cache, positions, block_table, rope_base,
 *              rope_style   as in rope_append_kv (bf16 inputs); q, k_new,
 *              v_new and the caches 16-byte aligned (EINVAL otherwise)
 *   max_seq_len_host  a host bound on positions[b] + 1, in [1, max_seq_len];
 *              attention covers min(positions[b] + 1, max_seq_len_host)
 *              tokens (none for a negative position)
 *   scale, out, lse, workspace, options   as in gqa_decode_attn_multi with
 *              n_query = 1 (the same workspace size); options may not ask
 *              for the VALU kernel
 *   q_rot      [B, H, D] fp32 output of the rotated q, or NULL; written for
 *              every sequence with a non-negative position
 * Errors: as rope_append_kv and gqa_decode_attn_multi; EUNSUPPORTED for a
 * cache that is not bf16 (INT8: gqa_decode_step_int8) or more query heads
 * per KV head than above (use the two calls); ERANGE for max_seq_len_host
 * < 1.
 *
 * gqa_decode_step_multi: n_query = T new tokens per sequence (1 <= T <= 16,
 * T x query heads per KV head <= 32), bf16 caches: rope_append_kv_multi
 * then gqa_decode_attn_multi with seq_lens[b] = positions[b] + T; q, q_rot,
 * out [B, T, H, D], k_new, v_new [B, T, G, D], lse [B, T, H]; workspace
 * gqa_decode_workspace_size_multi(shape, T, ..).  Each split's workgroup
 * appends the window tokens its split holds (the last one also those past
 * max_seq_len_host).  EUNSUPPORTED for T outside [1, 16], more than 32
 * query rows per KV head, or a cache that is not bf16.
 *
 * gqa_decode_step_int8: the same on an INT8 cache with per-head scales
 * k_scale, v_scale [G] (rope_append_kv_int8 then gqa_decode_attn_multi);
 * the new token's codes are those rope_append_kv_int8 writes.
 */
kvd_status gqa_decode_step(const kvd_shape* shape, const void* q, const void* k_new,
                           const void* v_new, void* k_cache, void* v_cache,
                           const int32_t* positions, const int32_t* block_table,
                           int32_t max_seq_len_host, double rope_base, int32_t rope_style,
                           float scale, float* q_rot, float* out, float* lse, void* workspace,
                           size_t workspace_bytes, const kvd_options* options, void* stream);
kvd_status gqa_decode_step_multi(const kvd_shape* shape, int32_t n_query, const void* q,
                                 const void* k_new, const void* v_new, void* k_cache,
                                 void* v_cache, const int32_t* positions,
                                 const int32_t* block_table, int32_t max_seq_len_host,
                                 double rope_base, int32_t rope_style, float scale, float* q_rot,
                                 float* out, float* lse, void* workspace, size_t workspace_bytes,
                                 const kvd_options* options, void* stream);
kvd_status gqa_decode_step_int8(const kvd_shape* shape, const void* q, const void* k_new,
                                const void* v_new, int8_t* k_cache, int8_t* v_cache,
                                const float* k_scale, const float* v_scale,
                                const int32_t* positions, const int32_t* block_table,
                                int32_t max_seq_len_host, double rope_base, int32_t rope_style,
                                float scale, float* q_rot, float* out, float* lse,
                                void* workspace, size_t workspace_bytes,
                                const kvd_options* options, void* stream);

/* Workspace bytes of gqa_decode_attn_multi with these options (NULL:
 * automatic); 0 also for an invalid shape or invalid options. */
size_t gqa_decode_workspace_size_multi(const kvd_shape* shape, int32_t n_query,
                                       int32_t max_seq_len_host, const kvd_options* options);

/* Static, NUL-terminated description of a status code. */
const char* kvd_status_string(int32_t status);

/*
 * Plan inspection.  kvd_get_plan reports how gqa_decode_attn would run:
 * plan[0] = tokens per split (a multiple of 16), plan[1] = number of splits,
 * plan[2] = the kernel (a kvd_kernel value other than AUTO), plan[3] =
 * workgroups launched by the split kernel.  `plan` is a host array of 4
 * int32.  kvd_get_plan_multi does the same for gqa_decode_attn_multi with
 * n_query new tokens and the given options (NULL: automatic).
 * Errors: as the attention calls (EUNSUPPORTED when a requested kernel
 * cannot run the shape).
 */
kvd_status kvd_get_plan(const kvd_shape* shape, int32_t max_seq_len_host, int32_t* plan);
kvd_status kvd_get_plan_multi(const kvd_shape* shape, int32_t n_query, int32_t max_seq_len_host,
                              const kvd_options* options, int32_t* plan);

/*
 * kvd_read_probe -- measurement utility, not part of the decode step: reads
 * `bytes` (a multiple of 16; of 1024 with KVD_PROBE_LDS) of the
 * 16-byte-aligned device buffer `buf` with coalesced 16-byte loads
 * (`unroll` in {1, 4, 8, 16} loads in flight per lane, `n_workgroups`
 * workgroups of 256 threads) and writes one XOR word per workgroup to `sink`
 * (device, n_workgroups uint32).  `mode` is an OR of
 *   KVD_PROBE_CHUNKED      each workgroup streams one contiguous
 *                          1/n_workgroups of the buffer (else the grid
 *                          strides over it together);
 *   KVD_PROBE_NONTEMPORAL  loads carry the non-temporal (streaming) hint;
 *   KVD_PROBE_LDS          the decode kernels' V path: each wave copies 1 KiB
 *                          pieces HBM -> LDS with buffer loads that bypass
 *                          the registers (implies chunked; each workgroup's
 *                          range must stay below 2 GiB).
 * Its duration gives the device's practical streaming-read bandwidth, the
 * roof the decode kernels are compared with beside the nominal HBM peak.
 * Errors: EINVAL, EUNSUPPORTED (unroll), EHIP.
 */
enum { KVD_PROBE_CHUNKED = 1, KVD_PROBE_NONTEMPORAL = 2, KVD_PROBE_LDS = 4 };
kvd_status kvd_read_probe(const void* buf, size_t bytes, uint32_t* sink, int32_t n_workgroups,
                          int32_t unroll, int32_t mode, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVDECODE_H */
