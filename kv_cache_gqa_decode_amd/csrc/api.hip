// Host side of libkvdecode.so: the C ABI declared in include/kvdecode.h.
//
// Validation happens entirely on the host before any HIP call, so an invalid
// call returns its status with nothing enqueued.  Planning turns the shape
// and the host bound on sequence lengths into a split size (tokens per
// workgroup, a multiple of 16 so paged and contiguous caches split at the
// same token boundaries) and a grid that fills the device's compute units.
#include <atomic>
#include <cmath>
#include <cstdint>

#include "kvd_internal.h"

using namespace kvd;

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];   // 0 = not yet queried
std::atomic<int> g_xcc_count[kMaxDevices];  // 0 = not yet queried

// Plan overrides and timing events of one call (kvd_options, resolved):
// kernel -1 automatic, 0 VALU, 1 MFMA, 2 INT8 MFMA; order -1 automatic, a
// decode grid order 0-4 or a prefill grid order 5-7 (DecodeParams::grid_order
// 0-2 of the prefill kernel).
struct Tuning {
  int kernel = -1;
  int split = 0;          // tokens per split, 0 automatic
  int tail_split = 0;     // tokens per split near the end, 0 none
  int tail_span = -1;     // tokens covered by those splits, -1 automatic
  int order = -1;
  hipEvent_t ev_start = nullptr;
  hipEvent_t ev_stop = nullptr;
};

// prefill: the options of gqa_prefill_attn (its own dispatch orders; key
// splits of whole 32-token tiles, any length)
kvd_status read_options(const kvd_options* o, Tuning* t, bool prefill = false) {
  *t = Tuning{};
  if (!o) return KVD_OK;
  if (o->kernel < KVD_KERNEL_AUTO || o->kernel > KVD_KERNEL_INT8) return KVD_EINVAL;
  if (o->split_tokens < 0) return KVD_EINVAL;
  if (prefill ? o->split_tokens % kPrefillTile != 0
              : (o->split_tokens % 16 != 0 || o->split_tokens > kMaxChunk))
    return KVD_EINVAL;
  if (o->tail_split_tokens < 0 || o->tail_split_tokens % 16 != 0) return KVD_EINVAL;
  if (o->tail_span_tokens < 0) return KVD_EINVAL;
  if (o->dispatch_order < KVD_ORDER_AUTO || o->dispatch_order > KVD_ORDER_PREFILL_XCD_RUNS)
    return KVD_EINVAL;
  if (o->dispatch_order != KVD_ORDER_AUTO &&
      (o->dispatch_order >= KVD_ORDER_PREFILL_PAIRS_FASTEST) != prefill)
    return KVD_EINVAL;
  if (o->reserved != 0) return KVD_EINVAL;
  if ((o->event_start == nullptr) != (o->event_stop == nullptr)) return KVD_EINVAL;
  t->kernel = o->kernel - 1;
  t->split = o->split_tokens;
  t->tail_split = o->tail_split_tokens;
  t->tail_span = o->tail_span_tokens > 0 ? o->tail_span_tokens : -1;
  t->order = o->dispatch_order - 1;
  t->ev_start = static_cast<hipEvent_t>(o->event_start);
  t->ev_stop = static_cast<hipEvent_t>(o->event_stop);
  return KVD_OK;
}

int device_cu_count(int* cu) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (dev < 0 || dev >= kMaxDevices) return -1;
  int v = g_cu_count[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      return -1;
    g_cu_count[dev].store(v, std::memory_order_relaxed);
  }
  *cu = v;
  return 0;
}

// XCDs of the current device (1 where the runtime does not say)
int device_xcc_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 1;
  int v = g_xcc_count[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || v <= 0)
      v = 1;
    g_xcc_count[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

kvd_status check_shape(const kvd_shape* s) {
  if (!s) return KVD_EINVAL;
  if (s->batch < 0 || s->batch > 65535) return KVD_EINVAL;
  if (s->n_heads < 1 || s->n_kv_heads < 1 || s->n_heads > 4096) return KVD_EINVAL;
  if (s->n_heads % s->n_kv_heads != 0) return KVD_EINVAL;
  if (s->head_dim != 64 && s->head_dim != 128) return KVD_EUNSUPPORTED;
  if (s->kv_dtype != KVD_FP32 && s->kv_dtype != KVD_BF16 && s->kv_dtype != KVD_INT8)
    return KVD_EUNSUPPORTED;
  if (s->block_size != 0 && s->block_size != 16 && s->block_size != 32) return KVD_EUNSUPPORTED;
  if (s->max_seq_len < 1) return KVD_EINVAL;
  // INT8 V is grouped by 16 tokens: a contiguous capacity of whole groups
  if (s->kv_dtype == KVD_INT8 && s->max_seq_len % 16 != 0) return KVD_EUNSUPPORTED;
  if (s->block_size != 0) {
    if (s->num_blocks < 1 || s->max_blocks_per_seq < 1) return KVD_EINVAL;
    if (static_cast<int64_t>(s->max_blocks_per_seq) * s->block_size != s->max_seq_len) return KVD_EINVAL;
    // the kernels address the pool in 16-token groups
    if (static_cast<int64_t>(s->num_blocks) * (s->block_size / 16) > 0x7fffffff) return KVD_EINVAL;
  }
  return KVD_OK;
}

struct Plan {
  int chunk = 0;        // tokens per split (the first n_big splits)
  int chunk2 = 0;       // tokens per split after those
  int n_big = 0;
  int n_splits = 0;
  int kernel = 0;       // 0 VALU, 1 MFMA, 2 INT8 MFMA
  int grid_order = 0;   // matrix-core dispatch order (DecodeParams::grid_order)
  size_t units_offset = 0;   // work list in the workspace (grid_order 3)
  int head_groups = 1;  // VALU: query-head groups per KV head
  int row_groups = 1;   // INT8: workgroups of 16 query rows per KV head (DecodeParams)
  int rb = 1;           // VALU: heads per pass
  int64_t wgs = 0;
  size_t workspace = 0;
};

int round_up(int64_t x, int64_t m) { return static_cast<int>((x + m - 1) / m * m); }

// Splits of [0, max_len): `chunk` tokens each, except that the last
// `tail span` tokens (tuning; none by default) are cut into splits of
// `tail` tokens, so that the units dispatched last are short.
void set_splits(Plan* pl, int chunk, int max_len, const Tuning& tu, bool tail = true) {
  int t2 = tail ? tu.tail_split : 0;
  int span = tu.tail_span;
  if (t2 <= 0 || t2 > chunk) t2 = chunk;
  if (span < 0 || t2 == chunk) span = 0;
  int n_big = span >= max_len ? 0 : (max_len - span) / chunk;
  const int rest = max_len - n_big * chunk;
  pl->chunk = chunk;
  pl->chunk2 = t2;
  pl->n_big = n_big;
  pl->n_splits = n_big + (rest + t2 - 1) / t2;
}

// T new tokens (queries) per sequence: the matrix-core kernels take the
// R * T query rows of a KV head as the columns of one tile.
kvd_status make_plan(const kvd_shape* s, int32_t max_len_host, int cu, const Tuning& tu,
                     Plan* pl, int T = 1) {
  const int R = s->n_heads / s->n_kv_heads;
  if (T < 1 || T > 32) return KVD_EUNSUPPORTED;
  const int RT = R * T;
  int kernel = tu.kernel;
  if (s->kv_dtype == KVD_INT8) {
    // INT8 caches: the INT8 matrix-core kernel, up to 32 query rows per KV head
    if (RT > 32) return KVD_EUNSUPPORTED;
    if (kernel < 0) kernel = 2;
    if (kernel != 2) return KVD_EUNSUPPORTED;
  } else {
    // matrix cores for bf16 caches with up to 32 query rows per KV head; the
    // VALU kernel takes one new token per sequence
    const bool mfma_ok = s->kv_dtype == KVD_BF16 && RT <= 32;
    if (kernel < 0) kernel = mfma_ok ? 1 : 0;
    if ((kernel == 1 && !mfma_ok) || kernel == 2) return KVD_EUNSUPPORTED;
    if (kernel == 0 && T > 1) return KVD_EUNSUPPORTED;
  }
  pl->kernel = kernel;
  // The INT8 kernel with 17 to 32 query rows per KV head holds one
  // workgroup per CU (its registers); when the KV bytes at the bound fit in
  // half of the 256 MB memory-side cache, two workgroups of 16 rows each
  // (two per CU) read each tile instead, the second read served from that
  // cache.  Measured on larger caches, where it is not (5 new tokens on the
  // batched workload), the same split was slower: 151 against 130 us; on a
  // 1024-token sequence with 5 new tokens (8 KV heads) the kernel went from
  // 12.2 to 9.4 us.  Its units are sized for one round at one workgroup per
  // CU: longer units amortise each workgroup's start (a 128K MQA sequence:
  // 1024-token splits 16.1 us, 512 18.3, 256 24.7, 2048 20.9).
  pl->row_groups = 1;
  if (kernel == 2 && RT > 16 &&
      static_cast<int64_t>(s->batch) * s->n_kv_heads * max_len_host * 2 * s->head_dim <=
          (int64_t{128} << 20))
    pl->row_groups = 2;
  if (kernel >= 1) {
    pl->rb = R;
    pl->head_groups = 1;
  } else {
    pl->rb = valu_heads_per_pass(R);
    pl->head_groups = (R + pl->rb - 1) / pl->rb;
  }
  // a workgroup advances kWaves tiles of kMfmaTileTokens (MFMA) or
  // kI8TileTokens (INT8) tokens per step
  const int granule = kernel == 1 ? kMfmaWaves * kMfmaTileTokens
                    : kernel == 2 ? kMfmaWaves * kI8TileTokens : 64;
  if (max_len_host <= 0 || s->batch == 0) {
    pl->chunk = 16; pl->n_splits = 0; pl->wgs = 0; pl->workspace = 0;
    return KVD_OK;
  }
  int chunk = tu.split;
  if (chunk <= 0) {
    // Resident workgroups: two per CU for the MFMA kernel (also with two
    // column blocks, held to 256 registers), four for the VALU kernel, two
    // for the INT8 kernel (one with more than 16 query rows per KV head).
    // The MFMA kernel aims for about four rounds of them over the
    // (sequence, KV head) pairs and their tokens: the workgroups that share a CU run at
    // different speeds (the older one is served first), and smaller units
    // let the dispatcher even that out at a small cost in merges.  With
    // more than 8 query rows per KV head (several new tokens, or n_rep
    // above 8) each unit ends with a heavier merge of its waves and writes
    // more partial rows: one round of splits of up to 2048 tokens then
    // measured faster (c3 shape with 5 new tokens: 215 against 226 us),
    // and with more than 16 rows, as long as one workgroup per CU would
    // make them (a 128K MQA sequence: 512-token splits 20 us, 256-token
    // 31 us).  The VALU kernel aims for two rounds of at most 2048 tokens.
    // The INT8 kernel aims for a single round of at most 2048 tokens (4096
    // with more than 16 query rows, one workgroup per CU): its workgroups
    // keep two 64-token tiles in flight per wave from the first tile on,
    // and each one pays a full memory latency before its first tile, so
    // fewer, longer units measured faster (a 128K sequence: 2048-token
    // splits 46 us, 512-token splits 63 us).  A batch with up to 16 rows
    // takes eight rounds of the bound instead (about four of the real
    // work), as the MFMA kernel does: the batch of contexts up to 8K went
    // from 2048- to 1024-token splits, 106.7 -> 101.3 us (its mixed-cache
    // history kernel 119.6 -> 114.1 us), while the paged batch up to 32K
    // stays at 2048 (1024: 186.5 against 171.4 us).  The 17-32-row kernel
    // keeps one round: 5 new tokens on the 8K batch, 2048-token splits
    // took 150 against 131 us at 4096.
    //
    // The rounds are counted over the host bound on lengths.  For a batch
    // the bound overstates the work: lengths spread over [0, bound] average
    // about half of it.  The MFMA kernel with up to 8 rows therefore aims
    // for eight rounds of the bound with several sequences (about four of
    // the real work) and two with one, up to 2048 tokens per split
    // (measured with the caches evicted before each step: the paged batch
    // of contexts up to 32K, 2048-token splits 321 us against 328 us at
    // 1024; the batch of contexts up to 8K, 1024 tokens 179 us against 180
    // us at 2048; one 128K sequence with 8 KV heads, 1024 tokens 87.7 us
    // against 89.6 at 512, 87.4 at 896, 90.5 at 2048 and 92.9 at 384, with
    // 4 KV heads 47.6 against 48.6 us at 512).
    const bool one_per_cu = RT > 16 && pl->row_groups == 1;
    const int64_t rows = static_cast<int64_t>(s->batch) * s->n_kv_heads * pl->head_groups *
                         pl->row_groups * static_cast<int64_t>(max_len_host);
    const int64_t slots =
        static_cast<int64_t>(cu) * (kernel == 0 ? 4 : (one_per_cu || pl->row_groups > 1 ? 1 : 2));
    const int64_t rounds = kernel == 0 ? 2
                         : kernel == 2 ? (s->batch > 1 && RT <= 16 ? 8 : 1)
                         : (RT > 8 ? 1 : (s->batch > 1 ? 8 : 2));
    const int cap = kernel == 2 && one_per_cu ? 4096 : 2048;
    chunk = round_up((rows + slots * rounds - 1) / (slots * rounds), granule);
    if (chunk < granule) chunk = granule;
    // Short units pay the workgroup's fixed cost (q loads, merge, partial
    // rows) too often: the MFMA kernel with up to 8 rows takes no fewer than
    // 512 tokens per split while that still makes a full round of units at
    // the bound, else no fewer than 256 under the same condition (measured:
    // 16 sequences of 8K, 256-token splits 74% of the peak, 512 83%, 1024
    // 85%; 8 sequences of 2K, 128 tokens 38%, 256 47%).
    if (kernel == 1 && RT <= 8) {
      for (const int floor_tokens : {512, 256}) {
        if (chunk < floor_tokens && rows / floor_tokens >= slots) {
          chunk = floor_tokens;
          break;
        }
      }
    }
    if (chunk > cap) chunk = cap;
  }
  if (chunk > kMaxChunk) chunk = kMaxChunk;
  // the split index is a grid dimension: at most 65535 splits
  if ((max_len_host + chunk - 1) / chunk > 65535) chunk = round_up((max_len_host + 65534) / 65535, 16);
  if (chunk > round_up(max_len_host, 16)) chunk = round_up(max_len_host, 16);
  set_splits(pl, chunk, max_len_host, tu);
  // split is a grid dimension: at most 65535 of them
  if (pl->n_splits > 65535) {
    chunk = round_up((max_len_host + 65534) / 65535, 16);
    set_splits(pl, chunk, max_len_host, tu, false);
  }
  // Dispatch order of the matrix-core kernels.  One sequence: consecutive
  // splits of one head side by side.  Several sequences with more than one
  // split: a work list built on the device from the lengths (units.hip), so
  // that the (sequence, split) slots past a sequence's end, which only the
  // device can tell, are not interleaved with the real units; heads fastest,
  // full splits sequence by sequence, the partial last splits longest first.
  // Measured on the batched workloads: the split kernel 4% (contiguous) to
  // 10% (paged) faster than without the list.  Grid
  // orders 1 (contiguous) and 2 (paged) without the list: heads fastest,
  // then sequences, splits slowest (resp. sequences slowest).
  const int64_t list_wgs =
      static_cast<int64_t>(s->n_kv_heads) * pl->row_groups * s->batch * pl->n_splits;
  const bool list_ok = kernel >= 1 && pl->n_splits > 1 && list_wgs <= 0x7fffffff;
  // Up to 64 sequences the split kernel's waves derive the list themselves
  // from the lengths (order 4, one sequence per lane): the same order
  // without the launch that builds it.
  const bool wave_list_ok = list_ok && s->batch <= 64;
  pl->grid_order = s->batch == 1 ? 0
                 : (wave_list_ok ? 4 : (list_ok ? 3 : (s->block_size != 0 ? 2 : 1)));
  const int ord = tu.order;
  if (ord >= 0 && ord <= 2) pl->grid_order = ord;
  if (ord == 3 && list_ok) pl->grid_order = 3;   // a single split (or the VALU kernel): no list
  if (ord == 4 && wave_list_ok) pl->grid_order = 4;
  pl->wgs = static_cast<int64_t>(pl->n_splits) * s->n_kv_heads * pl->head_groups *
            pl->row_groups * s->batch;
  if (pl->n_splits > 1) {
    const size_t rows = static_cast<size_t>(s->batch) * T * s->n_heads * pl->n_splits;
    size_t o_bytes = rows * s->head_dim * sizeof(float);
    o_bytes = (o_bytes + 255) / 256 * 256;
    pl->workspace = o_bytes + (rows * sizeof(float) + 255) / 256 * 256;
    if (pl->grid_order == 3) {
      // [count][entries]: one int32 per (sequence, split) slot
      pl->units_offset = pl->workspace;
      const size_t n = static_cast<size_t>(s->batch) * pl->n_splits + 64;
      pl->workspace += (n * sizeof(int32_t) + 255) / 256 * 256;
    }
  } else {
    pl->workspace = 0;
  }
  return KVD_OK;
}

}  // namespace


namespace {

// The softmax scale of a call: `scale`, or 1/sqrt(head_dim) when it is 0
// (the default of "Transformer推理核心：KV Cache、GQA与RoPE原理与工程实践" §2.1,
// d_k being the per-head dimension), times log2(e) for the exp2 the kernels use.
float log2_scale(float scale, int head_dim) {
  const double s = scale == 0.f ? 1.0 / std::sqrt(static_cast<double>(head_dim))
                                 : static_cast<double>(scale);
  return static_cast<float>(s * 1.4426950408889634);
}

// Report a plan in the C ABI's terms: plan[2] is a kvd_kernel value.
void export_plan(const Plan& pl, int32_t* plan) {
  plan[0] = pl.chunk;
  plan[1] = pl.n_splits;
  plan[2] = pl.kernel + 1;
  plan[3] = static_cast<int32_t>(pl.wgs);
}

kvd_status plan_for(const kvd_shape* shape, int32_t n_query, int32_t max_seq_len_host,
                    const kvd_options* options, Plan* pl) {
  kvd_status st = check_shape(shape);
  if (st != KVD_OK) return st;
  if (max_seq_len_host < 0 || max_seq_len_host > shape->max_seq_len) return KVD_ERANGE;
  if (n_query < 1 || n_query > 32) return KVD_EUNSUPPORTED;
  Tuning tu;
  st = read_options(options, &tu);
  if (st != KVD_OK) return st;
  int cu = 0;
  if (device_cu_count(&cu) != 0) return KVD_EHIP;
  return make_plan(shape, max_seq_len_host, cu, tu, pl, n_query);
}

// Key splits of a prefill call.  Each workgroup owns 128 query rows of one
// (sequence, KV head) pair and walks their keys; when those workgroups
// would not fill two rounds of the device (three per CU), each row tile's
// keys are cut into splits of whole tiles, at least 2048 keys each (so that
// a workgroup's start and its partial write stay small beside its tiles),
// written to the workspace as (o, log2 lse) and merged by lse_reduce.
constexpr int kPrefillMinSplit = 2048;

struct PfPlan {
  int n_splits = 1;     // 1: no split, out and lse written directly
  int chunk = 0;        // keys per split
  size_t lse_offset = 0;
  size_t workspace = 0;
};

// Validation shared by the prefill calls and their workspace size, and the
// plan (may_split: a workspace is or will be given; dtype: the cache dtype
// the call takes, -1 for either of bf16 and INT8).
kvd_status prefill_setup(const kvd_shape* s, int32_t T, int32_t max_len, const kvd_options* options,
                         bool may_split, Tuning* tu, PfPlan* pl, int dtype = KVD_BF16) {
  *pl = PfPlan{};
  kvd_status st = check_shape(s);
  if (st != KVD_OK) return st;
  if (dtype < 0 ? (s->kv_dtype != KVD_BF16 && s->kv_dtype != KVD_INT8) : s->kv_dtype != dtype)
    return KVD_EUNSUPPORTED;
  if (T < 1 || T > s->max_seq_len) return KVD_EUNSUPPORTED;
  if (max_len < 0 || max_len > s->max_seq_len) return KVD_ERANGE;
  st = read_options(options, tu, true);
  if (st != KVD_OK) return st;
  // the prefill kernel has no kernel choice and no tail splits
  if (tu->kernel >= 0 || tu->tail_split != 0 || tu->tail_span >= 0) return KVD_EINVAL;
  const int64_t R = s->n_heads / s->n_kv_heads;
  const int64_t nqt = (static_cast<int64_t>(T) * R + kPrefillRows - 1) / kPrefillRows;
  const int64_t wgs = nqt * s->batch * s->n_kv_heads;
  const int64_t rows = static_cast<int64_t>(s->batch) * T * s->n_heads;
  if (wgs > 0x7fffffff || rows > 0x7fffffff) return KVD_EUNSUPPORTED;
  int64_t chunk = 0;
  if (tu->split > 0) {
    chunk = tu->split;
  } else if (may_split && wgs > 0 && max_len > kPrefillMinSplit) {
    int cu = 0;
    if (device_cu_count(&cu) != 0) return KVD_EHIP;
    const int64_t target = 2 * 3 * static_cast<int64_t>(cu);
    if (wgs < target) {
      const int64_t n = (target + wgs - 1) / wgs;
      chunk = (max_len + n - 1) / n;
      if (chunk < kPrefillMinSplit) chunk = kPrefillMinSplit;
      chunk = (chunk + kPrefillTile - 1) / kPrefillTile * kPrefillTile;
    }
  }
  if (chunk > 0 && max_len > chunk) {
    const int64_t n = (max_len + chunk - 1) / chunk;
    if (wgs * n > 0x7fffffff) return KVD_EUNSUPPORTED;
    pl->n_splits = static_cast<int>(n);
    pl->chunk = static_cast<int>(chunk);
    const size_t parts = static_cast<size_t>(rows) * pl->n_splits;
    pl->lse_offset = (parts * s->head_dim * sizeof(float) + 255) / 256 * 256;
    pl->workspace = pl->lse_offset + (parts * sizeof(float) + 255) / 256 * 256;
  }
  return KVD_OK;
}

// The prefill calls: a bf16 cache (no scales) or an INT8 cache (scales).
kvd_status prefill_impl(const kvd_shape* shape, int32_t n_query, const float* q_rot,
                        const void* k_cache, const void* v_cache, const float* k_scale,
                        const float* v_scale, const int32_t* seq_lens,
                        const int32_t* block_table, int32_t max_seq_len_host, float scale,
                        float* out, float* lse, void* workspace, size_t workspace_bytes,
                        const kvd_options* options, void* stream) {
  const bool i8 = k_scale != nullptr;
  if (!q_rot || !k_cache || !v_cache || !seq_lens || !out) return KVD_EINVAL;
  if (!aligned16(q_rot) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return KVD_EINVAL;
  if (static_cast<const void*>(out) == static_cast<const void*>(q_rot)) return KVD_EINVAL;
  if (!std::isfinite(scale)) return KVD_EINVAL;
  if (shape && (shape->block_size != 0) != (block_table != nullptr)) return KVD_EINVAL;
  Tuning tu;
  PfPlan pl;
  kvd_status st = prefill_setup(shape, n_query, max_seq_len_host, options, workspace != nullptr,
                                &tu, &pl, i8 ? KVD_INT8 : KVD_BF16);
  if (st != KVD_OK) return st;
  if (pl.workspace > 0 && (!workspace || workspace_bytes < pl.workspace ||
                           (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0))
    return KVD_EWORKSPACE;
  if (shape->batch == 0) return KVD_OK;
  DecodeParams p{};
  p.q_rot = q_rot; p.k = k_cache; p.v = v_cache; p.seq_lens = seq_lens; p.table = block_table;
  p.k_scale = k_scale; p.v_scale = v_scale;
  p.out = out; p.lse = lse;
  p.B = shape->batch; p.H = shape->n_heads; p.G = shape->n_kv_heads; p.D = shape->head_dim;
  p.R = p.H / p.G; p.T = n_query;
  p.max_seq_len = shape->max_seq_len; p.max_len_host = max_seq_len_host;
  p.num_blocks = shape->num_blocks; p.max_blocks_per_seq = shape->max_blocks_per_seq;
  p.block_shift = shape->block_size == 32 ? 1 : 0;
  p.qscale = log2_scale(scale, shape->head_dim);
  p.n_xcd = device_xcc_count();
  // -1: the launcher's choice
  p.grid_order = tu.order >= 0 ? tu.order - (KVD_ORDER_PREFILL_PAIRS_FASTEST - 1) : -1;
  p.n_splits = pl.n_splits;
  p.part_stride = pl.n_splits;
  p.direct = pl.n_splits == 1 ? 1 : 0;
  if (!p.direct) {
    // uniform splits (n_big = n_splits), as the merge counts them
    p.chunk = p.chunk2 = pl.chunk;
    p.n_big = pl.n_splits;
    p.part_o = static_cast<float*>(workspace);
    p.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.lse_offset);
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const Launch l{s, tu.ev_start, tu.ev_stop};
  const bool paged = shape->block_size != 0;
  const hipError_t e = i8 ? launch_prefill_i8(p, paged, l) : launch_prefill_mfma(p, paged, l);
  if (e != hipSuccess) return KVD_EHIP;
  if (!p.direct && launch_lse_reduce(p, s) != hipSuccess) return KVD_EHIP;
  return KVD_OK;
}

}  // namespace

extern "C" {

const char* kvd_status_string(int32_t status) {
  switch (status) {
    case KVD_OK: return "ok";
    case KVD_EINVAL: return "invalid argument (null pointer, inconsistent shape, options or aliasing)";
    case KVD_EUNSUPPORTED: return "unsupported head_dim, dtype, block_size, rope style or kernel";
    case KVD_ERANGE: return "max_seq_len_host outside [0, max_seq_len]";
    case KVD_EWORKSPACE: return "workspace missing or too small";
    case KVD_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

kvd_status kvd_get_plan(const kvd_shape* shape, int32_t max_seq_len_host, int32_t* plan) {
  return kvd_get_plan_multi(shape, 1, max_seq_len_host, nullptr, plan);
}

kvd_status kvd_get_plan_multi(const kvd_shape* shape, int32_t n_query, int32_t max_seq_len_host,
                              const kvd_options* options, int32_t* plan) {
  if (!plan) return KVD_EINVAL;
  Plan pl;
  const kvd_status st = plan_for(shape, n_query, max_seq_len_host, options, &pl);
  if (st != KVD_OK) return st;
  export_plan(pl, plan);
  return KVD_OK;
}

size_t gqa_decode_workspace_size_multi(const kvd_shape* shape, int32_t n_query,
                                       int32_t max_seq_len_host, const kvd_options* options) {
  Plan pl;
  if (plan_for(shape, n_query, max_seq_len_host, options, &pl) != KVD_OK) return 0;
  return pl.workspace;
}

size_t gqa_decode_workspace_size(const kvd_shape* shape, int32_t max_seq_len_host) {
  return gqa_decode_workspace_size_multi(shape, 1, max_seq_len_host, nullptr);
}

}  // extern "C"

namespace {

// window > 0: the append into a mixed-precision cache (k_recent / v_recent
// the bf16 rings of the `window` newest tokens, shape the INT8 history)
kvd_status append_impl(const kvd_shape* shape, const void* q, const void* k_new,
                       const void* v_new, float* q_rot, void* k_cache, void* v_cache,
                       const float* k_scale, const float* v_scale, const int32_t* positions,
                       const int32_t* block_table, double rope_base, int32_t rope_style,
                       void* stream, int32_t T = 1, void* k_recent = nullptr,
                       void* v_recent = nullptr, int32_t window = 0) {
  kvd_status st = check_shape(shape);
  if (st != KVD_OK) return st;
  if (T < 1 || T > shape->max_seq_len) return KVD_EUNSUPPORTED;
  if (rope_style != KVD_ROPE_INTERLEAVED && rope_style != KVD_ROPE_HALF) return KVD_EUNSUPPORTED;
  if (!k_new || !v_new || !k_cache || !v_cache || !positions) return KVD_EINVAL;
  if (q && !q_rot) return KVD_EINVAL;
  if (q && static_cast<const void*>(q_rot) == q) return KVD_EINVAL;
  if (!(rope_base > 0.0) || !std::isfinite(rope_base)) return KVD_EINVAL;
  const bool paged = shape->block_size != 0;
  if (paged != (block_table != nullptr)) return KVD_EINVAL;
  if (shape->batch == 0) return KVD_OK;
  RopeParams p{};
  p.q = q; p.k_new = k_new; p.v_new = v_new; p.q_rot = q ? q_rot : nullptr;
  p.k_cache = k_cache; p.v_cache = v_cache; p.k_scale = k_scale; p.v_scale = v_scale;
  p.positions = positions; p.table = block_table;
  p.base = rope_base; p.B = shape->batch; p.H = shape->n_heads; p.G = shape->n_kv_heads;
  p.D = shape->head_dim; p.T = T; p.style = rope_style; p.max_seq_len = shape->max_seq_len;
  p.num_blocks = shape->num_blocks; p.max_blocks_per_seq = shape->max_blocks_per_seq;
  p.block_shift = shape->block_size == 32 ? 1 : 0;
  p.k_recent = k_recent; p.v_recent = v_recent; p.window = window;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = window > 0 ? launch_rope_append_mixed(p, paged, s)
                                  : launch_rope_append(p, shape->kv_dtype, paged, s);
  return e == hipSuccess ? KVD_OK : KVD_EHIP;
}

kvd_status decode_impl(const kvd_shape* shape, const float* q_rot, const void* k_cache,
                       const void* v_cache, const float* k_scale, const float* v_scale,
                       const int32_t* seq_lens, const int32_t* block_table,
                       int32_t max_seq_len_host, float scale, float* out, float* lse,
                       void* workspace, size_t workspace_bytes, const kvd_options* options,
                       void* stream, int32_t T = 1);

// The decode step in one launch (gqa_decode_step / _int8): scales given
// for an INT8 cache, NULL for bf16.
kvd_status step_impl(const kvd_shape* shape, int32_t T, const void* q, const void* k_new,
                     const void* v_new, void* k_cache, void* v_cache, const float* k_scale,
                     const float* v_scale, const int32_t* positions, const int32_t* block_table,
                     int32_t max_seq_len_host, double rope_base, int32_t rope_style, float scale,
                     float* q_rot, float* out, float* lse, void* workspace,
                     size_t workspace_bytes, const kvd_options* options, void* stream) {
  kvd_status st = check_shape(shape);
  if (st != KVD_OK) return st;
  const bool i8 = k_scale != nullptr;
  // new tokens: up to 16 on bf16 caches (the INT8 kernel's fused form takes one)
  if (T < 1 || T > (i8 ? 1 : 16) || T > shape->max_seq_len) return KVD_EUNSUPPORTED;
  // query heads per KV head: up to 32 on bf16 caches (one or two column
  // blocks), up to 16 on INT8 ones (the one-block kernel)
  if (shape->kv_dtype != (i8 ? KVD_INT8 : KVD_BF16) ||
      shape->n_heads / shape->n_kv_heads * T > (i8 ? 16 : 32))
    return KVD_EUNSUPPORTED;
  if (rope_style != KVD_ROPE_INTERLEAVED && rope_style != KVD_ROPE_HALF) return KVD_EUNSUPPORTED;
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !positions || !out) return KVD_EINVAL;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned16(out) || (q_rot && !aligned16(q_rot)))
    return KVD_EINVAL;
  if (static_cast<const void*>(out) == q || (q_rot && static_cast<const void*>(q_rot) == q) ||
      (q_rot && q_rot == out))
    return KVD_EINVAL;
  if (!(rope_base > 0.0) || !std::isfinite(rope_base) || !std::isfinite(scale)) return KVD_EINVAL;
  const bool paged = shape->block_size != 0;
  if (paged != (block_table != nullptr)) return KVD_EINVAL;
  if (max_seq_len_host < 1 || max_seq_len_host > shape->max_seq_len) return KVD_ERANGE;
  Tuning tu;
  st = read_options(options, &tu);
  if (st != KVD_OK) return st;
  if (tu.kernel >= 0 && tu.kernel != (i8 ? 2 : 1)) return KVD_EINVAL;
  if (shape->batch == 0) return KVD_OK;
  int cu = 0;
  if (device_cu_count(&cu) != 0) return KVD_EHIP;
  Plan pl;
  st = make_plan(shape, max_seq_len_host, cu, tu, &pl, T);
  if (st != KVD_OK) return st;
  if (pl.kernel != (i8 ? 2 : 1) || pl.row_groups > 1 || pl.n_splits < 1) return KVD_EUNSUPPORTED;
  if (pl.workspace > 0 && (!workspace || workspace_bytes < pl.workspace)) return KVD_EWORKSPACE;
  if (pl.workspace > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return KVD_EWORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  DecodeParams p{};
  // lengths: positions[b] + T
  p.seq_lens = positions; p.len_bias = T;
  p.q_in = q; p.k_new = k_new; p.v_new = v_new; p.q_rot_out = q_rot;
  p.rope_base = rope_base; p.rope_style = rope_style;
  p.q_rot = nullptr; p.k = k_cache; p.v = v_cache; p.table = block_table;
  p.k_scale = k_scale; p.v_scale = v_scale;
  p.out = out; p.lse = lse;
  p.B = shape->batch; p.H = shape->n_heads; p.G = shape->n_kv_heads; p.D = shape->head_dim;
  p.R = p.H / p.G; p.T = T;
  p.max_seq_len = shape->max_seq_len; p.max_len_host = max_seq_len_host;
  p.num_blocks = shape->num_blocks; p.max_blocks_per_seq = shape->max_blocks_per_seq;
  p.block_shift = shape->block_size == 32 ? 1 : 0;
  p.chunk = pl.chunk; p.chunk2 = pl.chunk2; p.n_big = pl.n_big;
  p.n_splits = pl.n_splits; p.head_groups = pl.head_groups; p.row_groups = pl.row_groups;
  p.part_stride = pl.n_splits;
  p.qscale = log2_scale(scale, shape->head_dim);
  p.direct = pl.n_splits <= 1 ? 1 : 0;
  p.grid_order = pl.grid_order;
  if (pl.n_splits > 1) {
    char* ws = static_cast<char*>(workspace);
    const size_t rows = static_cast<size_t>(p.B) * p.T * p.H * p.n_splits;
    const size_t o_bytes = (rows * p.D * sizeof(float) + 255) / 256 * 256;
    p.part_o = reinterpret_cast<float*>(ws);
    p.part_lse = reinterpret_cast<float*>(ws + o_bytes);
    if (pl.grid_order == 3) {
      p.n_units = reinterpret_cast<int32_t*>(ws + pl.units_offset);
      p.units = p.n_units + 64;
    }
  }
  if (p.grid_order == 3 && launch_build_units(p, s) != hipSuccess) return KVD_EHIP;
  const Launch l{s, tu.ev_start, tu.ev_stop};
  if ((i8 ? launch_decode_i8(p, paged, l) : launch_decode_mfma(p, paged, l)) != hipSuccess)
    return KVD_EHIP;
  if (!p.direct && launch_lse_reduce(p, s) != hipSuccess) return KVD_EHIP;
  return KVD_OK;
}

}  // namespace

extern "C" {

kvd_status rope_append_kv(const kvd_shape* shape, const void* q, const void* k_new,
                          const void* v_new, float* q_rot, void* k_cache, void* v_cache,
                          const int32_t* positions, const int32_t* block_table,
                          double rope_base, int32_t rope_style, void* stream) {
  // INT8 caches need their scales: rope_append_kv_int8
  if (shape && shape->kv_dtype == KVD_INT8) return KVD_EUNSUPPORTED;
  return append_impl(shape, q, k_new, v_new, q_rot, k_cache, v_cache, nullptr, nullptr,
                     positions, block_table, rope_base, rope_style, stream);
}

kvd_status rope_append_kv_int8(const kvd_shape* shape, const void* q, const void* k_new,
                               const void* v_new, float* q_rot, int8_t* k_cache, int8_t* v_cache,
                               const float* k_scale, const float* v_scale,
                               const int32_t* positions, const int32_t* block_table,
                               double rope_base, int32_t rope_style, void* stream) {
  if (!shape) return KVD_EINVAL;
  if (shape->kv_dtype != KVD_INT8) return KVD_EUNSUPPORTED;
  if (!k_scale || !v_scale) return KVD_EINVAL;
  return append_impl(shape, q, k_new, v_new, q_rot, k_cache, v_cache, k_scale, v_scale,
                     positions, block_table, rope_base, rope_style, stream);
}

kvd_status gqa_decode_step(const kvd_shape* shape, const void* q, const void* k_new,
                           const void* v_new, void* k_cache, void* v_cache,
                           const int32_t* positions, const int32_t* block_table,
                           int32_t max_seq_len_host, double rope_base, int32_t rope_style,
                           float scale, float* q_rot, float* out, float* lse, void* workspace,
                           size_t workspace_bytes, const kvd_options* options, void* stream) {
  if (shape && shape->kv_dtype == KVD_INT8) return KVD_EUNSUPPORTED;   // gqa_decode_step_int8
  return step_impl(shape, 1, q, k_new, v_new, k_cache, v_cache, nullptr, nullptr, positions,
                   block_table, max_seq_len_host, rope_base, rope_style, scale, q_rot, out, lse,
                   workspace, workspace_bytes, options, stream);
}

kvd_status gqa_decode_step_multi(const kvd_shape* shape, int32_t n_query, const void* q,
                                 const void* k_new, const void* v_new, void* k_cache,
                                 void* v_cache, const int32_t* positions,
                                 const int32_t* block_table, int32_t max_seq_len_host,
                                 double rope_base, int32_t rope_style, float scale, float* q_rot,
                                 float* out, float* lse, void* workspace, size_t workspace_bytes,
                                 const kvd_options* options, void* stream) {
  if (shape && shape->kv_dtype == KVD_INT8) return KVD_EUNSUPPORTED;
  return step_impl(shape, n_query, q, k_new, v_new, k_cache, v_cache, nullptr, nullptr,
                   positions, block_table, max_seq_len_host, rope_base, rope_style, scale, q_rot,
                   out, lse, workspace, workspace_bytes, options, stream);
}

kvd_status gqa_decode_step_int8(const kvd_shape* shape, const void* q, const void* k_new,
                                const void* v_new, int8_t* k_cache, int8_t* v_cache,
                                const float* k_scale, const float* v_scale,
                                const int32_t* positions, const int32_t* block_table,
                                int32_t max_seq_len_host, double rope_base, int32_t rope_style,
                                float scale, float* q_rot, float* out, float* lse,
                                void* workspace, size_t workspace_bytes,
                                const kvd_options* options, void* stream) {
  if (!shape) return KVD_EINVAL;
  if (shape->kv_dtype != KVD_INT8) return KVD_EUNSUPPORTED;
  if (!k_scale || !v_scale) return KVD_EINVAL;
  return step_impl(shape, 1, q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, positions,
                   block_table, max_seq_len_host, rope_base, rope_style, scale, q_rot, out, lse,
                   workspace, workspace_bytes, options, stream);
}

kvd_status gqa_decode_attn(const kvd_shape* shape, const float* q_rot, const void* k_cache,
                           const void* v_cache, const int32_t* seq_lens,
                           const int32_t* block_table, int32_t max_seq_len_host, float scale,
                           float* out, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (shape && shape->kv_dtype == KVD_INT8) return KVD_EUNSUPPORTED;
  return decode_impl(shape, q_rot, k_cache, v_cache, nullptr, nullptr, seq_lens, block_table,
                     max_seq_len_host, scale, out, lse, workspace, workspace_bytes, nullptr,
                     stream);
}

kvd_status gqa_decode_attn_int8(const kvd_shape* shape, const float* q_rot,
                                const int8_t* k_cache, const int8_t* v_cache,
                                const float* k_scale, const float* v_scale,
                                const int32_t* seq_lens, const int32_t* block_table,
                                int32_t max_seq_len_host, float scale, float* out, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (!shape) return KVD_EINVAL;
  if (shape->kv_dtype != KVD_INT8) return KVD_EUNSUPPORTED;
  if (!k_scale || !v_scale) return KVD_EINVAL;
  return decode_impl(shape, q_rot, k_cache, v_cache, k_scale, v_scale, seq_lens, block_table,
                     max_seq_len_host, scale, out, lse, workspace, workspace_bytes, nullptr,
                     stream);
}

kvd_status rope_append_kv_multi(const kvd_shape* shape, int32_t n_query, const void* q,
                                const void* k_new, const void* v_new, float* q_rot,
                                void* k_cache, void* v_cache, const float* k_scale,
                                const float* v_scale, const int32_t* positions,
                                const int32_t* block_table, double rope_base, int32_t rope_style,
                                void* stream) {
  if (!shape) return KVD_EINVAL;
  // INT8 caches take their scales, the others none
  const bool i8 = shape->kv_dtype == KVD_INT8;
  if (i8 != (k_scale != nullptr) || i8 != (v_scale != nullptr)) return KVD_EINVAL;
  return append_impl(shape, q, k_new, v_new, q_rot, k_cache, v_cache, k_scale, v_scale,
                     positions, block_table, rope_base, rope_style, stream, n_query);
}

kvd_status gqa_decode_attn_multi(const kvd_shape* shape, int32_t n_query, const float* q_rot,
                                 const void* k_cache, const void* v_cache, const float* k_scale,
                                 const float* v_scale, const int32_t* seq_lens,
                                 const int32_t* block_table, int32_t max_seq_len_host,
                                 float scale, float* out, float* lse, void* workspace,
                                 size_t workspace_bytes, const kvd_options* options,
                                 void* stream) {
  if (!shape) return KVD_EINVAL;
  const bool i8 = shape->kv_dtype == KVD_INT8;
  if (i8 != (k_scale != nullptr) || i8 != (v_scale != nullptr)) return KVD_EINVAL;
  return decode_impl(shape, q_rot, k_cache, v_cache, k_scale, v_scale, seq_lens, block_table,
                     max_seq_len_host, scale, out, lse, workspace, workspace_bytes, options,
                     stream, n_query);
}

size_t gqa_prefill_workspace_size(const kvd_shape* shape, int32_t n_query,
                                  int32_t max_seq_len_host, const kvd_options* options) {
  Tuning tu;
  PfPlan pl;
  if (prefill_setup(shape, n_query, max_seq_len_host, options, true, &tu, &pl, -1) != KVD_OK)
    return 0;
  return pl.workspace;
}

kvd_status gqa_prefill_attn(const kvd_shape* shape, int32_t n_query, const float* q_rot,
                            const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                            const int32_t* block_table, int32_t max_seq_len_host, float scale,
                            float* out, float* lse, void* workspace, size_t workspace_bytes,
                            const kvd_options* options, void* stream) {
  return prefill_impl(shape, n_query, q_rot, k_cache, v_cache, nullptr, nullptr, seq_lens,
                      block_table, max_seq_len_host, scale, out, lse, workspace,
                      workspace_bytes, options, stream);
}

kvd_status gqa_prefill_attn_int8(const kvd_shape* shape, int32_t n_query, const float* q_rot,
                                 const void* k_cache, const void* v_cache, const float* k_scale,
                                 const float* v_scale, const int32_t* seq_lens,
                                 const int32_t* block_table, int32_t max_seq_len_host,
                                 float scale, float* out, float* lse, void* workspace,
                                 size_t workspace_bytes, const kvd_options* options,
                                 void* stream) {
  if (!k_scale || !v_scale) return KVD_EINVAL;
  return prefill_impl(shape, n_query, q_rot, k_cache, v_cache, k_scale, v_scale, seq_lens,
                      block_table, max_seq_len_host, scale, out, lse, workspace,
                      workspace_bytes, options, stream);
}

}  // extern "C"

namespace {

kvd_status decode_impl(const kvd_shape* shape, const float* q_rot, const void* k_cache,
                       const void* v_cache, const float* k_scale, const float* v_scale,
                       const int32_t* seq_lens, const int32_t* block_table,
                       int32_t max_seq_len_host, float scale, float* out, float* lse,
                       void* workspace, size_t workspace_bytes, const kvd_options* options,
                       void* stream, int32_t T) {
  kvd_status st = check_shape(shape);
  if (st != KVD_OK) return st;
  if (!q_rot || !k_cache || !v_cache || !seq_lens || !out) return KVD_EINVAL;
  if (!aligned16(q_rot) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return KVD_EINVAL;
  if (static_cast<const void*>(out) == static_cast<const void*>(q_rot)) return KVD_EINVAL;
  if (!std::isfinite(scale)) return KVD_EINVAL;
  const bool paged = shape->block_size != 0;
  if (paged != (block_table != nullptr)) return KVD_EINVAL;
  if (max_seq_len_host < 0 || max_seq_len_host > shape->max_seq_len) return KVD_ERANGE;
  if (T < 1 || T > 32) return KVD_EUNSUPPORTED;
  Tuning tu;
  st = read_options(options, &tu);
  if (st != KVD_OK) return st;
  if (shape->batch == 0) return KVD_OK;
  int cu = 0;
  if (device_cu_count(&cu) != 0) return KVD_EHIP;
  Plan pl;
  st = make_plan(shape, max_seq_len_host, cu, tu, &pl, T);
  if (st != KVD_OK) return st;
  if (pl.workspace > 0 && (!workspace || workspace_bytes < pl.workspace)) return KVD_EWORKSPACE;
  if (pl.workspace > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return KVD_EWORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  DecodeParams p{};
  p.q_rot = q_rot; p.k = k_cache; p.v = v_cache; p.seq_lens = seq_lens; p.table = block_table;
  p.k_scale = k_scale; p.v_scale = v_scale;
  p.out = out; p.lse = lse;
  p.B = shape->batch; p.H = shape->n_heads; p.G = shape->n_kv_heads; p.D = shape->head_dim;
  p.R = p.H / p.G; p.T = T;
  p.max_seq_len = shape->max_seq_len; p.max_len_host = max_seq_len_host;
  p.num_blocks = shape->num_blocks; p.max_blocks_per_seq = shape->max_blocks_per_seq;
  p.block_shift = shape->block_size == 32 ? 1 : 0;
  p.chunk = pl.chunk; p.chunk2 = pl.chunk2; p.n_big = pl.n_big;
  p.n_splits = pl.n_splits; p.head_groups = pl.head_groups; p.row_groups = pl.row_groups;
  p.part_stride = pl.n_splits;
  p.qscale = log2_scale(scale, shape->head_dim);
  p.direct = pl.n_splits <= 1 ? 1 : 0;
  p.grid_order = pl.grid_order;
  p.units = nullptr; p.n_units = nullptr;
  // workspace layout: [partial O][partial lse]
  p.part_o = nullptr; p.part_lse = nullptr;
  if (pl.n_splits > 1) {
    char* ws = static_cast<char*>(workspace);
    const size_t rows = static_cast<size_t>(p.B) * p.T * p.H * p.n_splits;
    const size_t o_bytes = (rows * p.D * sizeof(float) + 255) / 256 * 256;
    p.part_o = reinterpret_cast<float*>(ws);
    p.part_lse = reinterpret_cast<float*>(ws + o_bytes);
    if (pl.grid_order == 3) {
      p.n_units = reinterpret_cast<int32_t*>(ws + pl.units_offset);
      p.units = p.n_units + 64;
    }
  }

  if (pl.n_splits == 0) {
    // no sequence can hold a token: the merge kernel writes zeros and -inf
    p.chunk = 16; p.chunk2 = 16; p.n_big = 1; p.n_splits = 1;
    return launch_lse_reduce(p, s) == hipSuccess ? KVD_OK : KVD_EHIP;
  }

  if (p.grid_order == 3 && launch_build_units(p, s) != hipSuccess) return KVD_EHIP;
  const Launch l{s, tu.ev_start, tu.ev_stop};
  const hipError_t e = pl.kernel == 1 ? launch_decode_mfma(p, paged, l)
                     : pl.kernel == 2 ? launch_decode_i8(p, paged, l)
                                      : launch_decode_valu(p, shape->kv_dtype, paged, pl.rb, l);
  if (e != hipSuccess) return KVD_EHIP;
  if (!p.direct && launch_lse_reduce(p, s) != hipSuccess) return KVD_EHIP;
  return KVD_OK;
}

// Attention over a mixed-precision cache: the history (tokens older than
// the window) on the INT8 kernel, the rings (the window's tokens) on the
// bf16 kernels, read as a contiguous cache of `window` rows in ring order
// (a softmax does not depend on the order of its keys).  Both write their
// split partials side by side in one workspace -- the history's in slots
// [0, n1), the rings' in [n1, n1 + n2) -- and one merge combines them.
struct MixedPlan {
  Plan hist, ring;
  kvd_shape ring_shape;
  int n1 = 0, n2 = 0;
  size_t lse_offset = 0, units1 = 0, units2 = 0, workspace = 0;
};

kvd_status mixed_plan(const kvd_shape* s, int32_t window, int32_t max_len,
                      const kvd_options* options, Tuning* tu, MixedPlan* mp) {
  *mp = MixedPlan{};
  kvd_status st = check_shape(s);
  if (st != KVD_OK) return st;
  // the INT8 kernel takes up to 32 query rows per KV head
  if (s->kv_dtype != KVD_INT8 || s->n_heads / s->n_kv_heads > 32) return KVD_EUNSUPPORTED;
  if (window < 1 || window > s->max_seq_len) return KVD_ERANGE;
  if (max_len < 0 || max_len > s->max_seq_len) return KVD_ERANGE;
  st = read_options(options, tu);
  if (st != KVD_OK) return st;
  // each part takes its own kernel; the two-level tail split is not offered
  if (tu->kernel >= 0 || tu->tail_split != 0 || tu->tail_span >= 0) return KVD_EINVAL;
  mp->ring_shape = *s;
  mp->ring_shape.kv_dtype = KVD_BF16;
  mp->ring_shape.block_size = 0;
  mp->ring_shape.max_seq_len = window;
  mp->ring_shape.num_blocks = 0;
  mp->ring_shape.max_blocks_per_seq = 0;
  if (s->batch == 0) return KVD_OK;
  int cu = 0;
  if (device_cu_count(&cu) != 0) return KVD_EHIP;
  const int hist_bound = max_len > window ? max_len - window : 0;
  const int ring_bound = max_len < window ? max_len : window;
  if (hist_bound > 0) {
    st = make_plan(s, hist_bound, cu, *tu, &mp->hist, 1);
    if (st != KVD_OK) return st;
    mp->n1 = mp->hist.n_splits;
  }
  if (ring_bound > 0) {
    st = make_plan(&mp->ring_shape, ring_bound, cu, *tu, &mp->ring, 1);
    if (st != KVD_OK) return st;
    mp->n2 = mp->ring.n_splits;
  }
  const size_t parts = static_cast<size_t>(s->batch) * s->n_heads * (mp->n1 + mp->n2);
  mp->lse_offset = (parts * s->head_dim * sizeof(float) + 255) / 256 * 256;
  size_t off = mp->lse_offset + (parts * sizeof(float) + 255) / 256 * 256;
  // work lists ([count][entries]) of the parts that dispatch from one
  const auto list_bytes = [&](int n) {
    return ((static_cast<size_t>(s->batch) * n + 64) * sizeof(int32_t) + 255) / 256 * 256;
  };
  if (mp->n1 > 0 && mp->hist.grid_order == 3) { mp->units1 = off; off += list_bytes(mp->n1); }
  if (mp->n2 > 0 && mp->ring.grid_order == 3) { mp->units2 = off; off += list_bytes(mp->n2); }
  mp->workspace = parts > 0 ? off : 0;
  return KVD_OK;
}

kvd_status mixed_impl(const kvd_shape* shape, int32_t window, const float* q_rot,
                      const void* k_cache, const void* v_cache, const float* k_scale,
                      const float* v_scale, const void* k_recent, const void* v_recent,
                      const int32_t* seq_lens, const int32_t* block_table,
                      int32_t max_seq_len_host, float scale, float* out, float* lse,
                      void* workspace, size_t workspace_bytes, const kvd_options* options,
                      void* stream) {
  if (!shape) return KVD_EINVAL;
  if (!q_rot || !k_cache || !v_cache || !k_scale || !v_scale || !k_recent || !v_recent ||
      !seq_lens || !out)
    return KVD_EINVAL;
  if (!aligned16(q_rot) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      !aligned16(k_recent) || !aligned16(v_recent))
    return KVD_EINVAL;
  if (static_cast<const void*>(out) == static_cast<const void*>(q_rot)) return KVD_EINVAL;
  if (!std::isfinite(scale)) return KVD_EINVAL;
  const bool paged = shape->block_size != 0;
  if (paged != (block_table != nullptr)) return KVD_EINVAL;
  Tuning tu;
  MixedPlan mp;
  kvd_status st = mixed_plan(shape, window, max_seq_len_host, options, &tu, &mp);
  if (st != KVD_OK) return st;
  if (shape->batch == 0) return KVD_OK;
  if (mp.workspace > 0 && (!workspace || workspace_bytes < mp.workspace ||
                           (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0))
    return KVD_EWORKSPACE;

  const hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  DecodeParams p{};
  p.q_rot = q_rot; p.seq_lens = seq_lens;
  p.out = out; p.lse = lse;
  p.B = shape->batch; p.H = shape->n_heads; p.G = shape->n_kv_heads; p.D = shape->head_dim;
  p.R = p.H / p.G; p.T = 1;
  p.max_len_host = max_seq_len_host;
  p.qscale = log2_scale(scale, shape->head_dim);
  p.window = window;
  p.direct = 0;
  p.part_stride = mp.n1 + mp.n2;
  if (mp.n1 + mp.n2 > 0) {
    p.part_o = reinterpret_cast<float*>(ws);
    p.part_lse = reinterpret_cast<float*>(ws + mp.lse_offset);
  }
  // the timing events bracket both parts: start at the first, stop at the last
  const bool two = mp.n1 > 0 && mp.n2 > 0;
  if (mp.n1 > 0) {
    DecodeParams h = p;
    h.k = k_cache; h.v = v_cache; h.k_scale = k_scale; h.v_scale = v_scale; h.table = block_table;
    h.max_seq_len = shape->max_seq_len;
    h.num_blocks = shape->num_blocks; h.max_blocks_per_seq = shape->max_blocks_per_seq;
    h.block_shift = shape->block_size == 32 ? 1 : 0;
    h.chunk = mp.hist.chunk; h.chunk2 = mp.hist.chunk2; h.n_big = mp.hist.n_big;
    h.n_splits = mp.n1; h.head_groups = mp.hist.head_groups; h.grid_order = mp.hist.grid_order;
    h.row_groups = mp.hist.row_groups;
    h.len_mode = 1; h.split_base = 0;
    if (h.grid_order == 3) {
      h.n_units = reinterpret_cast<int32_t*>(ws + mp.units1);
      h.units = h.n_units + 64;
      if (launch_build_units(h, s) != hipSuccess) return KVD_EHIP;
    }
    const Launch l{s, tu.ev_start, two ? nullptr : tu.ev_stop};
    if (launch_decode_i8(h, paged, l) != hipSuccess) return KVD_EHIP;
  }
  if (mp.n2 > 0) {
    DecodeParams r = p;
    r.k = k_recent; r.v = v_recent; r.table = nullptr;
    r.max_seq_len = window;
    r.chunk = mp.ring.chunk; r.chunk2 = mp.ring.chunk2; r.n_big = mp.ring.n_big;
    r.n_splits = mp.n2; r.head_groups = mp.ring.head_groups; r.grid_order = mp.ring.grid_order;
    r.len_mode = 2; r.split_base = mp.n1;
    if (r.grid_order == 3) {
      r.n_units = reinterpret_cast<int32_t*>(ws + mp.units2);
      r.units = r.n_units + 64;
      if (launch_build_units(r, s) != hipSuccess) return KVD_EHIP;
    }
    const Launch l{s, two ? nullptr : tu.ev_start, tu.ev_stop};
    const hipError_t e = mp.ring.kernel == 1 ? launch_decode_mfma(r, false, l)
                                             : launch_decode_valu(r, KVD_BF16, false, mp.ring.rb, l);
    if (e != hipSuccess) return KVD_EHIP;
  }
  // the merge: history slots under the history's split layout, ring slots
  // in splits of the ring's (uniform) size; no part at all (a zero bound):
  // zeros and -inf
  p.len_mode = 3;
  p.n_splits = mp.n1 + mp.n2;
  p.seg2_base = mp.n1;
  p.seg2_chunk = mp.n2 > 0 ? mp.ring.chunk : 16;
  p.chunk = mp.n1 > 0 ? mp.hist.chunk : 16;
  p.chunk2 = mp.n1 > 0 ? mp.hist.chunk2 : 16;
  p.n_big = mp.n1 > 0 ? mp.hist.n_big : 1;
  if (p.n_splits == 0) p.n_splits = 1;
  return launch_lse_reduce(p, s) == hipSuccess ? KVD_OK : KVD_EHIP;
}

}  // namespace

extern "C" {

kvd_status rope_append_kv_mixed(const kvd_shape* shape, int32_t window, const void* q,
                                const void* k_new, const void* v_new, float* q_rot,
                                void* k_cache, void* v_cache, const float* k_scale,
                                const float* v_scale, void* k_recent, void* v_recent,
                                const int32_t* positions, const int32_t* block_table,
                                double rope_base, int32_t rope_style, void* stream) {
  if (!shape) return KVD_EINVAL;
  if (shape->kv_dtype != KVD_INT8) return KVD_EUNSUPPORTED;
  if (window < 1 || window > shape->max_seq_len) return KVD_ERANGE;
  if (!k_scale || !v_scale || !k_recent || !v_recent) return KVD_EINVAL;
  return append_impl(shape, q, k_new, v_new, q_rot, k_cache, v_cache, k_scale, v_scale,
                     positions, block_table, rope_base, rope_style, stream, 1, k_recent,
                     v_recent, window);
}

kvd_status gqa_decode_attn_mixed(const kvd_shape* shape, int32_t window, const float* q_rot,
                                 const void* k_cache, const void* v_cache, const float* k_scale,
                                 const float* v_scale, const void* k_recent,
                                 const void* v_recent, const int32_t* seq_lens,
                                 const int32_t* block_table, int32_t max_seq_len_host,
                                 float scale, float* out, float* lse, void* workspace,
                                 size_t workspace_bytes, const kvd_options* options,
                                 void* stream) {
  return mixed_impl(shape, window, q_rot, k_cache, v_cache, k_scale, v_scale, k_recent,
                    v_recent, seq_lens, block_table, max_seq_len_host, scale, out, lse,
                    workspace, workspace_bytes, options, stream);
}

size_t gqa_decode_workspace_size_mixed(const kvd_shape* shape, int32_t window,
                                       int32_t max_seq_len_host, const kvd_options* options) {
  Tuning tu;
  MixedPlan mp;
  if (mixed_plan(shape, window, max_seq_len_host, options, &tu, &mp) != KVD_OK) return 0;
  return mp.workspace;
}

}  // extern "C"
