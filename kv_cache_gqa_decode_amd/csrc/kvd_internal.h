// Internal declarations shared by the HIP sources of libkvdecode.so.
// Nothing here is part of the C ABI (include/kvdecode.h is).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvdecode.h"

namespace kvd {

// Everything a decode-attention launch needs, passed by value.
struct DecodeParams {
  const float* q_rot;       // [B, H, D] fp32
  const void* k;            // cache or pool
  const void* v;
  const float* k_scale;     // INT8 caches: [G] per-head scales, else null
  const float* v_scale;
  const int32_t* seq_lens;  // [B]
  const int32_t* table;     // [B, max_blocks_per_seq] or null
  float* out;               // [B, H, D]
  float* lse;               // [B, H] or null
  float* part_o;            // [B * H, n_splits, D]  (split results, normalised)
  float* part_lse;          // [B * H, n_splits]     (log2 of the split's exp-sum)
  int32_t B, H, G, D, R;    // R = H / G
  int32_t T;                // new tokens (queries) per sequence; query t of
                            // sequence b attends the tokens j < L_b - T + 1 + t
  int32_t max_seq_len;      // contiguous S_max, or max_blocks_per_seq * 16
  int32_t max_len_host;     // lengths are clamped to this
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t block_shift;      // paged: log2(block_size / 16), 0 or 1
  // Splits of a sequence: n_big splits of `chunk` tokens, then splits of
  // `chunk2` tokens (both multiples of 16; n_big == n_splits: all equal).
  // Small last splits keep the units that are dispatched last short.
  int32_t chunk;
  int32_t chunk2;
  int32_t n_big;
  int32_t n_splits;
  int32_t head_groups;      // query-head groups per KV head (VALU kernel)
  float qscale;             // softmax scale * log2(e)
  int32_t direct;           // 1: one split, write out / lse directly
  int32_t grid_order;       // matrix-core kernels: 0 (split, G, B), 1 (G, B, split),
                            // 2 (G, split, B), 3 work list (heads fastest; units.hip),
                            // 4 the same list derived by each wave (B <= 64)
  int32_t* units;           // work list (grid_order 3): b | split << 16, in the workspace
  int32_t* n_units;         // its length
  int32_t n_xcd;            // prefill, grid_order 2: XCDs the workgroups are dealt to
  // Partial slots: row h's split s goes to slot h * part_stride + split_base
  // + s (one launch's splits inside a wider set, for the mixed-precision
  // cache; else part_stride = n_splits, split_base = 0).
  int32_t part_stride;
  int32_t split_base;
  // Tokens a launch covers of a cache whose `window` newest tokens are kept
  // apart (mixed precision): len_mode 0 all, 1 the older ones, 2 the newest
  // ones (see attended_len); 3 (the merge only): split slots [0, seg2_base)
  // are those of mode 1 under chunk / chunk2 / n_big, slots seg2_base + s
  // those of mode 2 in splits of seg2_chunk tokens.
  int32_t len_mode;
  int32_t window;
  int32_t seg2_base;
  int32_t seg2_chunk;
  // INT8 kernel: the query rows of a KV head split over row_groups
  // workgroups of 16 rows each (0 or 1: one workgroup takes all); units then
  // run over G * row_groups (KV head, row group) pairs
  int32_t row_groups;
  // Fused decode step (gqa_decode_step, one new token, the MFMA kernel):
  // seq_lens points at the positions and len_bias is 1, so sequence b
  // attends positions[b] + 1 tokens; the split kernel rotates q_in itself,
  // and the workgroup of each (sequence, KV head)'s last split appends the
  // new token's rotated k and v before it requests any tile.  len_bias 0:
  // the plain calls.
  int32_t len_bias;
  int32_t rope_style;
  double rope_base;
  const void* q_in;         // [B, H, D] bf16, not rotated
  const void* k_new;        // [B, G, D] bf16, not rotated
  const void* v_new;        // [B, G, D] bf16
  float* q_rot_out;         // [B, H, D] fp32, or null
};

// Tokens sequence b holds, from its entry in seq_lens (plus len_bias;
// saturating, so that a position of INT32_MAX stays positive).
__host__ __device__ __forceinline__ int len_of(const DecodeParams& p, int raw) {
  return raw > 0x7fffffff - p.len_bias ? 0x7fffffff : raw + p.len_bias;
}

// (KV head, row group) pairs the units of a split kernel run over
__host__ __device__ __forceinline__ int unit_heads(const DecodeParams& p) {
  return p.row_groups > 1 ? p.G * p.row_groups : p.G;
}

struct RopeParams {
  const void* q;            // [B, H, D] or null
  const void* k_new;        // [B, G, D]
  const void* v_new;        // [B, G, D]
  float* q_rot;             // [B, H, D]
  void* k_cache;
  void* v_cache;
  const float* k_scale;     // INT8 caches: [G] per-head scales, else null
  const float* v_scale;
  const int32_t* positions; // [B] slot of each sequence's first new token
  const int32_t* table;
  double base;
  int32_t B, H, G, D;
  int32_t T;                // new tokens per sequence (rows b * T + t of q / k_new / v_new)
  int32_t style;
  int32_t max_seq_len;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t block_shift;      // paged: log2(block_size / 16), 0 or 1
  // mixed precision: the bf16 rings [B, window, G, D] of the newest tokens
  // (window 0: a plain cache)
  void* k_recent;
  void* v_recent;
  int32_t window;
  // set by the launcher: workgroup slices y < rot_slices of a token take its
  // q and k items (which need the rotation factors), the others its v items;
  // rot_slices = gridDim.y: every slice takes items of both kinds
  int32_t rot_slices;
};

// Where a main kernel goes: its stream and, for measurement, a pair of
// events tied to the dispatch itself (hipExtLaunchKernel records them at
// the kernel's own start and end, so their interval is the kernel's
// execution as a profiler's kernel trace sees it, without the gap between
// a separately recorded event and the dispatch).
struct Launch {
  hipStream_t stream = nullptr;
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// kernel<<<grid, block, 0, l.stream>>>(p), with l's events when it has them.
template <typename P>
inline hipError_t launch_kernel(void (*kernel)(P), dim3 grid, dim3 block, const Launch& l, P p) {
  if (l.start || l.stop) {
    void* args[] = {&p};
    return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0,
                              l.stream, l.start, l.stop, 0);
  }
  hipLaunchKernelGGL(kernel, grid, block, 0, l.stream, p);
  return hipGetLastError();
}

// Launchers (each returns the hipError_t of its launch).
hipError_t launch_rope_append(const RopeParams& p, int32_t kv_dtype, bool paged,
                              hipStream_t stream);
// the append into a mixed-precision cache (INT8 history, bf16 rings)
hipError_t launch_rope_append_mixed(const RopeParams& p, bool paged, hipStream_t stream);
hipError_t launch_decode_valu(const DecodeParams& p, int32_t kv_dtype, bool paged,
                              int rb, const Launch& l);
hipError_t launch_decode_mfma(const DecodeParams& p, bool paged, const Launch& l);
hipError_t launch_decode_i8(const DecodeParams& p, bool paged, const Launch& l);
// causal prefill of p.T new tokens per sequence (p.qscale, no splits)
// n_splits 1: out and lse directly; more: (o, log2 lse) per key split into
// part_o / part_lse, merged by launch_lse_reduce
hipError_t launch_prefill_mfma(const DecodeParams& p, bool paged, const Launch& l);
// the same on an INT8 cache (k_scale / v_scale set)
hipError_t launch_prefill_i8(const DecodeParams& p, bool paged, const Launch& l);
hipError_t launch_lse_reduce(const DecodeParams& p, hipStream_t stream);
hipError_t launch_build_units(const DecodeParams& p, hipStream_t stream);
// Heads per pass of the VALU kernel for a given n_rep (1, 2, 4 or 8).
int valu_heads_per_pass(int n_rep);
// Workgroups and tokens per workgroup-iteration of the MFMA kernel.
constexpr int kMfmaWaves = 4;
constexpr int kMfmaTileTokens = 32;   // tokens per wave per iteration
constexpr int kI8TileTokens = 64;     // INT8 kernel: tokens per wave per iteration
constexpr int kMaxChunk = 8192;       // tokens per split, upper bound
constexpr int kPrefillRows = 128;     // prefill: query rows per workgroup
constexpr int kPrefillTile = 32;      // prefill: keys per tile (key splits are whole tiles)
constexpr int kMfmaMaxChunk = kMaxChunk;

// ------------------------------------------------------------ device helpers

// first token, size and count of the splits of a sequence (see DecodeParams)
__host__ __device__ __forceinline__ int split_start(const DecodeParams& p, int s) {
  return s < p.n_big ? s * p.chunk : p.n_big * p.chunk + (s - p.n_big) * p.chunk2;
}
__host__ __device__ __forceinline__ int split_size(const DecodeParams& p, int s) {
  return s < p.n_big ? p.chunk : p.chunk2;
}
// splits holding at least one of L tokens
// The tokens of sequence b a launch attends, from its stored length: clamped
// to [0, max_len_host], then all of them (len_mode 0), the ones older than
// the `window` newest (1), or the newest ones (2).
__host__ __device__ __forceinline__ int attended_len(const DecodeParams& p, int L) {
  L = L < 0 ? 0 : (L > p.max_len_host ? p.max_len_host : L);
  return p.len_mode == 1 ? (L > p.window ? L - p.window : 0)
       : p.len_mode == 2 ? (L < p.window ? L : p.window) : L;
}

__host__ __device__ __forceinline__ int split_count(const DecodeParams& p, int L) {
  const int big = p.n_big * p.chunk;
  return L <= big ? (L + p.chunk - 1) / p.chunk : p.n_big + (L - big + p.chunk2 - 1) / p.chunk2;
}

// Paged caches: the pool's 16-token group that holds token group j (tokens
// 16j .. 16j+15) of sequence b.  A block of block_size tokens is block_size/16
// consecutive groups of the pool, so every kernel addresses the pool in
// 16-token groups.  -1 when the table entry is outside the pool.
__device__ __forceinline__ int paged_group(const DecodeParams& p, int b, int j) {
  const int blk = p.table[static_cast<int64_t>(b) * p.max_blocks_per_seq + (j >> p.block_shift)];
  if (blk < 0 || blk >= p.num_blocks) return -1;
  return (blk << p.block_shift) | (j & ((1 << p.block_shift) - 1));
}

// Row of q_rot / out / lse / the split partials that column c of KV head g's
// tile stands for: the columns are the n_rep query heads of each of the T new
// tokens, c = t * R + r.  With T = 1 this is query head g * R + c.
__host__ __device__ __forceinline__ int64_t query_row(const DecodeParams& p, int b, int g, int c) {
  const int t = c / p.R, r = c - t * p.R;
  return (static_cast<int64_t>(b) * p.T + t) * p.H + g * p.R + r;
}

// bf16 pair in a 32-bit word -> two floats (exact).
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// Nearest-even bf16 of a double, in one rounding (no detour through fp32,
// which would round twice).  Works on the binary64 fields directly.
__device__ __forceinline__ uint16_t double_to_bf16_rne(double x) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
  const uint32_t sign = static_cast<uint32_t>(u >> 63) << 15;
  const int e = static_cast<int>((u >> 52) & 0x7ff);
  const uint64_t frac = u & ((1ull << 52) - 1);
  if (e == 0x7ff) return static_cast<uint16_t>(sign | (frac ? 0x7fc0u : 0x7f80u));
  if (e == 0) return static_cast<uint16_t>(sign);          // |x| < 2^-1022 rounds to 0
  int E = e - 1023;
  if (E > 127) return static_cast<uint16_t>(sign | 0x7f80u);
  const uint64_t sig = (1ull << 52) | frac;                 // 53-bit significand
  if (E >= -126) {                                          // bf16 normal range
    uint64_t keep = sig >> 45;                              // 8 significant bits
    const uint64_t rem = sig & ((1ull << 45) - 1);
    const uint64_t halfway = 1ull << 44;
    if (rem > halfway || (rem == halfway && (keep & 1))) ++keep;
    if (keep == 256) { keep = 128; ++E; }
    if (E > 127) return static_cast<uint16_t>(sign | 0x7f80u);
    return static_cast<uint16_t>(sign | (static_cast<uint32_t>(E + 127) << 7) |
                                 static_cast<uint32_t>(keep & 0x7f));
  }
  // bf16 subnormal: value = sig * 2^(E-52), unit 2^-133 -> sig >> (-(E + 81))
  const int shift = -(E + 81);                              // > 45 here
  if (shift > 54) return static_cast<uint16_t>(sign);       // below half a unit
  uint64_t keep = sig >> shift;
  const uint64_t rem = sig & ((1ull << shift) - 1);
  const uint64_t halfway = 1ull << (shift - 1);
  if (rem > halfway || (rem == halfway && (keep & 1))) ++keep;
  return static_cast<uint16_t>(sign | static_cast<uint32_t>(keep));  // 128 -> min normal
}

// INT8 code of x under scale s: nearest integer to the fp64 quotient, ties
// to even (v_rndne_f64), saturating at +-127; a NaN quotient gives 0.
__device__ __forceinline__ int8_t quantize_i8(double x, float s) {
  const double q = x / static_cast<double>(s);
  if (q != q) return 0;
  if (q >= 127.0) return 127;
  if (q <= -127.0) return -127;
  return static_cast<int8_t>(static_cast<int>(__builtin_rint(q)));
}

__device__ __forceinline__ float bf16_to_float(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

}  // namespace kvd
