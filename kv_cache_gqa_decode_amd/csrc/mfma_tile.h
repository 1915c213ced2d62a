// Device helpers shared by the matrix-core kernels (decode on bf16 and INT8
// caches, prefill): operand types, the bf16 hi/lo split, buffer descriptors
// for the K/V reads, the staged V-tile geometry in LDS, the inline-assembly
// LDS accesses of that tile, the work-unit order and the merge of the
// waves.  Not part of the C ABI.
#pragma once

#include <type_traits>

#include "kvd_internal.h"
#include "uniform_join.h"

namespace kvd {
namespace mt {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr float kNegInf = -__builtin_inff();
// the running max moves only when a tile's max exceeds it by more than this
// (log2 units): probabilities stay below 2^8, far inside fp32 / bf16 range
constexpr float kRescaleSlack = 8.f;

// bf16 bits of a finite float, nearest-even.
__device__ __forceinline__ unsigned short bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<unsigned short>(u >> 16);
}
__device__ __forceinline__ float bf16_value(unsigned short h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// x ~= hi + lo with both bf16 (the residual x - hi is exact in fp32)
__device__ __forceinline__ void split_bf16(float x, unsigned short& hi, unsigned short& lo) {
  hi = bf16_bits(x);
  lo = bf16_bits(x - bf16_value(hi));
}

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// At most N of this wave's vector-memory loads (HBM -> LDS copies included)
// are still outstanding; loads complete in issue order.
template <int N>
__device__ __forceinline__ void vmem_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
  __builtin_amdgcn_wave_barrier();
}

// A 64-bit value made wave-uniform (readfirstlane of both halves, joined
// without sign-extending the low half: uniform_join.h).
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  return join_uniform_halves(v, [](uint32_t x) {
    return __builtin_amdgcn_readfirstlane(static_cast<int>(x));
  });
}

// Raw buffer descriptor over `bytes` bytes from `base` (stride 0: byte
// offsets; word 3 = the gfx9-family default format).  A load at an offset
// >= bytes is out of range: it touches no memory and returns zeros.  Both
// arguments are wave-uniform by construction; readfirstlane keeps the
// descriptor in scalar registers even where the compiler cannot prove it
// (a descriptor it believes divergent costs a loop around every load).
__device__ __forceinline__ rsrc_t make_rsrc(const char* base, uint32_t bytes) {
  char* ub = reinterpret_cast<char*>(uniform_u64(reinterpret_cast<uint64_t>(base)));
  const int n = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  return __builtin_amdgcn_make_buffer_rsrc(ub, 0, n, 0x00020000);
}
// Cache policy of the V copies: non-temporal.  Every V byte is read exactly
// once and each copy instruction reads whole 128-byte lines, so keeping
// them in the caches only displaces other traffic; marking them streaming
// measured +15% (long single sequences) to +5% (batches) of bandwidth.  The
// K loads keep the default policy: each K instruction reads half of a line
// whose other half the next instruction reads, and a non-temporal first
// half is fetched twice.
constexpr int kCopyPolicyNT = 2;
// 16 bytes per lane from `r` at byte offset `off` into LDS at dst + 16*lane
// (MUBUF rather than global: the compiler treats a pending global HBM -> LDS
// copy like a FLAT access and then turns its own waits for unrelated
// register loads into waits for everything)
__device__ __forceinline__ void copy16_to_lds(rsrc_t r, lds_char* dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, off, 0, 0, kCopyPolicyNT);
}
__device__ __forceinline__ uint4 load16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// A wave-uniform 32-bit read through the scalar cache (as constant memory:
// only for data the kernel does not write).  Counted apart
// from vector-memory loads, so waiting for it leaves those -- and an atomic
// issued by one lane under a branch, whose place in their order the
// compiler cannot pin down -- outstanding.
__device__ __forceinline__ int scalar_load_i32(const int32_t* p) {
  typedef __attribute__((address_space(4))) const int32_t const_i32;
  return *reinterpret_cast<const_i32*>(uniform_u64(reinterpret_cast<uint64_t>(p)));
}

// Prefill dispatch order 2 with the batch a multiple of n_xcd (at most 64
// sequences): the sequence that slot `slot` of the unit list holds.  The
// list's n_xcd contiguous runs, one per XCD, then hold B / n_xcd whole
// sequences each; run x takes the sequences of length ranks x, 2 n_xcd - 1 -
// x, 2 n_xcd + x, .. (longest first, ties by index, dealt back and forth),
// so that the runs' summed lengths -- each XCD's share of the work -- come
// out nearly equal whatever order the lengths arrive in.  Every lane of the
// wave takes part; the result is wave-uniform.
__device__ __forceinline__ int balanced_run_seq(const DecodeParams& p, int slot) {
  const int per = p.B / p.n_xcd;
  const int x = slot / per, j = slot - x * per;
  const int r = j * p.n_xcd + ((j & 1) ? p.n_xcd - 1 - x : x);
  const int l = static_cast<int>(threadIdx.x & 63);
  int len = -1;
  if (l < p.B) {
    const int v = p.seq_lens[l];
    len = v < 0 ? 0 : (v > p.max_len_host ? p.max_len_host : v);
  }
  int rank = 0;                              // sequences ahead of lane l's
  for (int m = 0; m < p.B; ++m) {
    const int lm = __builtin_amdgcn_readlane(len, m);
    rank += (lm > len || (lm == len && m < l)) ? 1 : 0;
  }
  // the ranks of lanes 0..B-1 are a permutation of 0..B-1, and r < B
  const uint64_t hit = __ballot(l < p.B && rank == r);
  return __builtin_amdgcn_readfirstlane(static_cast<int>(__builtin_ctzll(hit)));
}

__device__ __forceinline__ uint32_t lds_addr(const lds_char* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

template <int D>
struct Geo {
  static constexpr int KB = D / 32;          // 32-dim blocks of the score contraction
  static constexpr int CB = D / 16;          // 16-dim blocks of the output
  static constexpr int TT = kMfmaTileTokens; // 32 tokens per wave tile
  static constexpr int LPR = D / 8;          // lanes per V row (16 bytes each)
  static constexpr int RPI = 64 / LPR;       // V rows per load instruction
  static constexpr int NVL = TT / RPI;       // V load instructions per tile
  static constexpr int NLOADS = 2 * KB + NVL;  // vector-memory loads per tile
  // every V copy instruction writes 1 KiB; instruction blocks are padded by
  // 32 bytes, so the four lane groups' transposing reads (rows 4 grp ..)
  // start 8 banks apart
  static constexpr int BLOCK = 1024 + 32;
  static constexpr int kTileBytes = NVL * BLOCK;
  // byte offset of (token row r, byte c within the row) in a staged tile
  __device__ __forceinline__ static constexpr int at(int r, int c) {
    return (r / RPI) * BLOCK + (r % RPI) * (2 * D) + c;
  }
};

// The V^T operand of lane (n, grp) for output dims 16 cb + n: the tokens
// the score left in lane group grp (tile_row(4 grp + s), s < 4, and the same
// 16 tokens further) of the staged tile, from two ds_read_b64_tr_b16.  That
// instruction hands lane i of each 16-lane group 16-bit element i % 4 of the
// 8-byte rows addressed by lanes 4k + i / 4, k = 0..3 (measured on gfx950);
// so lane j of the group addresses token row tile_row(4 grp + j / 4), dims
// 16 cb + 4 (j % 4) .. +3, and lane i receives dim 16 cb + i of the four
// rows.  `addr` is that address; the rows 16 further lie `kHalf` bytes
// further; dims 16 cb .. at kOff = 32 cb.
// Issued from inline assembly on purpose: the compiler cannot tell that
// these reads do not touch the buffer an HBM -> LDS copy is still filling,
// and would otherwise wait for every outstanding copy first, which
// serialises the pipeline.
template <int kOff, int kHalf>
__device__ __forceinline__ bf16x8 read_vt_tr(uint32_t addr) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  u32x2 a, b;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %2 offset:%3\n\t"
      "ds_read_b64_tr_b16 %1, %2 offset:%4\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a), "=&v"(b)
      : "v"(addr), "i"(kOff), "i"(kOff + kHalf));
  const u32x4 r = {a[0], a[1], b[0], b[1]};
  return __builtin_bit_cast(bf16x8, r);
}

// The token of a 16-token half that row n of the score MFMA's A operand (K)
// stands for: n = 4 g + s takes token 4 s + g.  The score then leaves lane
// (n, grp) the tokens tile_row(4 grp + j) = 4 j + grp, and the V^T operand
// must follow: each 16-lane group of a transposing read addresses the four
// tokens 4 k + grp, k = 0..3, which lie in four different staged copy blocks
// (1056 bytes apart, 8 banks) -- with the identity order they were four rows
// of one block, 256 bytes apart, all in the same 8 banks: a 4-way conflict
// on every V^T read (measured: 6.6 M conflict cycles per launch on the
// batched workload, 4.5 per LDS instruction).
__device__ __forceinline__ constexpr int tile_row(int n) { return 4 * (n & 3) + (n >> 2); }

// Query rows staged once per workgroup, for the kernels with two column
// blocks (17 to 32 query rows per KV head): there every wave needs all rows
// (16 KB of fp32 at D = 128), and four waves loading them each while the
// first tiles go out measured a start-up twice as long (128K MQA: q in
// registers after 2.8 us, against 1.3 us with no q load at all).  Wave w
// loads rows 8w .. 8w + 7 (lane l of load i: row 8w + i RPI + l / LPR,
// floats 4 (l % LPR) .. +3; rows past RT read row 0), and `publish` writes
// them to the second staging buffer of wave r / 8, which no copy touches
// before the first tile's successor is requested, rows ROW bytes apart (16
// bytes of padding: the 8 lanes of a b128 read pass, rows apart, fall in
// different banks).  The LDS accesses are inline assembly and the barrier
// carries no memory fence, for the reason given at read_vt_tr: the first
// tile's HBM -> LDS copies are still in flight.  After reading its rows
// (read_b128x2), every wave passes a second barrier before any reuse.
template <int D>
struct QStage {
  static constexpr int LPR = D / 4;
  static constexpr int RPI = 64 / LPR;
  static constexpr int NI = 8 / RPI;
  static constexpr int ROW = D * 4 + 16;
  float4 v[NI];

  __device__ __forceinline__ void load(const DecodeParams& p, int b, int g, int RT, int wave,
                                       int lane) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = 8 * wave + i * RPI + lane / LPR;
      v[i] = *reinterpret_cast<const float4*>(p.q_rot + query_row(p, b, g, r < RT ? r : 0) * D +
                                              4 * (lane % LPR));
    }
  }
  // LDS address of staged row r (buffers of `tile_bytes`, two per wave)
  __device__ __forceinline__ static uint32_t row_addr(uint32_t stage, int tile_bytes, int r) {
    return stage + static_cast<uint32_t>((2 * (r >> 3) + 1) * tile_bytes + (r & 7) * ROW);
  }
  __device__ __forceinline__ void publish(uint32_t stage, int tile_bytes, int wave,
                                          int lane) const {
    // the smallest staging buffer: the INT8 kernel's, 4 groups of 16 x D bytes
    static_assert(8 * ROW <= 4 * D * 16, "eight rows fit a staging buffer");
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t a = row_addr(stage, tile_bytes, 8 * wave + i * RPI + lane / LPR) +
                         16 * (lane % LPR);
      const u32x4 x = __builtin_bit_cast(u32x4, v[i]);
      asm volatile("ds_write_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(a), "v"(x) : "memory");
    }
    __builtin_amdgcn_s_barrier();
  }
};

// Two 16-byte LDS reads at addr + kOff and addr + kOff + 16, waited for.
template <int kOff>
__device__ __forceinline__ void read_b128x2(uint32_t addr, float4& x0, float4& x1) {
  u32x4 a, b;
  asm volatile(
      "ds_read_b128 %0, %2 offset:%3\n\t"
      "ds_read_b128 %1, %2 offset:%4\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a), "=&v"(b)
      : "v"(addr), "i"(kOff), "i"(kOff + 16)
      : "memory");
  x0 = __builtin_bit_cast(float4, a);
  x1 = __builtin_bit_cast(float4, b);
}

// f(std::integral_constant<int, i>) for i = 0 .. N-1 (compile-time indices).
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// Two floats to packed bf16, nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// 16 zero bytes at LDS address `addr` (inline assembly for the same reason
// as read_vt_tr; ordered after the copies by an explicit vmcnt wait)
__device__ __forceinline__ void lds_zero16(uint32_t addr) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  asm volatile("ds_write_b128 %0, %1" ::"v"(addr), "v"(z) : "memory");
}

// The dispatch order (chosen by the planner) of the (sequence, KV head,
// split) units, slot x fastest (orders 0-2; orders 3 and 4 follow a work
// list): which of them run side by side decides how
// the workgroups reading the same DRAM rows (the heads of one token range)
// and the longest chunks are spread in time and across the XCDs.
struct Unit { int b, g, split; };
__device__ __forceinline__ Unit unit_of(const DecodeParams& p, int x, int y, int z) {
  const int o = p.grid_order;
  return Unit{o == 1 ? y : z, o == 0 ? y : x, o == 0 ? x : (o == 1 ? z : y)};
}
// Order 4, batches of at most 64 sequences: the order-3 list without its
// launch.  Every wave derives its entry k = id / G from the lengths, one
// sequence per lane: an inclusive scan of the full-split counts places the
// full units (sequence by sequence); the partial last splits are ranked by
// the key (16-token bucket of their length + 1) << 6 | (63 - b), unique per
// lane, largest first -- longest bucket first, then by sequence -- and the
// (k - n_full)-th largest is picked bit by bit with ballots (a radix
// select: 16 steps of one compare and one popcount).  The KV heads of an
// entry are rotated across the XCDs as in order 3 (see unit_at).
__device__ __forceinline__ bool unit_from_lengths(const DecodeParams& p, Unit& u) {
  const int lane = threadIdx.x & 63;
  const int id = static_cast<int>(blockIdx.x);
  const int k = id / unit_heads(p);
  const int L = lane < p.B ? attended_len(p, len_of(p, p.seq_lens[lane])) : 0;
  const int n = split_count(p, L);
  int full = 0, part = 0;
  if (n > 0) {
    const int tail = L - split_start(p, n - 1);
    if (tail == split_size(p, n - 1)) full = n;
    else { full = n - 1; part = tail; }
  }
  int incl = full;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  const int n_full = __builtin_amdgcn_readlane(incl, 63);
  int b, split;
  if (k < n_full) {
    const uint64_t hit = __ballot(incl - full <= k && k < incl);
    b = __builtin_ctzll(hit);
    split = k - __builtin_amdgcn_readlane(incl - full, b);
  } else {
    // part <= kMaxChunk: the key fits in 16 bits
    const int key = part > 0 ? ((((part - 1) >> 4) + 1) << 6) | (63 - lane) : 0;
    uint64_t cand = __ballot(part > 0);
    int j = k - n_full;
    if (j >= __popcll(cand)) return false;
#pragma unroll
    for (int bit = 15; bit >= 0; --bit) {
      const uint64_t ones = cand & __ballot((key >> bit) & 1);
      const int c1 = __popcll(ones);
      if (j < c1) {
        cand = ones;
      } else {
        j -= c1;
        cand &= ~ones;
      }
    }
    b = __builtin_ctzll(cand);
    split = __builtin_amdgcn_readlane(full, b);
  }
  const int uh = unit_heads(p);
  u = Unit{b, (id - k * uh + (k >> 4)) % uh, split};
  return true;
}

// This workgroup's unit; false when it has none (orders 3 and 4: past the
// end of the work list; order 3 reads entries b | split << 16 built by
// units.hip, and the KV heads of an entry are its G consecutive
// workgroups).  The hardware hands
// workgroups to the 8 XCDs round-robin by id, so with the heads in a fixed
// order every XCD would serve one KV head (G = 8) for the whole dispatch;
// the heads of entries k are rotated by k / 16 instead, so each XCD stays
// on one head for 16 consecutive entries (neighbouring token ranges of one
// sequence) and then moves on.  Measured on the batched workload's split
// kernel: fixed heads 198 us, rotation by k 195, by k / 2 187, by k / 16
// 185; 64 uniform 8K sequences 373, 356, 343, 338 us.
__device__ __forceinline__ bool unit_at(const DecodeParams& p, Unit& u) {
  if (p.grid_order == 4) return unit_from_lengths(p, u);
  if (p.grid_order == 3) {
    const int id = static_cast<int>(blockIdx.x);
    const int uh = unit_heads(p);
    const int k = id / uh;
    if (k >= scalar_load_i32(p.n_units)) return false;
    const uint32_t e = static_cast<uint32_t>(scalar_load_i32(p.units + k));
    u = Unit{static_cast<int>(e & 0xffffu), (id - k * uh + (k >> 4)) % uh,
             static_cast<int>(e >> 16)};
    return true;
  }
  u = unit_of(p, blockIdx.x, blockIdx.y, blockIdx.z);
  return true;
}
// The split kernels' grid for the dispatch order.
inline dim3 split_grid(const DecodeParams& p) {
  switch (p.grid_order) {
    case 0: return dim3(p.n_splits, unit_heads(p), p.B);
    case 1: return dim3(unit_heads(p), p.B, p.n_splits);
    case 2: return dim3(unit_heads(p), p.n_splits, p.B);
    default: return dim3(static_cast<unsigned>(unit_heads(p)) * p.B * p.n_splits);   // orders 3, 4
  }
}

// The waves of a split workgroup each hold (acc, m, l) for the same 16 query
// rows over different tiles: the column block's accumulator acc[cb] (rows
// 16 cb + 4 grp + j of lane column n), its running max m (log2 units) and
// its exp-sum l.  They are combined through LDS with the log-sum-exp weights
// and the split's normalised rows (times out_scale) and log2-sum-exp written
// -- as the final output when the split is the whole sequence.
//
// LDS rows are padded by 16 bytes so that the 16 lanes of a lane group,
// which write rows 528 bytes apart, fall into different banks; each thread
// then reduces one row over D / 16 consecutive dims, with the row's weights
// computed once.
template <int D>
constexpr int merge_row_floats() { return D + 4; }
template <int D>
constexpr int merge_bytes() {
  return (kMfmaWaves * 16 * merge_row_floats<D>() + 2 * kMfmaWaves * 16) * 4;
}

template <int D>
__device__ __forceinline__ void merge_waves(const DecodeParams& p, char* smem, int b, int g,
                                            int split, int hb, int nh,
                                            const f32x4 (&acc)[D / 16], float m, float l,
                                            float out_scale) {
  constexpr int CB = D / 16, SD = merge_row_floats<D>();
  constexpr int TPR = 16, DPT = D / TPR;    // threads per row, dims per thread
  static_assert(DPT % 4 == 0, "float4 columns");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, grp = lane >> 4;
  float* so = reinterpret_cast<float*>(smem);           // [waves][16][SD]
  float* sm_m = so + kMfmaWaves * 16 * SD;              // [waves][16]
  float* sm_l = sm_m + kMfmaWaves * 16;                 // [waves][16]
  __syncthreads();                  // staging tiles / previous pass no longer read
  if (n < nh) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      *reinterpret_cast<f32x4*>(so + (wave * 16 + n) * SD + 16 * cb + 4 * grp) = acc[cb];
    if (grp == 0) { sm_m[wave * 16 + n] = m; sm_l[wave * 16 + n] = l; }
  }
  __syncthreads();
  const int r = threadIdx.x / TPR, c = threadIdx.x - r * TPR;
  if (r >= nh) return;
  float mw[kMfmaWaves];
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < kMfmaWaves; ++w) {
    mw[w] = sm_m[w * 16 + r];
    M = fmaxf(M, mw[w]);
  }
  const float ref = M == kNegInf ? 0.f : M;
  float a[kMfmaWaves];
  float sum = 0.f;
#pragma unroll
  for (int w = 0; w < kMfmaWaves; ++w) {
    a[w] = exp2f(mw[w] - ref);
    sum += sm_l[w * 16 + r] * a[w];
  }
  // every token of the split masked (invalid blocks, the window's bound):
  // an empty softmax
  const float inv = sum > 0.f ? out_scale / sum : 0.f;
  const float lse2 = sum > 0.f ? ref + log2f(sum) : kNegInf;
  f32x4 o[DPT / 4];
#pragma unroll
  for (int k = 0; k < DPT / 4; ++k) o[k] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < kMfmaWaves; ++w)
#pragma unroll
    for (int k = 0; k < DPT / 4; ++k)
      o[k] += *reinterpret_cast<const f32x4*>(so + (w * 16 + r) * SD + c * DPT + 4 * k) * a[w];
  const int64_t h = query_row(p, b, g, hb + r);
  float* dst;
  if (p.direct) {
    dst = p.out + h * D;
    if (c == 0 && p.lse) p.lse[h] = lse2 * 0.69314718055994531f;
  } else {
    const int64_t pr = h * p.part_stride + p.split_base + split;
    dst = p.part_o + pr * D;
    if (c == 0) p.part_lse[pr] = lse2;
  }
#pragma unroll
  for (int k = 0; k < DPT / 4; ++k)
    *reinterpret_cast<f32x4*>(dst + c * DPT + 4 * k) = o[k] * inv;
}

}  // namespace mt
}  // namespace kvd
