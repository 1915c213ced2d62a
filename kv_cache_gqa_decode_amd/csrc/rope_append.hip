// Fused RoPE + KV-cache append (one launch per decode step).
//
// "Transformer推理核心：KV Cache、GQA与RoPE原理与工程实践" §3: theta_i =
// base^(-2i/d), angle = position * theta_i, each (real, imag) pair of q and k
// multiplied by cos + i sin; only the new token is rotated, the cache keeps
// rotated keys.  "4. 自注意力机制推理" §4.5 and "Transformer架构优化实战2026"
// §四: the new K/V go into a preallocated cache at the step's position
// (contiguous, or through a 16-token block table).
//
// Workgroup (new token, slice): the token's D/2 rotation factors are
// computed in fp64 into LDS, then each thread rotates one pair of q or k or
// copies one element of v (the scalar kernel), or four pairs or eight v
// elements (the vector kernel, for aligned buffers and many tokens).  The
// rotation runs in fp64 and the stored key is rounded once to the cache
// dtype, so the appended row is bit-identical to the exact rotation rounded
// to nearest-even.
//
// INT8 caches (same page, §4.3: 8-bit K and V with per-head quantisation
// parameters): the inputs are bf16 and each stored element is the code in
// [-127, 127] nearest to x / scale[g], the quotient taken in fp64 from the
// exact rotated key (or v_new), ties to even, saturating.  Tokens are grouped
// by 16 (group r: the physical block, or b * S_max/16 + pos/16), each group
// holding per KV head its 16 K rows and its V block transposed: K element
// (pos, g, d) at ((r * G + g) * 16 + pos % 16) * D + d, V element at
// ((r * G + g) * D + d) * 16 + pos % 16.
//
// Mixed precision (the same §4.3 names caches that keep the most recent
// tokens at high precision and quantise the older history): the W newest
// tokens of a sequence sit in bf16 rings [B, W, G, D], token p in row p mod
// W, the older ones in an INT8 cache as above.  The append of the token at
// position P first moves token P - W (when P >= W) out of row P mod W into
// the INT8 cache, as codes of its stored bf16 values, then writes the
// rotated k (rounded once to bf16) and v_new there.  Each thread reads and
// rewrites only its own ring elements, so the move needs no ordering.
#include <type_traits>

#include "kvd_internal.h"

namespace kvd {
namespace {

// T = cache element type; int8_t stands for an INT8 cache fed with bf16
template <typename T> __device__ __forceinline__ double load_d(const void* p, int64_t i);
template <> __device__ __forceinline__ double load_d<float>(const void* p, int64_t i) {
  return static_cast<double>(static_cast<const float*>(p)[i]);
}
template <> __device__ __forceinline__ double load_d<uint16_t>(const void* p, int64_t i) {
  return static_cast<double>(bf16_to_float(static_cast<const uint16_t*>(p)[i]));
}
template <> __device__ __forceinline__ double load_d<int8_t>(const void* p, int64_t i) {
  return load_d<uint16_t>(p, i);
}

template <typename T> __device__ __forceinline__ void store_rounded(void* p, int64_t i, double x);
template <> __device__ __forceinline__ void store_rounded<float>(void* p, int64_t i, double x) {
  static_cast<float*>(p)[i] = static_cast<float>(x);       // v_cvt_f32_f64: nearest-even
}
template <> __device__ __forceinline__ void store_rounded<uint16_t>(void* p, int64_t i, double x) {
  static_cast<uint16_t*>(p)[i] = double_to_bf16_rne(x);
}

// Row (in units of D elements) of slot `pos` of sequence b, KV head g, or -1.
template <bool PAGED>
__device__ __forceinline__ int64_t slot_row(const RopeParams& p, int b, int pos, int g) {
  if (pos < 0 || pos >= p.max_seq_len) return -1;
  if (!PAGED) return (static_cast<int64_t>(b) * p.max_seq_len + pos) * p.G + g;
  const int blk = p.table[static_cast<int64_t>(b) * p.max_blocks_per_seq + (pos >> (4 + p.block_shift))];
  if (blk < 0 || blk >= p.num_blocks) return -1;
  // a block of 16 << shift tokens is that many consecutive rows
  const int64_t tok = (static_cast<int64_t>(blk) << (4 + p.block_shift)) + (pos & ((16 << p.block_shift) - 1));
  return tok * p.G + g;
}

// INT8 caches: the 16-token group of a slot whose token-major row is `row`
// (paged: group row/G/16 of the pool, a block being block_size/16 groups;
// contiguous: group pos/16 of sequence b), and the slot's K row in the
// group-major layout.
template <bool PAGED>
__device__ __forceinline__ int64_t i8_group(const RopeParams& p, int b, int pos, int64_t row) {
  return PAGED ? (row / p.G) >> 4 : static_cast<int64_t>(b) * (p.max_seq_len >> 4) + (pos >> 4);
}
template <bool PAGED>
__device__ __forceinline__ int64_t i8_krow(const RopeParams& p, int b, int pos, int g, int64_t row) {
  return (i8_group<PAGED>(p, b, pos, row) * p.G + g) * 16 + (pos & 15);
}

template <typename T, bool PAGED, bool MIXED = false>
__global__ __launch_bounds__(256) void rope_append_kernel(RopeParams p) {
  static_assert(!MIXED || std::is_same<T, int8_t>::value, "a mixed cache's history is INT8");
  // workgroup (new token bt = b * T + t, slice y): the token's items are
  // its q and k pairs (nq + nk, rotated) and its v elements (nv, copied).
  // With rot_slices < gridDim.y, slices y < rot_slices take the pairs in
  // 256-item strides and the rest the v elements; otherwise every slice
  // takes items y * 256, y * 256 + 256 * gridDim.y, .. of both kinds.  A
  // slice with pairs computes the D/2 rotation factors of the token's
  // position once (fp64) and shares them through LDS; the v slices skip
  // that serial fp64 work.
  __shared__ double cs[64], sn[64];
  const int bt = blockIdx.x;
  const int b = bt / p.T;
  const int half = p.D >> 1;
  const int64_t pos64 = static_cast<int64_t>(p.positions[b]) + (bt - b * p.T);
  // a slot past any cache (the rotation still uses the true position)
  const int pos = pos64 > 0x7fffffff ? -1 : static_cast<int>(pos64);
  const int nq = p.q ? p.H * half : 0;
  const int nk = p.G * half;
  const int nv = p.G * p.D;
  const int ys = static_cast<int>(blockIdx.y), ny = static_cast<int>(gridDim.y);
  const bool split = p.rot_slices < ny;
  const int first = split && ys >= p.rot_slices ? nq + nk + (ys - p.rot_slices) * 256 : ys * 256;
  const int stride = 256 * (split ? (ys < p.rot_slices ? p.rot_slices : ny - p.rot_slices) : ny);
  const int end = split && ys < p.rot_slices ? nq + nk : nq + nk + nv;
  if (first < nq + nk) {                    // the same for the whole workgroup
    for (int i = threadIdx.x; i < half; i += 256) {
      const double theta = pow(p.base, -2.0 * i / p.D);
      sincos(static_cast<double>(pos64) * theta, &sn[i], &cs[i]);
    }
    __syncthreads();
  }
  for (int i = first + static_cast<int>(threadIdx.x); i < end; i += stride) {
    if (i < nq + nk) {
      const bool is_q = i < nq;
      const int j = is_q ? i : i - nq;
      const int head = j / half, pi = j - head * half;
      const int ia = p.style == KVD_ROPE_HALF ? pi : 2 * pi;
      const int ib = p.style == KVD_ROPE_HALF ? pi + half : 2 * pi + 1;
      const int heads = is_q ? p.H : p.G;
      const int64_t src = (static_cast<int64_t>(bt) * heads + head) * p.D;
      const void* x = is_q ? p.q : p.k_new;
      const double a = load_d<T>(x, src + ia), c = load_d<T>(x, src + ib);
      const double ra = a * cs[pi] - c * sn[pi];    // (a + ic)(cos + i sin)
      const double rb = a * sn[pi] + c * cs[pi];
      if (is_q) {
        p.q_rot[src + ia] = static_cast<float>(ra);
        p.q_rot[src + ib] = static_cast<float>(rb);
      } else if constexpr (MIXED) {
        if (pos >= 0 && pos < p.max_seq_len) {
          uint16_t* kr = static_cast<uint16_t*>(p.k_recent) +
                         ((static_cast<int64_t>(b) * p.window + pos % p.window) * p.G + head) * p.D;
          if (pos >= p.window) {
            // token pos - window leaves the ring for the INT8 history
            const int old = pos - p.window;
            const int64_t row = slot_row<PAGED>(p, b, old, head);
            if (row >= 0) {
              int8_t* kc = static_cast<int8_t*>(p.k_cache) + i8_krow<PAGED>(p, b, old, head, row) * p.D;
              const float ks = p.k_scale[head];
              kc[ia] = quantize_i8(load_d<uint16_t>(kr, ia), ks);
              kc[ib] = quantize_i8(load_d<uint16_t>(kr, ib), ks);
            }
          }
          kr[ia] = double_to_bf16_rne(ra);
          kr[ib] = double_to_bf16_rne(rb);
        }
      } else {
        const int64_t row = slot_row<PAGED>(p, b, pos, head);
        if (row >= 0) {
          if constexpr (std::is_same<T, int8_t>::value) {
            int8_t* kc = static_cast<int8_t*>(p.k_cache) + i8_krow<PAGED>(p, b, pos, head, row) * p.D;
            const float ks = p.k_scale[head];
            kc[ia] = quantize_i8(ra, ks);
            kc[ib] = quantize_i8(rb, ks);
          } else {
            store_rounded<T>(p.k_cache, row * p.D + ia, ra);
            store_rounded<T>(p.k_cache, row * p.D + ib, rb);
          }
        }
      }
    } else if constexpr (MIXED) {
      const int j = i - nq - nk;
      const int g = j / p.D, d = j - g * p.D;
      if (pos >= 0 && pos < p.max_seq_len) {
        uint16_t* vr = static_cast<uint16_t*>(p.v_recent) +
                       ((static_cast<int64_t>(b) * p.window + pos % p.window) * p.G + g) * p.D + d;
        if (pos >= p.window) {
          const int old = pos - p.window;
          const int64_t row = slot_row<PAGED>(p, b, old, g);
          if (row >= 0) {
            const int64_t vi = ((i8_group<PAGED>(p, b, old, row) * p.G + g) * p.D + d) * 16 + (old & 15);
            static_cast<int8_t*>(p.v_cache)[vi] = quantize_i8(load_d<uint16_t>(vr, 0), p.v_scale[g]);
          }
        }
        *vr = static_cast<const uint16_t*>(p.v_new)[(static_cast<int64_t>(bt) * p.G + g) * p.D + d];
      }
    } else {
      const int j = i - nq - nk;
      const int g = j / p.D, d = j - g * p.D;
      const int64_t row = slot_row<PAGED>(p, b, pos, g);
      if (row >= 0) {
        const int64_t src = (static_cast<int64_t>(bt) * p.G + g) * p.D + d;
        if constexpr (std::is_same<T, int8_t>::value) {
          const int64_t vi = ((i8_group<PAGED>(p, b, pos, row) * p.G + g) * p.D + d) * 16 + (pos & 15);
          static_cast<int8_t*>(p.v_cache)[vi] = quantize_i8(load_d<int8_t>(p.v_new, src), p.v_scale[g]);
        } else {
          static_cast<T*>(p.v_cache)[row * p.D + d] = static_cast<const T*>(p.v_new)[src];
        }
      }
    }
  }
}

// ------------------------------------------------------------ vector form
//
// The same arithmetic, eight elements of a head row per thread: a q or k
// item is four rotation pairs (elements 8c..8c+7 for interleaved pairs,
// 4c..4c+3 with their partners 4c+D/2.. for half pairs; pair k uses factor
// 4c + k in both), a v item eight consecutive elements.  Every access is a
// run of 4 elements (8 or 16 bytes), so the pointers need 16-byte alignment
// (checked by the launcher).  A thread requests the inputs of up to kBatch
// items before it computes any, and a workgroup's first batch is in flight
// while one wave computes the rotation factors; the scalar kernel above,
// with one request per pair, left the append latency-bound on large
// prompts.

template <typename In> struct Quads;             // two runs of 4 input elements
template <> struct Quads<float> { float4 a, b; };
template <> struct Quads<uint16_t> { uint2 a, b; };

__device__ __forceinline__ void load_quads(Quads<float>& r, const void* base, int64_t e1,
                                           int64_t e2) {
  const float* f = static_cast<const float*>(base);
  r.a = *reinterpret_cast<const float4*>(f + e1);
  r.b = *reinterpret_cast<const float4*>(f + e2);
}
__device__ __forceinline__ void load_quads(Quads<uint16_t>& r, const void* base, int64_t e1,
                                           int64_t e2) {
  const uint16_t* h = static_cast<const uint16_t*>(base);
  r.a = *reinterpret_cast<const uint2*>(h + e1);
  r.b = *reinterpret_cast<const uint2*>(h + e2);
}
__device__ __forceinline__ void widen(const Quads<float>& r, double (&x)[8]) {
  x[0] = r.a.x; x[1] = r.a.y; x[2] = r.a.z; x[3] = r.a.w;
  x[4] = r.b.x; x[5] = r.b.y; x[6] = r.b.z; x[7] = r.b.w;
}
__device__ __forceinline__ void widen(const Quads<uint16_t>& r, double (&x)[8]) {
  const uint32_t w[4] = {r.a.x, r.a.y, r.b.x, r.b.y};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = bf16_to_float(static_cast<uint16_t>(w[j] & 0xffffu));
    x[2 * j + 1] = bf16_to_float(static_cast<uint16_t>(w[j] >> 16));
  }
}
// the 8 rounded values of y into runs at dst + e1 and dst + e2
__device__ __forceinline__ void store_runs(float* dst, int64_t e1, int64_t e2, const double (&y)[8]) {
  *reinterpret_cast<float4*>(dst + e1) = make_float4(static_cast<float>(y[0]), static_cast<float>(y[1]),
                                                     static_cast<float>(y[2]), static_cast<float>(y[3]));
  *reinterpret_cast<float4*>(dst + e2) = make_float4(static_cast<float>(y[4]), static_cast<float>(y[5]),
                                                     static_cast<float>(y[6]), static_cast<float>(y[7]));
}
__device__ __forceinline__ void store_runs(uint16_t* dst, int64_t e1, int64_t e2, const double (&y)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    w[j] = static_cast<uint32_t>(double_to_bf16_rne(y[2 * j])) |
           (static_cast<uint32_t>(double_to_bf16_rne(y[2 * j + 1])) << 16);
  *reinterpret_cast<uint2*>(dst + e1) = make_uint2(w[0], w[1]);
  *reinterpret_cast<uint2*>(dst + e2) = make_uint2(w[2], w[3]);
}
// the 8 INT8 codes of y under scale s into runs at dst + e1 and dst + e2
__device__ __forceinline__ void store_codes(int8_t* dst, int64_t e1, int64_t e2, const double (&y)[8],
                                            float s) {
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j)
    w[j >> 2] |= (static_cast<uint32_t>(quantize_i8(y[j], s)) & 0xffu) << (8 * (j & 3));
  *reinterpret_cast<uint32_t*>(dst + e1) = w[0];
  *reinterpret_cast<uint32_t*>(dst + e2) = w[1];
}
// INT8 V (transposed 16-token groups): the codes of elements d0..d0+7 of
// token `pos` into group column pos % 16, starting at vt = ((group * G + g)
// * D + d0) * 16
__device__ __forceinline__ void store_v_codes(int8_t* v, int64_t vt, int pos, const double (&y)[8],
                                              float s) {
#pragma unroll
  for (int j = 0; j < 8; ++j) v[vt + j * 16 + (pos & 15)] = quantize_i8(y[j], s);
}

template <typename T, bool PAGED, bool MIXED, int D>
__global__ __launch_bounds__(256) void rope_append_vec_kernel(RopeParams p) {
  static_assert(!MIXED || std::is_same<T, int8_t>::value, "a mixed cache's history is INT8");
  constexpr bool kGroupV = std::is_same<T, int8_t>::value && !MIXED;
  using In = typename std::conditional<std::is_same<T, float>::value, float, uint16_t>::type;
  constexpr int N8 = D / 8;        // items per head row
  constexpr int HALF = D / 2;
  constexpr int kBatch = 4;        // items a thread requests before computing
  __shared__ double cs[HALF], sn[HALF];
  const int bt = blockIdx.x;
  const int b = bt / p.T;
  const int64_t pos64 = static_cast<int64_t>(p.positions[b]) + (bt - b * p.T);
  const int pos = pos64 > 0x7fffffff ? -1 : static_cast<int>(pos64);
  const int nq = p.q ? p.H * N8 : 0;
  const int nrot = nq + p.G * N8;
  // INT8 cache, 16 tokens per sequence or more: v goes by 16-token groups of
  // the transposed layout.  The token that starts a group's run in this
  // call (the chunk's first token, or one at a multiple of 16) takes its
  // G * D items, each the codes of one (g, d) for the run's tokens -- one
  // 16-byte store for a whole group, instead of a one-byte store 16 bytes
  // from its neighbour per token and element.
  const int tt = bt - b * p.T;
  const bool group_v = kGroupV && p.T >= 16;
  const int nall = nrot + (group_v ? (tt == 0 || (pos & 15) == 0 ? p.G * D : 0) : p.G * N8);
  // slices as in the scalar kernel, counted in items
  const int ys = static_cast<int>(blockIdx.y), ny = static_cast<int>(gridDim.y);
  const bool split = p.rot_slices < ny;
  const int first = split && ys >= p.rot_slices ? nrot + (ys - p.rot_slices) * 256 : ys * 256;
  const int stride = 256 * (split ? (ys < p.rot_slices ? p.rot_slices : ny - p.rot_slices) : ny);
  const int end = split && ys < p.rot_slices ? nrot : nall;
  const bool inter = p.style != KVD_ROPE_HALF;

  // item i: kind (q, k, v), head, chunk c, and the two runs' offsets in the row
  auto decode = [&](int i, int& head, int& c, int& o1, int& o2) {
    const int j = i < nq ? i : (i < nrot ? i - nq : i - nrot);
    head = j / N8;
    c = j - head * N8;
    const bool rot = i < nrot;
    o1 = rot && !inter ? 4 * c : 8 * c;
    o2 = rot && !inter ? 4 * c + HALF : 8 * c + 4;
  };
  auto load = [&](int i, Quads<In>& r) {
    if (group_v && i >= nrot) return;        // loaded where it is used
    int head, c, o1, o2;
    decode(i, head, c, o1, o2);
    const bool is_q = i < nq;
    const int heads = is_q ? p.H : p.G;
    const int64_t row = (static_cast<int64_t>(bt) * heads + head) * D;
    const void* x = is_q ? p.q : (i < nrot ? p.k_new : p.v_new);
    load_quads(r, x, row + o1, row + o2);
  };
  // the codes of v element (g, d) for the tokens of this group's run
  auto group_v_item = [&](int i) {
    const int j = i - nrot;
    const int g = j / D, d = j - g * D;
    if (pos < 0 || pos >= p.max_seq_len) return;
    const int64_t row = slot_row<PAGED>(p, b, pos, g);
    if (row < 0) return;
    // the run stays inside pos's group, whose slots all lie below max_seq_len
    const int cnt = (16 - (pos & 15)) < (p.T - tt) ? 16 - (pos & 15) : p.T - tt;
    const uint16_t* src = static_cast<const uint16_t*>(p.v_new) +
                          (static_cast<int64_t>(bt) * p.G + g) * D + d;
    const int64_t tstride = static_cast<int64_t>(p.G) * D;
    int8_t* dst = static_cast<int8_t*>(p.v_cache) +
                  ((i8_group<PAGED>(p, b, pos, row) * p.G + g) * D + d) * 16 + (pos & 15);
    const float s = p.v_scale[g];
    if (cnt == 16) {                           // a whole group: pos % 16 == 0
      uint16_t x[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) x[k] = src[k * tstride];
      uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int k = 0; k < 16; ++k)
        w[k >> 2] |= (static_cast<uint32_t>(quantize_i8(bf16_to_float(x[k]), s)) & 0xffu) << (8 * (k & 3));
      *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      for (int k = 0; k < cnt; ++k) dst[k] = quantize_i8(bf16_to_float(src[k * tstride]), s);
    }
  };
  auto finish = [&](int i, const Quads<In>& r) {
    if (group_v && i >= nrot) {
      group_v_item(i);
      return;
    }
    int head, c, o1, o2;
    decode(i, head, c, o1, o2);
    double x[8];
    widen(r, x);
    if (i < nrot) {
      double y[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int ia = inter ? 2 * k : k, ib = inter ? 2 * k + 1 : 4 + k;
        const double cf = cs[4 * c + k], sf = sn[4 * c + k];
        y[ia] = x[ia] * cf - x[ib] * sf;            // (a + ic)(cos + i sin)
        y[ib] = x[ia] * sf + x[ib] * cf;
      }
      if (i < nq) {
        const int64_t row = (static_cast<int64_t>(bt) * p.H + head) * D;
        store_runs(p.q_rot, row + o1, row + o2, y);
        return;
      }
      if constexpr (MIXED) {
        if (pos < 0 || pos >= p.max_seq_len) return;
        uint16_t* kr = static_cast<uint16_t*>(p.k_recent) +
                       ((static_cast<int64_t>(b) * p.window + pos % p.window) * p.G + head) * D;
        if (pos >= p.window) {
          // token pos - window leaves the ring for the INT8 history
          const int old = pos - p.window;
          const int64_t row = slot_row<PAGED>(p, b, old, head);
          if (row >= 0) {
            Quads<uint16_t> o;
            load_quads(o, kr, o1, o2);
            double xo[8];
            widen(o, xo);
            store_codes(static_cast<int8_t*>(p.k_cache) + i8_krow<PAGED>(p, b, old, head, row) * D,
                        o1, o2, xo, p.k_scale[head]);
          }
        }
        store_runs(kr, o1, o2, y);
      } else {
        const int64_t row = slot_row<PAGED>(p, b, pos, head);
        if (row < 0) return;
        if constexpr (std::is_same<T, int8_t>::value) {
          store_codes(static_cast<int8_t*>(p.k_cache) + i8_krow<PAGED>(p, b, pos, head, row) * D,
                      o1, o2, y, p.k_scale[head]);
        } else {
          store_runs(static_cast<T*>(p.k_cache), row * D + o1, row * D + o2, y);
        }
      }
      return;
    }
    const int g = head;
    if constexpr (MIXED) {
      if (pos < 0 || pos >= p.max_seq_len) return;
      uint16_t* vr = static_cast<uint16_t*>(p.v_recent) +
                     ((static_cast<int64_t>(b) * p.window + pos % p.window) * p.G + g) * D;
      if (pos >= p.window) {
        const int old = pos - p.window;
        const int64_t row = slot_row<PAGED>(p, b, old, g);
        if (row >= 0) {
          Quads<uint16_t> o;
          load_quads(o, vr, o1, o2);
          double xo[8];
          widen(o, xo);
          store_v_codes(static_cast<int8_t*>(p.v_cache),
                        ((i8_group<PAGED>(p, b, old, row) * p.G + g) * D + o1) * 16, old, xo,
                        p.v_scale[g]);
        }
      }
      *reinterpret_cast<uint2*>(vr + o1) = r.a;
      *reinterpret_cast<uint2*>(vr + o2) = r.b;
    } else {
      const int64_t row = slot_row<PAGED>(p, b, pos, g);
      if (row < 0) return;
      if constexpr (std::is_same<T, int8_t>::value) {
        store_v_codes(static_cast<int8_t*>(p.v_cache),
                      ((i8_group<PAGED>(p, b, pos, row) * p.G + g) * D + o1) * 16, pos, x,
                      p.v_scale[g]);
      } else {
        T* v = static_cast<T*>(p.v_cache) + row * D;
        *reinterpret_cast<decltype(r.a)*>(v + o1) = r.a;   // bit copy
        *reinterpret_cast<decltype(r.b)*>(v + o2) = r.b;
      }
    }
  };

  int i0 = first + static_cast<int>(threadIdx.x);
  Quads<In> r[kBatch];
#pragma unroll
  for (int k = 0; k < kBatch; ++k)
    if (i0 + k * stride < end) load(i0 + k * stride, r[k]);
  if (first < nrot) {                        // the same for the whole workgroup
    for (int j = threadIdx.x; j < HALF; j += 256) {
      const double theta = pow(p.base, -2.0 * j / D);
      sincos(static_cast<double>(pos64) * theta, &sn[j], &cs[j]);
    }
    __syncthreads();
  }
  for (;;) {
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
      if (i0 + k * stride < end) finish(i0 + k * stride, r[k]);
    i0 += kBatch * stride;
    if (i0 >= end) break;
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
      if (i0 + k * stride < end) load(i0 + k * stride, r[k]);
  }
}


// Workgroup slices per token: many tokens (a prompt), one workgroup per
// token, so the rotation factors are computed once per token; fewer, the v
// items in slices of 256 of their own and the q and k items over enough
// slices that the pair workgroups number about kRotWorkgroups (every pair
// workgroup repeats the token's fp64 factors, the serial part of the
// kernel, so more of them only add that work).  nrot / nv: items per token.
constexpr int kRotWorkgroups = 1024;

dim3 rope_grid(RopeParams& p, int tokens, int nrot, int nv) {
  if (tokens >= 4096) {
    p.rot_slices = 1;
    return dim3(static_cast<unsigned>(tokens), 1);
  }
  const int rmax = (nrot + 255) / 256;
  const int want = (kRotWorkgroups + tokens - 1) / tokens;
  p.rot_slices = want < 1 ? 1 : (want > rmax ? rmax : want);
  return dim3(static_cast<unsigned>(tokens), p.rot_slices + (nv + 255) / 256);
}

bool aligned16(const void* x) { return (reinterpret_cast<uintptr_t>(x) & 15u) == 0; }

// every buffer the vector kernel touches with runs of 4 elements
bool vector_ok(const RopeParams& p) {
  return (!p.q || (aligned16(p.q) && aligned16(p.q_rot))) && aligned16(p.k_new) &&
         aligned16(p.v_new) && aligned16(p.k_cache) && aligned16(p.v_cache) &&
         (p.window <= 0 || (aligned16(p.k_recent) && aligned16(p.v_recent)));
}

// Tokens from which the vector kernel runs.  Below, a step is one memory
// round trip after the factors, and the scalar kernel's shorter per-thread
// work over more workgroups finishes first (measured: 64 tokens 4.7 against
// 4.9 us, 32 paged 4.6 against 5.5 us); from a few hundred tokens the
// vector kernel's wider requests win (320 tokens 7.0 against 13.6 us, 32768
// tokens 203 against 449 us).
constexpr int kVectorTokens = 128;

template <typename T, bool PAGED, bool MIXED>
hipError_t launch_rope(RopeParams p, hipStream_t stream) {
  const int tokens = p.B * p.T;
  if (tokens >= kVectorTokens && vector_ok(p)) {
    const int n8 = p.D / 8;
    // an INT8 cache with 16 tokens per sequence or more: v items per (g, d)
    // (fewer tokens leave runs of a few tokens, and the per-token v items
    // spread the work better: 5 tokens 9.6 against 12.1 us)
    const bool group_v = std::is_same<T, int8_t>::value && !MIXED && p.T >= 16;
    const dim3 grid = rope_grid(p, tokens, ((p.q ? p.H : 0) + p.G) * n8, p.G * (group_v ? p.D : n8));
    if (p.D == 64) rope_append_vec_kernel<T, PAGED, MIXED, 64><<<grid, 256, 0, stream>>>(p);
    else rope_append_vec_kernel<T, PAGED, MIXED, 128><<<grid, 256, 0, stream>>>(p);
  } else {
    const int half = p.D / 2;
    const dim3 grid = rope_grid(p, tokens, ((p.q ? p.H : 0) + p.G) * half, p.G * p.D);
    rope_append_kernel<T, PAGED, MIXED><<<grid, 256, 0, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope_append(const RopeParams& p, int32_t kv_dtype, bool paged,
                              hipStream_t stream) {
  if (p.T < 1 || static_cast<int64_t>(p.B) * p.T > 0x7fffffff) return hipErrorInvalidValue;
  if (kv_dtype == KVD_FP32)
    return paged ? launch_rope<float, true, false>(p, stream) : launch_rope<float, false, false>(p, stream);
  if (kv_dtype == KVD_INT8)
    return paged ? launch_rope<int8_t, true, false>(p, stream) : launch_rope<int8_t, false, false>(p, stream);
  return paged ? launch_rope<uint16_t, true, false>(p, stream) : launch_rope<uint16_t, false, false>(p, stream);
}

hipError_t launch_rope_append_mixed(const RopeParams& p, bool paged, hipStream_t stream) {
  if (p.T != 1 || p.window < 1 || !p.k_recent || !p.v_recent) return hipErrorInvalidValue;
  return paged ? launch_rope<int8_t, true, true>(p, stream) : launch_rope<int8_t, false, true>(p, stream);
}

}  // namespace kvd
