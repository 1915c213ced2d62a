// Fused RoPE + KV-cache append (one launch per decode step).
//
// "Transformer推理核心：KV Cache、GQA与RoPE原理与工程实践" §3: theta_i =
// base^(-2i/d), angle = position * theta_i, each (real, imag) pair of q and k
// multiplied by cos + i sin; only the new token is rotated, the cache keeps
// rotated keys.  "4. 自注意力机制推理" §4.5 and "Transformer架构优化实战2026"
// §四: the new K/V go into a preallocated cache at the step's position
// (contiguous, or through a 16-token block table).
//
// Workgroup (sequence, slice): the sequence's D/2 rotation factors are
// computed in fp64 into LDS, then each thread rotates one pair of q or k or
// copies one element of v.  The rotation runs in fp64 and the stored key is
// rounded once to the cache dtype, so the appended row is bit-identical to
// the exact rotation rounded to nearest-even.
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

// Nearest-even bf16 of a double, in one rounding (no detour through fp32,
// which would round twice).  Works on the binary64 fields directly.
__device__ uint16_t double_to_bf16_rne(double x) {
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
  // workgroup (new token bt = b * T + t, slices y, y + gridDim.y, .. of 256
  // items): the D/2 rotation factors of the token's position are computed
  // once per workgroup (fp64) and shared by its threads through LDS
  __shared__ double cs[64], sn[64];
  const int bt = blockIdx.x;
  const int b = bt / p.T;
  const int half = p.D >> 1;
  const int64_t pos64 = static_cast<int64_t>(p.positions[b]) + (bt - b * p.T);
  // a slot past any cache (the rotation still uses the true position)
  const int pos = pos64 > 0x7fffffff ? -1 : static_cast<int>(pos64);
  for (int i = threadIdx.x; i < half; i += 256) {
    const double theta = pow(p.base, -2.0 * i / p.D);
    sincos(static_cast<double>(pos64) * theta, &sn[i], &cs[i]);
  }
  __syncthreads();
  const int nq = p.q ? p.H * half : 0;
  const int nk = p.G * half;
  const int nv = p.G * p.D;
  for (int i = blockIdx.y * 256 + threadIdx.x; i < nq + nk + nv; i += 256 * gridDim.y) {
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

}  // namespace

hipError_t launch_rope_append(const RopeParams& p, int32_t kv_dtype, bool paged,
                              hipStream_t stream) {
  const int work = (p.q ? p.H : 0) * (p.D / 2) + p.G * (p.D / 2) + p.G * p.D;
  if (p.T < 1 || static_cast<int64_t>(p.B) * p.T > 0x7fffffff) return hipErrorInvalidValue;
  // a few tokens (a decode step): one workgroup per 256 items, for
  // parallelism; many (a prompt): one workgroup per token, so the rotation
  // factors are computed once per token
  const int tokens = p.B * p.T;
  const int slices = tokens >= 4096 ? 1 : (work + 255) / 256;
  const dim3 grid(static_cast<unsigned>(tokens), slices);
  if (kv_dtype == KVD_FP32) {
    if (paged) rope_append_kernel<float, true><<<grid, 256, 0, stream>>>(p);
    else rope_append_kernel<float, false><<<grid, 256, 0, stream>>>(p);
  } else if (kv_dtype == KVD_INT8) {
    if (paged) rope_append_kernel<int8_t, true><<<grid, 256, 0, stream>>>(p);
    else rope_append_kernel<int8_t, false><<<grid, 256, 0, stream>>>(p);
  } else {
    if (paged) rope_append_kernel<uint16_t, true><<<grid, 256, 0, stream>>>(p);
    else rope_append_kernel<uint16_t, false><<<grid, 256, 0, stream>>>(p);
  }
  return hipGetLastError();
}

hipError_t launch_rope_append_mixed(const RopeParams& p, bool paged, hipStream_t stream) {
  if (p.T != 1 || p.window < 1 || !p.k_recent || !p.v_recent) return hipErrorInvalidValue;
  const int work = (p.q ? p.H : 0) * (p.D / 2) + p.G * (p.D / 2) + p.G * p.D;
  const dim3 grid(static_cast<unsigned>(p.B), (work + 255) / 256);
  if (paged) rope_append_kernel<int8_t, true, true><<<grid, 256, 0, stream>>>(p);
  else rope_append_kernel<int8_t, false, true><<<grid, 256, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace kvd
