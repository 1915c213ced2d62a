// Split-K decode attention with VALU dot products (fp32 or bf16 KV).
//
// softmax(q K^T * scale) V for one query per (b, h) over L_b cached tokens
// ("Transformer推理核心：KV Cache、GQA与RoPE原理与工程实践" §2.1, §4.2; "4. 自注意力
// 机制推理" §4.5).  The sequence is cut into chunks of `chunk` tokens; one
// workgroup (4 waves) handles one chunk of one KV head for RB query heads of
// that head's group, so every K/V row fetched from HBM serves RB heads
// (the GQA sharing of §2.2 without materialising the broadcast).
//
// Data movement: a K or V row of one head is D * sizeof(T) contiguous bytes
// (256 B for bf16 D = 128).  Each lane loads 16 bytes per row, so LPR lanes
// cover a row with one fully coalesced load and a wave fetches RPW rows per
// instruction; U rows of K and U rows of V are in flight per lane before any
// arithmetic.  Rows go straight from HBM into registers: each is used once,
// by the lanes that loaded it, so staging through LDS would only add
// instructions.
//
// Arithmetic: per row, each lane forms EPL products per head, a butterfly
// over the LPR lanes of the row (DPP within 16-lane rows) gives the score,
// and each row-lane keeps its own online softmax (running max m, running
// sum l, accumulator) -- the blockwise softmax of the FlashAttention
// approach (§4.2 of the same page).  Scores are kept in log2 units
// (q pre-multiplied by scale * log2 e) so exp2 is used throughout.  At the
// end the row streams of a wave merge through cross-lane shuffles, the four
// waves through LDS, and the workgroup writes one (o, lse) partial.
#include "kvd_internal.h"

namespace kvd {
namespace {

constexpr float kNegInf = -__builtin_inff();

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kPerLoad = 4;
  __device__ __forceinline__ static void unpack(const uint4& w, float* f) {
    f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y);
    f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
  }
};
template <> struct Elem<uint16_t> {
  static constexpr int kPerLoad = 8;
  __device__ __forceinline__ static void unpack(const uint4& w, float* f) {
    f[0] = bf16lo(w.x); f[1] = bf16hi(w.x); f[2] = bf16lo(w.y); f[3] = bf16hi(w.y);
    f[4] = bf16lo(w.z); f[5] = bf16hi(w.z); f[6] = bf16lo(w.w); f[7] = bf16hi(w.w);
  }
};

// Sum over the LPR consecutive lanes that share a row, result in every one
// of them.  LPR in {8, 16, 32}.
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  // quad_perm [1,0,3,2], quad_perm [2,3,0,1]: every lane holds its quad's sum
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
  // row_half_mirror: lane i of each 8 reads lane 7 - i (the other quad)
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
  if constexpr (LPR >= 16) {
    // row_mirror: lane i of each 16 reads lane 15 - i (the other half-row)
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
  }
  if constexpr (LPR >= 32) x += __shfl_xor(x, 16);
  return x;
}

template <bool PAGED>
__device__ __forceinline__ int64_t kv_row(const DecodeParams& p, int b, int t, int g, bool& ok) {
  if (!PAGED) return (static_cast<int64_t>(b) * p.max_seq_len + t) * p.G + g;
  int grp = paged_group(p, b, t >> 4);
  if (grp < 0) { ok = false; grp = 0; }
  return (static_cast<int64_t>(grp) * 16 + (t & 15)) * p.G + g;
}

template <typename T, int D, int RB, bool PAGED>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeParams p) {
  constexpr int EPL = Elem<T>::kPerLoad;      // elements per lane per row
  constexpr int LPR = D / EPL;                // lanes per row
  constexpr int RPW = 64 / LPR;               // rows per wave per load
  constexpr int U = 4;                        // rows in flight per lane
  constexpr int TW = RPW * U;                 // tokens per wave tile
  constexpr int kWaves = 4;
  static_assert(LPR >= 8 && LPR <= 32, "unsupported row shape");

  __shared__ float sm_acc[kWaves][RB][D];
  __shared__ float sm_m[kWaves][RB];
  __shared__ float sm_l[kWaves][RB];

  // grid (B, G * head_groups, n_splits): first chunks are dispatched first
  const int b = blockIdx.x;
  const int g = blockIdx.y / p.head_groups;
  const int hg = blockIdx.y - g * p.head_groups;
  const int split = blockIdx.z;
  const int L = attended_len(p, __builtin_amdgcn_readfirstlane(p.seq_lens[b]));
  const int h0 = g * p.R + hg * RB;
  const int nh = min(RB, p.R - hg * RB);
  const int t0 = split_start(p, split);
  if (t0 >= L) {
    if (p.direct && split == 0) {      // empty sequence: out = 0, lse = -inf
      for (int idx = threadIdx.x; idx < nh * D; idx += 256) {
        const int r = idx / D, d = idx - r * D;
        p.out[(static_cast<int64_t>(b) * p.H + h0 + r) * D + d] = 0.f;
        if (d == 0 && p.lse) p.lse[static_cast<int64_t>(b) * p.H + h0 + r] = kNegInf;
      }
    }
    return;
  }
  const int t1 = min(t0 + split_size(p, split), L);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rg = lane / LPR, c = lane - rg * LPR;

  // unconditional vector loads from a valid head, then a select (a load under
  // a per-lane branch would serialise into one round trip per element)
  float q[RB][EPL];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const bool live = r < nh;
    const float* src = p.q_rot + (static_cast<int64_t>(b) * p.H + h0 + (live ? r : 0)) * D + c * EPL;
    const float qs = live ? p.qscale : 0.f;
#pragma unroll
    for (int e = 0; e < EPL; e += 4) {
      const float4 x = *reinterpret_cast<const float4*>(src + e);
      q[r][e] = x.x * qs; q[r][e + 1] = x.y * qs; q[r][e + 2] = x.z * qs; q[r][e + 3] = x.w * qs;
    }
  }

  float m[RB], l[RB], acc[RB][EPL];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    m[r] = kNegInf; l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[r][e] = 0.f;
  }

  const char* kbase = static_cast<const char*>(p.k);
  const char* vbase = static_cast<const char*>(p.v);
  constexpr int64_t kRowBytes = static_cast<int64_t>(D) * sizeof(T);

  for (int tile = t0 + wave * TW; tile < t1; tile += kWaves * TW) {
    uint4 kr[U], vr[U];
    bool valid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = tile + u * RPW + rg;
      bool ok = t < t1;
      const int64_t row = kv_row<PAGED>(p, b, ok ? t : t0, g, ok);
      valid[u] = ok;
      kr[u] = *reinterpret_cast<const uint4*>(kbase + row * kRowBytes + c * 16);
      vr[u] = *reinterpret_cast<const uint4*>(vbase + row * kRowBytes + c * 16);
    }
    float s[RB][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[EPL];
      Elem<T>::unpack(kr[u], kf);
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) d += q[r][e] * kf[e];
        s[r][u] = d;
      }
    }
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float t = row_sum<LPR>(s[r][u]);
        s[r][u] = valid[u] ? t : kNegInf;
      }
    float vf[U][EPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint4 w = valid[u] ? vr[u] : make_uint4(0, 0, 0, 0);  // padding may hold NaN
      Elem<T>::unpack(w, vf[u]);
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      float mt = s[r][0];
#pragma unroll
      for (int u = 1; u < U; ++u) mt = fmaxf(mt, s[r][u]);
      const float mn = fmaxf(m[r], mt);
      const float ref = mn == kNegInf ? 0.f : mn;
      const float alpha = exp2f(m[r] - ref);
      float pu[U], ps = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) { pu[u] = exp2f(s[r][u] - ref); ps += pu[u]; }
      l[r] = l[r] * alpha + ps;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        float a = acc[r][e] * alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) a += pu[u] * vf[u][e];
        acc[r][e] = a;
      }
      m[r] = mn;
    }
  }

  // merge the RPW row streams of this wave (lanes c, c + LPR, ...)
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const float mo = __shfl_xor(m[r], off);
      const float lo = __shfl_xor(l[r], off);
      const float mn = fmaxf(m[r], mo);
      const float ref = mn == kNegInf ? 0.f : mn;
      const float a = exp2f(m[r] - ref), ao = exp2f(mo - ref);
      l[r] = l[r] * a + lo * ao;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float x = __shfl_xor(acc[r][e], off);
        acc[r][e] = acc[r][e] * a + x * ao;
      }
      m[r] = mn;
    }
  }
  if (rg == 0) {
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_acc[wave][r][c * EPL + e] = acc[r][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < RB; ++r) { sm_m[wave][r] = m[r]; sm_l[wave][r] = l[r]; }
  }
  __syncthreads();

  // merge the four waves; thread -> (head r, dim d)
  for (int idx = threadIdx.x; idx < nh * D; idx += 256) {
    const int r = idx / D, d = idx - r * D;
    float M = sm_m[0][r];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_m[w][r]);
    const float ref = M == kNegInf ? 0.f : M;
    float o = 0.f, sum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float a = exp2f(sm_m[w][r] - ref);
      o += sm_acc[w][r][d] * a;
      sum += sm_l[w][r] * a;
    }
    const int h = h0 + r;
    const float val = o / sum;
    const float lse2 = ref + log2f(sum);
    if (p.direct) {
      p.out[(static_cast<int64_t>(b) * p.H + h) * D + d] = val;
      if (d == 0 && p.lse) p.lse[static_cast<int64_t>(b) * p.H + h] = lse2 * 0.69314718055994531f;
    } else {
      const int64_t pr = (static_cast<int64_t>(b) * p.H + h) * p.part_stride + p.split_base + split;
      p.part_o[pr * D + d] = val;
      if (d == 0) p.part_lse[pr] = lse2;
    }
  }
}

template <typename T, int D, bool PAGED>
hipError_t launch_t(const DecodeParams& p, int rb, const Launch& l) {
  const dim3 grid(p.B, p.G * p.head_groups, p.n_splits);
  void (*k)(DecodeParams) = rb == 1 ? decode_valu_kernel<T, D, 1, PAGED>
                          : rb == 2 ? decode_valu_kernel<T, D, 2, PAGED>
                          : rb == 4 ? decode_valu_kernel<T, D, 4, PAGED>
                                    : decode_valu_kernel<T, D, 8, PAGED>;
  return launch_kernel(k, grid, dim3(256), l, p);
}

template <typename T, int D>
hipError_t launch_d(const DecodeParams& p, bool paged, int rb, const Launch& l) {
  return paged ? launch_t<T, D, true>(p, rb, l) : launch_t<T, D, false>(p, rb, l);
}

}  // namespace

int valu_heads_per_pass(int n_rep) {
  if (n_rep <= 1) return 1;
  if (n_rep <= 2) return 2;
  if (n_rep <= 4) return 4;
  return 8;
}

hipError_t launch_decode_valu(const DecodeParams& p, int32_t kv_dtype, bool paged, int rb,
                              const Launch& l) {
  if (p.T != 1) return hipErrorInvalidValue;    // one new token per sequence
  if (kv_dtype == KVD_FP32) {
    return p.D == 64 ? launch_d<float, 64>(p, paged, rb, l) : launch_d<float, 128>(p, paged, rb, l);
  }
  return p.D == 64 ? launch_d<uint16_t, 64>(p, paged, rb, l)
                   : launch_d<uint16_t, 128>(p, paged, rb, l);
}

}  // namespace kvd
