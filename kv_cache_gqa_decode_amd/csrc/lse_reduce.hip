// Cross-split log-sum-exp merge.
//
// Attention over the union of disjoint token chunks is the combination of
// the per-chunk results weighted by exp(lse_s - lse): with M = max_s lse_s,
// w_s = 2^(lse_s - M) (lse kept in log2 units), out = sum_s w_s o_s / sum_s
// w_s and lse = M + log2(sum_s w_s).  This is the exact blockwise-softmax
// algebra behind the tiled attention of "Transformer推理核心：KV Cache、GQA与
// RoPE原理与工程实践" §4.2 applied across workgroups.
//
// Only the splits that hold tokens of the sequence contribute: the first
// split_count(L) slots, or for a mixed-precision cache (len_mode 3) the
// history's splits in slots [0, seg2_base) and the recent tokens' splits
// from seg2_base on, each counted from its own share of L.  The kernel
// is a handful of microseconds of memory latency around a few MB of
// partials, so it is written to wait for memory once: the sequence length
// and every partial a thread merges are requested together (all reads stay
// inside the workspace; the splits past the sequence's end are masked after
// the loads land), each thread keeps its own running maximum, and the split
// lanes are combined with wave shuffles and two barriers.
#include "kvd_internal.h"

namespace kvd {
namespace {

constexpr float kNegInf = -__builtin_inff();
// rows from which each row's merge is one wave (four rows per workgroup):
// enough waves to occupy every CU, and no barrier or LDS round in the merge
constexpr int64_t kMergeWaveRows = 1024;

// Workgroup (b*T*H + t*H + h, dim group): 256 threads = SL split lanes x
// DT/4 float4 columns merge DT output dims of one query row; split lane sl
// takes splits sl, sl + SL, ... in batches of U whose loads are issued
// together.  With few splits one workgroup takes all D dims; with many,
// D/DT workgroups share a row.  kWaveRow: each of the 4 waves merges a row
// of its own (all D dims, 64 / (D/4) split lanes), rows 4x + wave.
template <int D, int DT, int U, bool kWaveRow = false>
__global__ __launch_bounds__(256) void lse_reduce_kernel(DecodeParams p) {
  constexpr int C4 = DT / 4;          // float4 columns
  constexpr int SL = (kWaveRow ? 64 : 256) / C4;   // split lanes
  static_assert(C4 <= 32 && SL * C4 == (kWaveRow ? 64 : 256), "columns within a wave");
  static_assert(!kWaveRow || DT == D, "a wave merges whole rows");
  __shared__ float4 sm_acc[4][C4];
  __shared__ float sm_m[4], sm_w[4];

  const int bh = kWaveRow ? blockIdx.x * 4 + (threadIdx.x >> 6) : blockIdx.x;
  if (kWaveRow && bh >= static_cast<int64_t>(p.B) * p.H * p.T) return;   // the whole wave: no barrier follows
  const int d0 = blockIdx.y * DT;
  const int b = bh / (p.H * p.T);       // rows b * T * H + t * H + h
  const int tid = kWaveRow ? static_cast<int>(threadIdx.x & 63) : static_cast<int>(threadIdx.x);
  const int sl = tid / C4, c4 = tid - sl * C4;
  // no workspace: no sequence can hold a token (the host planned no split)
  const int n_splits = p.part_lse ? p.n_splits : 0;
  const float* plse = p.part_lse + static_cast<int64_t>(bh) * p.n_splits;
  const float* po = p.part_o + static_cast<int64_t>(bh) * p.n_splits * D + d0 + c4 * 4;

  // the length through a vector-memory (buffer) load: a scalar load would
  // be waited for before the partials below are requested
  const __amdgpu_buffer_rsrc_t lens = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(p.seq_lens), 0, p.B * static_cast<int>(sizeof(int32_t)), 0x00020000);
  const int L = len_of(p, static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(lens, b * 4, 0, 0)));
  float m = kNegInf, wsum = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float ls[U];
  float4 o[U];
  // request batch s0 (split lane sl's splits s0, s0 + SL, ..., in bounds)
  auto request = [&](int s0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u * SL;
      const int sc = s < n_splits ? s : s0;          // in bounds; masked below
      ls[u] = plse[sc];
      o[u] = *reinterpret_cast<const float4*>(po + static_cast<int64_t>(sc) * D);
    }
  };
  // fold the landed batch s0 into (m, wsum, acc); slot s holds tokens when
  // s < ns, or with two segments when s < ns (the first) or s - seg2_base <
  // ns2 (the second)
  auto fold = [&](int s0, int ns, int ns2) {
    float mt = m;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u * SL;
      const bool held = p.len_mode == 3 ? (s < p.seg2_base ? s < ns : s - p.seg2_base < ns2)
                                        : s < ns;
      if (!held) ls[u] = kNegInf;                   // never weighs in, even if NaN was read
      mt = fmaxf(mt, ls[u]);
    }
    if (mt == kNegInf) return;
    const float a = exp2f(m - mt);                  // m = -inf: 0
    acc.x *= a; acc.y *= a; acc.z *= a; acc.w *= a;
    wsum *= a;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ls[u] == kNegInf) continue;               // masked, or a split without valid tokens
      const float w = exp2f(ls[u] - mt);
      acc.x += w * o[u].x; acc.y += w * o[u].y; acc.z += w * o[u].z; acc.w += w * o[u].w;
      wsum += w;
    }
    m = mt;
  };
  // The first batch is requested before the length is used, in the same
  // block, so that a single wait covers both; the rest (more than SL * U
  // splits) follow one batch at a time.
  if (sl < n_splits) {
    request(sl);
    // the splits holding tokens (the length clamped as in the split kernels)
    const int Lc = L < 0 ? 0 : (L > p.max_len_host ? p.max_len_host : L);
    int ns, ns2 = 0;
    if (p.len_mode == 3) {
      const int lh = Lc > p.window ? Lc - p.window : 0, lr = Lc < p.window ? Lc : p.window;
      ns = p.seg2_base > 0 ? split_count(p, lh) : 0;
      ns2 = (lr + p.seg2_chunk - 1) / p.seg2_chunk;
    } else {
      ns = split_count(p, Lc);
    }
    fold(sl, ns, ns2);
    for (int s0 = sl + SL * U; s0 < n_splits; s0 += SL * U) {
      request(s0);
      fold(s0, ns, ns2);
    }
  }
  // Combine the split lanes: the row's maximum (wave shuffles, then the 4
  // waves through LDS unless the wave holds the whole row), each lane's sums
  // rescaled to it, then summed over the split lanes of a column -- shuffles
  // inside a wave (the lanes C4 apart hold the same column), then the 4
  // waves through LDS.
  constexpr int kW = 4;
  const int lane = tid & 63, wave = tid >> 6;
  float M = m;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
  if constexpr (!kWaveRow) {
    if (lane == 0) sm_m[wave] = M;
    __syncthreads();
    M = fmaxf(fmaxf(sm_m[0], sm_m[1]), fmaxf(sm_m[2], sm_m[3]));
  }
  const float sc = m == kNegInf ? 0.f : exp2f(m - M);   // a lane without tokens adds 0
  float4 a = make_float4(acc.x * sc, acc.y * sc, acc.z * sc, acc.w * sc);
  float ws = wsum * sc;
#pragma unroll
  for (int off = C4; off < 64; off <<= 1) {
    a.x += __shfl_xor(a.x, off); a.y += __shfl_xor(a.y, off);
    a.z += __shfl_xor(a.z, off); a.w += __shfl_xor(a.w, off);
    ws += __shfl_xor(ws, off);
  }
  if constexpr (kWaveRow) {
    if (tid >= C4) return;
  } else {
    if (lane < C4) {
      sm_acc[wave][lane] = a;
      if (lane == 0) sm_w[wave] = ws;
    }
    __syncthreads();
    if (tid >= C4) return;
    a = sm_acc[0][tid];
    ws = sm_w[0];
#pragma unroll
    for (int w = 1; w < kW; ++w) {
      const float4 x = sm_acc[w][tid];
      a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
      ws += sm_w[w];
    }
  }
  // no split saw a valid token (an empty sequence, or every block invalid):
  // an empty softmax, out = 0 and lse = -inf
  const float inv = ws > 0.f ? 1.f / ws : 0.f;
  float* out = p.out + static_cast<int64_t>(bh) * D + d0;
  reinterpret_cast<float4*>(out)[tid] = make_float4(a.x * inv, a.y * inv, a.z * inv, a.w * inv);
  if (tid == 0 && blockIdx.y == 0 && p.lse)
    p.lse[bh] = ws > 0.f ? (M + log2f(ws)) * 0.69314718055994531f : kNegInf;
}

}  // namespace

hipError_t launch_lse_reduce(const DecodeParams& p, hipStream_t stream) {
  // Many rows (a batch, several new tokens, a prefill's key splits): a wave
  // per row, all D columns (D/4 float4 lanes) x 64/(D/4) split lanes, each
  // lane taking up to 8 splits per batch of loads.  Fewer rows: a workgroup
  // per row -- up to 8 splits all D columns x 256/(D/4) split lanes; more
  // splits (one long sequence) the row's dims over several workgroups, up to
  // 64 splits 32-dim groups (32 split lanes x 8 columns, 2 splits per lane
  // per batch), more 16-dim groups (64 split lanes x 4 columns, 4 per batch).
  const int ns = p.n_splits;
  const int64_t rows = static_cast<int64_t>(p.B) * p.H * p.T;
  if (rows > 0x7fffffff) return hipErrorInvalidValue;   // rows index the grid
  if (rows >= kMergeWaveRows) {
    const dim3 grid(static_cast<unsigned>((rows + 3) / 4), 1);
    const int sl = 64 / (p.D / 4);
    const int u = ns <= sl ? 1 : ns <= 2 * sl ? 2 : ns <= 4 * sl ? 4 : 8;
    if (p.D == 64) {
      if (u == 1) lse_reduce_kernel<64, 64, 1, true><<<grid, 256, 0, stream>>>(p);
      else if (u == 2) lse_reduce_kernel<64, 64, 2, true><<<grid, 256, 0, stream>>>(p);
      else if (u == 4) lse_reduce_kernel<64, 64, 4, true><<<grid, 256, 0, stream>>>(p);
      else lse_reduce_kernel<64, 64, 8, true><<<grid, 256, 0, stream>>>(p);
    } else {
      if (u == 1) lse_reduce_kernel<128, 128, 1, true><<<grid, 256, 0, stream>>>(p);
      else if (u == 2) lse_reduce_kernel<128, 128, 2, true><<<grid, 256, 0, stream>>>(p);
      else if (u == 4) lse_reduce_kernel<128, 128, 4, true><<<grid, 256, 0, stream>>>(p);
      else lse_reduce_kernel<128, 128, 8, true><<<grid, 256, 0, stream>>>(p);
    }
    return hipGetLastError();
  }
  const int groups = ns <= 8 ? 1 : (ns <= 64 ? p.D / 32 : p.D / 16);
  const dim3 grid(static_cast<unsigned>(rows), groups);
  if (p.D == 64) {
    if (ns <= 8) lse_reduce_kernel<64, 64, 1><<<grid, 256, 0, stream>>>(p);
    else if (ns <= 64) lse_reduce_kernel<64, 32, 2><<<grid, 256, 0, stream>>>(p);
    else lse_reduce_kernel<64, 16, 4><<<grid, 256, 0, stream>>>(p);
  } else {
    if (ns <= 8) lse_reduce_kernel<128, 128, 1><<<grid, 256, 0, stream>>>(p);
    else if (ns <= 64) lse_reduce_kernel<128, 32, 2><<<grid, 256, 0, stream>>>(p);
    else lse_reduce_kernel<128, 16, 4><<<grid, 256, 0, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace kvd
