// Cross-split log-sum-exp merge.
//
// Attention over the union of disjoint token chunks is the combination of
// the per-chunk results weighted by exp(lse_s - lse): with M = max_s lse_s,
// w_s = 2^(lse_s - M) (lse kept in log2 units), out = sum_s w_s o_s / sum_s
// w_s and lse = M + log2(sum_s w_s).  This is the exact blockwise-softmax
// algebra behind the tiled attention of "Transformer推理核心：KV Cache、GQA与
// RoPE原理与工程实践" §4.2 applied across workgroups.
//
// Only the splits that hold tokens of the sequence are read.
#include "kvd_internal.h"

namespace kvd {
namespace {

constexpr float kNegInf = -__builtin_inff();

// Workgroup (b*H + h, dim group): 256 threads = SL split lanes x DT/4 float4
// columns merge DT output dims of one (b, h).  With few splits one
// workgroup takes all D dims; with many, D/32 workgroups share a (b, h).
template <int D, int DT>
__global__ __launch_bounds__(256) void lse_reduce_kernel(DecodeParams p) {
  constexpr int C4 = DT / 4;          // float4 columns
  constexpr int SL = 256 / C4;        // split lanes
  __shared__ float sm_red[256];
  __shared__ float4 sm_acc[SL][C4];
  __shared__ float sm_w[SL];

  const int bh = blockIdx.x;
  const int d0 = blockIdx.y * DT;
  const int b = bh / (p.H * p.T);       // rows b * T * H + t * H + h
  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > p.max_len_host ? p.max_len_host : L);
  const int ns = split_count(p, L);
  const int tid = threadIdx.x;
  float* out = p.out + static_cast<int64_t>(bh) * D + d0;
  if (ns == 0) {
    if (tid < DT) out[tid] = 0.f;
    if (tid == 0 && blockIdx.y == 0 && p.lse) p.lse[bh] = kNegInf;
    return;
  }
  const float* plse = p.part_lse + static_cast<int64_t>(bh) * p.n_splits;
  const float* po = p.part_o + static_cast<int64_t>(bh) * p.n_splits * D + d0;

  // 1) M = max over splits
  float M = kNegInf;
  for (int s = tid; s < ns; s += 256) M = fmaxf(M, plse[s]);
  sm_red[tid] = M;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) sm_red[tid] = fmaxf(sm_red[tid], sm_red[tid + w]);
    __syncthreads();
  }
  M = sm_red[0];
  const float ref = M == kNegInf ? 0.f : M;

  // 2) weighted sums, SL partial rows at a time
  const int sl = tid / C4, c4 = tid - sl * C4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float wsum = 0.f;
  for (int s = sl; s < ns; s += SL) {
    const float w = exp2f(plse[s] - ref);
    const float4 o = *reinterpret_cast<const float4*>(po + static_cast<int64_t>(s) * D + c4 * 4);
    acc.x += w * o.x; acc.y += w * o.y; acc.z += w * o.z; acc.w += w * o.w;
    wsum += w;
  }
  sm_acc[sl][c4] = acc;
  if (c4 == 0) sm_w[sl] = wsum;
  __syncthreads();
  if (tid < C4) {
    float4 a = sm_acc[0][tid];
    float ws = sm_w[0];
#pragma unroll
    for (int r = 1; r < SL; ++r) {
      const float4 x = sm_acc[r][tid];
      a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
      ws += sm_w[r];
    }
    // no split saw a valid token (every block invalid): empty softmax
    const float inv = ws > 0.f ? 1.f / ws : 0.f;
    reinterpret_cast<float4*>(out)[tid] = make_float4(a.x * inv, a.y * inv, a.z * inv, a.w * inv);
    if (tid == 0 && blockIdx.y == 0 && p.lse)
      p.lse[bh] = ws > 0.f ? (ref + log2f(ws)) * 0.69314718055994531f : kNegInf;
  }
}

}  // namespace

hipError_t launch_lse_reduce(const DecodeParams& p, hipStream_t stream) {
  const bool wide = p.n_splits > 16;
  const dim3 grid(p.B * p.H * p.T, wide ? p.D / 32 : 1);
  if (p.D == 64) {
    if (wide) lse_reduce_kernel<64, 32><<<grid, 256, 0, stream>>>(p);
    else lse_reduce_kernel<64, 64><<<grid, 256, 0, stream>>>(p);
  } else {
    if (wide) lse_reduce_kernel<128, 32><<<grid, 256, 0, stream>>>(p);
    else lse_reduce_kernel<128, 128><<<grid, 256, 0, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace kvd
