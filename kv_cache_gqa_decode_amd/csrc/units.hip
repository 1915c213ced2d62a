// Work list of the matrix-core split kernels for batches of sequences.
//
// A batch with ragged lengths has many (sequence, split) slots past the end
// of their sequence: with the splits as a grid dimension each of them is a
// workgroup that starts, finds no token and exits, and they are interleaved
// with the real units all through the dispatch, so a fifth of the resident
// slots of a 64-sequence batch sat idle on them (measured with per-workgroup
// timestamps).  This kernel turns the lengths, which only the device knows,
// into a dense list of the units that hold tokens, so that the split kernel's
// grid carries its empty slots at the very end:
//   1. the full-size units (every split but possibly the last of each
//      sequence), sequence by sequence (measured as fast as or faster than
//      split by split on every workload);
//   2. then the last, partial split of each sequence, longest first, so the
//      units dispatched last are the shortest ones (longest-processing-time
//      order for the tail).
// Entries are b | split << 16.  The order only decides which units run side
// by side: each unit writes its own partial and the merge reads them in split
// order, so results do not depend on it.
//
// One workgroup of 1024 threads: per-thread ranges of sequences, wave-shuffle
// scans joined through LDS, partial units counted per 16-token bucket with LDS
// atomics.  It runs before the split kernel on every call, so it is kept to a
// few barriers.
#include "kvd_internal.h"

namespace kvd {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBuckets = kMaxChunk / 16;     // partial units binned by tokens / 16
static_assert(kBuckets <= kThreads, "one bucket per thread");

// Exclusive scan of one value per thread over the workgroup; `total` gets
// the sum.  Two barriers.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_sums, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wave_sums[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int s = wave_sums[w];
    before += w < wave ? s : 0;
    all += s;
  }
  __syncthreads();
  total = all;
  return before + x - v;
}

__global__ __launch_bounds__(kThreads) void build_units_kernel(DecodeParams p) {
  __shared__ int wave_sums[kWaves];
  __shared__ int bucket[kBuckets];
  const int t = threadIdx.x;
  const int B = p.B;
  const int per = (B + kThreads - 1) / kThreads;
  const int b0 = min(B, t * per), b1 = min(B, b0 + per);

  // full units of sequence b (all splits but the last, plus the last one when
  // it is full-size) and the tokens of its partial last split (0 if none)
  auto counts = [&](int b, int& full, int& last_tokens) {
    const int L = attended_len(p, len_of(p, p.seq_lens[b]));
    const int n = split_count(p, L);
    full = 0;
    last_tokens = 0;
    if (n == 0) return;
    const int tail = L - split_start(p, n - 1);
    if (tail == split_size(p, n - 1)) {
      full = n;
    } else {
      full = n - 1;
      last_tokens = tail;
    }
  };

  if (t < kBuckets) bucket[t] = 0;
  int my_full = 0;
  for (int b = b0; b < b1; ++b) {
    int f, lt;
    counts(b, f, lt);
    my_full += f;
  }
  int n_full = 0;
  int pos = block_exclusive_scan(my_full, wave_sums, n_full);   // barriers also cover `bucket`

  // full units, sequence by sequence; count the partial ones per bucket
  for (int b = b0; b < b1; ++b) {
    int f, lt;
    counts(b, f, lt);
    for (int s = 0; s < f; ++s)
      p.units[pos++] = static_cast<int32_t>(static_cast<uint32_t>(b) | (static_cast<uint32_t>(s) << 16));
    if (lt > 0) atomicAdd(&bucket[(lt - 1) >> 4], 1);
  }
  __syncthreads();
  // bucket offsets, longest bucket first: exclusive scan over buckets taken
  // in descending order (thread t holds bucket kBuckets - 1 - t)
  const int cnt = t < kBuckets ? bucket[kBuckets - 1 - t] : 0;
  int n_part = 0;
  const int off = block_exclusive_scan(cnt, wave_sums, n_part);
  if (t < kBuckets) bucket[kBuckets - 1 - t] = n_full + off;
  if (t == 0) *p.n_units = n_full + n_part;
  __syncthreads();
  for (int b = b0; b < b1; ++b) {
    int f, lt;
    counts(b, f, lt);
    if (lt > 0) {
      const int at = atomicAdd(&bucket[(lt - 1) >> 4], 1);
      // the partial last split is split f
      p.units[at] = static_cast<int32_t>(static_cast<uint32_t>(b) | (static_cast<uint32_t>(f) << 16));
    }
  }
}

}  // namespace

hipError_t launch_build_units(const DecodeParams& p, hipStream_t stream) {
  if (p.B > 65535 || p.n_splits > 65535 || p.chunk > kMaxChunk || !p.units || !p.n_units)
    return hipErrorInvalidValue;
  build_units_kernel<<<1, kThreads, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace kvd
