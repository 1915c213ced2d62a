// HBM streaming-read ceiling: what a plain, perfectly coalesced read of a
// large buffer achieves on this device, the practical roof beside the
// nominal 8 TB/s for the bandwidth-bound decode kernels.
//
// Each thread reads 16-byte words in a grid-stride loop, UNROLL words in
// flight per iteration, and folds them into an XOR; one word per workgroup
// is written so the loads cannot be elided.
#include "kvd_internal.h"

namespace kvd {
namespace {

// CHUNKED: workgroup w reads words [w * per, (w + 1) * per) (one contiguous
// stream per workgroup, like the split-K kernels); otherwise the whole grid
// strides over the buffer together.
template <int UNROLL, bool CHUNKED>
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ src,
                                                         int64_t n16, uint32_t* sink) {
  int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (CHUNKED) {
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const int64_t lo = static_cast<int64_t>(blockIdx.x) * per;
    const int64_t hi = lo + per < n16 ? lo + per : n16;
    src += lo;
    n16 = hi > lo ? hi - lo : 0;
    stride = 256;
    i = threadIdx.x;
  }
  uint32_t x = 0;
  for (; i + (UNROLL - 1) * stride < n16; i += UNROLL * stride) {
    uint4 w[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) w[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) x ^= w[u].x ^ w[u].y ^ w[u].z ^ w[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 w = src[i];
    x ^= w.x ^ w.y ^ w.z ^ w.w;
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
    for (int t = 0; t < 256; ++t) y ^= red[t];
    sink[blockIdx.x] = y;
  }
}

}  // namespace
}  // namespace kvd

namespace {
template <bool CHUNKED>
void launch_probe(const uint4* src, int64_t n16, uint32_t* sink, int nwg, int unroll,
                  hipStream_t s) {
  if (unroll == 1) kvd::read_probe_kernel<1, CHUNKED><<<nwg, 256, 0, s>>>(src, n16, sink);
  else if (unroll == 4) kvd::read_probe_kernel<4, CHUNKED><<<nwg, 256, 0, s>>>(src, n16, sink);
  else if (unroll == 8) kvd::read_probe_kernel<8, CHUNKED><<<nwg, 256, 0, s>>>(src, n16, sink);
  else kvd::read_probe_kernel<16, CHUNKED><<<nwg, 256, 0, s>>>(src, n16, sink);
}
}  // namespace

extern "C" kvd_status kvd_read_probe(const void* buf, size_t bytes, uint32_t* sink,
                                     int32_t n_workgroups, int32_t unroll, int32_t chunked,
                                     void* stream) {
  if (!buf || !sink || n_workgroups < 1 || (bytes % 16) != 0 ||
      (reinterpret_cast<uintptr_t>(buf) & 15u) != 0)
    return KVD_EINVAL;
  if (unroll != 1 && unroll != 4 && unroll != 8 && unroll != 16) return KVD_EUNSUPPORTED;
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint4* src = static_cast<const uint4*>(buf);
  if (chunked) launch_probe<true>(src, n16, sink, n_workgroups, unroll, s);
  else launch_probe<false>(src, n16, sink, n_workgroups, unroll, s);
  return hipGetLastError() == hipSuccess ? KVD_OK : KVD_EHIP;
}
