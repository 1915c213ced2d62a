// HBM streaming-read ceiling: what a plain, perfectly coalesced read of a
// large buffer achieves on this device, the practical roof beside the
// nominal 8 TB/s for the bandwidth-bound decode kernels.
//
// Two load paths, the two the decode kernels use:
//   * registers: each thread reads 16-byte words, UNROLL in flight per
//     iteration, and folds them into an XOR (optionally non-temporal);
//   * HBM -> LDS: each wave streams 1 KiB pieces (16 bytes per lane) with
//     buffer_load_dwordx4 ... lds straight into a ring of LDS slots, UNROLL
//     pieces in flight, the way the decode kernels stage their V tiles
//     (optionally non-temporal, as those copies are).
// One word per workgroup is written so the loads cannot be elided.
#include "kvd_internal.h"

namespace kvd {
namespace {

typedef __attribute__((address_space(3))) char lds_char;

// CHUNKED: workgroup w reads words [w * per, (w + 1) * per) (one contiguous
// stream per workgroup, like the split-K kernels); otherwise the whole grid
// strides over the buffer together.
template <int UNROLL, bool CHUNKED, bool NT>
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
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  auto load = [&](int64_t k) -> uint4 {
    if constexpr (NT) {
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + k));
      return make_uint4(v[0], v[1], v[2], v[3]);
    } else {
      return src[k];
    }
  };
  uint32_t x = 0;
  for (; i + (UNROLL - 1) * stride < n16; i += UNROLL * stride) {
    uint4 w[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) w[u] = load(i + u * stride);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) x ^= w[u].x ^ w[u].y ^ w[u].z ^ w[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 w = load(i);
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

// HBM -> LDS streaming.  Workgroup w owns the contiguous range [w * per,
// (w + 1) * per) of 1 KiB pieces (below 2 GiB, the host checks, so one
// buffer descriptor with 32-bit offsets covers it); wave v takes pieces v, v + 4, ... and
// keeps UNROLL of them in flight in a ring of 2 * UNROLL slots: group g of
// UNROLL copies goes to half g & 1, and before group g + 1 reuses the half
// of group g - 1, "vmcnt <= UNROLL" says group g - 1 has landed.  The
// buffer length is a whole number of pieces (the host checks), and the
// descriptor spans exactly the workgroup's range, so every copy is in
// bounds.  At the end each lane reads one dword of the ring.
template <int UNROLL, bool NT>
__global__ __launch_bounds__(256) void read_probe_lds_kernel(const char* __restrict__ src,
                                                             int64_t n_pieces, uint32_t* sink) {
  __shared__ __align__(16) char ring[4][2 * UNROLL][1024];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t per = (n_pieces + gridDim.x - 1) / gridDim.x;
  const int64_t lo = static_cast<int64_t>(blockIdx.x) * per;
  const int64_t hi = lo + per < n_pieces ? lo + per : n_pieces;
  const int64_t mine = hi > lo ? hi - lo : 0;               // pieces of this workgroup
  const uint32_t bytes = static_cast<uint32_t>(mine * 1024);
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(src) + lo * 1024, 0, static_cast<int>(bytes), 0x00020000);
  // pieces of this wave: wave, wave + 4, ...; groups of UNROLL of them
  const int64_t nw = mine > wave ? (mine - wave + 3) / 4 : 0;
  const int64_t groups = nw / UNROLL;
  lds_char* base = (lds_char*)(&ring[wave][0][0]);
  for (int64_t g = 0; g < groups; ++g) {
    const int half = static_cast<int>(g & 1);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t piece = wave + 4 * (g * UNROLL + u);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, base + (half * UNROLL + u) * 1024, 16,
                                               static_cast<uint32_t>(piece * 1024 + lane * 16),
                                               0, 0, NT ? 2 : 0);
    }
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(UNROLL) : "memory");
  }
  // the wave's last pieces (fewer than UNROLL), one group into half 0 (the
  // drain below orders them after the copies still writing there)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  for (int64_t k = groups * UNROLL; k < nw; ++k) {
    const int64_t piece = wave + 4 * k;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, base + (k - groups * UNROLL) * 1024, 16,
                                             static_cast<uint32_t>(piece * 1024 + lane * 16), 0,
                                             0, NT ? 2 : 0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  uint32_t x = reinterpret_cast<const uint32_t*>(&ring[wave][0][0])[lane];
  __shared__ uint32_t red[256];
  red[threadIdx.x] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
    for (int t = 0; t < 256; ++t) y ^= red[t];
    sink[blockIdx.x] = y;
  }
}

template <bool CHUNKED, bool NT>
void launch_probe(const uint4* src, int64_t n16, uint32_t* sink, int nwg, int unroll,
                  hipStream_t s) {
  if (unroll == 1) read_probe_kernel<1, CHUNKED, NT><<<nwg, 256, 0, s>>>(src, n16, sink);
  else if (unroll == 4) read_probe_kernel<4, CHUNKED, NT><<<nwg, 256, 0, s>>>(src, n16, sink);
  else if (unroll == 8) read_probe_kernel<8, CHUNKED, NT><<<nwg, 256, 0, s>>>(src, n16, sink);
  else read_probe_kernel<16, CHUNKED, NT><<<nwg, 256, 0, s>>>(src, n16, sink);
}

template <bool NT>
void launch_probe_lds(const char* src, int64_t n_pieces, uint32_t* sink, int nwg, int unroll,
                      hipStream_t s) {
  if (unroll == 1) read_probe_lds_kernel<1, NT><<<nwg, 256, 0, s>>>(src, n_pieces, sink);
  else if (unroll == 4) read_probe_lds_kernel<4, NT><<<nwg, 256, 0, s>>>(src, n_pieces, sink);
  else if (unroll == 8) read_probe_lds_kernel<8, NT><<<nwg, 256, 0, s>>>(src, n_pieces, sink);
  else read_probe_lds_kernel<16, NT><<<nwg, 256, 0, s>>>(src, n_pieces, sink);
}

}  // namespace
}  // namespace kvd

extern "C" kvd_status kvd_read_probe(const void* buf, size_t bytes, uint32_t* sink,
                                     int32_t n_workgroups, int32_t unroll, int32_t mode,
                                     void* stream) {
  using namespace kvd;
  if (!buf || !sink || n_workgroups < 1 || (bytes % 16) != 0 ||
      (reinterpret_cast<uintptr_t>(buf) & 15u) != 0 || (mode & ~7) != 0)
    return KVD_EINVAL;
  if (unroll != 1 && unroll != 4 && unroll != 8 && unroll != 16) return KVD_EUNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool chunked = mode & KVD_PROBE_CHUNKED, nt = mode & KVD_PROBE_NONTEMPORAL;
  if (mode & KVD_PROBE_LDS) {
    // whole 1 KiB pieces, and each workgroup's range addressable with
    // 32-bit offsets
    if (bytes % 1024 != 0) return KVD_EINVAL;
    const int64_t pieces = static_cast<int64_t>(bytes / 1024);
    const int64_t per = (pieces + n_workgroups - 1) / n_workgroups;
    if (per * 1024 > 0x7fffffffLL) return KVD_EINVAL;
    const char* src = static_cast<const char*>(buf);
    if (nt) launch_probe_lds<true>(src, pieces, sink, n_workgroups, unroll, s);
    else launch_probe_lds<false>(src, pieces, sink, n_workgroups, unroll, s);
  } else {
    const int64_t n16 = static_cast<int64_t>(bytes / 16);
    const uint4* src = static_cast<const uint4*>(buf);
    if (chunked) {
      if (nt) launch_probe<true, true>(src, n16, sink, n_workgroups, unroll, s);
      else launch_probe<true, false>(src, n16, sink, n_workgroups, unroll, s);
    } else {
      if (nt) launch_probe<false, true>(src, n16, sink, n_workgroups, unroll, s);
      else launch_probe<false, false>(src, n16, sink, n_workgroups, unroll, s);
    }
  }
  return hipGetLastError() == hipSuccess ? KVD_OK : KVD_EHIP;
}
