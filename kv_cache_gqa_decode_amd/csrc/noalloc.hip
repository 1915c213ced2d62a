// gqa_decode_attn_multi_noalloc: gqa_decode_attn_multi for callers that
// cannot allocate device memory (code under graph capture, tight serving
// loops, harnesses that forbid hipMalloc).  The split partials and the work
// list live in a file-scope device array instead of a caller workspace.
//
// The array's name is a host-side stand-in in host code, not a device
// address: its address on each device is looked up once with
// hipGetSymbolAddress (with that device current) and only that pointer is
// ever handed to kernels.  Every device that runs the library holds its own
// copy of the array until the process ends.
//
// Nothing in the array needs clearing between calls: every byte a call
// reads (partials of splits that hold tokens, the work list and its count)
// is written earlier in the same call.  Calls that overlap in time on one
// device share the array and race.
#include <atomic>
#include <mutex>

#include "kvd_internal.h"

namespace {

static __device__ __align__(256) char scratch[KVD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's address of `scratch`, looked up on the first call
// on that device; null on a HIP error.
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!ptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

}  // namespace

extern "C" kvd_status gqa_decode_attn_multi_noalloc(
    const kvd_shape* shape, int32_t n_query, const float* q_rot, const void* k_cache,
    const void* v_cache, const float* k_scale, const float* v_scale, const int32_t* seq_lens,
    const int32_t* block_table, int32_t max_seq_len_host, float scale, float* out, float* lse,
    const kvd_options* options, void* stream) {
  // the size check comes first, so an oversized call is refused before any
  // HIP call; a shape or option error reports as gqa_decode_attn_multi would
  const size_t need = gqa_decode_workspace_size_multi(shape, n_query, max_seq_len_host, options);
  if (need > KVD_NOALLOC_SCRATCH_BYTES) return KVD_EWORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    ws = device_scratch();
    if (!ws) return KVD_EHIP;
  }
  return gqa_decode_attn_multi(shape, n_query, q_rot, k_cache, v_cache, k_scale, v_scale,
                               seq_lens, block_table, max_seq_len_host, scale, out, lse, ws,
                               need, options, stream);
}
