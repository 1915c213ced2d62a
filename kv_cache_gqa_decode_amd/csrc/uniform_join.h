// Joining the two 32-bit halves of a wave-uniform 64-bit value (an address)
// after each half went through a wave broadcast.  Plain C++ (no HIP types)
// so that the host test suite compiles this very header and checks it.
#pragma once

#include <stdint.h>

namespace kvd {

// `bcast` broadcasts a 32-bit lane value and returns it as a signed int, as
// the readfirstlane builtin does.  Each half goes back through uint32_t
// before the join: joining the signed low half directly would sign-extend
// it, and an address whose low word has bit 31 set would become
// 0xffffffff'xxxxxxxx.  (constexpr: host and device function in HIP.)
template <typename Bcast>
constexpr uint64_t join_uniform_halves(uint64_t v, Bcast bcast) {
  const uint32_t lo = static_cast<uint32_t>(bcast(static_cast<uint32_t>(v)));
  const uint32_t hi = static_cast<uint32_t>(bcast(static_cast<uint32_t>(v >> 32)));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

}  // namespace kvd
