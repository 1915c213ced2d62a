// INT8 cache codes on the fp16 matrix cores: exact code -> fp16 conversion
// and the fp16 MFMA, shared by the INT8 decode and prefill kernels.
#pragma once

#include "mfma_tile.h"

namespace kvd {
namespace mt {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Eight codes (two words, token order) -> eight exact fp16 values: c XOR
// 0x80 is c + 128 as an unsigned byte; under the exponent byte 0x64 it is the
// half 1024 + (c + 128), and one packed subtract of 1152 leaves c.
__device__ __forceinline__ f16x8 codes_to_f16(uint32_t w0, uint32_t w1) {
  constexpr uint32_t kExp = 0x64646464u;            // fp16 exponent byte of 1024
  const f16x2 off = {static_cast<_Float16>(-1152.f), static_cast<_Float16>(-1152.f)};
  const uint32_t x0 = w0 ^ 0x80808080u, x1 = w1 ^ 0x80808080u;   // c + 128, unsigned
  const f16x2 h0 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(kExp, x0, 0x04010400u)) + off;
  const f16x2 h1 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(kExp, x0, 0x04030402u)) + off;
  const f16x2 h2 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(kExp, x1, 0x04010400u)) + off;
  const f16x2 h3 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(kExp, x1, 0x04030402u)) + off;
  return f16x8{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// Two floats -> two fp16 in one word, nearest-even (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){a, b}, f16x2));
}

}  // namespace mt
}  // namespace kvd
