// Expansion of int4 latent codes into 16-bit MFMA operands (device code,
// internal to the library).  The decode consumes the int4 latent
// z_hat = code * scale (PALU page, section "Rollout", route C: quantization
// on top of the low-rank cache): a 4-bit two's-complement code times its
// chunk's binary16 scale is exact in fp32 and is rounded once, to nearest
// even, into the activation format.
#pragma once
#include "common.h"

#include <type_traits>

namespace palu {

// Eight codes (one 32-bit word: element i in nibble i) times the scale s ->
// eight T values as four 32-bit words (element 2k low, 2k+1 high).
template <class T>
__device__ __forceinline__ uint4 expand8(unsigned w, float s) {
  unsigned out[4];
  if constexpr (std::is_same<T, _Float16>::value) {
    // packed fp16: the nibble pair (2k, 2k+1) of byte k becomes the halves
    // 1024 + (q + 8) (bits 0x6400 | (nibble ^ 8)); subtracting 1032 gives q
    // exactly, and one fp16 multiply rounds q * s to nearest even, which is
    // the exact product rounded once
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const unsigned lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    const h2 s2 = {(_Float16)s, (_Float16)s};
    const h2 bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      // bytes [lo byte k, 0, hi byte k, 0]
      const unsigned sel = (unsigned)k | (0x0Cu << 8) | ((4u + k) << 16) | (0x0Cu << 24);
      const unsigned pr = (__builtin_amdgcn_perm(hi, lo, sel) ^ 0x00080008u) | 0x64006400u;
      out[k] = __builtin_bit_cast(unsigned, (__builtin_bit_cast(h2, pr) + bias) * s2);
    }
  } else {
    T v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = (int)(w << (28 - 4 * i)) >> 28;   // nibble i, 4-bit two's complement
      v[i] = from_f32<T>((float)q * s);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) out[k] = *(const unsigned*)&v[2 * k];
  }
  return uint4{out[0], out[1], out[2], out[3]};
}

// Eight codes (one 32-bit word: element i in nibble i) -> the eight integers
// as T, exactly (four 32-bit words, element 2k low, 2k+1 high).  The decode
// multiplies them by their scale only after the matrix product, so the
// latent code * scale enters unrounded.
template <class T>
__device__ __forceinline__ uint4 codes8(unsigned w) {
  unsigned out[4];
  if constexpr (std::is_same<T, _Float16>::value) {
    // the nibble pair (2k, 2k+1) of byte k becomes the halves 1024 + (q + 8)
    // (bits 0x6400 | (nibble ^ 8)); subtracting 1032 leaves q exactly
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const unsigned lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    const h2 bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const unsigned sel = (unsigned)k | (0x0Cu << 8) | ((4u + k) << 16) | (0x0Cu << 24);
      const unsigned pr = (__builtin_amdgcn_perm(hi, lo, sel) ^ 0x00080008u) | 0x64006400u;
      out[k] = __builtin_bit_cast(unsigned, __builtin_bit_cast(h2, pr) + bias);
    }
  } else {
    // bf16: a small integer is exact in binary32, and its upper half is the
    // bfloat16 of the same value
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float a = (float)((int)(w << (28 - 8 * k)) >> 28);        // nibble 2k
      const float b = (float)((int)(w << (24 - 8 * k)) >> 28);        // nibble 2k + 1
      out[k] = __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
    }
  }
  return uint4{out[0], out[1], out[2], out[3]};
}

// Eight codes times the scale s as hi + lo pairs of T: hi = T(code * s)
// (round to nearest even), lo = T(code * s - hi); both conversions of the
// second are exact, so hi + lo == code * s.
template <class T>
__device__ __forceinline__ void split8(unsigned w, float s, uint4& hi, uint4& lo) {
  T h[8], g[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float z = (float)((int)(w << (28 - 4 * i)) >> 28) * s;   // exact
    h[i] = from_f32<T>(z);
    g[i] = from_f32<T>(z - to_f32(h[i]));
  }
  hi = *(const uint4*)h;
  lo = *(const uint4*)g;
}

}  // namespace palu
