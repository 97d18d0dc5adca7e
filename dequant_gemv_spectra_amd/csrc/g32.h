// Group-32 quantizer helpers shared by the weight packer and the KV-cache
// append kernel.  Also compiled for the host, so that a CPU test can check the
// conversion against numpy on every binary16 value and rounding midpoint.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spectra {

__host__ __device__ __forceinline__ double g32_h2d(uint16_t b) {
  return (double)__builtin_bit_cast(_Float16, b);
}

// binary64 -> binary16, round to nearest, ties to even.  Written from the IEEE
// 754 formats: keep 11 significant bits (fewer in the subnormal range, whose
// unit is 2^-24), round on the dropped bits, let a carry ripple into the
// exponent field, saturate to infinity past the largest finite value.
__host__ __device__ inline uint16_t f64_to_f16_rne(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  const int ex = (int)((b >> 52) & 0x7FF);
  const uint64_t frac = b & 0x000FFFFFFFFFFFFFull;
  if (ex == 0x7FF) return sign | 0x7C00u | (frac ? 0x0200u : 0u);
  if (ex == 0) return sign;  // binary64 subnormals are far below half of 2^-24
  const int e = ex - 1023;
  if (e > 15) return sign | 0x7C00u;
  const uint64_t m = frac | (1ull << 52);  // 53-bit significand
  int shift = 42;                          // 52 - 10 fraction bits kept
  int biased = e + 15;
  if (e < -14) {                           // half subnormal
    shift += (-14 - e);
    biased = 0;
  }
  if (shift > 60) return sign;
  uint64_t r = m >> shift;
  const uint64_t rem = m & ((1ull << shift) - 1);
  const uint64_t halfway = 1ull << (shift - 1);
  if (rem > halfway || (rem == halfway && (r & 1))) r += 1;
  uint32_t bits;
  if (biased == 0) {
    bits = (uint32_t)r;  // r == 1024 becomes the smallest normal on its own
  } else {
    bits = ((uint32_t)biased << 10) + (uint32_t)(r - 1024);
  }
  if (bits >= 0x7C00u) bits = 0x7C00u;
  return sign | (uint16_t)bits;
}

// Bit position of member e (0..31) in its code word e / 8.
__host__ __device__ __forceinline__ uint32_t member_shift(int e) {
  return 16u * (uint32_t)(e & 1) + 4u * (uint32_t)((e & 7) >> 1);
}

}  // namespace spectra
