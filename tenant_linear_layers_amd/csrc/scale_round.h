// Final rounding of the BitDelta scale, shared by host and device code.
//
// alpha = mean|Delta| (page "BitDelta: Tek bir GPU kümesinden 14 Zen modeli
// sunmak", section "Matematiksel temel", alpha equation) is defined here as
// S / (n * 2^48) with S the exact integer sum of floor(|d| * 2^48), rounded
// once to float32, nearest with ties to even.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bd {

// float32 bits of S / (n * 2^48), S = s_hi * 2^64 + s_lo, 0 < n < 2^62.
//
// Fast path (S < 2^64, n < 2^53): q = double(S) / double(n) carries two
// roundings to nearest, so |q - S/n| < 2^-51.9 S/n, i.e. less than three
// units in the last place of q.  The nearest float of S/n is the nearest
// float of q unless a point halfway between two floats lies between them,
// which needs the 29 bits of q below the float significand to be within 3 of
// the halfway pattern 2^28.  Such q (within 8) are still right when q is S/n
// exactly (S < 2^53 and the fused S - q*n is zero; with n a power of two and
// S of few significant bits, as row sums of bf16 differences often are, q is
// often exactly halfway); the others, and results outside the normal float
// range, go to the long division.  Scaling by 2^-48 is exact, so the float
// conversion of q * 2^-48 rounds the same significand.
//
// Long division: restoring, one quotient bit per dividend bit, from the top
// bit of S downwards (then through zero fraction bits) until 25 significant
// quotient bits exist: 24 for the significand and one rounding bit.  Every
// dividend bit not yet brought down and the final remainder form the sticky
// bit.  The remainder stays below n, so it fits in 64 bits.
__host__ __device__ inline uint32_t ratio_to_f32_bits(uint64_t s_hi, uint64_t s_lo, uint64_t n) {
  if (n == 0) return 0x7FC00000u;
  if (s_hi == 0 && s_lo == 0) return 0u;
  if (s_hi == 0 && n < (uint64_t(1) << 53)) {
    const double q = (double)s_lo / (double)n;
    const uint64_t qb = __builtin_bit_cast(uint64_t, q);
    const uint64_t tail = qb & ((uint64_t(1) << 29) - 1);
    const uint64_t half = uint64_t(1) << 28;
    const int e = (int)((qb >> 52) & 0x7FF) - 1023 - 48;  // alpha in [2^e, 2^(e+1))
    if (e >= -126 && e <= 127) {
      bool ok = tail + 8 < half || tail > half + 8;
      if (!ok && s_lo < (uint64_t(1) << 53))
        ok = __builtin_fma(-q, (double)n, (double)s_lo) == 0.0;  // q == S/n
      if (ok) return __builtin_bit_cast(uint32_t, (float)(q * 0x1p-48));
    }
  }
  int top;  // index of the highest set bit of S
  if (s_hi) {
    top = 127 - __builtin_clzll(s_hi);
  } else {
    top = 63 - __builtin_clzll(s_lo);
  }
  uint64_t r = 0;
  uint32_t q = 0;
  int qbits = 0;
  int first = 0;  // weight exponent (relative to S/n) of the leading quotient bit
  int i = top;
  for (;; --i) {
    uint64_t bit = 0;
    if (i >= 64) {
      bit = (s_hi >> (i - 64)) & 1u;
    } else if (i >= 0) {
      bit = (s_lo >> i) & 1u;
    }
    r = (r << 1) | bit;
    uint32_t qb = 0;
    if (r >= n) {
      r -= n;
      qb = 1;
    }
    if (qbits > 0 || qb) {
      if (qbits == 0) first = i;
      q = (q << 1) | qb;
      ++qbits;
      if (qbits == 25) break;
    }
  }
  // Dividend bits below position i that were never brought down.
  bool sticky = r != 0;
  if (i > 0) {
    if (i >= 64) {
      sticky = sticky || s_lo != 0 || (s_hi & ((uint64_t(1) << (i - 64)) - 1)) != 0;
    } else {
      sticky = sticky || (s_lo & ((uint64_t(1) << i) - 1)) != 0;
    }
  }
  uint32_t mant = q >> 1;
  const uint32_t round = q & 1u;
  int e = first - 48;  // S/n in [2^first, 2^(first+1)); alpha = S/n * 2^-48
  if (round && (sticky || (mant & 1u))) {
    ++mant;
    if (mant == (1u << 24)) {
      mant >>= 1;
      ++e;
    }
  }
  if (e > 127) return 0x7F800000u;
  if (e < -126) return 0u;  // not reachable for the shapes the ABI accepts
  return (uint32_t(e + 127) << 23) | (mant & 0x7FFFFFu);
}

}  // namespace bd
