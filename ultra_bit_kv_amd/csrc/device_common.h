// Device helpers shared by the liboscar_kv kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "oscar_internal.h"

namespace oscar {

// ---------------------------------------------------------------------------
// Single round-to-nearest-even conversions from fp64.
//
// The cache stores the bf16 rounding of each rotated row and fp16 scale /
// zero-point values (OSCAR summary page, sections 3-4).  Both conversions go
// straight from the fp64 value: |x| is scaled by an exact power of two so
// that its quantum becomes 1, rounded to an integer with rint (IEEE
// round-half-even), and the integer is placed into the target's fields.  A
// significand that rounds up to the next power of two carries into the
// exponent field by the addition itself.
// ---------------------------------------------------------------------------
__host__ __device__ __forceinline__ uint16_t round_f64_to_short_float(double x, int emin,
                                                                      int mant_bits, int bias,
                                                                      uint32_t inf_bits,
                                                                      uint32_t nan_bits) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  const uint32_t sign = (uint32_t)(b >> 48) & 0x8000u;
  const double a = __builtin_fabs(x);
  if (a != a) return (uint16_t)(sign | nan_bits);
  if (a == __builtin_inf()) return (uint16_t)(sign | inf_bits);
  const int expf = (int)((b >> 52) & 0x7FFu);
  if (expf == 0) return (uint16_t)sign;       // zero or below 2^-1022: rounds to zero
  const int e = expf - 1023;                  // floor(log2 |x|)
  const int eq = (e > emin ? e : emin) - mant_bits;
  const double m = __builtin_ldexp(a, -eq);   // exact: power-of-two scaling
  const uint32_t mi = (uint32_t)__builtin_rint(m);
  uint32_t bits;
  if (e >= emin)
    bits = ((uint32_t)(e + bias) << mant_bits) + mi - (1u << mant_bits);
  else
    bits = mi;                                  // subnormal (mi == 2^mant_bits is the min normal)
  if (bits >= inf_bits) bits = inf_bits;
  return (uint16_t)(sign | bits);
}

__host__ __device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
  return round_f64_to_short_float(x, -126, 7, 127, 0x7F80u, 0x7FC0u);
}

__host__ __device__ __forceinline__ uint16_t f64_to_f16_rne(double x) {
  return round_f64_to_short_float(x, -14, 10, 15, 0x7C00u, 0x7E00u);
}

// fp64 -> bf16 round-to-nearest-even on the bit pattern for results in the
// bf16 normal range (exponent field 897 .. 1150): the 45 dropped significand
// bits round by adding 2^44 - 1 plus the kept lowest bit, a carry moving into
// the exponent; zeros, subnormals and overflow take f64_to_bf16_rne.
__host__ __device__ __forceinline__ uint16_t f64_to_bf16_rne_normal(double x) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  const uint32_t e = (uint32_t)(b >> 52) & 0x7FFu;
  if (e < 897u || e > 1150u) return f64_to_bf16_rne(x);
  const uint64_t mag = b & 0x7FFFFFFFFFFFFFFFull;
  const uint64_t r = mag + 0xFFFFFFFFFFFull + ((mag >> 45) & 1ull);
  uint32_t bits = (uint32_t)(r >> 45) - (896u << 7);
  if (bits >= 0x7F80u) bits = 0x7F80u;
  return (uint16_t)(((uint32_t)(b >> 48) & 0x8000u) | bits);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ double f16_bits_to_f64(uint32_t bits16) {
  _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)bits16);
  return (double)h;
}

// ---------------------------------------------------------------------------
// Positions, windows and pages of one cache row (the placement rule of the
// OSCAR summary page, section 4, with the WUSH-KV flush boundary S_quant).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int s_quant_of(int len, int s_sink, int s_keep, int s_flush) {
  int num = len - s_sink - s_keep;
  int k = num >= 0 ? num / s_flush : 0;
  return s_sink + s_flush * k;
}

// Structured rotations (kind 1: R = H / sqrt(128), kind 2: R = H P_br / sqrt(128),
// Sylvester's H[i][k] = (-1)^popcount(i & k), P_br the 7-bit bit reversal of
// the column index): entry R[i][k] in fp32.
constexpr float kInvSqrtDf = 0x1.6a09e6p-4f;   // fp32(sqrt(2)) / 16

__device__ __forceinline__ int bitrev7(int k) { return (int)(__brev((unsigned)k) >> 25); }

// x / d and x % d (r) for 0 <= x < 2^31 and d >= 1, with m = floor(2^32 / d)
// (m = 0 for d = 1): umulhi(x, m) is the quotient or one less (x m / 2^32
// lies within x / 2^32 < 1 below x / d), so one correction makes it exact.
__device__ __forceinline__ uint32_t div_by_magic(uint32_t x, uint32_t d, uint32_t m, uint32_t& r) {
  uint32_t q = m ? __umulhi(x, m) : x;
  r = x - q * d;
  if (r >= d) {
    q += 1;
    r -= d;
  }
  return q;
}

__device__ __forceinline__ float hadamard_entry(int kind, int i, int k) {
  const int c = kind == 2 ? bitrev7(k) : k;
  return (__popc((unsigned)(i & c)) & 1) ? -kInvSqrtDf : kInvSqrtDf;
}

}  // namespace oscar
