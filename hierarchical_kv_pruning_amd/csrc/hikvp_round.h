// hikvp_round.h -- one-step rounding of fp64 values to the storage types,
// for queries formed as exact sums (shared group queries, folded queries).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hikvp {

// fp64 -> bf16, nearest with ties to even, from the bit pattern (one
// rounding).  Zero keeps its sign; magnitudes outside the bf16 normal range
// saturate the exponent field.
__device__ inline uint16_t f64_to_bf16_rne(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint32_t sign = (uint32_t)(u >> 63);
  if ((u << 1) == 0) return (uint16_t)(sign << 15);
  int e = (int)((u >> 52) & 0x7ffu) - 1023 + 127;
  const uint64_t sig = (u & ((1ull << 52) - 1)) | (1ull << 52);  // 53 significant bits
  uint64_t keep = sig >> 45;                                     // 8 of them
  const uint64_t rest = sig & ((1ull << 45) - 1), half = 1ull << 44;
  if (rest > half || (rest == half && (keep & 1))) ++keep;
  if (keep >> 8) { keep >>= 1; ++e; }
  e = e < 0 ? 0 : (e > 255 ? 255 : e);
  return (uint16_t)((sign << 15) | ((uint32_t)e << 7) | (uint32_t)(keep & 0x7fu));
}

__device__ inline double bf16_value(uint16_t h) { return (double)__uint_as_float((uint32_t)h << 16); }

// An exact value as the sum of two bf16 values: hi = x rounded, lo = the
// residual x - hi (exact in fp64) rounded, and what the pair leaves out.
struct Bf16Split {
  uint16_t hi, lo;
  double rest;                 // x - hi - lo
};
__device__ inline Bf16Split split_bf16(double x) {
  Bf16Split s;
  s.hi = f64_to_bf16_rne(x);
  const double r = x - bf16_value(s.hi);
  s.lo = f64_to_bf16_rne(r);
  s.rest = r - bf16_value(s.lo);
  return s;
}

}  // namespace hikvp
