// The 2:4 eligibility and compression rules on packed NVFP4 codes, shared by the 2:4 codec
// kernels and the fused producer.
//
// Rule ("Sparse GPU FLOPS Need the Right Zeros in the Right Places", leviathansystems.co,
// section "The operation determines which four entries belong together"): a group of four
// consecutive codes along K is eligible when at least two are zero; a code is zero when its
// three magnitude bits are 0 (so 0x8, the FP4 negative zero, is zero).
// Compressed form ("NVFP4 vs 2:4 sparse", robertz.co, section "What 2:4 actually is"): the two
// kept codes plus a 2-bit position each. Kept positions are the nonzero codes first, then the
// lowest-index zeros, in ascending order; a failing group is written as vals 0x00 with
// positions (0, 1) and counted.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssn {

// bit 4i of the result is set when nibble i of w has zero magnitude bits
__device__ __forceinline__ uint32_t zero_nibbles(uint32_t w) {
  return ~(w | (w >> 1) | (w >> 2)) & 0x11111111u;
}

// Compress one group (16-bit word of four codes): returns vals byte | pos nibble << 8 | fail << 12
__device__ __forceinline__ uint32_t compress_group(uint32_t g) {
  const uint32_t z = zero_nibbles(g) & 0x1111u;
  // nonzero mask over the 4 positions
  const uint32_t nz = (~((z & 1u) | ((z >> 3) & 2u) | ((z >> 6) & 4u) | ((z >> 9) & 8u))) & 0xFu;
  const uint32_t cnt = __builtin_popcount(nz);
  if (cnt > 2) return 0x0u | (0x4u << 8) | (1u << 12);
  uint32_t sel = nz;
  if (cnt == 1) sel |= (~nz & 0xFu) & (0u - (~nz & 0xFu));   // add the lowest zero position
  if (cnt == 0) sel = 0x3u;                                    // two lowest zero positions
  const uint32_t i0 = __builtin_ctz(sel);
  const uint32_t i1 = 31u - __builtin_clz(sel);
  const uint32_t c0 = (g >> (4 * i0)) & 0xFu, c1 = (g >> (4 * i1)) & 0xFu;
  return (c0 | (c1 << 4)) | ((i0 | (i1 << 2)) << 8);
}

}  // namespace ssn
