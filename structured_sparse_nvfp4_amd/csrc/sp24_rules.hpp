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

// ---- the same rule as a 16-entry table, for the streaming kernels. Index: the nonzero
// pattern n of a group (bit i set when code i has a nonzero magnitude). Entry: bits 0-4 the
// bit offset 4 i0 of the first kept code, bits 8-12 that of the second (16 for a failing
// group: read from the group's 16 bits zero-extended, both give 0, so vals is 0x00), bits
// 16-19 the position nibble i0 | i1 << 2, bit 26 the failure flag. The fields below bit 20
// of 32 entries sum to less than 2^25, so a running sum of up to 32 entries holds its failure
// count (at most 32) in bits 26-31, clear of carries.
constexpr uint32_t kFailShift = 26;

__device__ __forceinline__ uint32_t compress_entry(uint32_t n) {
  uint32_t g = 0;
  for (int i = 0; i < 4; ++i) g |= ((n >> i) & 1u) << (4 * i);   // code 1 where nonzero, 0 elsewhere
  const uint32_t r = compress_group(g);
  const uint32_t pos = (r >> 8) & 0xFu, fail = r >> 12;
  const uint32_t o0 = fail ? 16u : 4u * (pos & 3u), o1 = fail ? 16u : 4u * (pos >> 2);
  return o0 | (o1 << 8) | (pos << 16) | (fail << kFailShift);
}

// nonzero-magnitude flags of the eight codes of w, at bits 4i
__device__ __forceinline__ uint32_t nonzero_nibbles(uint32_t w) { return (w | (w >> 1) | (w >> 2)) & 0x11111111u; }

// the flags at bits 0, 4, 8, 12 of f gathered into bits 0-3: the 24-bit product with 0x1248
// moves flag j to bit 12 + j, and every partial product of the flags at bits 0..20 lands on a
// bit of its own, so nothing carries into bits 12-15
__device__ __forceinline__ uint32_t gather_flags4(uint32_t f) { return (__umul24(f, 0x1248u) >> 12) & 0xFu; }

// Compress the two groups of the word w with table lut: vals bytes (low group in bits 0-7),
// position nibbles (low group in bits 0-3); acc collects the two entries.
__device__ __forceinline__ void compress_word(uint32_t w, const uint32_t* lut, uint32_t& vals16, uint32_t& meta8,
                                              uint32_t& acc) {
  const uint32_t nz = nonzero_nibbles(w);
  const uint32_t ea = lut[gather_flags4(nz)], eb = lut[gather_flags4(nz >> 16)];
  const uint32_t ga = w & 0xFFFFu, gb = w >> 16;
  const uint32_t va = __builtin_amdgcn_ubfe(ga, ea & 31u, 4) | (__builtin_amdgcn_ubfe(ga, (ea >> 8) & 31u, 4) << 4);
  const uint32_t vb = __builtin_amdgcn_ubfe(gb, eb & 31u, 4) | (__builtin_amdgcn_ubfe(gb, (eb >> 8) & 31u, 4) << 4);
  vals16 = va | (vb << 8);
  meta8 = ((ea >> 16) & 0xFu) | (((eb >> 16) & 0xFu) << 4);
  acc += ea + eb;
}

}  // namespace ssn
