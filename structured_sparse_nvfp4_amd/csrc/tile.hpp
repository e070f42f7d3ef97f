// Device helpers shared by the tiled matrix-core kernels (square/prefill products and the
// grouped-expert products).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace ssn {

// weight form of a tiled kernel: dense codes, or 2:4 vals + meta
enum WForm { kDense = 0, kSp24 = 1 };

// Chunk swizzle of the activation tile: eight consecutive rows (one 128-byte bank sweep each)
// and the eight same-parity rows of any sixteen get distinct chunks, so 16-byte operand reads
// of 8 or 16 lanes (rows r..r+7 or r..r+15, one chunk each) never share a bank.
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// Scheduling hint for the region just issued: LEAD matrix instructions first, then GROUPS of
// (one matrix instruction, VALU vector-ALU instructions), so the weight decode fills the
// matrix pipe's shadow instead of running ahead of or behind it.
template <int LEAD, int GROUPS, int VALU>
__device__ __forceinline__ void interleave_mfma_valu() {
  __builtin_amdgcn_sched_group_barrier(0x008, LEAD, 0);
#pragma unroll
  for (int i = 0; i < GROUPS; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x002, VALU, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  }
}

// Two kept codes (byte vb) at positions (nib & 3, nib >> 2) of a group of four nibbles.
__device__ __forceinline__ uint32_t expand_group(uint32_t vb, uint32_t nib) {
  return ((vb & 0xFu) << ((nib & 3u) << 2)) | (((vb >> 4) & 0xFu) << ((nib >> 2) << 2));
}

// Codes word of MFMA step s (8 codes, k = 8s..8s+7 of the lane's 32-wide slice)
template <int WF>
__device__ __forceinline__ uint32_t codes_step(const u32x4& w, int s) {
  if constexpr (WF == kDense) {
    return w[s];
  } else {
    const uint32_t vb = w[s >> 1] >> (16 * (s & 1));          // groups 2s, 2s+1: two vals bytes
    const uint32_t nb = w[2] >> (8 * s);                      // their two position nibbles
    return expand_group(vb & 0xFFu, nb & 0xFu) | (expand_group((vb >> 8) & 0xFFu, (nb >> 4) & 0xFu) << 16);
  }
}

__device__ __forceinline__ void store_val(void* Y, int y_bf16, size_t idx, float v) {
  if (y_bf16) ((uint16_t*)Y)[idx] = (uint16_t)f32_to_bf16_rne(v);
  else ((float*)Y)[idx] = v;
}

// Four consecutive outputs Y[m][n..n+3] (already scaled) of a row-major Y with row stride ld
// and N columns. `vec`: the piece is 16-byte (f32) or 8-byte (bf16) aligned (ld % 4 == 0 and an
// aligned Y); otherwise, and at the right edge, element by element.
__device__ __forceinline__ void store4_ld(void* Y, int y_bf16, int ld, int N, int m, int n, f32x4 v, bool vec) {
  const size_t idx = (size_t)m * ld + n;
  if (vec && n + 3 < N) {
    if (y_bf16) {
      u32x2 o;
      o[0] = pk_bf16_rne(v[0], v[1]);
      o[1] = pk_bf16_rne(v[2], v[3]);
      *(u32x2*)((uint16_t*)Y + idx) = o;
    } else {
      *(f32x4*)((float*)Y + idx) = v;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (n + i < N) store_val(Y, y_bf16, idx + i, v[i]);
  }
}

// the same for a dense row-major Y (row stride N)
__device__ __forceinline__ void store4(void* Y, int y_bf16, int N, int m, int n, f32x4 v, bool vec) {
  store4_ld(Y, y_bf16, N, N, m, n, v, vec);
}

// Eight consecutive bf16 outputs Y[m][n..n+7] of a row-major Y with row stride ld and N
// columns, packed in pairs (element 2i in the low half of v[i]). `vec`: the piece is 16-byte
// aligned (ld % 8 == 0 and an aligned Y); otherwise, and at the right edge, element by element.
__device__ __forceinline__ void store8_bf16_ld(void* Y, int ld, int N, int m, int n, u32x4 v, bool vec) {
  uint16_t* y = (uint16_t*)Y + (size_t)m * ld + n;
  if (vec && n + 7 < N) {
    *(u32x4*)y = v;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (n + i < N) y[i] = (uint16_t)(v[i >> 1] >> (16 * (i & 1)));
  }
}

// the same for a dense row-major Y (row stride N)
__device__ __forceinline__ void store8_bf16(void* Y, int N, int m, int n, u32x4 v, bool vec) {
  store8_bf16_ld(Y, N, N, m, n, v, vec);
}

}  // namespace ssn
