// Calibration (measurement only, not part of any product path): the matrix-core rate the GPU
// sustains on register-resident operands whose bits are random, i.e. under the power limit that
// a real product's data meets. Each wave keeps NACC independent accumulators and issues
// back-to-back matrix ops on fixed operands drawn once from a hash of its lane; nothing is read
// from memory inside the loop. The published peaks assume the full clock, which random operands
// at full issue rate do not hold.
#include "common.hpp"
#include "device_once.hpp"
#include "launch.hpp"

namespace ssn {
namespace {

typedef int i32x8p __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t mix32(uint32_t x) {   // a 32-bit integer hash (xorshift-multiply)
  x ^= x >> 16; x *= 0x7feb352du; x ^= x >> 15; x *= 0x846ca68bu; x ^= x >> 16;
  return x;
}

// KIND 0: v_mfma_f32_32x32x16_bf16 on bf16 values uniform in [-0.5, 0.5);
// KIND 1: v_mfma_scale_f32_32x32x64_f8f6f4 on random E2M1 codes (scale bytes 1.0)
template <int KIND, int NACC>
__global__ __launch_bounds__(256) void k_mfma_probe(int iters, uint32_t seed, float* __restrict__ sink) {
  const uint32_t t = threadIdx.x + 977u * blockIdx.x + 131u * seed;
  f32x16 acc[NACC];
#pragma unroll
  for (int j = 0; j < NACC; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;
  if constexpr (KIND == 0) {
    u32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = (mix32(t + i) & 0x3F7F3F7Fu) ^ (mix32(t + 64 + i) & 0x80008000u);   // |x| < 1, random sign
      b[i] = (mix32(t + 31 + i) & 0x3F7F3F7Fu) ^ (mix32(t + 97 + i) & 0x80008000u);
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < NACC; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), acc[j], 0, 0, 0);
  } else {
    i32x8p a = {0, 0, 0, 0, 0, 0, 0, 0}, b = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = (int)mix32(t + i);
      b[i] = (int)mix32(t + 31 + i);
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < NACC; ++j)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], 4, 4, 0, 127, 0, 127);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NACC; ++j) s += acc[j][threadIdx.x & 15];
  sink[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_mfma_probe(int kind, int waves_per_simd, int iters, uint32_t seed, float* sink, hipStream_t s) {
  // one 256-thread workgroup puts one wave on each SIMD of a CU; the register budget allows 16
  // accumulators at one wave per SIMD and 8 at two
  const unsigned blocks = (unsigned)(cu_count() * waves_per_simd);
  if (kind == 0 && waves_per_simd == 1)
    hipLaunchKernelGGL((k_mfma_probe<0, 16>), dim3(blocks), dim3(256), 0, s, iters, seed, sink);
  else if (kind == 0)
    hipLaunchKernelGGL((k_mfma_probe<0, 8>), dim3(blocks), dim3(256), 0, s, iters, seed, sink);
  else if (waves_per_simd == 1)
    hipLaunchKernelGGL((k_mfma_probe<1, 16>), dim3(blocks), dim3(256), 0, s, iters, seed, sink);
  else
    hipLaunchKernelGGL((k_mfma_probe<1, 8>), dim3(blocks), dim3(256), 0, s, iters, seed, sink);
  return hipGetLastError();
}

}  // namespace ssn
