// 2:4 check, compress and decompress of NVFP4 codes on gfx950. HBM-bound streaming kernels:
// each lane moves 16 B of codes (32 codes = 8 groups of four) per step with a 128-bit load.
// The eligibility and compression rules themselves are in sp24_rules.hpp; the check is per
// group ("Sparse GPU FLOPS Need the Right Zeros in the Right Places", leviathansystems.co,
// section "Two half-zero vectors produce different pattern answers").
#include "common.hpp"
#include "launch.hpp"
#include "sp24_rules.hpp"

namespace ssn {
namespace {

constexpr int kThreads = 256;

__global__ void k_init_counters(int64_t* bad, int64_t* first) {
  *bad = 0;
  if (first) *first = -1;  // as uint64 this is the largest value, so atomicMin keeps real indices
}

// Block-wide sum (and min) of per-thread values; thread 0 gets the result.
__device__ __forceinline__ void block_reduce(uint32_t& cnt, uint64_t& mn) {
  for (int off = 32; off > 0; off >>= 1) {
    cnt += __shfl_xor(cnt, off, 64);
    const uint64_t o = __shfl_xor(mn, off, 64);
    mn = o < mn ? o : mn;
  }
  __shared__ uint32_t sc[kThreads / 64];
  __shared__ uint64_t sm[kThreads / 64];
  if ((threadIdx.x & 63) == 0) { sc[threadIdx.x >> 6] = cnt; sm[threadIdx.x >> 6] = mn; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kThreads / 64; ++w) { cnt += sc[w]; mn = sm[w] < mn ? sm[w] : mn; }
  }
}

// Each thread checks kUnroll chunks of 16 bytes (8 groups each), loaded together; chunks of a
// block are lane-consecutive so every load instruction is coalesced. Flat group index = byte
// offset / 2. One atomic per block (only when it found failing groups).
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kThreads) void k_check(const u32x4* codes, size_t n16, int64_t* bad,
                                                    int64_t* first) {
  const size_t base = (size_t)blockIdx.x * kThreads * kUnroll + threadIdx.x;
  u32x4 w[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const size_t i = base + (size_t)u * kThreads;
    w[u] = ld_nt(codes + (i < n16 ? i : 0));
  }
  uint32_t nbad = 0;
  uint64_t fb = ~0ull;
#pragma unroll
  for (int u = kUnroll - 1; u >= 0; --u) {
    const size_t i = base + (size_t)u * kThreads;
    if (i >= n16) continue;
    for (int d = 3; d >= 0; --d) {          // descending so the last write is the smallest index
      const uint32_t z = zero_nibbles(w[u][d]);
      const uint32_t c0 = __builtin_popcount(z & 0xFFFFu), c1 = __builtin_popcount(z >> 16);
      if (c1 < 2) { ++nbad; fb = i * 8 + 2 * d + 1; }
      if (c0 < 2) { ++nbad; fb = i * 8 + 2 * d; }
    }
  }
  block_reduce(nbad, fb);
  if (threadIdx.x == 0 && nbad) {
    atomicAdd((unsigned long long*)bad, (unsigned long long)nbad);
    if (first) atomicMin((unsigned long long*)first, (unsigned long long)fb);
  }
}

__global__ __launch_bounds__(kThreads) void k_compress(const u32x4* codes, size_t n16, u32x2* vals,
                                                       uint32_t* meta, int64_t* bad) {
  static_assert(kUnroll * 8 <= 32, "the entry sum counts the failures of at most 32 groups");
  __shared__ uint32_t lut[16];
  if (threadIdx.x < 16) lut[threadIdx.x] = compress_entry(threadIdx.x);
  const size_t base = (size_t)blockIdx.x * kThreads * kUnroll + threadIdx.x;
  u32x4 w[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const size_t i = base + (size_t)u * kThreads;
    w[u] = ld_nt(codes + (i < n16 ? i : 0));
  }
  __syncthreads();
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const size_t i = base + (size_t)u * kThreads;
    if (i >= n16) continue;
    uint32_t v[2] = {0u, 0u}, m = 0u;
#pragma unroll
    for (int d = 0; d < 4; ++d) {              // word d holds groups 2d and 2d + 1
      uint32_t v16, m8;
      compress_word(w[u][d], lut, v16, m8, acc);
      v[d >> 1] |= v16 << (16 * (d & 1));
      m |= m8 << (8 * d);
    }
    u32x2 vo; vo[0] = v[0]; vo[1] = v[1];
    vals[i] = vo;
    meta[i] = m;
  }
  uint32_t nbad = acc >> kFailShift;
  uint64_t unused = 0;
  block_reduce(nbad, unused);
  if (threadIdx.x == 0 && nbad) atomicAdd((unsigned long long*)bad, (unsigned long long)nbad);
}

__global__ __launch_bounds__(kThreads) void k_decompress(const u32x2* vals, const uint32_t* meta, size_t n16,
                                                         u32x4* codes) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n16) return;
  u32x2 v = vals[i];
  uint32_t m = meta[i];
  u32x4 out;
  for (int d = 0; d < 4; ++d) {
    uint32_t word = 0;
    for (int h = 0; h < 2; ++h) {
      const int g = 2 * d + h;
      const uint32_t vb = (v[g >> 2] >> (8 * (g & 3))) & 0xFFu;
      const uint32_t pos = (m >> (4 * g)) & 0xFu;
      const uint32_t i0 = pos & 3u, i1 = pos >> 2;
      uint32_t grp = 0;
      for (uint32_t p = 0; p < 4; ++p) {
        uint32_t c = (p == i1) ? (vb >> 4) : (p == i0) ? (vb & 0xFu) : 0u;  // i1 wins on a clash
        grp |= c << (4 * p);
      }
      word |= grp << (16 * h);
    }
    out[d] = word;
  }
  codes[i] = out;
}

inline unsigned grid_for(size_t n) { return (unsigned)((n + kThreads - 1) / kThreads); }
inline unsigned grid_unrolled(size_t n) {
  return (unsigned)((n + (size_t)kThreads * kUnroll - 1) / ((size_t)kThreads * kUnroll));
}

}  // namespace

hipError_t launch_check(const uint8_t* codes, int64_t N, int64_t K, int64_t* bad, int64_t* first,
                        hipStream_t s) {
  const size_t n16 = (size_t)N * (size_t)K / 32;  // K % 32 == 0: rows are whole 16-byte chunks
  hipLaunchKernelGGL(k_init_counters, dim3(1), dim3(1), 0, s, bad, first);
  if (n16) hipLaunchKernelGGL(k_check, dim3(grid_unrolled(n16)), dim3(kThreads), 0, s, (const u32x4*)codes, n16, bad, first);
  return hipGetLastError();
}

hipError_t launch_compress(const uint8_t* codes, int64_t N, int64_t K, uint8_t* vals, uint8_t* meta,
                           int64_t* bad, hipStream_t s) {
  const size_t n16 = (size_t)N * (size_t)K / 32;
  hipLaunchKernelGGL(k_init_counters, dim3(1), dim3(1), 0, s, bad, (int64_t*)nullptr);
  if (n16) hipLaunchKernelGGL(k_compress, dim3(grid_unrolled(n16)), dim3(kThreads), 0, s, (const u32x4*)codes, n16,
                              (u32x2*)vals, (uint32_t*)meta, bad);
  return hipGetLastError();
}

hipError_t launch_decompress(const uint8_t* vals, const uint8_t* meta, int64_t N, int64_t K, uint8_t* codes,
                             hipStream_t s) {
  const size_t n16 = (size_t)N * (size_t)K / 32;
  if (n16) hipLaunchKernelGGL(k_decompress, dim3(grid_for(n16)), dim3(kThreads), 0, s, (const u32x2*)vals,
                              (const uint32_t*)meta, n16, (u32x4*)codes);
  return hipGetLastError();
}

}  // namespace ssn
