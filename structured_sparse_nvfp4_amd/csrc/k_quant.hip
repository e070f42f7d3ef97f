// NVFP4 quantisation, decode and 2:4 magnitude pruning on gfx950.
//
// Quantisation follows "NVFP4 Without FP4 Hardware" (ai-muninn.com), section "Convert BF16 to
// NVFP4 yourself": a tensor scale s_t = amax / (6 * 448), one E4M3 scale per 16 values along K
// and E2M1 values; a group of tensors may share s_t (section "The shared global scale").
// All rounding decisions are exact. The block scale is decided on a float64 quotient: w has 24
// significant bits and s_t * S at most 28, so a quotient that is not exactly on a grid midpoint
// is further than half a float64 ulp from it. Each E2M1 code is decided by comparing |w| with
// the midpoints times s_t * S (exact float64 products), each rounded once to f32 in the
// direction that preserves the comparison.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "sp24_rules.hpp"

namespace ssn {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float load_w(const void* W, int w_bf16, size_t i) {
  if (w_bf16) return __uint_as_float((uint32_t)((const uint16_t*)W)[i] << 16);
  return ((const float*)W)[i];
}

// ---- amax over the tensor: one pass of one-shot blocks, each reading a contiguous run of
// kThreads * kAmaxUnroll 16-byte pieces and writing its block maximum to a partial slot; the
// scale kernel reduces the partials. No accumulator has to be cleared first.
constexpr int kAmaxUnroll = 8, kAmaxIters = 1;
constexpr size_t kAmaxPiece = (size_t)kThreads * kAmaxUnroll;   // 16-byte pieces per span; a block reads kAmaxIters spans

__device__ __forceinline__ float absmax4(f32x4 v) {
  return fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
}
__device__ __forceinline__ float absmax_bf16x8(u32x4 v) {
  float m = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t) m = fmaxf(m, fmaxf(fabsf(bf16_lo(v[t])), fabsf(bf16_hi(v[t]))));
  return m;
}

__global__ __launch_bounds__(kThreads) void k_amax(const void* W, int w_bf16, size_t n, float* part) {
  const size_t per16 = w_bf16 ? 8 : 4;                       // values per 16-byte piece
  const size_t n16 = n / per16;
  const u32x4* p = (const u32x4*)W;
  float m = 0.f;
  for (int it = 0; it < kAmaxIters; ++it) {
    const size_t base = ((size_t)blockIdx.x * kAmaxIters + it) * kAmaxPiece + threadIdx.x;
    u32x4 v[kAmaxUnroll];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      const size_t i = base + (size_t)u * kThreads;
      const u32x4* q = p + (i < n16 ? i : 0);                // piece 0 again past the end: harmless for a max
      v[u] = *q;
    }
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u)
      m = fmaxf(m, w_bf16 ? absmax_bf16x8(v[u]) : absmax4(__builtin_bit_cast(f32x4, v[u])));
  }
  if (blockIdx.x == gridDim.x - 1)                           // values after the last whole piece
    for (size_t j = n16 * per16 + threadIdx.x; j < n; j += kThreads) m = fmaxf(m, fabsf(load_w(W, w_bf16, j)));
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  __shared__ float red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
    for (int k = 1; k < kThreads / 64; ++k) r = fmaxf(r, red[k]);
    part[blockIdx.x] = r;
  }
}

// s_t = fl32(amax / 2688): float64 division then conversion is the correctly rounded f32
// quotient (2688 = 2^7 * 21 and 21 is odd, so the quotient is never an f32 midpoint).
// One block: the maximum of the nparts block maxima, or ts_in when the caller gives s_t.
constexpr int kFinThreads = 1024, kFinBatch = 8;
__global__ __launch_bounds__(kFinThreads) void k_finalize_scale(const float* part, unsigned nparts, const float* ts_in,
                                                                float* ts_out) {
  if (ts_in) {
    if (threadIdx.x == 0) *ts_out = *ts_in;
    return;
  }
  float m = 0.f;
  for (unsigned i0 = 0; i0 < nparts; i0 += kFinBatch * kFinThreads) {   // one batch of loads in flight
    float v[kFinBatch];
#pragma unroll
    for (int j = 0; j < kFinBatch; ++j) {
      const unsigned i = i0 + j * kFinThreads + threadIdx.x;
      v[j] = i < nparts ? part[i] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kFinBatch; ++j) m = fmaxf(m, v[j]);
  }
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  __shared__ float red[kFinThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
    for (int k = 1; k < kFinThreads / 64; ++k) r = fmaxf(r, red[k]);
    *ts_out = (float)((double)r / 2688.0);
  }
}

// E4M3 nearest-even of q >= 0, saturating at 448 (0x7E); q is an exactly rounded float64.
__device__ __forceinline__ uint32_t e4m3_rne(double q) {
  if (!(q < 448.0)) return 0x7Eu;
  if (q < 0.015625) {                          // below 2^-6: subnormal spacing 2^-9
    double m = rint(q * 512.0);                // exact scaling; rint ties to even
    return (uint32_t)m;                        // 8 -> 0x08 (= 2^-6), still correct
  }
  int e = ilogb(q);                            // -6 .. 8
  double mant = ldexp(q, -e) - 1.0;            // [0, 1), exact
  double m8 = rint(mant * 8.0);
  if (m8 >= 8.0) { m8 = 0.0; e += 1; }
  return (uint32_t)(((e + 7) << 3) | (int)m8);
}

__device__ __forceinline__ double e4m3_f64(uint32_t b) {
  int e = (b >> 3) & 15, m = b & 7;
  return e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
}

// Per block of 16 values: S, then 16 codes packed into 8 bytes.
//
// E2M1 decision thresholds m * d (exact float64 products): ties at 0.25, 1.25, 2.5 and 5 go
// down, at 0.75, 1.75 and 3.5 up, so code = [a > 0.25d] + [a >= 0.75d] + [a > 1.25d] +
// [a >= 1.75d] + [a > 2.5d] + [a >= 3.5d] + [a > 5d]. For a float x: x > T <=> x > RD(T), and
// x >= T <=> x >= RU(T), so rounding each threshold once to f32 (down, resp. up) keeps every
// decision exact. The seven tests are evaluated as a three-level search: bit 2 of the code is
// [a >= 1.75d], bit 1 is [a >= 0.75d] or [a >= 3.5d], bit 0 the remaining test of that quarter.
struct Thresholds {
  float e175, e075, e35, g025, g125, g25, g5;
};

// The thresholds are passed by value so that they stay in registers: the quarter's threshold is
// picked with two selects, not by indexing a spilled copy of the struct.
__device__ __forceinline__ uint32_t e2m1_code(float a, float e175, float e075, float e35, float g025, float g125,
                                              float g25, float g5) {
  const bool b2 = a >= e175;
  const float t1 = b2 ? e35 : e075;
  const bool b1 = a >= t1;
  const float lo = b1 ? g125 : g025;
  const float hi = b1 ? g5 : g25;
  const bool b0 = a > (b2 ? hi : lo);
  return ((uint32_t)b2 << 2) | ((uint32_t)b1 << 1) | (uint32_t)b0;
}

// S and the 16 codes of one block.
__device__ __forceinline__ void quantize_block(const float (&w)[16], double st, u32x2& code, uint32_t& S) {
  float amax = 0.f;
#pragma unroll
  for (int t = 0; t < 16; ++t) amax = fmaxf(amax, fabsf(w[t]));
  S = 0;
  if (st > 0.0) S = e4m3_rne((double)amax / (6.0 * st));
  const double d = st * e4m3_f64(S);           // exact: <= 24 + 4 significant bits
  uint32_t lo = 0, hi = 0;                     // a block whose scale is zero stores code 0x0
  if (d > 0.0) {
    Thresholds th;
    th.g025 = __double2float_rd(0.25 * d); th.g125 = __double2float_rd(1.25 * d);
    th.g25 = __double2float_rd(2.5 * d);   th.g5 = __double2float_rd(5.0 * d);
    th.e075 = __double2float_ru(0.75 * d); th.e175 = __double2float_ru(1.75 * d);
    th.e35 = __double2float_ru(3.5 * d);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      uint32_t c = e2m1_code(fabsf(w[t]), th.e175, th.e075, th.e35, th.g025, th.g125, th.g25, th.g5);
      c |= (__float_as_uint(w[t]) >> 28) & 8u;  // sign bit -> bit 3 (keeps -0 for tiny negatives)
      if (t < 8) lo |= c << (4 * t); else hi |= c << (4 * (t - 8));
    }
  }
  code[0] = lo; code[1] = hi;
}

// A wave takes chunks of 64 blocks (4 KB of f32, 2 KB of bf16). Its loads are contiguous: load
// u of lane l reads 16-byte piece 64u + l of the chunk. An LDS transpose then hands lane b the
// whole block b, so codes (8 bytes) and scales (1 byte) leave as contiguous runs. The pieces of a
// block sit at swizzled slots x ^ sw(b), which keeps both the writes and the reads free of bank
// conflicts. Chunks are visited from the end of W backwards, so the tail that the amax pass left
// in the Infinity Cache is read first.
constexpr int kQBlocks = 64;     // blocks per wave-chunk
// chunks per wave: quantise (2 measured faster than 4 on 13824 x 5120 f32: 59 vs 63 us) and
// the fused producer (4, with more arithmetic per block)
constexpr int kQIter = 2, kPIter = 4;

template <int BF16>
__device__ __forceinline__ int q_swz(int b) {
  return BF16 ? (((b >> 2) ^ (b >> 3)) & 1) : (((b >> 1) ^ (b >> 3)) & 3);
}

template <int BF16>
__global__ __launch_bounds__(kThreads) void k_quantize(const void* W, size_t nblocks, const float* ts,
                                                       uint8_t* codes, uint8_t* scales, float* ts_copy) {
  constexpr int P = BF16 ? 2 : 4;              // 16-byte pieces per block
  __shared__ u32x4 tr[kThreads / 64][kQBlocks * P];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  u32x4* t = tr[wave];
  const size_t nchunks = (nblocks + kQBlocks - 1) / kQBlocks;
  const size_t c0 = ((size_t)blockIdx.x * (kThreads / 64) + wave) * kQIter;
  const double st = (double)*ts;
  if (ts_copy && blockIdx.x == 0 && threadIdx.x == 0) *ts_copy = (float)st;   // the caller's s_t, passed on
  for (int it = 0; it < kQIter; ++it) {
    if (c0 + it >= nchunks) break;                               // uniform per wave
    const size_t b0 = (nchunks - 1 - (c0 + it)) * kQBlocks;      // first block of the chunk
    const u32x4* src = (const u32x4*)W + b0 * P;
    u32x4 v[P];
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const int p = 64 * u + lane;
      v[u] = b0 + p / P < nblocks ? ld_nt(src + p) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const int p = 64 * u + lane, b = p / P;
      t[b * P + ((p % P) ^ q_swz<BF16>(b))] = v[u];
    }
    __asm__ volatile("" ::: "memory");          // this wave's LDS reads stay after its writes
    float w[16];
#pragma unroll
    for (int x = 0; x < P; ++x) {
      const u32x4 r = t[lane * P + (x ^ q_swz<BF16>(lane))];
      if (BF16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) { w[8 * x + 2 * e] = bf16_lo(r[e]); w[8 * x + 2 * e + 1] = bf16_hi(r[e]); }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) w[4 * x + e] = __uint_as_float(r[e]);
      }
    }
    __asm__ volatile("" ::: "memory");          // ... and before the next chunk's writes
    if (b0 + lane < nblocks) {
      u32x2 code;
      uint32_t S;
      quantize_block(w, st, code, S);
      *(u32x2*)(codes + (b0 + lane) * 8) = code;
      scales[b0 + lane] = (uint8_t)S;
    }
  }
}

// ---- fused 2:4 producer: prune -> quantise -> compress in one pass over W.
// ("NVFP4 vs 2:4 sparse", robertz.co, section "Where it is supported in software": the tool that
// pruned and packed 2:4 checkpoints was withdrawn; "NVFP4 Without FP4 Hardware", ai-muninn.com,
// section "Convert BF16 to NVFP4 yourself".) The result is bit-identical to sp24_prune, then
// nvfp4_quantize, then sp24_compress:
//  - pruning keeps the two largest |w| of every group of four, so the largest |w| of any block
//    of 16 and of the whole tensor survives: the tensor scale and every block scale equal those
//    of the unpruned tensor, and the amax pass runs on W itself;
//  - the pruned entries become +0.0 (code 0x0) before the block is quantised exactly as in
//    k_quantize, and each group's four codes are compressed by the shared 2:4 rule (which still
//    decides, so a kept value that rounds to zero is handled as compress would).
// Layout and traversal as k_quantize (wave chunks of 64 blocks, LDS transpose, lane = block).
// Per block: vals 4 bytes, meta 2 bytes, scale 1 byte, and (optional) the 8 code bytes of the
// pruned tensor. A group that still has fewer than two zero codes (impossible after pruning) is
// counted in *bad like sp24_compress does.
template <int BF16>
__global__ __launch_bounds__(kThreads) void k_produce24(const void* W, size_t nblocks, const float* ts,
                                                        uint8_t* vals, uint8_t* meta, uint8_t* scales,
                                                        uint8_t* codes, int64_t* bad, float* ts_copy) {
  constexpr int P = BF16 ? 2 : 4;              // 16-byte pieces per block
  __shared__ u32x4 tr[kThreads / 64][kQBlocks * P];
  __shared__ uint32_t lut[16];                 // the 2:4 compression table
  if (threadIdx.x < 16) lut[threadIdx.x] = compress_entry(threadIdx.x);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  u32x4* t = tr[wave];
  const size_t nchunks = (nblocks + kQBlocks - 1) / kQBlocks;
  const size_t c0 = ((size_t)blockIdx.x * (kThreads / 64) + wave) * kPIter;
  const double st = (double)*ts;
  if (ts_copy && blockIdx.x == 0 && threadIdx.x == 0) *ts_copy = (float)st;   // the caller's s_t, passed on
  uint32_t nbad = 0;
  for (int it = 0; it < kPIter; ++it) {
    if (c0 + it >= nchunks) break;                               // uniform per wave
    const size_t b0 = (nchunks - 1 - (c0 + it)) * kQBlocks;      // first block of the chunk
    const u32x4* src = (const u32x4*)W + b0 * P;
    u32x4 v[P];
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const int p = 64 * u + lane;
      v[u] = b0 + p / P < nblocks ? ld_nt(src + p) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const int p = 64 * u + lane, b = p / P;
      t[b * P + ((p % P) ^ q_swz<BF16>(b))] = v[u];
    }
    __asm__ volatile("" ::: "memory");
    float w[16];
#pragma unroll
    for (int x = 0; x < P; ++x) {
      const u32x4 r = t[lane * P + (x ^ q_swz<BF16>(lane))];
      if (BF16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) { w[8 * x + 2 * e] = bf16_lo(r[e]); w[8 * x + 2 * e + 1] = bf16_hi(r[e]); }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) w[4 * x + e] = __uint_as_float(r[e]);
      }
    }
    __asm__ volatile("" ::: "memory");
    if (b0 + lane < nblocks) {
      // prune: entry i of a group is dropped when two entries outrank it (|w_j| > |w_i|, or equal
      // with j < i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = fabsf(w[4 * g + i]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int outrank = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) outrank += (a[j] > a[i]) || (a[j] == a[i] && j < i);
          if (outrank >= 2) w[4 * g + i] = 0.0f;
        }
      }
      u32x2 code;
      uint32_t S;
      quantize_block(w, st, code, S);
      const size_t b = b0 + lane;
      uint32_t v0, v1, m0, m1, acc = 0;
      compress_word(code[0], lut, v0, m0, acc);
      compress_word(code[1], lut, v1, m1, acc);
      nbad += acc >> kFailShift;
      const uint32_t vw = v0 | (v1 << 16), mw = m0 | (m1 << 8);
      *(uint32_t*)(vals + b * 4) = vw;
      *(uint16_t*)(meta + b * 2) = (uint16_t)mw;
      scales[b] = (uint8_t)S;
      if (codes) *(u32x2*)(codes + b * 8) = code;
    }
  }
  for (int off = 32; off > 0; off >>= 1) nbad += __shfl_xor(nbad, off, 64);
  if (lane == 0 && nbad) atomicAdd((unsigned long long*)bad, (unsigned long long)nbad);
}

// double -> f32 rounded to odd: truncate, then set the last bit if anything was dropped. A
// later rounding to bf16 (16 fewer bits) is then the correctly rounded bf16 of the double.
__device__ __forceinline__ float to_f32_round_odd(double x) {
  float t = __double2float_rz(x);
  if ((double)t != x) t = __uint_as_float(__float_as_uint(t) | 1u);
  return t;
}

// Decode: one thread per block of 16. f32 output: the exact product e2m1 * S times s_t, rounded
// once. bf16 output: the exact float64 product rounded once to bf16 (via round-to-odd f32).
__global__ __launch_bounds__(kThreads) void k_dequantize(const uint8_t* codes, const uint8_t* scales,
                                                         const float* ts, size_t nblocks, void* out,
                                                         int out_bf16) {
  size_t b = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  u32x2 c = *(const u32x2*)(codes + b * 8);
  const float s = e4m3_f32(scales[b]);
  const float st = *ts;
  float v[16];
  for (int h = 0; h < 2; ++h) {
    f32x2 p0 = fp4x2_f32<0>(c[h]), p1 = fp4x2_f32<1>(c[h]), p2 = fp4x2_f32<2>(c[h]), p3 = fp4x2_f32<3>(c[h]);
    float* o = v + 8 * h;
    o[0] = p0[0]; o[1] = p0[1]; o[2] = p1[0]; o[3] = p1[1]; o[4] = p2[0]; o[5] = p2[1]; o[6] = p3[0]; o[7] = p3[1];
  }
  if (!out_bf16) {
    f32x4* o = (f32x4*)((float*)out + b * 16);
    for (int t = 0; t < 4; ++t) {
      f32x4 r;
      for (int u = 0; u < 4; ++u) r[u] = (v[4 * t + u] * s) * st;  // e2m1*S exact, then one rounding
      o[t] = r;
    }
  } else {
    u32x4* o = (u32x4*)((uint16_t*)out + b * 16);
    for (int t = 0; t < 2; ++t) {
      u32x4 r;
      for (int u = 0; u < 4; ++u) {
        float a = to_f32_round_odd((double)(v[8 * t + 2 * u] * s) * (double)st);
        float c2 = to_f32_round_odd((double)(v[8 * t + 2 * u + 1] * s) * (double)st);
        r[u] = pk_bf16_rne(a, c2);
      }
      o[t] = r;
    }
  }
}

// 2:4 magnitude prune of one group of four held as raw bits (f32: u32x4, bf16: u32x2), in
// place. Entry i is kept when fewer than two entries outrank it, where j outranks i if
// |w_j| > |w_i|, or |w_j| == |w_i| and j < i. Returns the group's largest magnitude (NaN
// entries ignored, as in k_amax).
template <int BF16>
__device__ __forceinline__ float prune_group(typename std::conditional<BF16 != 0, u32x2, u32x4>::type& v) {
  float a[4];
  uint32_t raw[4];
  if (!BF16) {
    for (int i = 0; i < 4; ++i) { raw[i] = v[i]; a[i] = fabsf(__uint_as_float(v[i])); }
  } else {
    raw[0] = v[0] & 0xFFFFu; raw[1] = v[0] >> 16; raw[2] = v[1] & 0xFFFFu; raw[3] = v[1] >> 16;
    for (int i = 0; i < 4; ++i) a[i] = fabsf(__uint_as_float(raw[i] << 16));
  }
  for (int i = 0; i < 4; ++i) {
    int outrank = 0;
    for (int j = 0; j < 4; ++j) outrank += (a[j] > a[i]) || (a[j] == a[i] && j < i);
    if (outrank >= 2) raw[i] = 0u;
  }
  if (!BF16) {
    for (int i = 0; i < 4; ++i) v[i] = raw[i];
  } else {
    v[0] = raw[0] | (raw[1] << 16); v[1] = raw[2] | (raw[3] << 16);
  }
  return fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3]));
}

// Blocks stride over tiles of kThreads * U groups; in a tile every thread issues its U loads
// before it prunes and stores any of them. The plain prune runs one group per thread and one
// block per tile. With AMAX the block also folds the maximum |w| it saw into *amax_bits
// (cleared beforehand) with one atomic max; for non-negative floats the order of the bit
// patterns is the order of the values. Pruning keeps the largest entry of every group, so that
// is the maximum of the pruned tensor too. Atomics on one address are serialised, so the AMAX
// form runs a capped grid (kPruneAmaxGrid blocks) that strides over the tiles. Measured on
// 13824 x 5120 f32: one group per thread 94 us without the maximum; with it, 4 groups per
// thread on 2048 blocks 105 us (one block per tile: 69120 atomics, 795 us).
constexpr int kPruneAmaxUnroll = 4;
constexpr unsigned kPruneAmaxGrid = 2048;
template <int BF16, bool AMAX, int U>
__global__ __launch_bounds__(kThreads) void k_prune(const void* W, size_t ngroups, void* out, unsigned* amax_bits) {
  using V = typename std::conditional<BF16 != 0, u32x2, u32x4>::type;
  constexpr size_t tile = (size_t)kThreads * U;
  float m = 0.f;
  for (size_t base = (size_t)blockIdx.x * tile + threadIdx.x; base < ngroups; base += (size_t)gridDim.x * tile) {
    V v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t g = base + (size_t)u * kThreads;
      if (g < ngroups) v[u] = ((const V*)W)[g];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t g = base + (size_t)u * kThreads;
      if (g < ngroups) {
        m = fmaxf(m, prune_group<BF16>(v[u]));
        ((V*)out)[g] = v[u];
      }
    }
  }
  if (!AMAX) return;
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  __shared__ float red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
    for (int k = 1; k < kThreads / 64; ++k) r = fmaxf(r, red[k]);
    atomicMax(amax_bits, __float_as_uint(r));
  }
}

__global__ void k_zero_u32(unsigned* p) { *p = 0u; }

// In place: the maximum's bits -> s_t = fl32(amax / 2688), the rule of k_finalize_scale.
__global__ void k_scale_of_amax(float* ts) { *ts = (float)((double)*ts / 2688.0); }

__global__ void k_zero_i64(int64_t* p) { *p = 0; }

inline unsigned grid_for(size_t n, int per_block) { return (unsigned)((n + per_block - 1) / per_block); }

}  // namespace

hipError_t launch_quantize(const void* W, int w_bf16, int64_t N, int64_t K, const float* ts_in,
                           uint8_t* codes, uint8_t* scales, float* ts_out, hipStream_t s) {
  const size_t n = (size_t)N * (size_t)K;
  // The block maxima are parked in the codes output (N*K/2 bytes >= 4 bytes per amax block for
  // any K % 16 == 0 tensor); the quantisation kernel overwrites them afterwards.
  float* part = (float*)codes;
  unsigned nparts = 0;
  if (!ts_in && n) {                               // an empty tensor has no maximum: s_t = 0
    const size_t n16 = n / (w_bf16 ? 8 : 4);
    nparts = (unsigned)std::max<size_t>(1, (n16 + kAmaxPiece * kAmaxIters - 1) / (kAmaxPiece * kAmaxIters));
    hipLaunchKernelGGL(k_amax, dim3(nparts), dim3(kThreads), 0, s, W, w_bf16, n, part);
  }
  const size_t nb = n / 16;
  // with the caller's s_t and blocks to quantise, the quantisation kernel passes s_t on itself
  const bool pass_on = ts_in && nb;
  if (!pass_on)
    hipLaunchKernelGGL(k_finalize_scale, dim3(1), dim3(kFinThreads), 0, s, (const float*)part, nparts, ts_in, ts_out);
  const float* st = pass_on ? ts_in : ts_out;
  float* copy = pass_on ? ts_out : nullptr;
  if (nb) {
    const size_t waves = ((nb + kQBlocks - 1) / kQBlocks + kQIter - 1) / kQIter;
    const dim3 grid(grid_for(waves, kThreads / 64));
    if (w_bf16)
      hipLaunchKernelGGL(k_quantize<1>, grid, dim3(kThreads), 0, s, W, nb, st, codes, scales, copy);
    else
      hipLaunchKernelGGL(k_quantize<0>, grid, dim3(kThreads), 0, s, W, nb, st, codes, scales, copy);
  }
  return hipGetLastError();
}

hipError_t launch_produce24(const void* W, int w_bf16, int64_t N, int64_t K, const float* ts_in, uint8_t* vals,
                            uint8_t* meta, uint8_t* scales, float* ts_out, uint8_t* codes, int64_t* bad,
                            hipStream_t s) {
  const size_t n = (size_t)N * (size_t)K;
  // block maxima parked in the vals output (N*K/4 bytes, >= 4 bytes per amax block)
  float* part = (float*)vals;
  unsigned nparts = 0;
  if (!ts_in && n) {
    const size_t n16 = n / (w_bf16 ? 8 : 4);
    nparts = (unsigned)std::max<size_t>(1, (n16 + kAmaxPiece * kAmaxIters - 1) / (kAmaxPiece * kAmaxIters));
    hipLaunchKernelGGL(k_amax, dim3(nparts), dim3(kThreads), 0, s, W, w_bf16, n, part);
  }
  const size_t nb = n / 16;
  const bool pass_on = ts_in && nb;              // as in launch_quantize
  if (!pass_on)
    hipLaunchKernelGGL(k_finalize_scale, dim3(1), dim3(kFinThreads), 0, s, (const float*)part, nparts, ts_in, ts_out);
  hipLaunchKernelGGL(k_zero_i64, dim3(1), dim3(1), 0, s, bad);
  const float* st = pass_on ? ts_in : ts_out;
  float* copy = pass_on ? ts_out : nullptr;
  if (nb) {
    const size_t waves = ((nb + kQBlocks - 1) / kQBlocks + kPIter - 1) / kPIter;
    const dim3 grid(grid_for(waves, kThreads / 64));
    if (w_bf16)
      hipLaunchKernelGGL(k_produce24<1>, grid, dim3(kThreads), 0, s, W, nb, st, vals, meta, scales, codes, bad, copy);
    else
      hipLaunchKernelGGL(k_produce24<0>, grid, dim3(kThreads), 0, s, W, nb, st, vals, meta, scales, codes, bad, copy);
  }
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* ts, int64_t N,
                             int64_t K, void* out, int out_bf16, hipStream_t s) {
  const size_t nb = (size_t)N * (size_t)K / 16;
  hipLaunchKernelGGL(k_dequantize, dim3(grid_for(nb, kThreads)), dim3(kThreads), 0, s, codes, scales, ts,
                     nb, out, out_bf16);
  return hipGetLastError();
}

hipError_t launch_prune(const void* W, int w_bf16, int64_t N, int64_t K, void* out, float* ts_out, hipStream_t s) {
  const size_t ng = (size_t)N * (size_t)K / 4;
  unsigned* amax = (unsigned*)ts_out;
  if (ts_out) hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(1), 0, s, amax);
  if (ng && !ts_out) {
    const dim3 grid(grid_for(ng, kThreads));
    if (w_bf16) hipLaunchKernelGGL((k_prune<1, false, 1>), grid, dim3(kThreads), 0, s, W, ng, out, amax);
    else hipLaunchKernelGGL((k_prune<0, false, 1>), grid, dim3(kThreads), 0, s, W, ng, out, amax);
  } else if (ng) {
    const dim3 grid(std::min(grid_for(ng, kThreads * kPruneAmaxUnroll), kPruneAmaxGrid));
    if (w_bf16)
      hipLaunchKernelGGL((k_prune<1, true, kPruneAmaxUnroll>), grid, dim3(kThreads), 0, s, W, ng, out, amax);
    else
      hipLaunchKernelGGL((k_prune<0, true, kPruneAmaxUnroll>), grid, dim3(kThreads), 0, s, W, ng, out, amax);
  }
  if (ts_out) hipLaunchKernelGGL(k_scale_of_amax, dim3(1), dim3(1), 0, s, ts_out);
  return hipGetLastError();
}

}  // namespace ssn
