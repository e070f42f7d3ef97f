// Decode-shaped products (M <= 16 activation rows) and the plain vector-ALU products.
//
// Decode is bound by the weight read ("NVFP4 vs 2:4 sparse", robertz.co, section "Where a
// decode step actually spends itself"), so these kernels stream the 4-bit weights once with
// 128-bit loads, decode them in registers ("NVFP4 Without FP4 Hardware", ai-muninn.com,
// section "Why NVFP4 helps without FP4 hardware") and hand them to the matrix cores with the
// weights as the 16-row A operand and the (zero-padded) activations as the 16-column B operand,
// so that even M = 1..16 costs one MFMA per 16x16x32 (dense) or 16x16x64 (2:4) slice.
//
// gfx950 operand layouts used here (lane l, r = l % 16, q = l / 16):
//  v_mfma_f32_16x16x32_bf16   A: row r, k = 8q..8q+7;  B: col r, k = 8q..8q+7;
//                             D: rows 4q..4q+3, col r.
//  v_smfmac_f32_16x16x64_bf16 A (compressed): row r, 8 kept values of the four groups covering
//                             k = 16q..16q+15, kept value j at group j/2; its position in the
//                             group is index bits [2j+1:2j] (the abid operand selects the low or
//                             high 16 bits of the index register);
//                             B: col r, k = 8q..8q+7 then 32+8q..32+8q+7;  D as above.
// The compressed layout of this library (vals byte = two kept codes, meta nibble = i0 | i1 << 2)
// is therefore the SMFMAC A operand and index operand as stored: no permutation.
#include "common.hpp"
#include "launch.hpp"

namespace ssn {
namespace {

constexpr int kWaves = 4;

__device__ __forceinline__ u32x4 zero4() { u32x4 z = {0u, 0u, 0u, 0u}; return z; }

// Epilogue for a 16x16 D tile: lane (m = l%16, q = l/16) holds Y[m][n0+4q .. n0+4q+3].
// The per-wave partials are summed through LDS first.
__device__ __forceinline__ void store_tile16(f32x4 acc, float* red, int M, int N, int n0, float st,
                                             void* Y, int y_bf16) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = 0; i < 4; ++i) red[(wave * 4 + i) * 64 + lane] = acc[i];
  __syncthreads();
  if (wave != 0) return;
  f32x4 s;
  for (int i = 0; i < 4; ++i) {
    float v = 0.f;
    for (int w = 0; w < kWaves; ++w) v += red[(w * 4 + i) * 64 + lane];
    s[i] = v * st;
  }
  const int m = lane & 15, n = n0 + 4 * (lane >> 4);
  if (m >= M) return;
  if (!y_bf16) {
    float* y = (float*)Y + (size_t)m * N + n;
    if (n + 3 < N && ((N & 3) == 0)) {
      *(f32x4*)y = s;
    } else {
      for (int i = 0; i < 4; ++i) if (n + i < N) y[i] = s[i];
    }
  } else {
    uint16_t* y = (uint16_t*)Y + (size_t)m * N + n;
    if (n + 3 < N && ((N & 3) == 0)) {
      u32x2 o; o[0] = f32_to_bf16_rne(s[0]) | (f32_to_bf16_rne(s[1]) << 16);
      o[1] = f32_to_bf16_rne(s[2]) | (f32_to_bf16_rne(s[3]) << 16);
      *(u32x2*)y = o;
    } else {
      for (int i = 0; i < 4; ++i) if (n + i < N) y[i] = (uint16_t)f32_to_bf16_rne(s[i]);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Dense, M <= 16. One block = 16 weight rows; the 4 waves split K in 128-wide slices
// (lane group q takes 32 consecutive k of the slice: 16 B of codes, 2 scale bytes).
// SRC_SP24: the weights come as vals+meta and are expanded to dense codes in registers first
// (the decompress-then-dense-MFMA variant of the 2:4 product).
template <bool SRC_SP24>
__global__ __launch_bounds__(256) void k_gemv_mfma(const uint16_t* __restrict__ X, int M, int N, int K,
                                                   const uint8_t* __restrict__ w0, const uint8_t* __restrict__ w1,
                                                   const uint8_t* __restrict__ scales, const float* __restrict__ ts,
                                                   void* __restrict__ Y, int y_bf16) {
  __shared__ float red[kWaves * 4 * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int n = min(n0 + r, N - 1);
  const bool xv = r < M;
  const uint16_t* xrow = X + (size_t)(xv ? r : 0) * K;
  const uint8_t* srow = scales + (size_t)n * (K / 16);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int nslices = (K + 127) / 128;
  for (int c = wave; c < nslices; c += kWaves) {
    const int k = c * 128 + 32 * q;
    u32x4 cw = zero4();
    uint32_t sw = 0;
    u32x4 xw[4] = {zero4(), zero4(), zero4(), zero4()};
    if (k < K) {
      if constexpr (!SRC_SP24) {
        cw = ld_nt((const u32x4*)(w0 + (size_t)n * (K / 2) + k / 2));
      } else {
        // 8 groups: 8 vals bytes + 4 meta bytes -> 32 dense codes
        const u32x2 v = ld_nt((const u32x2*)(w0 + (size_t)n * (K / 4) + k / 4));
        const uint32_t mt = ld_nt((const uint32_t*)(w1 + (size_t)n * (K / 8) + k / 8));
        for (int g = 0; g < 8; ++g) {
          const uint32_t vb = (v[g >> 2] >> (8 * (g & 3))) & 0xFFu;
          const uint32_t pos = (mt >> (4 * g)) & 0xFu;
          const uint32_t grp = ((vb & 0xFu) << (4 * (pos & 3u))) | ((vb >> 4) << (4 * (pos >> 2)));
          cw[g >> 1] |= grp << (16 * (g & 1));
        }
      }
      sw = *(const uint16_t*)(srow + k / 16);
      if (xv) {
        const u32x4* xp = (const u32x4*)(xrow + k);
        xw[0] = xp[0]; xw[1] = xp[1]; xw[2] = xp[2]; xw[3] = xp[3];
      }
    }
    const float s0 = e4m3_f32_sel<0>(sw), s1 = e4m3_f32_sel<1>(sw);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 a = fp4x8_bf16(cw[j], j < 2 ? s0 : s1);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(xw[j]), acc, 0, 0, 0);
    }
  }
  store_tile16(acc, red, M, N, n0, *ts, Y, y_bf16);
}

// ---------------------------------------------------------------------------------------------
// 2:4, M <= 16, sparse MFMA. One block = 16 weight rows; waves split K in 256-wide slices.
// Lane group q of a slice takes 16 consecutive groups (64 k): 16 B vals, 8 B meta, 4 B scales,
// feeding four v_smfmac_f32_16x16x64_bf16 (j = 0..3). For SMFMAC j the instruction's k index
// kappa = 16q + t maps to k = slice + 64q + 16j + t, so the B lane (col r, group q) needs the
// activations at slice + 64(q>>1) + 16j + 8(q&1) (+8 contiguous) and the same +128.
__global__ __launch_bounds__(256) void k_gemv_smfmac(const uint16_t* __restrict__ X, int M, int N, int K,
                                                     const uint8_t* __restrict__ vals, const uint8_t* __restrict__ meta,
                                                     const uint8_t* __restrict__ scales, const float* __restrict__ ts,
                                                     void* __restrict__ Y, int y_bf16) {
  __shared__ float red[kWaves * 4 * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int n = min(n0 + r, N - 1);
  const bool xv = r < M;
  const uint16_t* xrow = X + (size_t)(xv ? r : 0) * K;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int nslices = (K + 255) / 256;
  for (int c = wave; c < nslices; c += kWaves) {
    const int kbase = c * 256;
    const int k = kbase + 64 * q;                 // this lane's weight k range [k, k+64)
    u32x4 vw = zero4();
    u32x2 mw; mw[0] = 0u; mw[1] = 0u;
    uint32_t sw = 0;
    if (k < K) {
      vw = ld_nt((const u32x4*)(vals + (size_t)n * (K / 4) + k / 4));
      mw = ld_nt((const u32x2*)(meta + (size_t)n * (K / 8) + k / 8));
      sw = ld_nt((const uint32_t*)(scales + (size_t)n * (K / 16) + k / 16));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x8 b;
      const int kb = kbase + 64 * (q >> 1) + 16 * j + 8 * (q & 1);
      u32x4 lo = zero4(), hi = zero4();
      if (xv && kb < K) lo = *(const u32x4*)(xrow + kb);
      if (xv && kb + 128 < K) hi = *(const u32x4*)(xrow + kb + 128);
      b[0] = lo[0]; b[1] = lo[1]; b[2] = lo[2]; b[3] = lo[3];
      b[4] = hi[0]; b[5] = hi[1]; b[6] = hi[2]; b[7] = hi[3];
      const float s = j == 0 ? e4m3_f32_sel<0>(sw) : j == 1 ? e4m3_f32_sel<1>(sw)
                    : j == 2 ? e4m3_f32_sel<2>(sw) : e4m3_f32_sel<3>(sw);
      const u32x4 a = fp4x8_bf16(vw[j], s);
      if (j < 2)
        acc = (j == 0) ? __builtin_amdgcn_smfmac_f32_16x16x64_bf16(as_bf16x8(a), as_bf16x16(b), acc, (int)mw[0], 0, 0)
                       : __builtin_amdgcn_smfmac_f32_16x16x64_bf16(as_bf16x8(a), as_bf16x16(b), acc, (int)mw[0], 0, 1);
      else
        acc = (j == 2) ? __builtin_amdgcn_smfmac_f32_16x16x64_bf16(as_bf16x8(a), as_bf16x16(b), acc, (int)mw[1], 0, 0)
                       : __builtin_amdgcn_smfmac_f32_16x16x64_bf16(as_bf16x8(a), as_bf16x16(b), acc, (int)mw[1], 0, 1);
    }
  }
  store_tile16(acc, red, M, N, n0, *ts, Y, y_bf16);
}

// ---------------------------------------------------------------------------------------------
// Vector-ALU products, any M, K % 32 == 0. One wave per weight row n and block of 16
// activation rows; lanes stride over 32-wide K chunks; f32 FMAs; a wave reduction at the end.
// Dense: every weight is multiplied. 2:4 (skip-and-gather): only the two kept values of each
// group are multiplied, each with the activation gathered at its stored position.
constexpr int kRowsPerWave = 16;

template <bool SP24>
__global__ __launch_bounds__(256) void k_gemm_valu(const uint16_t* __restrict__ X, int M, int N, int K,
                                                   const uint8_t* __restrict__ w0, const uint8_t* __restrict__ w1,
                                                   const uint8_t* __restrict__ scales, const float* __restrict__ ts,
                                                   void* __restrict__ Y, int y_bf16) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = blockIdx.x * kWaves + wave;
  const int m0 = blockIdx.y * kRowsPerWave;
  if (n >= N) return;
  float acc[kRowsPerWave];
  for (int i = 0; i < kRowsPerWave; ++i) acc[i] = 0.f;
  const int mcount = min(kRowsPerWave, M - m0);
  for (int c = lane; c < K / 32; c += 64) {
    const int k = c * 32;
    const uint16_t sw = *(const uint16_t*)(scales + (size_t)n * (K / 16) + k / 16);
    const float s0 = e4m3_f32_sel<0>(sw), s1 = e4m3_f32_sel<1>(sw);
    if constexpr (!SP24) {
      const u32x4 cw = *(const u32x4*)(w0 + (size_t)n * (K / 2) + k / 2);
      float w[32];
      for (int d = 0; d < 4; ++d) {
        const float s = d < 2 ? s0 : s1;
        f32x2 p0 = fp4x2_f32<0>(cw[d]), p1 = fp4x2_f32<1>(cw[d]), p2 = fp4x2_f32<2>(cw[d]), p3 = fp4x2_f32<3>(cw[d]);
        w[8 * d + 0] = p0[0] * s; w[8 * d + 1] = p0[1] * s; w[8 * d + 2] = p1[0] * s; w[8 * d + 3] = p1[1] * s;
        w[8 * d + 4] = p2[0] * s; w[8 * d + 5] = p2[1] * s; w[8 * d + 6] = p3[0] * s; w[8 * d + 7] = p3[1] * s;
      }
      for (int i = 0; i < mcount; ++i) {
        const u32x4* xp = (const u32x4*)(X + (size_t)(m0 + i) * K + k);
        float a = acc[i];
        for (int t = 0; t < 4; ++t) {
          const u32x4 xv = xp[t];
          for (int u = 0; u < 4; ++u) {
            a = fmaf(bf16_lo(xv[u]), w[8 * t + 2 * u], a);
            a = fmaf(bf16_hi(xv[u]), w[8 * t + 2 * u + 1], a);
          }
        }
        acc[i] = a;
      }
    } else {
      // 8 groups of this chunk: 8 vals bytes (16 kept codes), 4 meta bytes (positions)
      const u32x2 v = *(const u32x2*)(w0 + (size_t)n * (K / 4) + k / 4);
      const uint32_t mt = *(const uint32_t*)(w1 + (size_t)n * (K / 8) + k / 8);
      float w[16];
      int kk[16];
      for (int d = 0; d < 2; ++d) {
        f32x2 p0 = fp4x2_f32<0>(v[d]), p1 = fp4x2_f32<1>(v[d]), p2 = fp4x2_f32<2>(v[d]), p3 = fp4x2_f32<3>(v[d]);
        const float s = d == 0 ? s0 : s1;     // groups 0..3 -> k 0..15 (block 0), 4..7 -> block 1
        w[8 * d + 0] = p0[0] * s; w[8 * d + 1] = p0[1] * s; w[8 * d + 2] = p1[0] * s; w[8 * d + 3] = p1[1] * s;
        w[8 * d + 4] = p2[0] * s; w[8 * d + 5] = p2[1] * s; w[8 * d + 6] = p3[0] * s; w[8 * d + 7] = p3[1] * s;
      }
      for (int g = 0; g < 8; ++g) {
        const uint32_t pos = (mt >> (4 * g)) & 0xFu;
        kk[2 * g] = k + 4 * g + (int)(pos & 3u);
        kk[2 * g + 1] = k + 4 * g + (int)(pos >> 2);
      }
      for (int i = 0; i < mcount; ++i) {
        const uint16_t* xr = X + (size_t)(m0 + i) * K;
        float a = acc[i];
        for (int t = 0; t < 16; ++t) a = fmaf(__uint_as_float((uint32_t)xr[kk[t]] << 16), w[t], a);
        acc[i] = a;
      }
    }
  }
  const float st = *ts;
  for (int i = 0; i < kRowsPerWave; ++i) {
    float a = acc[i];
    for (int off = 32; off > 0; off >>= 1) a += __shfl_xor(a, off, 64);
    acc[i] = a * st;
  }
  if (lane < mcount) {
    float v = 0.f;
    for (int i = 0; i < kRowsPerWave; ++i) v = (lane == i) ? acc[i] : v;
    const size_t o = (size_t)(m0 + lane) * N + n;
    if (!y_bf16) ((float*)Y)[o] = v;
    else ((uint16_t*)Y)[o] = (uint16_t)f32_to_bf16_rne(v);
  }
}

}  // namespace

hipError_t launch_gemv_dense_mfma(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_gemv_mfma<false>, dim3((unsigned)((a.N + 15) / 16)), dim3(256), 0, s, a.X, (int)a.M,
                     (int)a.N, (int)a.K, a.w0, a.w1, a.scales, a.ts, a.Y, a.y_bf16);
  return hipGetLastError();
}

hipError_t launch_gemv_sp24_decomp(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_gemv_mfma<true>, dim3((unsigned)((a.N + 15) / 16)), dim3(256), 0, s, a.X, (int)a.M,
                     (int)a.N, (int)a.K, a.w0, a.w1, a.scales, a.ts, a.Y, a.y_bf16);
  return hipGetLastError();
}

hipError_t launch_gemv_sp24_smfmac(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_gemv_smfmac, dim3((unsigned)((a.N + 15) / 16)), dim3(256), 0, s, a.X, (int)a.M,
                     (int)a.N, (int)a.K, a.w0, a.w1, a.scales, a.ts, a.Y, a.y_bf16);
  return hipGetLastError();
}

hipError_t launch_gemm_dense_valu(const GemmArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.N + kWaves - 1) / kWaves), (unsigned)((a.M + kRowsPerWave - 1) / kRowsPerWave));
  hipLaunchKernelGGL(k_gemm_valu<false>, grid, dim3(256), 0, s, a.X, (int)a.M, (int)a.N, (int)a.K, a.w0, a.w1,
                     a.scales, a.ts, a.Y, a.y_bf16);
  return hipGetLastError();
}

hipError_t launch_gemm_sp24_valu(const GemmArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.N + kWaves - 1) / kWaves), (unsigned)((a.M + kRowsPerWave - 1) / kRowsPerWave));
  hipLaunchKernelGGL(k_gemm_valu<true>, grid, dim3(256), 0, s, a.X, (int)a.M, (int)a.N, (int)a.K, a.w0, a.w1,
                     a.scales, a.ts, a.Y, a.y_bf16);
  return hipGetLastError();
}

}  // namespace ssn
