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
#include <algorithm>

#include "common.hpp"
#include "device_once.hpp"
#include "launch.hpp"
#include "pipeline.hpp"

namespace ssn {
namespace {

constexpr int kWaves = 4;
// Post-scale decode slabs: up to this many workgroups per CU, one 32-row group each, so that the
// hardware starts a new group's loads while other groups on the CU finish (vocabulary-sized N
// measured 11% faster than two workgroups looping over their groups).
// 32 zero bytes: activation loads of K-slices outside the problem read here, so that the weights
// loaded (from a clamped, valid address) for those slices are multiplied by zero.
__device__ __attribute__((aligned(16))) uint32_t g_zero32[8];
// Slices in flight per wave (ring depth).
constexpr int kDenseRing = 2;    // 128-wide slices (dense)
constexpr int kSparseRing = 1;  // 256-wide slices (2:4)

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
      u32x2 o; o[0] = pk_bf16_rne(s[0], s[1]);
      o[1] = pk_bf16_rne(s[2], s[3]);
      *(u32x2*)y = o;
    } else {
      for (int i = 0; i < 4; ++i) if (n + i < N) y[i] = (uint16_t)f32_to_bf16_rne(s[i]);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Dense, M <= 16. One block = 16 weight rows over the whole K; the 4 waves take contiguous
// quarters of K in 128-wide slices (lane group q takes 32 consecutive k of a slice: 16 B of
// codes, 2 scale bytes and the 64 B of activations that meet them).
// The kernel streams the weights once, so it is a software pipeline: a ring of PW slices
// (weights + activations, in registers) is kept in flight, and the slot just consumed is
// refilled with the slice PW ahead. Compute then overlaps the loads of later slices instead of
// waiting for a whole batch. Loads are unconditional with selected addresses only (so the
// compiler counts outstanding loads exactly); slices past the wave's range read activations
// from a zero block, so the (clamped, valid) weights loaded for them contribute nothing. Lanes
// of activation rows >= M read row 0: those output columns are never stored.
// SRC_SP24: the weights come as vals+meta and are expanded to dense codes in registers first
// (the decompress-then-dense-MFMA variant of the 2:4 product).
template <bool SRC_SP24, int PW>
__global__ __launch_bounds__(256) void k_gemv_mfma(const uint16_t* __restrict__ X, int M, int N, int K,
                                                   const uint8_t* __restrict__ w0, const uint8_t* __restrict__ w1,
                                                   const uint8_t* __restrict__ scales, const float* __restrict__ ts,
                                                   void* __restrict__ Y, int y_bf16) {
  __shared__ float red[kWaves * 4 * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int n = min(n0 + r, N - 1);
  const uint16_t* xrow = X + (size_t)(r < M ? r : 0) * K;
  const uint8_t* srow = scales + (size_t)n * (K / 16);
  const int S = (K + 127) / 128;
  const int s_lo = (S * wave) / kWaves, s_hi = (S * (wave + 1)) / kWaves;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};

  struct Slot { u32x4 w; uint32_t sc; u32x4 x[4]; };
  auto load_slot = [&](int s) -> Slot {
    Slot o;
    const bool ok = s < s_hi && s * 128 + 32 * q < K;
    const int k = ok ? s * 128 + 32 * q : 0;
    if constexpr (!SRC_SP24) {
      o.w = ld_nt((const u32x4*)(w0 + (size_t)n * (K / 2) + k / 2));
    } else {
      const u32x2 v = ld_nt((const u32x2*)(w0 + (size_t)n * (K / 4) + k / 4));
      o.w[0] = v[0]; o.w[1] = v[1]; o.w[3] = 0u;
      o.w[2] = ld_nt((const uint32_t*)(w1 + (size_t)n * (K / 8) + k / 8));
    }
    o.sc = ld_nt((const uint16_t*)(srow + k / 16));
    const u32x4* xp = ok ? (const u32x4*)(xrow + k) : (const u32x4*)g_zero32;
    const int xs = ok ? 1 : 0;                     // the zero block is 32 B: do not step through it
#pragma unroll
    for (int j = 0; j < 4; ++j) o.x[j] = xp[j * xs];
    return o;
  };

  Slot ring[PW];
#pragma unroll
  for (int u = 0; u < PW; ++u) ring[u] = load_slot(s_lo + u);
  for (int s = s_lo; s < s_hi; s += PW) {
#pragma unroll
    for (int u = 0; u < PW; ++u) {
      const Slot cur = ring[u];
      ring[u] = load_slot(s + u + PW);             // refill: PW slices ahead
      u32x4 c = cur.w;
      if constexpr (SRC_SP24) {
        // 8 groups: vals bytes in c[0..1], meta nibbles in c[2] -> 32 dense codes
        const u32x2 v = {c[0], c[1]};
        const uint32_t mt = c[2];
        c = zero4();
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          const uint32_t vb = (v[g >> 2] >> (8 * (g & 3))) & 0xFFu;
          const uint32_t pos = (mt >> (4 * g)) & 0xFu;
          const uint32_t grp = ((vb & 0xFu) << (4 * (pos & 3u))) | ((vb >> 4) << (4 * (pos >> 2)));
          c[g >> 1] |= grp << (16 * (g & 1));
        }
      }
      const float sc0 = e4m3_f32_sel<0>(cur.sc), sc1 = e4m3_f32_sel<1>(cur.sc);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 a = fp4x8_bf16(c[j], j < 2 ? sc0 : sc1);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(cur.x[j]), acc, 0, 0, 0);
      }
    }
  }
  store_tile16(acc, red, M, N, n0, *ts, Y, y_bf16);
}

// ---------------------------------------------------------------------------------------------
// Dense, M <= 16, "slab" kernel: one block per CU owns a contiguous slab of R weight rows and
// streams it once through LDS.
//  * Weights reach LDS with gfx950 direct-to-LDS loads (global_load_lds_dwordx4, no registers):
//    every load instruction reads contiguous 256-byte runs of a row (4 rows per instruction), so
//    HBM sees long runs instead of 16 rows x 64 B per instruction.
//  * K is streamed in stages of kSK values; kD stages are in flight (a ring of LDS buffers).
//    Every wave issues a fixed number of loads per stage (clamped addresses), so "stage st has
//    landed" is an exact s_waitcnt vmcnt on each wave followed by a barrier. Rows past the
//    block's own range repeat its last row, so no other block's rows are read.
//  * Inside a 256-byte row run the 16-byte chunks are stored XOR-swizzled by the row index, so
//    the MFMA operand reads (16 rows x one chunk) hit 16 different LDS bank groups.
//  * The activations of the stage (M rows x kSK bf16) are loaded once per block (wave m loads
//    row m) and shared by its waves.
// Rows are processed in groups of 64 (four 16-row MFMA tiles); 16 waves: wave w computes tile
// w & 3 on slice w >> 2 of each stage's four 128-wide slices; the four partial tiles of each row
// tile are summed at the end.
constexpr int kSK = 512;                          // K values per stage
constexpr int kD = 4;                             // stages in flight
constexpr int kSlabWaves = 16;                    // 4 per SIMD; wave w: tile w & 3, slice w >> 2
constexpr int kSRow = kSK / 16;                   // scale bytes per row per stage (32)
constexpr int kXRow = kSK * 2 + 16;               // activation bytes per row per stage (+ pad)

template <int L>   // wait until at most `ahead` stages of L loads each are still in flight
__device__ __forceinline__ void wait_stages(int ahead) {
  switch (ahead) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<L>(); break;
    case 2: wait_vmcnt<2 * L>(); break;
    default: wait_vmcnt<3 * L>(); break;
  }
}

// Stage layout of one ring slot (G = 4 W rows of the current row group, W waves):
//   dense: codes [G][256 B] (16-byte chunks XOR-swizzled by row & 15), scales [G][32 B]
//   2:4:   vals  [G][128 B] (16-byte chunks XOR-swizzled by row & 7), meta [G][64 B],
//          scales [G][32 B]
//   both:  activations [W][1024 B + 16 B pad] (rows >= M are not read; M <= W)
template <bool SP24, int W>
struct SlabLayout {
  static constexpr int kG = 4 * W;                       // weight rows per group
  static constexpr int kA = SP24 ? kSK / 4 : kSK / 2;   // main weight bytes per row per stage
  static constexpr int kMeta = SP24 ? kSK / 8 : 0;       // position bytes per row per stage
  static constexpr int kAOff = 0, kMetaOff = kG * kA, kScOff = kMetaOff + kG * kMeta;
  static constexpr int kXOff = kScOff + kG * kSRow;
  static constexpr int kBytes = kXOff + W * kXRow;
};

template <bool SP24, int W>
__global__ __launch_bounds__(W * 64) void k_gemv_slab(const uint16_t* __restrict__ X, int M, int N, int K,
                                                               const uint8_t* __restrict__ w0,
                                                               const uint8_t* __restrict__ w1,
                                                               const uint8_t* __restrict__ scales,
                                                               const float* __restrict__ ts, void* __restrict__ Y,
                                                               int y_bf16, int R) {
  using Lay = SlabLayout<SP24, W>;
  constexpr int NT = W / 4;                        // 16-row MFMA tiles per group
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // loads per wave per stage: weights (dense: 1 KB = 4 rows; 2:4: vals 512 B + meta 256 B),
  // scales (128 B), and for waves m < M the activation row m (1 KB): L loads, or L - 1 for waves
  // without an activation row; rows past this block's range repeat its last row (no HBM traffic
  // outside the block's own rows)
  constexpr int L = SP24 ? 4 : 3;
  static_assert((W == 8 || W == 16) && Lay::kG * (kSK / 2) / 1024 == W, "one 1 KB weight load per wave per stage");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int row_lo = blockIdx.x * R, row_hi = min(row_lo + R, N);
  const int nst = (K + kSK - 1) / kSK;
  const int rowA = SP24 ? K / 4 : K / 2;            // bytes per row of the main weight array

  for (int g0 = row_lo; g0 < row_hi; g0 += Lay::kG) {
    auto issue = [&](int st) {
      uint8_t* b = smem + (st % kD) * Lay::kBytes;
      const int k0 = st * kSK;
      if constexpr (!SP24) {                        // codes: 4 rows x 256 B
        const int rr = wave * 4 + (lane >> 4);
        const int n = min(g0 + rr, row_hi - 1);
        const int cb = min(k0 / 2 + 16 * ((lane & 15) ^ (rr & 15)), rowA - 16);  // K tail: clamp
        lds_dma16(w0 + (size_t)n * rowA + cb, b + Lay::kAOff + wave * 4 * Lay::kA);
      } else {                                      // vals: 4 rows x 128 B (lanes 0..31)
        const int rr = wave * 4 + ((lane >> 3) & 3);
        const int n = min(g0 + rr, row_hi - 1);
        const int cb = min(k0 / 4 + 16 * ((lane & 7) ^ (rr & 7)), rowA - 16);
        if (lane < 32) lds_dma16(w0 + (size_t)n * rowA + cb, b + Lay::kAOff + wave * 4 * Lay::kA);
        // meta: 4 rows x 64 B (lanes 0..15)
        const int rm = wave * 4 + ((lane >> 2) & 3);
        const int nm = min(g0 + rm, row_hi - 1);
        const int mb = min(k0 / 8 + 16 * (lane & 3), K / 8 - 16);
        if (lane < 16) lds_dma16(w1 + (size_t)nm * (K / 8) + mb, b + Lay::kMetaOff + wave * 4 * Lay::kMeta);
      }
      {                                             // scales: 4 rows x 32 B (lanes 0..7)
        const int rr = wave * 4 + ((lane >> 1) & 3);
        const int n = min(g0 + rr, row_hi - 1);
        const int sb = min(k0 / 16 + 16 * (lane & 1), K / 16 - 16);
        if (lane < 8) lds_dma16(scales + (size_t)n * (K / 16) + sb, b + Lay::kScOff + wave * 4 * kSRow);
      }
      if (wave < M) {                               // activations: wave m < M loads row m, 1 KB
        const int xe = min(k0 + 8 * lane, K - 8);
        lds_dma16(X + (size_t)wave * K + xe, b + Lay::kXOff + wave * kXRow);
      }
    };

    const int tile = wave % NT, sl = wave / NT;     // row tile, 128-k slice within each stage
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int rt = tile * 16 + r;                   // this lane's A-operand row in the group
    const int xm = r < M ? r : 0;                   // B-operand rows >= M: any row, never stored

#pragma unroll
    for (int st = 0; st < kD - 1; ++st)
      if (st < nst) issue(st);
    for (int st = 0; st < nst; ++st) {
      if (wave < M) wait_stages<L>(min(kD - 2, nst - 1 - st));   // this wave's loads of stage st
      else wait_stages<L - 1>(min(kD - 2, nst - 1 - st));        // are in LDS
      stage_barrier();                              // ... every wave's; slot (st-1)%kD is free
      if (st + kD - 1 < nst) issue(st + kD - 1);
      const uint8_t* b = smem + (st % kD) * Lay::kBytes;
      const int k0 = st * kSK;
      const uint8_t* xrow = b + Lay::kXOff + xm * kXRow;
      if constexpr (!SP24) {
        // four 16x16x32 MFMAs: lane group q takes 32 consecutive k of the slice
        const int c = 4 * sl + q;                   // 16-byte chunk of the row run
        const bool ok = k0 + sl * 128 + 32 * q < K;
        const u32x4 cw = *(const u32x4*)(b + Lay::kAOff + rt * Lay::kA + 16 * (c ^ r));
        const uint32_t sw = *(const uint16_t*)(b + Lay::kScOff + rt * kSRow + 8 * sl + 2 * q);
        const uint8_t* xb = xrow + (sl * 128 + 32 * q) * 2;
        u32x4 x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = *(const u32x4*)(xb + 16 * j);
        const float s0 = e4m3_f32_sel<0>(sw), s1 = e4m3_f32_sel<1>(sw);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 a = fp4x8_bf16(cw[j], j < 2 ? s0 : s1);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(ok ? x[j] : zero4()), acc, 0, 0, 0);
        }
      } else {
        // two 16x16x64 SMFMACs: SMFMAC jj covers k = slice + 64 jj .. +64; lane group q of the
        // A operand holds its four groups k = slice + 64 jj + 16 q .. +16 (8 kept values, 16 bits
        // of positions); the B lane (col r, group q) holds k = slice + 64 jj + 8 q (8 values)
        // and the same + 32.
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int base = sl * 128 + 64 * jj;
          const bool ok_a = k0 + base + 16 * q < K;
          const int sidx = (2 * sl + jj) ^ (rt & 7);
          const uint32_t vw = *(const uint32_t*)(b + Lay::kAOff + rt * Lay::kA + 16 * sidx + 4 * q);
          const uint32_t mw = *(const uint16_t*)(b + Lay::kMetaOff + rt * Lay::kMeta + base / 8 + 2 * q);
          const uint32_t sc = *(const uint8_t*)(b + Lay::kScOff + rt * kSRow + base / 16 + q);
          u32x4 xl = *(const u32x4*)(xrow + (base + 8 * q) * 2);
          u32x4 xh = *(const u32x4*)(xrow + (base + 32 + 8 * q) * 2);
          xl = (k0 + base + 8 * q < K) ? xl : zero4();
          xh = (k0 + base + 32 + 8 * q < K) ? xh : zero4();
          const u32x4 a = fp4x8_bf16(ok_a ? vw : 0u, e4m3_f32(sc));
          u32x8 bx;
          bx[0] = xl[0]; bx[1] = xl[1]; bx[2] = xl[2]; bx[3] = xl[3];
          bx[4] = xh[0]; bx[5] = xh[1]; bx[6] = xh[2]; bx[7] = xh[3];
          acc = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(as_bf16x8(a), as_bf16x16(bx), acc, (int)mw, 0, 0);
        }
      }
    }
    // ---- sum the four slice-partials of each row tile, scale, store
    __syncthreads();                                // all stages consumed: reuse LDS for the sum
    float* red = (float*)smem;
    if (sl != 0)
      for (int i = 0; i < 4; ++i) red[((sl - 1) * 4 * NT + tile * 4 + i) * 64 + lane] = acc[i];
    __syncthreads();
    if (sl == 0) {
      const float st_ = *ts;
      f32x4 s;
      for (int i = 0; i < 4; ++i)
        s[i] = (acc[i] + red[(0 * 4 * NT + tile * 4 + i) * 64 + lane] + red[(1 * 4 * NT + tile * 4 + i) * 64 + lane] +
                red[(2 * 4 * NT + tile * 4 + i) * 64 + lane]) * st_;
      const int m = lane & 15, n = g0 + tile * 16 + 4 * q;
      if (m < M) {
        for (int i = 0; i < 4; ++i) {
          if (n + i < row_hi) {
            if (!y_bf16) ((float*)Y)[(size_t)m * N + n + i] = s[i];
            else ((uint16_t*)Y)[(size_t)m * N + n + i] = (uint16_t)f32_to_bf16_rne(s[i]);
          }
        }
      }
    }
    __syncthreads();                                // LDS is reused by the next row group
  }
}

// ---------------------------------------------------------------------------------------------
// 2:4, M <= 16, sparse MFMA. One block = 16 weight rows; the 4 waves take contiguous quarters of
// K in 256-wide slices. Lane group q of a slice takes 16 consecutive groups (64 k): 16 B vals,
// 8 B meta, 4 B scales, feeding four v_smfmac_f32_16x16x64_bf16 (j = 0..3). For SMFMAC j the
// instruction's k index kappa = 16q + t maps to k = slice + 64q + 16j + t, so the B lane
// (col r, group q) needs the activations at slice + 64(q>>1) + 16j + 8(q&1) (8 contiguous) and
// the same + 128. Same ring pipeline as the dense kernel.
template <int PW>
__global__ __launch_bounds__(256) void k_gemv_smfmac(const uint16_t* __restrict__ X, int M, int N, int K,
                                                     const uint8_t* __restrict__ vals, const uint8_t* __restrict__ meta,
                                                     const uint8_t* __restrict__ scales, const float* __restrict__ ts,
                                                     void* __restrict__ Y, int y_bf16) {
  __shared__ float red[kWaves * 4 * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int n = min(n0 + r, N - 1);
  const uint16_t* xrow = X + (size_t)(r < M ? r : 0) * K;
  const int S = (K + 255) / 256;
  const int s_lo = (S * wave) / kWaves, s_hi = (S * (wave + 1)) / kWaves;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};

  struct Slot { u32x4 v; u32x2 m; uint32_t sc; u32x4 x[8]; };
  auto load_slot = [&](int s) -> Slot {
    Slot o;
    const bool ok = s < s_hi && s * 256 + 64 * q < K;
    const int k = ok ? s * 256 + 64 * q : 0;
    o.v = ld_nt((const u32x4*)(vals + (size_t)n * (K / 4) + k / 4));
    o.m = ld_nt((const u32x2*)(meta + (size_t)n * (K / 8) + k / 8));
    o.sc = ld_nt((const uint32_t*)(scales + (size_t)n * (K / 16) + k / 16));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kb = s * 256 + 64 * (q >> 1) + 16 * j + 8 * (q & 1);
      const bool ok_lo = s < s_hi && kb < K, ok_hi = s < s_hi && kb + 128 < K;
      o.x[2 * j] = *(ok_lo ? (const u32x4*)(xrow + kb) : (const u32x4*)g_zero32);
      o.x[2 * j + 1] = *(ok_hi ? (const u32x4*)(xrow + kb + 128) : (const u32x4*)g_zero32);
    }
    return o;
  };

  Slot ring[PW];
#pragma unroll
  for (int u = 0; u < PW; ++u) ring[u] = load_slot(s_lo + u);
  for (int s = s_lo; s < s_hi; s += PW) {
#pragma unroll
    for (int u = 0; u < PW; ++u) {
      const Slot cur = ring[u];
      ring[u] = load_slot(s + u + PW);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float sc = j == 0 ? e4m3_f32_sel<0>(cur.sc) : j == 1 ? e4m3_f32_sel<1>(cur.sc)
                       : j == 2 ? e4m3_f32_sel<2>(cur.sc) : e4m3_f32_sel<3>(cur.sc);
        const u32x4 a = fp4x8_bf16(cur.v[j], sc);
        u32x8 b;
        b[0] = cur.x[2 * j][0]; b[1] = cur.x[2 * j][1]; b[2] = cur.x[2 * j][2]; b[3] = cur.x[2 * j][3];
        b[4] = cur.x[2 * j + 1][0]; b[5] = cur.x[2 * j + 1][1]; b[6] = cur.x[2 * j + 1][2]; b[7] = cur.x[2 * j + 1][3];
        const int idx = (int)cur.m[j >> 1];
        if ((j & 1) == 0)
          acc = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(as_bf16x8(a), as_bf16x16(b), acc, idx, 0, 0);
        else
          acc = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(as_bf16x8(a), as_bf16x16(b), acc, idx, 0, 1);
      }
    }
  }
  store_tile16(acc, red, M, N, n0, *ts, Y, y_bf16);
}

// ---------------------------------------------------------------------------------------------
// Dense, M <= 16, K % 512 == 0: the "post-scale" slab. 8-wave workgroups, each owning a contiguous
// range of weight rows (32-row groups), stream the rows through a 3-deep LDS ring of 512-wide K
// stages with direct-to-LDS buffer loads. The E4M3 block scale is
// applied after the matrix product instead of before it: one v_mfma_f32_32x32x16_bf16 per
// 16-wide scale block takes the E2M1 codes converted to bf16 unscaled (one
// v_cvt_scalef32_pk_bf16_fp4 per two codes, exact) and the activations, and its 32x32 result is
// accumulated with one f32 FMA per needed output row, times the block's scale. That costs about
// 0.6 vector instructions per weight instead of two. Operands: A = activations (row m = lane % 32,
// rows >= M read row 0 and are never stored), B = weights (column = weight row lane % 32); lane
// half h = lane / 32 holds codes 8h..8h+7 of the block. Wave w takes the four blocks 4w..4w+3 of
// every stage; the eight partial sums of a row are added at the end.
// Workgroups per CU: a ring slot holds the stage's weights and XR activation rows (XR = 1, 2, 4,
// 8, 16 for M = 1, 2, <= 4, <= 8, <= 16), so the ring takes 30.8 / 33.9 / 40.1 / 52.6 KB in
// three slots, and 51.7 KB in two for 16 rows; the buffer loads (one wave-uniform resource per
// row group, one 32-bit offset per lane) keep a wave to 64 registers up to M = 8 (79 for 16
// rows): four workgroups per CU for M <= 4, three above. Measured at N = 131072 against the earlier form (flat 64-bit
// addresses, 8-row slots, 78-84 registers, two or three workgroups per CU): M = 1 70-72 -> 66 us,
// M = 2 75-76 -> 69-70 us, M = 4 83 -> 75 us, M = 8 89 -> 86-88 us; M = 9 on the 16-wave slab
// 112 us, with 16-row slots 100-102 us in three slots and 96 us in two (alternated on one box;
// two slots for M <= 8 were 1-2% slower).
constexpr int kPsWaves = 8, kPsRows = 4 * kPsWaves, kPsStages = 3, kPsMaxM = 8, kPsMaxM16 = 16;
static_assert(kPsStages >= 2 && kPsStages <= 5, "wait_stages covers up to three stages in flight");
constexpr int kPsXRow = kSK * 2 + 16;                          // activation row stride in LDS
constexpr int kPsAOff = 0, kPsScOff = kPsRows * (kSK / 2), kPsXOff = kPsScOff + kPsRows * kSRow;
// a ring slot holds the stage's weights and XR >= M activation rows
template <int XR>
constexpr int ps_slot_bytes() { return kPsXOff + XR * kPsXRow; }
// ring slots: three, but two for 16 activation rows (three workgroups per CU instead of two)
template <int XR>
constexpr int ps_stages() { return XR > kPsWaves ? 2 : kPsStages; }

// F: output rows per lane (M = 1 -> 1, M = 2 -> 2, M <= 8 -> 4, M <= 16 -> 8). FOLD: each
// block's product is folded into the sums before the next block's is formed, so one 16-register
// result is live (M <= 2: 48-51 registers); without it the four products are formed together,
// which hides their latency better (M > 2: 4% faster at M = 4, N = 131072, within the same 64
// registers).
// XR activation rows per ring slot (XR = 16: wave w also loads row w + 8); WPE: waves per SIMD
// the registers must allow.
template <int F, bool FOLD, int XR, int WPE>
__global__ __launch_bounds__(kPsWaves * 64) __attribute__((amdgpu_waves_per_eu(WPE))) void k_gemv_ps(const uint16_t* __restrict__ X, int M, int N, int K,
                                                           const uint8_t* __restrict__ codes,
                                                           const uint8_t* __restrict__ scales,
                                                           const float* __restrict__ ts, void* __restrict__ Y,
                                                           int y_bf16, int R) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int S = ps_stages<XR>();
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row_lo = blockIdx.x * R, row_hi = min(row_lo + R, N);
  const int nst = K / kSK;
  const int h = lane >> 5, nl = lane & 31;
  const int xm = nl < M ? nl : 0;
  // per wave per stage: codes of rows 4w..4w+3 (1 KB; lane: row rc, 16-byte piece lane % 16 to
  // LDS piece (lane % 16) ^ (rc & 15)), their scales (lanes < 8: row rs, half lane % 2), and for
  // w < M activation row w (1 KB). Buffer loads: a wave-uniform resource per row group and one
  // 32-bit offset per lane (rows past the block's range repeat its last row); a stage adds its
  // wave-uniform K offset.
  const int rc = wave * 4 + (lane >> 4), rs = wave * 4 + ((lane >> 1) & 3);
  const uint32_t pc = 16u * ((lane & 15) ^ (rc & 15)), psc = 16u * (lane & 1);
  const auto xrs = buf_rsrc(X + (size_t)min(wave, M - 1) * K);
  const auto xrs2 = buf_rsrc(X + (size_t)min(wave + kPsWaves, M - 1) * K);   // XR = 16: row w + 8
  for (int g0 = row_lo; g0 < row_hi; g0 += kPsRows) {
    const auto crs = buf_rsrc(codes + (size_t)g0 * (K / 2));
    const auto srs = buf_rsrc(scales + (size_t)g0 * (K / 16));
    const uint32_t vc = (uint32_t)min(rc, row_hi - 1 - g0) * (uint32_t)(K / 2) + pc;
    const uint32_t vs = (uint32_t)min(rs, row_hi - 1 - g0) * (uint32_t)(K / 16) + psc;
    auto issue = [&](int st) {
      uint8_t* b = smem + (st % S) * ps_slot_bytes<XR>();
      lds_dma16(crs, vc, (uint32_t)st * (kSK / 2), b + kPsAOff + wave * 4 * (kSK / 2));
      if (lane < 8) lds_dma16(srs, vs, (uint32_t)st * (kSK / 16), b + kPsScOff + wave * 4 * kSRow);
      if (wave < M) lds_dma16(xrs, 16u * lane, (uint32_t)st * (2 * kSK), b + kPsXOff + wave * kPsXRow);
      if constexpr (XR > kPsWaves)
        if (wave + kPsWaves < M)
          lds_dma16(xrs2, 16u * lane, (uint32_t)st * (2 * kSK), b + kPsXOff + (wave + kPsWaves) * kPsXRow);
    };
    float acc[F];
#pragma unroll
    for (int i = 0; i < F; ++i) acc[i] = 0.f;
#pragma unroll
    for (int st = 0; st < S - 1; ++st)
      if (st < nst) issue(st);
    for (int st = 0; st < nst; ++st) {
      // this wave's loads of stage st have landed (later stages may be in flight), then every wave's
      const int ahead = min(S - 2, nst - 1 - st);
      if (XR > kPsWaves && wave + kPsWaves < M) wait_stages<4>(ahead);
      else if (wave < M) wait_stages<3>(ahead);
      else wait_stages<2>(ahead);
      stage_barrier();
      if (st + S - 1 < nst) issue(st + S - 1);
      const uint8_t* b = smem + (st % S) * ps_slot_bytes<XR>();
      // codes words of blocks 4w..4w+3 for this lane's half: 16-byte chunk c of the row run sits
      // at chunk c ^ (row & 15) (the slab's swizzle); block j's half h is word 2 (j & 1) + h
      const uint8_t* arow = b + kPsAOff + nl * (kSK / 2);
      uint32_t w[4];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const uint8_t* p = arow + 16 * ((2 * wave + jj) ^ (nl & 15)) + 4 * h;
        w[2 * jj] = *(const uint32_t*)p;
        w[2 * jj + 1] = *(const uint32_t*)(p + 8);
      }
      const uint32_t sw = *(const uint32_t*)(b + kPsScOff + nl * kSRow + 4 * wave);
      const uint8_t* xr = b + kPsXOff + xm * kPsXRow;
      // the products of blocks 0..3 times their scales enter each sum in block order (one FMA
      // per needed row: result row 4h + i, i < F, of the 32x32 tile, column nl)
      f32x16 d[FOLD ? 1 : 4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 xv = *(const u32x4*)(xr + 2 * (16 * (4 * wave + j) + 8 * h));
        u32x4 bw;
        bw[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], 1.0f, 0));
        bw[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], 1.0f, 1));
        bw[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], 1.0f, 2));
        bw[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], 1.0f, 3));
        f32x16 z = {};
        d[FOLD ? 0 : j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(xv), as_bf16x8(bw), z, 0, 0, 0);
        if (FOLD) {
          const float sj = j == 0 ? e4m3_f32_sel<0>(sw) : j == 1 ? e4m3_f32_sel<1>(sw)
                         : j == 2 ? e4m3_f32_sel<2>(sw) : e4m3_f32_sel<3>(sw);
#pragma unroll
          for (int i = 0; i < F; ++i) acc[i] = fmaf(sj, d[0][i], acc[i]);
        }
      }
      if (!FOLD) {
        const float s0 = e4m3_f32_sel<0>(sw), s1 = e4m3_f32_sel<1>(sw), s2 = e4m3_f32_sel<2>(sw),
                    s3 = e4m3_f32_sel<3>(sw);
#pragma unroll
        for (int i = 0; i < F; ++i)
          acc[i] = fmaf(s3, d[FOLD ? 0 : 3][i], fmaf(s2, d[FOLD ? 0 : 2][i], fmaf(s1, d[FOLD ? 0 : 1][i], fmaf(s0, d[0][i], acc[i]))));
      }
    }
    __syncthreads();                               // every stage consumed: LDS holds the partial sums
    float* red = (float*)smem;
    if (wave != 0)
      for (int i = 0; i < F; ++i) red[((wave - 1) * F + i) * 64 + lane] = acc[i];
    __syncthreads();
    if (wave == 0) {
      const float st_ = *ts;
      for (int i = 0; i < F; ++i) {
        float v = acc[i];
        for (int q = 0; q < kPsWaves - 1; ++q) v += red[(q * F + i) * 64 + lane];
        const int m = 8 * (i >> 2) + 4 * h + (i & 3), n = g0 + nl;   // row of result register i
        if (m < M && n < row_hi) {
          if (!y_bf16) ((float*)Y)[(size_t)m * N + n] = v * st_;
          else ((uint16_t*)Y)[(size_t)m * N + n] = (uint16_t)f32_to_bf16_rne(v * st_);
        }
      }
    }
    __syncthreads();                               // LDS is reused by the next row group
  }
}

// ---------------------------------------------------------------------------------------------
// 2:4, M <= 16, K % 512 == 0: the same pipeline as the post-scale slab (8-wave workgroups, 32-row
// groups, 512-wide K stages in a ring of S LDS slots), with every direct load a full 1 KB buffer
// load (one wave-uniform resource per group, one 32-bit offset per lane): waves 0-3 load the
// vals of rows 8w..8w+7 (128 B each), waves 4-5 the
// meta of rows 16(w-4)..+15 (64 B each), wave 6 the scales of all 32 rows (32 B each), and wave
// m < M activation row m. Wave w then multiplies the 64-wide K chunk w of the stage for all 32
// rows: two v_smfmac_f32_32x32x32_bf16 with the stored vals/meta as the compressed A operand and
// its index operand (lane (n = l % 32, h = l / 32) holds the 8 kept values of 16-blocks 2h and
// 2h + 1 of the chunk; step t takes block 2h + t), the kept values decoded with their E4M3 scale
// (exact in bf16). The activations are the B operand (row m = l % 32, rows >= M read row 0 and
// are never stored). The eight chunk partials of a row meet in LDS at the end.
// LDS slot: vals [32][128 B] (16-byte piece p of row r holds global piece p ^ (r & 7)), meta
// [32][64 B] (piece p holds global piece p ^ ((r >> 1) & 3)), scales [32][32 B], activations
// [XR][1 KB + 16 B]. The row group's partial sums meet in LDS through all eight waves' results
// (32 KB), and one thread per output adds them, so a wave keeps to 56-59 registers (a wave 0
// that added the seven other partials of its 16 results itself held 78 and took ~1 us per row
// group). Geometries: M <= 16 with XR = 16 and two slots (48 KB, three workgroups per CU; wave
// w also loads activation row w + 8; 4.5% faster at M = 9 than three slots with two workgroups
// per CU); M <= 8 with XR = 8 and three slots (46 KB, three per CU);
// M <= 4 with XR = 4 and three slots (34 KB), and M <= 2 with XR = 2 and four slots (37 KB):
// four workgroups per CU at eight waves per SIMD. Measured at N = 131072 against the wave-0
// reduction with three workgroups per CU: M = 1 72-75 -> 65-67 us, M = 2 71-72 -> 64-66 us,
// M = 4 72-73 -> 68-70 us, M = 8 unchanged (80 us).

// The weight part of a ring slot of the 2:4 slab (512-wide stage, 32 rows); XR activation rows
// follow it.
struct P4Slot {
  static constexpr int kV = kSK / 4, kMt = kSK / 8, kSc = kSK / 16;   // bytes per row per stage
  static constexpr int kVP = kV / 16, kMP = kMt / 16, kSP = kSc / 16;   // 16-byte pieces per row
  static constexpr int kVOff = 0, kMOff = kPsRows * kV, kSOff = kMOff + kPsRows * kMt;
  static constexpr int kXOff = kSOff + kPsRows * kSc;
  static constexpr int kVLoads = kPsRows * kV / 1024, kMLoads = kPsRows * kMt / 1024, kSLoads = kPsRows * kSc / 1024;
  static constexpr int kLoads = kVLoads + kMLoads + kSLoads;           // 1 KB weight loads per stage (7)
  static_assert(kLoads <= kPsWaves, "one weight load per wave");
};
template <int XR, int S>
struct P4Ring {
  static constexpr int kSlot = P4Slot::kXOff + XR * kPsXRow, kBytes = S * kSlot;
  static_assert(S >= 2 && S <= 5, "wait_stages covers up to three stages in flight");
  static_assert(kBytes >= kPsWaves * 16 * 64 * 4, "the partial sums of a row group fit the ring");
};

// 16-byte piece swizzles of a vals row (8 pieces) and a meta row (4 pieces)
__device__ __forceinline__ int p4_vswz(int r) { return r & 7; }
__device__ __forceinline__ int p4_mswz(int r) { return (r >> 1) & 3; }

template <int XR, int S, int WPE>
__global__ __launch_bounds__(kPsWaves * 64) __attribute__((amdgpu_waves_per_eu(WPE))) void k_gemv_ps24(const uint16_t* __restrict__ X, int M, int N, int K,
                                                             const uint8_t* __restrict__ vals,
                                                             const uint8_t* __restrict__ meta,
                                                             const uint8_t* __restrict__ scales,
                                                             const float* __restrict__ ts, void* __restrict__ Y,
                                                             int y_bf16, int R) {
  using L = P4Slot;
  constexpr int kSlot = P4Ring<XR, S>::kSlot;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row_lo = blockIdx.x * R, row_hi = min(row_lo + R, N);
  const int nst = K / kSK;
  const int h = lane >> 5, nl = lane & 31;
  const int xm = nl < M ? nl : 0;
  // direct loads of this wave per stage: weight load `wave` (waves < 7), activation row `wave`
  // and, with XR = 16, activation row wave + 8
  const int nload = (wave < L::kLoads ? 1 : 0) + (wave < M ? 1 : 0) + (XR > kPsWaves && wave + kPsWaves < M ? 1 : 0);
  const auto xr = buf_rsrc(X + (size_t)min(wave, M - 1) * K);
  const auto xr2 = buf_rsrc(X + (size_t)min(wave + kPsWaves, M - 1) * K);
  // this wave's weight load: row r of the group (rows past the block repeat its last row) and
  // byte offset poff in it, from a buffer resource at the group's first row; a stage adds its
  // wave-uniform K offset
  const uint8_t* wbase;
  int r;
  uint32_t poff, rowb, kstep, wdst;   // rowb: bytes of a row; kstep: bytes of a row per stage
  if (wave < L::kVLoads) {
    r = wave * (1024 / L::kV) + lane / L::kVP;
    poff = 16u * ((lane % L::kVP) ^ p4_vswz(r));
    wbase = vals; rowb = K / 4; kstep = L::kV; wdst = L::kVOff + wave * 1024;
  } else if (wave < L::kVLoads + L::kMLoads) {
    const int i = wave - L::kVLoads;
    r = i * (1024 / L::kMt) + lane / L::kMP;
    poff = 16u * ((lane % L::kMP) ^ p4_mswz(r));
    wbase = meta; rowb = K / 8; kstep = L::kMt; wdst = L::kMOff + i * 1024;
  } else {
    r = lane / L::kSP;
    poff = 16u * (lane % L::kSP);
    wbase = scales; rowb = K / 16; kstep = L::kSc; wdst = L::kSOff;
  }
  for (int g0 = row_lo; g0 < row_hi; g0 += kPsRows) {
    const auto wr = buf_rsrc(wbase + (size_t)g0 * rowb);
    const uint32_t voff = (uint32_t)min(r, row_hi - 1 - g0) * rowb + poff;
    auto issue = [&](int st) {
      uint8_t* b = smem + (st % S) * kSlot;
      if (wave < L::kLoads) lds_dma16(wr, voff, (uint32_t)st * kstep, b + wdst);
      if (wave < M) lds_dma16(xr, 16u * lane, (uint32_t)st * (2 * kSK), b + L::kXOff + wave * kPsXRow);
      if constexpr (XR > kPsWaves)
        if (wave + kPsWaves < M)
          lds_dma16(xr2, 16u * lane, (uint32_t)st * (2 * kSK), b + L::kXOff + (wave + kPsWaves) * kPsXRow);
    };
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int st = 0; st < S - 1; ++st)
      if (st < nst) issue(st);
    for (int st = 0; st < nst; ++st) {
      // this wave's loads of stage st have landed (later stages may be in flight), then every wave's
      const int ahead = min(S - 2, nst - 1 - st);
      if (XR > kPsWaves && nload == 3) wait_stages<3>(ahead);
      else if (nload == 2) wait_stages<2>(ahead);
      else if (nload == 1) wait_stages<1>(ahead);
      else wait_vmcnt<0>();
      stage_barrier();
      if (st + S - 1 < nst) issue(st + S - 1);
      const uint8_t* b = smem + (st % S) * kSlot;
      const u32x2 v = *(const u32x2*)(b + L::kVOff + nl * L::kV + 16 * (wave ^ p4_vswz(nl)) + 8 * h);
      const uint32_t mw = *(const uint32_t*)(b + L::kMOff + nl * L::kMt + 16 * ((wave >> 1) ^ p4_mswz(nl)) +
                                             8 * (wave & 1) + 4 * h);
      const uint32_t sw = *(const uint16_t*)(b + L::kSOff + nl * L::kSc + 4 * wave + 2 * h);
      const uint8_t* xrow = b + L::kXOff + xm * kPsXRow + 2 * (64 * wave + 8 * h);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const u32x4 lo = *(const u32x4*)(xrow + 2 * (16 * t));
        const u32x4 hi = *(const u32x4*)(xrow + 2 * (32 + 16 * t));
        u32x8 bx;
        bx[0] = lo[0]; bx[1] = lo[1]; bx[2] = lo[2]; bx[3] = lo[3];
        bx[4] = hi[0]; bx[5] = hi[1]; bx[6] = hi[2]; bx[7] = hi[3];
        const u32x4 a = fp4x8_bf16(v[t], t == 0 ? e4m3_f32_sel<0>(sw) : e4m3_f32_sel<1>(sw));
        acc = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(as_bf16x8(a), as_bf16x16(bx), acc, (int)((mw >> (16 * t)) & 0xFFFFu),
                                                        0, 0);
      }
    }
    __syncthreads();                               // every stage consumed: LDS holds the partial sums
    // lane (nl, h) of every wave holds D[8(i/4) + 4h + i%4][nl]: partial sums of weight rows of
    // the group for activation row nl; all of them go to LDS, then thread t < 32 M adds the eight
    // partials of output (row r = t % 32, activation row m = t / 32) in wave order
    float* red = (float*)smem;
#pragma unroll
    for (int i = 0; i < 16; ++i) red[(wave * 16 + i) * 64 + lane] = acc[i];
    __syncthreads();
    const int t = threadIdx.x;
    if (t < kPsRows * M) {
      const int r = t % kPsRows, m = t / kPsRows;
      const int i = 4 * (r >> 3) + (r & 3), src = 32 * ((r >> 2) & 1) + m;
      float v = red[i * 64 + src];
#pragma unroll
      for (int w = 1; w < kPsWaves; ++w) v += red[(w * 16 + i) * 64 + src];
      const int n = g0 + r;
      if (n < row_hi) {
        const float o = v * *ts;
        if (!y_bf16) ((float*)Y)[(size_t)m * N + n] = o;
        else ((uint16_t*)Y)[(size_t)m * N + n] = (uint16_t)f32_to_bf16_rne(o);
      }
    }
    __syncthreads();                               // LDS is reused by the next row group
  }
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
      for (int d = 0; d < 2; ++d) {
        f32x2 p0 = fp4x2_f32<0>(v[d]), p1 = fp4x2_f32<1>(v[d]), p2 = fp4x2_f32<2>(v[d]), p3 = fp4x2_f32<3>(v[d]);
        const float s = d == 0 ? s0 : s1;     // groups 0..3 -> k 0..15 (block 0), 4..7 -> block 1
        w[8 * d + 0] = p0[0] * s; w[8 * d + 1] = p0[1] * s; w[8 * d + 2] = p1[0] * s; w[8 * d + 3] = p1[1] * s;
        w[8 * d + 4] = p2[0] * s; w[8 * d + 5] = p2[1] * s; w[8 * d + 6] = p3[0] * s; w[8 * d + 7] = p3[1] * s;
      }
      // the chunk's 32 activations of a row arrive as four 16-byte loads; the kept value at
      // position p of group g is half p & 1 of word 2g + (p >> 1)
      for (int i = 0; i < mcount; ++i) {
        const u32x4* xp = (const u32x4*)(X + (size_t)(m0 + i) * K + k);
        u32x4 xv[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) xv[t] = xp[t];
        float a = acc[i];
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          const uint32_t d0 = xv[g >> 1][2 * (g & 1)], d1 = xv[g >> 1][2 * (g & 1) + 1];
          const uint32_t pos = (mt >> (4 * g)) & 0xFu;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const uint32_t p = e == 0 ? (pos & 3u) : (pos >> 2);
            const uint32_t d = (p & 2u) ? d1 : d0;
            const uint32_t bits = (p & 1u) ? (d & 0xFFFF0000u) : (d << 16);
            a = fmaf(__uint_as_float(bits), w[2 * g + e], a);
          }
        }
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

int slab_blocks(int64_t N) {
  const int64_t tiles = (N + 15) / 16;
  return (int)std::min<int64_t>(cu_count(), tiles);
}

hipError_t launch_gemv_dense_mfma(const GemmArgs& a, hipStream_t s) {
  static PerDeviceOnce attr_once;
  hipError_t e1 = once_per_device(attr_once, [] {
    return hipFuncSetAttribute((const void*)k_gemv_slab<false, kSlabWaves>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               kD * SlabLayout<false, kSlabWaves>::kBytes);
  });
  if (e1 != hipSuccess) return e1;
  if (a.K % 256) {   // the slab kernel stages scale rows in 16-byte pieces: K/16 must be a multiple of 16
    hipLaunchKernelGGL((k_gemv_mfma<false, kDenseRing>), dim3((unsigned)((a.N + 15) / 16)), dim3(256), 0, s, a.X,
                       (int)a.M, (int)a.N, (int)a.K, a.w0, a.w1, a.scales, a.ts, a.Y, a.y_bf16);
    return hipGetLastError();
  }
  // post-scale slab; its buffer offsets (32 rows of a row group, an activation row) are 32-bit,
  // so K stays below 2^27
  if (a.K % kSK == 0 && a.M <= kPsMaxM16 && a.K <= ((int64_t)1 << 27)) {
    static PerDeviceOnce ps_once;
    hipError_t e2 = once_per_device(ps_once, [] {
      for (const void* f : {(const void*)k_gemv_ps<1, true, 1, 8>, (const void*)k_gemv_ps<2, true, 2, 8>,
                            (const void*)k_gemv_ps<4, false, 4, 8>, (const void*)k_gemv_ps<4, false, 8, 6>,
                            (const void*)k_gemv_ps<8, false, 16, 6>}) {
        hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           kPsStages * ps_slot_bytes<kPsMaxM16>());
        if (e != hipSuccess) return e;
      }
      return hipSuccess;
    });
    if (e2 != hipSuccess) return e2;
    const int G = (int)std::min<int64_t>((int64_t)16 * cu_count(), (a.N + kPsRows - 1) / kPsRows);
    const int R = (int)((a.N + G - 1) / G);
    auto k = a.M == 1 ? k_gemv_ps<1, true, 1, 8> : a.M == 2 ? k_gemv_ps<2, true, 2, 8>
           : a.M <= 4 ? k_gemv_ps<4, false, 4, 8> : a.M <= kPsMaxM ? k_gemv_ps<4, false, 8, 6>
           : k_gemv_ps<8, false, 16, 6>;
    const int xr = a.M == 1 ? 1 : a.M == 2 ? 2 : a.M <= 4 ? 4 : a.M <= kPsMaxM ? kPsMaxM : kPsMaxM16;
    const int lds = (xr > kPsWaves ? ps_stages<kPsMaxM16>() : kPsStages) * (kPsXOff + xr * kPsXRow);
    hipLaunchKernelGGL(k, dim3(G), dim3(kPsWaves * 64), lds, s, a.X, (int)a.M, (int)a.N, (int)a.K,
                       a.w0, a.scales, a.ts, a.Y, a.y_bf16, R);
    return hipGetLastError();
  }
  const int G = slab_blocks(a.N);
  const int R = (int)((a.N + G - 1) / G);
  static_assert(kSlabWaves >= 16, "one activation row load per wave must cover M <= 16");
  constexpr int lds16 = kD * SlabLayout<false, kSlabWaves>::kBytes;
  hipLaunchKernelGGL((k_gemv_slab<false, kSlabWaves>), dim3(G), dim3(kSlabWaves * 64), lds16, s, a.X,
                     (int)a.M, (int)a.N, (int)a.K, a.w0, (const uint8_t*)nullptr, a.scales, a.ts, a.Y, a.y_bf16, R);
  return hipGetLastError();
}

hipError_t launch_gemv_sp24_decomp(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((k_gemv_mfma<true, kDenseRing>), dim3((unsigned)((a.N + 15) / 16)), dim3(256), 0, s, a.X, (int)a.M,
                     (int)a.N, (int)a.K, a.w0, a.w1, a.scales, a.ts, a.Y, a.y_bf16);
  return hipGetLastError();
}

hipError_t launch_gemv_sp24_smfmac(const GemmArgs& a, hipStream_t s) {
  static PerDeviceOnce attr_once;
  hipError_t e1 = once_per_device(attr_once, [] {
    for (const void* f : {(const void*)k_gemv_slab<true, 8>, (const void*)k_gemv_slab<true, kSlabWaves>}) {
      hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                                         kD * SlabLayout<true, kSlabWaves>::kBytes);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  });
  if (e1 != hipSuccess) return e1;
  if (a.K % 256) {   // the slab kernel stages scale rows in 16-byte pieces: K/16 must be a multiple of 16
    hipLaunchKernelGGL((k_gemv_smfmac<kSparseRing>), dim3((unsigned)((a.N + 15) / 16)), dim3(256), 0, s, a.X,
                       (int)a.M, (int)a.N, (int)a.K, a.w0, a.w1, a.scales, a.ts, a.Y, a.y_bf16);
    return hipGetLastError();
  }
  // full-width loads, 32x32x32 sparse MFMA per 64-k chunk; its buffer offsets (32 rows of a row
  // group, an activation row) are 32-bit, so K stays below 2^27
  if (a.M <= kPsMaxM16 && a.K % kSK == 0 && a.K <= ((int64_t)1 << 27)) {
    static PerDeviceOnce p4_once;
    hipError_t e2 = once_per_device(p4_once, [] {
      for (const auto& f : {std::make_pair((const void*)k_gemv_ps24<16, 2, 6>, P4Ring<16, 2>::kBytes),
                            std::make_pair((const void*)k_gemv_ps24<8, 3, 6>, P4Ring<8, 3>::kBytes),
                            std::make_pair((const void*)k_gemv_ps24<4, 3, 8>, P4Ring<4, 3>::kBytes),
                            std::make_pair((const void*)k_gemv_ps24<2, 4, 8>, P4Ring<2, 4>::kBytes)}) {
        hipError_t e = hipFuncSetAttribute(f.first, hipFuncAttributeMaxDynamicSharedMemorySize, f.second);
        if (e != hipSuccess) return e;
      }
      return hipSuccess;
    });
    if (e2 != hipSuccess) return e2;
    const int G = (int)std::min<int64_t>((int64_t)16 * cu_count(), (a.N + kPsRows - 1) / kPsRows);
    const int R = (int)((a.N + G - 1) / G);
    constexpr int lds2 = P4Ring<2, 4>::kBytes, lds4 = P4Ring<4, 3>::kBytes, lds8 = P4Ring<8, 3>::kBytes,
                  lds16 = P4Ring<16, 2>::kBytes;
    if (a.M <= 2)
      hipLaunchKernelGGL((k_gemv_ps24<2, 4, 8>), dim3(G), dim3(kPsWaves * 64), lds2, s, a.X, (int)a.M, (int)a.N,
                         (int)a.K, a.w0, a.w1, a.scales, a.ts, a.Y, a.y_bf16, R);
    else if (a.M <= 4)
      hipLaunchKernelGGL((k_gemv_ps24<4, 3, 8>), dim3(G), dim3(kPsWaves * 64), lds4, s, a.X, (int)a.M, (int)a.N,
                         (int)a.K, a.w0, a.w1, a.scales, a.ts, a.Y, a.y_bf16, R);
    else if (a.M <= kPsMaxM)
      hipLaunchKernelGGL((k_gemv_ps24<8, 3, 6>), dim3(G), dim3(kPsWaves * 64), lds8, s, a.X, (int)a.M, (int)a.N,
                         (int)a.K, a.w0, a.w1, a.scales, a.ts, a.Y, a.y_bf16, R);
    else
      hipLaunchKernelGGL((k_gemv_ps24<16, 2, 6>), dim3(G), dim3(kPsWaves * 64), lds16, s, a.X, (int)a.M, (int)a.N,
                         (int)a.K, a.w0, a.w1, a.scales, a.ts, a.Y, a.y_bf16, R);
    return hipGetLastError();
  }
  if (a.M <= 8) {    // 8-wave workgroups (two per CU at 94 registers), 32-row groups
    const int G = (int)std::min<int64_t>(2 * (int64_t)cu_count(), (a.N + 31) / 32);
    const int R = (int)((a.N + G - 1) / G);
    constexpr int lds8 = kD * SlabLayout<true, 8>::kBytes;
    hipLaunchKernelGGL((k_gemv_slab<true, 8>), dim3(G), dim3(8 * 64), lds8, s, a.X,
                       (int)a.M, (int)a.N, (int)a.K, a.w0, a.w1, a.scales, a.ts, a.Y, a.y_bf16, R);
    return hipGetLastError();
  }
  const int G = slab_blocks(a.N);
  const int R = (int)((a.N + G - 1) / G);
  constexpr int lds16 = kD * SlabLayout<true, kSlabWaves>::kBytes;
  hipLaunchKernelGGL((k_gemv_slab<true, kSlabWaves>), dim3(G), dim3(kSlabWaves * 64), lds16, s, a.X,
                     (int)a.M, (int)a.N, (int)a.K, a.w0, a.w1, a.scales, a.ts, a.Y, a.y_bf16, R);
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
