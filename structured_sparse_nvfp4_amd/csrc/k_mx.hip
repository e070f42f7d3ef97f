// W4A4 variant: MXFP4 quantisation (activations and weights) and the FP4 x FP4 product on the
// block-scaled matrix cores of gfx950.
//
// Block-scaled FP4 x FP4 is what the pages call the FP4 tensor cores' performance unlock
// ("Trying to beat the bandwidth", NVIDIA developer forum: W4A16 has to dequantise to BF16
// first). gfx950's v_mfma_scale_f32_32x32x64_f8f6f4 multiplies E2M1 operands and applies one
// E8M0 (power-of-two) scale per 32 values along K to each operand, the OCP MX format, so both
// operands of this variant are MXFP4: E2M1 codes plus an E8M0 scale per 32 along K, the scale
// exponent floor(log2(amax)) - 2 (the OCP reference rule).
//
// MFMA tile layout (SSN_MX_TILED): the quantiser can write codes and scales in the order the
// matrix-core operands are read, so the product streams 1 KB pieces straight into LDS and every
// lane reads its operand with one 16-byte LDS read:
//   codes  [R/32][K/64][64 lanes][16 B]: lane l holds row 32 rb + l % 32, codes of
//          k = 64 ks + 32 (l / 32) .. + 31 (two per byte, even k in the low nibble);
//   scales [R/32][K/256][64 lanes][4 B]: byte s of lane l is the scale of row 32 rb + l % 32 for
//          k = 256 kg + 64 s + 32 (l / 32) .. + 31 (the byte the MFMA selects for step s).
// R is padded to a multiple of 32 and K to a multiple of 256 with zero codes and scale byte 0
// (value 0 x 2^-127 = 0), so padding adds nothing to a product.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "device_once.hpp"
#include "launch.hpp"
#include "pipeline.hpp"
#include "tile.hpp"

namespace ssn {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------------------------
// quantisation. Row-major layout: four lanes per 32-value block, eight values per lane (one or
// two 16-byte loads), the block maximum by two lane exchanges. Tiled layout: one lane per block
// (see k_mx_quantize_tiled).

// E2M1 magnitude code of r >= 0 (exact), nearest with ties to the even code, saturating at 6:
// the boundaries are the midpoints 0.25 0.75 1.25 1.75 2.5 3.5 5, ties going down at 0.25, 1.25,
// 2.5, 5 (to codes 0, 2, 4, 6) and up at 0.75, 1.75, 3.5 (to codes 2, 4, 6)
__device__ __forceinline__ uint32_t e2m1_code(float r) {
  return (uint32_t)(r > 0.25f) + (uint32_t)(r >= 0.75f) + (uint32_t)(r > 1.25f) + (uint32_t)(r >= 1.75f) +
         (uint32_t)(r > 2.5f) + (uint32_t)(r >= 3.5f) + (uint32_t)(r > 5.0f);
}

// floor(log2(a)) - 2 clamped to [-127, 127] for a > 0 finite; -127 for a == 0
__device__ __forceinline__ int mx_exponent(float a) {
  if (!(a > 0.f)) return -127;
  const uint32_t u = __float_as_uint(a);
  int e = (int)((u >> 23) & 0xFF) - 127;
  if ((u >> 23) == 0) e = -127 - (__clz(u) - 9);   // subnormal: 2^-149 * m, m < 2^23
  return max(-127, min(127, e - 2));
}

template <bool BF16>
__device__ __forceinline__ void load8(const void* V, int64_t g, float (&v)[8]) {
  if constexpr (BF16) {
    const u32x4 w = *((const u32x4*)V + g);
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[2 * i] = bf16_lo(w[i]); v[2 * i + 1] = bf16_hi(w[i]); }
  } else {
    const f32x4 a = *((const f32x4*)V + 2 * g), b = *((const f32x4*)V + 2 * g + 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
  }
}

// groups g of eight values over [R, K] in row-major order; thread t of the grid takes
// g = t, t + stride, ...; the four lanes of a block share it (block = g / 4, lanes aligned to 4)
template <bool BF16>
__global__ __launch_bounds__(256) void k_mx_quantize(const void* __restrict__ V, int64_t R, int64_t K,
                                                     uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t groups = R * (K / 8);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < groups; g += stride) {
    float v[8];
    load8<BF16>(V, g, v);
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[i]));
    a = fmaxf(a, __shfl_xor(a, 1, 64));
    a = fmaxf(a, __shfl_xor(a, 2, 64));
    const int e = mx_exponent(a);
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float r = __builtin_amdgcn_ldexpf(fabsf(v[i]), -e);     // exact: a power-of-two scale
      const uint32_t c = e2m1_code(r) | ((__float_as_uint(v[i]) >> 28) & 8u);
      word |= c << (4 * i);
    }
    ((uint32_t*)codes)[g] = word;
    if ((g & 3) == 0) scales[g >> 2] = (uint8_t)(e + 127);
  }
}

// Matrix-core tiled layout: one wave per 32 rows x 256 k (four 64-k pieces). Lane l takes row
// 32 rb + l % 32 and the k half l / 32 of every piece, i.e. one whole 32-value block per piece,
// so its 16 code bytes are its slice of the piece (a piece leaves as one 1 KB store of the wave)
// and its four scale bytes, one per piece, are one word. Rows past R and k past K are written as
// zeros, so every byte of the layout is written once, by this kernel alone.
template <bool BF16>
__global__ __launch_bounds__(256) void k_mx_quantize_tiled(const void* __restrict__ V, int64_t R, int64_t K,
                                                           uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t k256 = (K + 255) / 256, k64 = 4 * k256;
  const int64_t items = (R + 31) / 32 * k256;
  const int lane = threadIdx.x & 63;
  const int64_t wstride = (int64_t)gridDim.x * (blockDim.x / 64);
  for (int64_t it = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6); it < items; it += wstride) {
    const int64_t rb = it / k256, kg = it - rb * k256;
    const int64_t r = 32 * rb + (lane & 31);
    uint32_t sword = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int64_t k0 = 256 * kg + 64 * s + 32 * (lane >> 5);
      u32x4 cw = {0u, 0u, 0u, 0u};
      if (r < R && k0 < K) {
        float v[32];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float w8[8];
          load8<BF16>(V, (r * K + k0) / 8 + j, w8);
#pragma unroll
          for (int i = 0; i < 8; ++i) v[8 * j + i] = w8[i];
        }
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) a = fmaxf(a, fabsf(v[i]));
        const int e = mx_exponent(a);
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const float q = __builtin_amdgcn_ldexpf(fabsf(v[i]), -e);   // exact: a power-of-two scale
          cw[i >> 3] |= (e2m1_code(q) | ((__float_as_uint(v[i]) >> 28) & 8u)) << (4 * (i & 7));
        }
        sword |= (uint32_t)(e + 127) << (8 * s);
      }
      *(u32x4*)(codes + ((size_t)((rb * k64 + 4 * kg + s) * 64 + lane) << 4)) = cw;
    }
    *(uint32_t*)(scales + ((size_t)((rb * k256 + kg) * 64 + lane) << 2)) = sword;
  }
}

// ---------------------------------------------------------------------------------------------
// product: Y = X_hat . W_hat^T on v_mfma_scale_f32_32x32x64_f8f6f4 (E2M1 x E2M1).
// 256 x 256 output tile per workgroup of NWV waves: wave (wm, wn) owns 128 rows x 256 / (NWV / 2)
// columns (4 x NBK blocks of 32 x 32). A K stage is 128 wide (two MFMA steps): X and W pieces of
// the tile's eight row blocks each (8 x 2 KB), and the scale pieces of the 256-wide group the
// stage belongs to (8 x 256 B each; the two stages of a group load the same piece). Four ring
// slots, so three stages are in flight while one is multiplied; a slot is refilled right after
// the barrier that shows every wave is done with it. Each step's operands are read from LDS while
// the previous step's MFMAs run. Eight waves (two per SIMD, 128 x 64 each) measured 7% faster
// than four (128 x 128 each) at 8192 x 27648 x 5120 and 10% at 4096^3: while one wave waits on
// LDS or the barrier the other's matrix ops run, and the operands need no decode, so the second
// wave adds no vector-ALU work.
constexpr int kMT = 256, kMN = 256;
constexpr int kMxBlocks = 8;                          // 32-row blocks per tile side
constexpr int kMxSlots = 4;                           // ring slots (stages of 128 K)
constexpr int kMxStageX = kMxBlocks * 2048;           // codes of the tile's rows for one stage
constexpr int kMxStageS = kMxBlocks * 256;            // the scale pieces of their 256-wide group
constexpr int kMxSlot = 2 * kMxStageX + 2 * kMxStageS;   // X codes, W codes, X scales, W scales
constexpr int kMxLds = kMxSlots * kMxSlot;
constexpr int kMxWaves = 8;
static_assert(kMxLds <= 160 * 1024, "LDS budget");

constexpr int kXcds = 8, kGroupM = 4;
__device__ __forceinline__ void mx_tile_of(int b, int total, int tiles_m, int tiles_n, int& tm, int& tn) {
  // consecutive logical tiles share an XCD (workgroups are dealt to the eight XCDs round-robin)
  // and walk down kGroupM tile rows before moving right (4, 8 and 16 measured alike)
  const int per = total / kXcds, extra = total % kXcds;
  const int x = b % kXcds, idx = b / kXcds;
  const int t = x * per + min(x, extra) + idx;
  const int span = kGroupM * tiles_n;
  const int first = (t / span) * kGroupM;
  const int gsize = min(kGroupM, tiles_m - first);
  const int tin = t % span;
  tm = first + tin % gsize;
  tn = tin / gsize;
}

// format 4 = E2M1 for both operands; the scale byte of step S of a 256-wide group is byte S of
// the lane's scale word (op_sel)
template <int S>
__device__ __forceinline__ f32x16 mfma_fp4(u32x4 a, u32x4 b, f32x16 c, uint32_t sa, uint32_t sb) {
  const i32x8 av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  const i32x8 bv = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 4, S, (int)sa, S, (int)sb);
}

template <int NWV, bool YB>
__global__ __launch_bounds__(64 * NWV) __attribute__((amdgpu_waves_per_eu(NWV / 4, NWV / 4)))
void k_gemm_mx(const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xs, int M, const uint8_t* __restrict__ wc,
               const uint8_t* __restrict__ ws, int N, int K, void* __restrict__ Y, int y_bf16) {
  constexpr int BPW = kMxBlocks / NWV;                // row blocks of X and of W each wave copies
  constexpr int WN = NWV / 2, NBK = kMxBlocks / WN;   // waves along N, W blocks per wave
  constexpr int kLoads = BPW * 2 * 2 + BPW * 2;       // per wave per stage: code copies, scale copies
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int tiles_m = (M + kMT - 1) / kMT, tiles_n = (N + kMN - 1) / kMN;
  int tm, tn;
  mx_tile_of(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, tm, tn);
  const int k64 = (K + 255) / 256 * 4, k256 = k64 / 4, nst = 2 * k256;   // nst is even
  const int mb_last = (M + 31) / 32 - 1, nb_last = (N + 31) / 32 - 1;
  // this wave copies row blocks BPW wave + i of X and of W (clamped to the last block of the
  // padded layout; their results are not stored) and their scale pieces
  int xbs[BPW], wbs[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    xbs[i] = min(8 * tm + BPW * wave + i, mb_last);
    wbs[i] = min(8 * tn + BPW * wave + i, nb_last);
  }
  // Loads go through buffer resources whose (wave-uniform) base is the copied block's piece of
  // the stage, moved on the scalar unit each stage; the lane offsets are fixed (16 bytes of a
  // 1 KB code piece, 4 bytes of a 256-byte scale piece).
  const uint8_t *xcb[BPW], *wcb[BPW], *xsb[BPW], *wsb[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    xcb[i] = xc + (size_t)xbs[i] * k64 * 1024;
    wcb[i] = wc + (size_t)wbs[i] * k64 * 1024;
    xsb[i] = xs + (size_t)xbs[i] * k256 * 256;
    wsb[i] = ws + (size_t)wbs[i] * k256 * 256;
  }
  auto issue = [&](int st, char* slot) {
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const auto xr = buf_rsrc(xcb[i] + (size_t)st * 2048), wr = buf_rsrc(wcb[i] + (size_t)st * 2048);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        lds_dma16(xr, 16u * lane + 1024u * s, 0u, slot + (BPW * wave + i) * 2048 + s * 1024);
        lds_dma16(wr, 16u * lane + 1024u * s, 0u, slot + kMxStageX + (BPW * wave + i) * 2048 + s * 1024);
      }
    }
    // scale pieces of the stage's 256-wide group: 256 bytes per block, 4 bytes per lane
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      lds_dma4(buf_rsrc(xsb[i] + (size_t)(st >> 1) * 256), 4u * lane, 0u, slot + 2 * kMxStageX + (BPW * wave + i) * 256);
      lds_dma4(buf_rsrc(wsb[i] + (size_t)(st >> 1) * 256), 4u * lane, 0u,
               slot + 2 * kMxStageX + kMxStageS + (BPW * wave + i) * 256);
    }
  };

  f32x16 acc[4][NBK];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NBK; ++j)
#pragma unroll
      for (int t = 0; t < 16; ++t) acc[i][j][t] = 0.f;

  auto read_ops = [&](const char* slot, int s, u32x4 (&a)[4], u32x4 (&b)[NBK]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *(const u32x4*)(slot + (4 * wm + i) * 2048 + s * 1024 + 16 * lane);
#pragma unroll
    for (int j = 0; j < NBK; ++j) b[j] = *(const u32x4*)(slot + kMxStageX + (NBK * wn + j) * 2048 + s * 1024 + 16 * lane);
  };
  // stage st (parity P: steps 2P, 2P + 1 of its 256-wide group) from slot st % kMxSlots
  auto stage = [&](auto parity, int st) {
    constexpr int P = decltype(parity)::value;
    const char* slot = lds + (st % kMxSlots) * kMxSlot;
    wait_vmcnt<2 * kLoads>();             // stage st has landed (st + 1, st + 2 may be in flight)
    stage_barrier();                      // ... for every wave; slot (st - 1) % kMxSlots is free
    issue(min(st + 3, nst - 1), lds + ((st + 3) % kMxSlots) * kMxSlot);   // past the end: a repeat, unused
    uint32_t sa[4], sb[NBK];
#pragma unroll
    for (int i = 0; i < 4; ++i) sa[i] = *(const uint32_t*)(slot + 2 * kMxStageX + (4 * wm + i) * 256 + 4 * lane);
#pragma unroll
    for (int j = 0; j < NBK; ++j)
      sb[j] = *(const uint32_t*)(slot + 2 * kMxStageX + kMxStageS + (NBK * wn + j) * 256 + 4 * lane);
    u32x4 a0[4], b0[NBK], a1[4], b1[NBK];
    read_ops(slot, 0, a0, b0);
    read_ops(slot, 1, a1, b1);            // step 1's operands are read while step 0 multiplies
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NBK; ++j) acc[i][j] = mfma_fp4<2 * P>(b0[j], a0[i], acc[i][j], sb[j], sa[i]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NBK; ++j) acc[i][j] = mfma_fp4<2 * P + 1>(b1[j], a1[i], acc[i][j], sb[j], sa[i]);
  };

  issue(0, lds);
  issue(1, lds + kMxSlot);
  issue(min(2, nst - 1), lds + 2 * kMxSlot);
  for (int st = 0; st < nst; st += 2) {
    stage(std::integral_constant<int, 0>{}, st);
    stage(std::integral_constant<int, 1>{}, st + 1);
  }
  wait_vmcnt<0>();
  __syncthreads();

  // epilogue: the blocks are Y^T (weights = A, activations = B), so lane l holds
  // Y[m][n .. n + 3] for m = 32 i + l % 32 and n = 32 j + 8 g + 4 (l / 32) (plus the wave's
  // offsets) in acc[i][j][4g .. 4g + 3]. Each 32-row block of the wave (32 x 32 NBK) is staged in
  // LDS and leaves as row-contiguous pieces: bf16 output rounded first, 16-byte pieces of 8 values
  // (piece c of row r at position c ^ (r & 7)); f32 output as 16-byte pieces of 4 values (piece
  // q at q ^ (r & 7)).
  const int r32 = lane & 31, h = lane >> 5;
  const int m0 = kMT * tm + 128 * wm, n0 = kMN * tn + 32 * NBK * wn;
  if constexpr (YB) {
    constexpr int kPR = 4 * NBK;                      // 16-byte pieces (8 bf16) per staged row
    static_assert(kPR >= 8, "swizzle spans eight pieces");
    char* T = lds + wave * (32 * kPR * 16);
    const bool vec = (N & 7) == 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < NBK; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 w;
          w[0] = pk_bf16_rne(acc[i][j][4 * g], acc[i][j][4 * g + 1]);
          w[1] = pk_bf16_rne(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
          const int c = 4 * j + g;
          *(u32x2*)(T + r32 * (16 * kPR) + 16 * (c ^ (r32 & 7)) + 8 * h) = w;
        }
      __builtin_amdgcn_s_waitcnt(0xC07F);
      const int c = lane % kPR;
#pragma unroll
      for (int q = 0; q < 32 * kPR / 64; ++q) {
        const int r = lane / kPR + (64 / kPR) * q;
        const u32x4 v = *(const u32x4*)(T + r * (16 * kPR) + 16 * (c ^ (r & 7)));
        const int m = m0 + 32 * i + r, n = n0 + 8 * c;
        if (m < M && n < N) store8_bf16(Y, N, m, n, v, vec);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);
    }
  } else {
    constexpr int kPR = 8 * NBK;                      // 16-byte pieces (4 f32) per staged row
    float* T = (float*)(lds + wave * (32 * kPR * 16));
    const bool vec = (N & 3) == 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < NBK; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 v;
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] = acc[i][j][4 * g + t];
          const int q = 8 * j + 2 * g + h;
          *(f32x4*)(T + r32 * (4 * kPR) + 4 * (q ^ (r32 & 7))) = v;
        }
      __builtin_amdgcn_s_waitcnt(0xC07F);
      const int p = lane % kPR;
#pragma unroll
      for (int q = 0; q < 32 * kPR / 64; ++q) {
        const int r = lane / kPR + (64 / kPR) * q;
        const f32x4 v = *(const f32x4*)(T + r * (4 * kPR) + 4 * (p ^ (r & 7)));
        const int m = m0 + 32 * i + r, n = n0 + 4 * p;
        if (m < M && n < N) store4(Y, 0, N, m, n, v, vec);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);
    }
  }
}

}  // namespace

int64_t mx_tiled_code_bytes(int64_t R, int64_t K) { return (R + 31) / 32 * 32 * ((K + 255) / 256 * 128); }
int64_t mx_tiled_scale_bytes(int64_t R, int64_t K) { return (R + 31) / 32 * 32 * ((K + 255) / 256 * 8); }

hipError_t launch_mx_quantize(const void* V, int v_bf16, int64_t R, int64_t K, int tiled, uint8_t* codes,
                              uint8_t* scales, hipStream_t s) {
  const int64_t groups = R * (K / 8);
  const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>((groups + 255) / 256, 64 * (int64_t)cu_count()));
  if (tiled) {
    const int64_t items = (R + 31) / 32 * ((K + 255) / 256);   // one wave each, four per workgroup
    const unsigned tg = (unsigned)std::min<int64_t>((items + 3) / 4, 64 * (int64_t)cu_count());
    if (items > 0) {
      if (v_bf16) hipLaunchKernelGGL((k_mx_quantize_tiled<true>), dim3(tg), dim3(256), 0, s, V, R, K, codes, scales);
      else hipLaunchKernelGGL((k_mx_quantize_tiled<false>), dim3(tg), dim3(256), 0, s, V, R, K, codes, scales);
    }
  } else if (groups > 0) {
    if (v_bf16) hipLaunchKernelGGL(k_mx_quantize<true>, dim3(grid), dim3(256), 0, s, V, R, K, codes, scales);
    else hipLaunchKernelGGL(k_mx_quantize<false>, dim3(grid), dim3(256), 0, s, V, R, K, codes, scales);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_mx(const uint8_t* xc, const uint8_t* xs, int64_t M, const uint8_t* wc, const uint8_t* ws,
                          int64_t N, int64_t K, void* Y, int y_bf16, hipStream_t s) {
  static PerDeviceOnce attr_once;
  hipError_t e = once_per_device(attr_once, [] {
    hipError_t e1 = hipFuncSetAttribute((const void*)k_gemm_mx<kMxWaves, true>, hipFuncAttributeMaxDynamicSharedMemorySize, kMxLds);
    if (e1 != hipSuccess) return e1;
    return hipFuncSetAttribute((const void*)k_gemm_mx<kMxWaves, false>, hipFuncAttributeMaxDynamicSharedMemorySize, kMxLds);
  });
  if (e != hipSuccess) return e;
  const unsigned tiles = (unsigned)(((M + kMT - 1) / kMT) * ((N + kMN - 1) / kMN));
  if (y_bf16)
    hipLaunchKernelGGL((k_gemm_mx<kMxWaves, true>), dim3(tiles), dim3(64 * kMxWaves), kMxLds, s, xc, xs, (int)M, wc, ws,
                       (int)N, (int)K, Y, y_bf16);
  else
    hipLaunchKernelGGL((k_gemm_mx<kMxWaves, false>), dim3(tiles), dim3(64 * kMxWaves), kMxLds, s, xc, xs, (int)M, wc, ws,
                       (int)N, (int)K, Y, y_bf16);
  return hipGetLastError();
}

}  // namespace ssn
