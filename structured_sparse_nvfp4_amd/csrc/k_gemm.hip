// Prefill-shaped and square products (M > 16): 256x256 output tiles on the matrix cores.
//
// The square and prefill shapes are compute-bound ("NVFP4 Without FP4 Hardware", ai-muninn.com,
// section on prefill: unpacking is extra work on top of the dense product), so the design keeps
// the matrix cores fed and spends as little vector-ALU time per weight as possible:
//  - the activation tile [256 rows][64 k] bf16 is copied HBM -> LDS by the direct-to-LDS loads
//    (three stages in flight), 16-byte chunks XOR-swizzled so that matrix-operand reads are free
//    of bank conflicts;
//  - every wave decodes its own weights straight from global memory into matrix operands: a
//    weight is decoded once per output tile and never written back to LDS.
//
// Dense and 2:4-decompressed products (v_mfma_f32_32x32x16_bf16, activations = A, weights = B):
//   wave w owns all 256 rows x columns [64w, 64w + 64) of the tile: 8 x 2 blocks of 32 x 32.
//   Lane l (r = l % 32, h = l / 32) feeds k = 8h..8h+7 of each 16-wide MFMA step. The kernel
//   maps MFMA step s of a 64-wide stage to k = 32h + 8s + j, so one lane's weights for a whole
//   stage are 16 contiguous code bytes (32 codes, two E4M3 scale blocks).
// 2:4 products on the sparse matrix cores (v_smfmac_f32_32x32x32_bf16, weights = compressed A,
//   activations = B): the roles swap, the tile computes Y^T, and wave (wn, wm) owns 128 weight
//   rows x 128 activation rows (4 x 4 blocks). The two 16-wide halves of MFMA step t take the
//   16-blocks 2H + t of the stage (H = 0, 1), so each lane's compressed weights for a stage are
//   8 contiguous vals bytes, 4 meta bytes and 2 scale bytes. The compressed layout of this
//   library is the SMFMAC A operand and index operand as stored ("NVFP4 vs 2:4 sparse",
//   robertz.co, section "What 2:4 actually is": two kept values plus a 2-bit index each).
#include "common.hpp"
#include "launch.hpp"
#include "pipeline.hpp"

namespace ssn {
namespace {

constexpr int kTM = 256, kTN = 256, kTK = 64;   // output tile and K-stage
constexpr int kStages = 3;                       // activation stages resident in LDS
constexpr int kXStage = kTM * kTK * 2;           // 32 KiB
constexpr int kThreads = 256;

// zero bytes that activation chunks and weight words beyond K are read from
__device__ __attribute__((aligned(16))) uint32_t g_zero_k[4];

enum WForm { kDense = 0, kSp24Expand = 1 };

// ---- tile scheduling: consecutive logical tiles share an XCD (workgroups are dealt to the
// eight XCDs round-robin), and go down GROUP tile rows before moving right, so the
// activation and weight panels a group touches stay in that XCD's L2.
constexpr int kXcds = 8, kGroupM = 4;

__device__ __forceinline__ void tile_of(int b, int total, int tiles_m, int tiles_n, int& tm, int& tn) {
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

// ---- activation stage: rows [m0, m0+256) x k [k0, k0+64) -> LDS, row r at r * 128 bytes,
// logical 16-byte chunk c at physical chunk c ^ ((r >> 1) & 7). Eight 1 KiB direct loads per
// wave; lane l of load i writes tile row 8 * (8 * wave + i) + l / 8, physical chunk l % 8.
template <bool FULL>   // FULL: the whole stage lies inside K (no zero-block select needed)
__device__ __forceinline__ void issue_x(const uint16_t* __restrict__ X, int M, int K, int m0, int k0,
                                        char* slot, int wave, int lane) {
  const int p = lane & 7;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 8 * (8 * wave + i) + (lane >> 3);
    const int c = p ^ ((r >> 1) & 7);
    const int k = k0 + 8 * c;
    const int m = min(m0 + r, M - 1);
    const void* src = (FULL || k < K) ? (const void*)(X + (size_t)m * K + k) : (const void*)g_zero_k;
    lds_dma16(src, slot + (8 * wave + i) * 1024);
  }
}

__device__ __forceinline__ void issue_x_stage(const uint16_t* __restrict__ X, int M, int K, int m0, int st,
                                              char* lds, int wave, int lane) {
  char* slot = lds + (st % kStages) * kXStage;
  if ((st + 1) * kTK <= K) issue_x<true>(X, M, K, m0, st * kTK, slot, wave, lane);
  else issue_x<false>(X, M, K, m0, st * kTK, slot, wave, lane);
}

// 16-byte activation chunk `c` of tile row r (bits 1..3 of r given as `sw`)
__device__ __forceinline__ u32x4 lds_x(const char* slot, int r, int c, int sw) {
  return *(const u32x4*)(slot + r * 128 + 16 * (c ^ sw));
}

// Two kept codes (byte vb) at positions (nib & 3, nib >> 2) of a group of four nibbles.
__device__ __forceinline__ uint32_t expand_group(uint32_t vb, uint32_t nib) {
  return ((vb & 0xFu) << ((nib & 3u) << 2)) | (((vb >> 4) & 0xFu) << ((nib >> 2) << 2));
}

// Weights of one lane for one stage (dense: 32 codes; 2:4: 8 groups) and its two scale bytes.
struct WStage {
  u32x4 c;        // dense codes, or (vals word 0, vals word 1, meta word, -) for 2:4
  uint32_t s;     // two E4M3 scale bytes (16-blocks 2h, 2h + 1 of the stage)
};

template <int WF, bool FULL>
__device__ __forceinline__ WStage load_w(const uint8_t* __restrict__ w0, const uint8_t* __restrict__ w1,
                                         const uint8_t* __restrict__ scales, int n, int K, int kk) {
  // kk = first k of this lane's 32-wide slice; a slice at or beyond K reads the zero block
  const bool ok = FULL || kk < K;
  WStage o;
  if constexpr (WF == kDense) {
    const u32x4* pc = ok ? (const u32x4*)(w0 + (size_t)n * (K / 2) + kk / 2) : (const u32x4*)g_zero_k;
    o.c = *pc;
  } else {
    const u32x2* pv = ok ? (const u32x2*)(w0 + (size_t)n * (K / 4) + kk / 4) : (const u32x2*)g_zero_k;
    const uint32_t* pm = ok ? (const uint32_t*)(w1 + (size_t)n * (K / 8) + kk / 8) : (const uint32_t*)g_zero_k;
    const u32x2 v = *pv;
    o.c[0] = v[0]; o.c[1] = v[1]; o.c[2] = *pm; o.c[3] = 0u;
  }
  const uint16_t* ps = ok ? (const uint16_t*)(scales + (size_t)n * (K / 16) + kk / 16) : (const uint16_t*)g_zero_k;
  o.s = *ps;
  return o;
}

// Codes word of MFMA step s (8 codes, k = 8s..8s+7 of the lane's slice)
template <int WF>
__device__ __forceinline__ uint32_t codes_step(const WStage& w, int s) {
  if constexpr (WF == kDense) {
    return w.c[s];
  } else {
    const uint32_t vb = w.c[s >> 1] >> (16 * (s & 1));        // groups 2s, 2s+1: two vals bytes
    const uint32_t nb = w.c[2] >> (8 * s);                    // their two position nibbles
    return expand_group(vb & 0xFFu, nb & 0xFu) | (expand_group((vb >> 8) & 0xFFu, (nb >> 4) & 0xFu) << 16);
  }
}

// weights of stage st for ROWS rows of this lane (slice k = 64 st + 32 half .. + 31)
template <int WF, int ROWS>
__device__ __forceinline__ void load_w_stage(WStage (&w)[ROWS], const uint8_t* __restrict__ w0,
                                             const uint8_t* __restrict__ w1, const uint8_t* __restrict__ scales,
                                             const int (&nrow)[ROWS], int K, int st, int half) {
  const int kk = st * kTK + 32 * half;
  if ((st + 1) * kTK <= K) {
#pragma unroll
    for (int i = 0; i < ROWS; ++i) w[i] = load_w<WF, true>(w0, w1, scales, nrow[i], K, kk);
  } else {
#pragma unroll
    for (int i = 0; i < ROWS; ++i) w[i] = load_w<WF, false>(w0, w1, scales, nrow[i], K, kk);
  }
}

__device__ __forceinline__ void store_val(void* Y, int y_bf16, size_t idx, float v) {
  if (y_bf16) ((uint16_t*)Y)[idx] = (uint16_t)f32_to_bf16_rne(v);
  else ((float*)Y)[idx] = v;
}

// ---------------------------------------------------------------------------------------------
// Dense (or 2:4 expanded to dense) x activations on v_mfma_f32_32x32x16_bf16.
template <int WF>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_mfma(const uint16_t* __restrict__ X, int M, int N, int K,
                                                        const uint8_t* __restrict__ w0,
                                                        const uint8_t* __restrict__ w1,
                                                        const uint8_t* __restrict__ scales,
                                                        const float* __restrict__ ts, void* __restrict__ Y,
                                                        int y_bf16) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tiles_m = (M + kTM - 1) / kTM, tiles_n = (N + kTN - 1) / kTN;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * kTM, n0 = tn * kTN;
  const int r32 = lane & 31, h = lane >> 5, sw = (lane >> 1) & 7;
  const int nst = (K + kTK - 1) / kTK;

  // this lane's two weight rows (clamped; columns beyond N are computed and not stored)
  int nrow[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) nrow[nt] = min(n0 + 64 * wave + 32 * nt + r32, N - 1);

  f32x16 acc[8][2];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.f;

  // Pipeline: activation stages st+1, st+2 and the weights of stage st+1 are in flight while
  // stage st is computed. Within an iteration the weight loads are issued before the
  // activation loads, so the register copy of the prefetched weights at the end of the
  // iteration waits only for them (they were issued a whole stage earlier), never for the
  // activation stages still meant to be in flight.
  constexpr int kWL = WF == kDense ? 2 : 3;     // weight loads per weight row per stage
  WStage wcur[2], wnext[2];
  issue_x_stage(X, M, K, m0, 0, lds, wave, lane);
  load_w_stage<WF, 2>(wcur, w0, w1, scales, nrow, K, 0, h);
  if (nst > 1) issue_x_stage(X, M, K, m0, 1, lds, wave, lane);
  __builtin_amdgcn_sched_barrier(0);

  for (int st = 0; st < nst; ++st) {
    // issued after activation stage st: weights st (2 kWL) and activation st+1 (8, if any)
    if (st + 1 < nst) wait_vmcnt<8 + 2 * kWL>();
    else wait_vmcnt<2 * kWL>();
    stage_barrier();   // stage st visible to all; every wave is done with slot (st - 1) % 3
    if (st + 1 < nst) load_w_stage<WF, 2>(wnext, w0, w1, scales, nrow, K, st + 1, h);
    if (st + 2 < nst) issue_x_stage(X, M, K, m0, st + 2, lds, wave, lane);
    __builtin_amdgcn_sched_barrier(0);

    // activation operands of MFMA step s+1 are read while step s runs
    const char* slot = lds + (st % kStages) * kXStage;
    u32x4 abuf[2][8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) abuf[0][mt] = lds_x(slot, 32 * mt + r32, 4 * h, sw);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) abuf[(s + 1) & 1][mt] = lds_x(slot, 32 * mt + r32, 4 * h + s + 1, sw);
      }
      bf16x8 b[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const float sc = s < 2 ? e4m3_f32_sel<0>(wcur[nt].s) : e4m3_f32_sel<1>(wcur[nt].s);
        b[nt] = as_bf16x8(fp4x8_bf16(codes_step<WF>(wcur[nt], s), sc));
      }
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const bf16x8 av = as_bf16x8(abuf[s & 1][mt]);
        acc[mt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b[0], acc[mt][0], 0, 0, 0);
        acc[mt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b[1], acc[mt][1], 0, 0, 0);
      }
    }
    if (st + 1 < nst) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) wcur[nt] = wnext[nt];
    }
  }

  // epilogue: lane holds rows 8(i/4) + 4h + i%4 of each 32x32 block, column r32
  const float st_scale = *ts;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int n = n0 + 64 * wave + 32 * nt + r32;
    if (n >= N) continue;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = m0 + 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3);
        if (m < M) store_val(Y, y_bf16, (size_t)m * N + n, acc[mt][nt][i] * st_scale);
      }
  }
}

// ---------------------------------------------------------------------------------------------
// 2:4 weights on the sparse matrix cores: Y^T tile = W (compressed A) x X^T (B).
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_smfmac(const uint16_t* __restrict__ X, int M, int N, int K,
                                                          const uint8_t* __restrict__ vals,
                                                          const uint8_t* __restrict__ meta,
                                                          const uint8_t* __restrict__ scales,
                                                          const float* __restrict__ ts, void* __restrict__ Y,
                                                          int y_bf16) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int tiles_m = (M + kTM - 1) / kTM, tiles_n = (N + kTN - 1) / kTN;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * kTM, n0 = tn * kTN;
  const int r32 = lane & 31, q = lane >> 5, sw = (lane >> 1) & 7;
  const int nst = (K + kTK - 1) / kTK;

  int nrow[4];
#pragma unroll
  for (int at = 0; at < 4; ++at) nrow[at] = min(n0 + 128 * wn + 32 * at + r32, N - 1);

  f32x16 acc[4][4];
#pragma unroll
  for (int at = 0; at < 4; ++at)
#pragma unroll
    for (int bt = 0; bt < 4; ++bt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[at][bt][i] = 0.f;

  constexpr int kWL = 4 * 3;   // 4 weight rows x (vals, meta, scales)
  WStage wcur[4], wnext[4];
  issue_x_stage(X, M, K, m0, 0, lds, wave, lane);
  load_w_stage<kSp24Expand, 4>(wcur, vals, meta, scales, nrow, K, 0, q);
  if (nst > 1) issue_x_stage(X, M, K, m0, 1, lds, wave, lane);
  __builtin_amdgcn_sched_barrier(0);

  for (int st = 0; st < nst; ++st) {
    if (st + 1 < nst) wait_vmcnt<8 + kWL>();
    else wait_vmcnt<kWL>();
    stage_barrier();
    if (st + 1 < nst) load_w_stage<kSp24Expand, 4>(wnext, vals, meta, scales, nrow, K, st + 1, q);
    if (st + 2 < nst) issue_x_stage(X, M, K, m0, st + 2, lds, wave, lane);
    __builtin_amdgcn_sched_barrier(0);

    const char* slot = lds + (st % kStages) * kXStage;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      // B (activations): col r32 of block bt; k = 16t + 8q + j (j < 8), 32 + 16t + 8q + j' (j >= 8)
      u32x8 bx[4];
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) {
        const int r = 128 * wm + 32 * bt + r32;
        const u32x4 lo = lds_x(slot, r, 2 * t + q, sw), hi = lds_x(slot, r, 4 + 2 * t + q, sw);
        bx[bt][0] = lo[0]; bx[bt][1] = lo[1]; bx[bt][2] = lo[2]; bx[bt][3] = lo[3];
        bx[bt][4] = hi[0]; bx[bt][5] = hi[1]; bx[bt][6] = hi[2]; bx[bt][7] = hi[3];
      }
#pragma unroll
      for (int at = 0; at < 4; ++at) {
        // A (weights): row r32, the 8 kept values of 16-block 2q + t; index bits = its 4 nibbles
        const float sc = t == 0 ? e4m3_f32_sel<0>(wcur[at].s) : e4m3_f32_sel<1>(wcur[at].s);
        const bf16x8 a = as_bf16x8(fp4x8_bf16(wcur[at].c[t], sc));
        const int idx = (int)((wcur[at].c[2] >> (16 * t)) & 0xFFFFu);
#pragma unroll
        for (int bt = 0; bt < 4; ++bt)
          acc[at][bt] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a, as_bf16x16(bx[bt]), acc[at][bt], idx, 0, 0);
      }
    }
    if (st + 1 < nst) {
#pragma unroll
      for (int at = 0; at < 4; ++at) wcur[at] = wnext[at];
    }
  }

  // epilogue: lane holds weight rows 8(i/4) + 4q + i%4 of each block, activation row r32
  const float st_scale = *ts;
  const bool vec_ok = (N & 3) == 0;   // 4 consecutive outputs of a row are then 16-B (8-B) aligned
#pragma unroll
  for (int bt = 0; bt < 4; ++bt) {
    const int m = m0 + 128 * wm + 32 * bt + r32;
    if (m >= M) continue;
#pragma unroll
    for (int at = 0; at < 4; ++at)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int nb = n0 + 128 * wn + 32 * at + 8 * g + 4 * q;
        if (vec_ok && nb + 3 < N) {
          if (y_bf16) {
            u32x2 o;
            o[0] = f32_to_bf16_rne(acc[at][bt][4 * g] * st_scale) | (f32_to_bf16_rne(acc[at][bt][4 * g + 1] * st_scale) << 16);
            o[1] = f32_to_bf16_rne(acc[at][bt][4 * g + 2] * st_scale) | (f32_to_bf16_rne(acc[at][bt][4 * g + 3] * st_scale) << 16);
            *(u32x2*)((uint16_t*)Y + (size_t)m * N + nb) = o;
          } else {
            f32x4 o;
            for (int i = 0; i < 4; ++i) o[i] = acc[at][bt][4 * g + i] * st_scale;
            *(f32x4*)((float*)Y + (size_t)m * N + nb) = o;
          }
        } else {
          for (int i = 0; i < 4; ++i)
            if (nb + i < N) store_val(Y, y_bf16, (size_t)m * N + nb + i, acc[at][bt][4 * g + i] * st_scale);
        }
      }
  }
}

}  // namespace

hipError_t launch_gemm_dense_mfma(const GemmArgs& a, hipStream_t s) {
  const int bytes = kStages * kXStage;
  hipError_t e = hipFuncSetAttribute((const void*)k_gemm_mfma<kDense>, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  const unsigned tiles = (unsigned)(((a.M + kTM - 1) / kTM) * ((a.N + kTN - 1) / kTN));
  hipLaunchKernelGGL(k_gemm_mfma<kDense>, dim3(tiles), dim3(kThreads), bytes, s, a.X, (int)a.M, (int)a.N,
                     (int)a.K, a.w0, a.w1, a.scales, a.ts, a.Y, a.y_bf16);
  return hipGetLastError();
}

hipError_t launch_gemm_sp24_decomp(const GemmArgs& a, hipStream_t s) {
  const int bytes = kStages * kXStage;
  hipError_t e = hipFuncSetAttribute((const void*)k_gemm_mfma<kSp24Expand>, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  const unsigned tiles = (unsigned)(((a.M + kTM - 1) / kTM) * ((a.N + kTN - 1) / kTN));
  hipLaunchKernelGGL(k_gemm_mfma<kSp24Expand>, dim3(tiles), dim3(kThreads), bytes, s, a.X, (int)a.M, (int)a.N,
                     (int)a.K, a.w0, a.w1, a.scales, a.ts, a.Y, a.y_bf16);
  return hipGetLastError();
}

hipError_t launch_gemm_sp24_smfmac(const GemmArgs& a, hipStream_t s) {
  const int bytes = kStages * kXStage;
  hipError_t e = hipFuncSetAttribute((const void*)k_gemm_smfmac, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  const unsigned tiles = (unsigned)(((a.M + kTM - 1) / kTM) * ((a.N + kTN - 1) / kTN));
  hipLaunchKernelGGL(k_gemm_smfmac, dim3(tiles), dim3(kThreads), bytes, s, a.X, (int)a.M, (int)a.N, (int)a.K,
                     a.w0, a.w1, a.scales, a.ts, a.Y, a.y_bf16);
  return hipGetLastError();
}

}  // namespace ssn
