// Grouped-expert (MoE) path: routing bookkeeping, grouped NVFP4 products (dense or 2:4) with the
// SiLU-gate epilogue, and the weighted combine.
//
// The pages describe a 512-expert, top-10 mixture whose expert weights are the thing every step
// reads ("NVFP4 vs 2:4 sparse", robertz.co, sections "Concurrency, not sparsity, is the lever"
// and "The sparsity that does pay is already running") and note that no grouped 2:4 product
// exists for it (same page, section "Why it cannot run on this cluster"). Here every expert's
// rows are a contiguous range of an expert-major row space (built by the routing kernels), and
// one launch runs every (expert, 64-row tile, 256-column tile) of a projection:
//  - rows per expert range from a handful to thousands, so the row tile is 64: small experts
//    waste little matrix-core work and the product stays bound by the expert weight read;
//  - the activation rows of a tile are gathered by row id straight into LDS by direct buffer
//    loads, and the expert's weights follow them through a two-slot LDS ring (one stage lands
//    while the other is multiplied);
//  - gate and up projections of one expert share a tile (128 gate + 128 up columns), so the
//    SiLU-gate product is formed in the epilogue and only H = bf16(silu(g) * u) is written.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "pipeline.hpp"
#include "tile.hpp"

namespace ssn {
namespace {

// ------------------------------------------------------------------------------ routing
// Rows are grouped by expert (ascending) and, inside an expert, follow the flat order
// f = t * k + j of the (token, slot) entries: a stable counting sort by expert id.
constexpr int kRouteChunk = 256;    // flat entries per block (one 256-thread round)
constexpr int kRouteThreads = 256;

__global__ __launch_bounds__(kRouteThreads) void k_route_hist(const int32_t* __restrict__ ids, int F, int E,
                                                              int32_t* __restrict__ hist) {
  extern __shared__ int32_t h[];   // [E]
  for (int e = threadIdx.x; e < E; e += kRouteThreads) h[e] = 0;
  __syncthreads();
  const int base = blockIdx.x * kRouteChunk;
  for (int i = threadIdx.x; i < kRouteChunk; i += kRouteThreads) {
    const int f = base + i;
    if (f < F) {
      const int e = ids[f];
      if (e >= 0 && e < E) atomicAdd(&h[e], 1);
    }
  }
  __syncthreads();
  int32_t* out = hist + (size_t)blockIdx.x * E;
  for (int e = threadIdx.x; e < E; e += kRouteThreads) out[e] = h[e];
}

// Exclusive scan of one value per thread over a block of 1024 threads.
__device__ __forceinline__ int block_excl_scan_1024(int v, int* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(inc, d, 64);
    if (lane >= d) inc += t;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    int w = lane < 16 ? wsum[lane] : 0;
    for (int d = 1; d < 16; d <<= 1) {
      const int t = __shfl_up(w, d, 64);
      if (lane >= d) w += t;
    }
    if (lane < 16) wsum[16 + lane] = w;   // inclusive sums of the wave totals
  }
  __syncthreads();
  return inc - v + (wave > 0 ? wsum[16 + wave - 1] : 0);
}

// Column scan, one wave per expert: the exclusive prefix of the expert's per-chunk counts over
// the chunks (written over the histogram) and its total. Lane l takes chunks l, l + 64, ...
__global__ __launch_bounds__(kRouteThreads) void k_route_colscan(int32_t* __restrict__ hist, int B, int E,
                                                                 int32_t* __restrict__ tot) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * (kRouteThreads / 64) + (threadIdx.x >> 6);
  if (e >= E) return;                               // uniform per wave
  int carry = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    const int c = b < B ? hist[(size_t)b * E + e] : 0;
    int inc = c;
    for (int d = 1; d < 64; d <<= 1) {
      const int t = __shfl_up(inc, d, 64);
      if (lane >= d) inc += t;
    }
    if (b < B) hist[(size_t)b * E + e] = carry + inc - c;
    carry += __shfl(inc, 63, 64);
  }
  if (lane == 0) tot[e] = carry;
}

// One block: expert offsets (exclusive scan of the totals), the placed-row count and the count
// of entries whose id is out of range. Null totals stand for all zero (no entries).
__global__ __launch_bounds__(1024) void k_route_scan(const int32_t* __restrict__ tot, int E, int F,
                                                     int32_t* __restrict__ offsets, int64_t* __restrict__ bad) {
  __shared__ int wsum[32];
  const int per = (E + 1023) / 1024;
  const int e0 = min(E, (int)threadIdx.x * per), e1 = min(E, e0 + per);
  int s = 0;
  if (tot)
    for (int e = e0; e < e1; ++e) s += tot[e];
  int ex = block_excl_scan_1024(s, wsum);
  for (int e = e0; e < e1; ++e) { offsets[e] = ex; ex += tot ? tot[e] : 0; }
  if (threadIdx.x == 1023) {
    offsets[E] = ex;                        // rows with a valid expert id
    if (bad) *bad = (int64_t)F - ex;        // entries whose id is outside [0, E)
  }
}

// Stable placement of the 256 entries [f0, f0 + 256): inside a wave the rank among equal ids
// comes from ballots over the id bits, across the four waves from per-wave counts wc[4][E]
// (zero on entry and on return); cur[e] (next output row of expert e) advances past the
// round's rows.
__device__ __forceinline__ void route_place_round(const int32_t* __restrict__ ids, int F, int k, int E, int f0,
                                                  int32_t* cur, int32_t* wc, int32_t* __restrict__ row_token,
                                                  int32_t* __restrict__ row_slot, int32_t* __restrict__ row_of) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int f = f0 + threadIdx.x;
  const int e = f < F ? ids[f] : -1;
  const bool valid = f < F && e >= 0 && e < E;
  // lanes of this wave holding the same expert id: one ballot per id bit, each lane keeping
  // the lanes that agree with it on that bit (no exchange of values between lanes)
  const int bits = E > 1 ? 32 - __clz(E - 1) : 0;
  unsigned long long same = __ballot(valid);
  for (int b = 0; b < bits; ++b) {
    const bool on = (e >> b) & 1;
    const unsigned long long s = __ballot(valid && on);
    same &= on ? s : ~s;
  }
  const int rank = __popcll(same & ((1ull << lane) - 1ull));
  const int cnt = __popcll(same);
  if (valid && rank == 0) wc[wave * E + e] = cnt;
  __syncthreads();
  if (valid) {
    int pos = cur[e] + rank;
    for (int w = 0; w < wave; ++w) pos += wc[w * E + e];
    row_token[pos] = f / k;
    row_slot[pos] = f % k;
    row_of[f] = pos;
  } else if (f < F) {
    row_of[f] = -1;
  }
  __syncthreads();
  for (int x = threadIdx.x; x < E; x += kRouteThreads) {
    cur[x] += wc[x] + wc[E + x] + wc[2 * E + x] + wc[3 * E + x];
    wc[x] = 0; wc[E + x] = 0; wc[2 * E + x] = 0; wc[3 * E + x] = 0;
  }
  __syncthreads();
}

// One chunk per block; the chunk's first row of each expert comes from the offsets and the
// column-scanned histogram.
__global__ __launch_bounds__(kRouteThreads) void k_route_scatter(const int32_t* __restrict__ ids, int F, int k,
                                                                 int E, const int32_t* __restrict__ hist,
                                                                 const int32_t* __restrict__ offsets,
                                                                 int32_t* __restrict__ row_token,
                                                                 int32_t* __restrict__ row_slot,
                                                                 int32_t* __restrict__ row_of) {
  extern __shared__ int32_t sm[];
  int32_t* cur = sm;            // [E]   next output row of each expert
  int32_t* wc = sm + E;         // [4][E] per-wave counts of the current round
  for (int e = threadIdx.x; e < E; e += kRouteThreads) {
    cur[e] = offsets[e] + hist[(size_t)blockIdx.x * E + e];
    for (int w = 0; w < 4; ++w) wc[w * E + e] = 0;
  }
  __syncthreads();
  for (int round = 0; round < kRouteChunk / kRouteThreads; ++round)
    route_place_round(ids, F, k, E, blockIdx.x * kRouteChunk + round * kRouteThreads, cur, wc, row_token, row_slot,
                      row_of);
}

// Small routings (decode: a few tokens) in one block and one launch: histogram, offsets and
// stable placement, the same results as the four kernels above.
constexpr int kRouteSmallMax = 4 * kRouteChunk;    // entries (one block is slower beyond)

__global__ __launch_bounds__(kRouteThreads) void k_route_small(const int32_t* __restrict__ ids, int F, int k, int E,
                                                               int32_t* __restrict__ offsets, int64_t* __restrict__ bad,
                                                               int32_t* __restrict__ row_token,
                                                               int32_t* __restrict__ row_slot,
                                                               int32_t* __restrict__ row_of) {
  extern __shared__ int32_t sm[];
  int32_t* cur = sm;            // [E] counts, then the next output row of each expert
  int32_t* wc = sm + E;         // [4][E]
  __shared__ int wsum[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += kRouteThreads) {
    cur[e] = 0;
    for (int w = 0; w < 4; ++w) wc[w * E + e] = 0;
  }
  __syncthreads();
  for (int f = threadIdx.x; f < F; f += kRouteThreads) {
    const int e = ids[f];
    if (e >= 0 && e < E) atomicAdd(&cur[e], 1);
  }
  __syncthreads();
  // exclusive scan of the counts: thread t takes experts [t per, (t + 1) per)
  const int per = (E + kRouteThreads - 1) / kRouteThreads;
  const int e0 = min(E, (int)threadIdx.x * per), e1 = min(E, e0 + per);
  int sum = 0;
  for (int e = e0; e < e1; ++e) sum += cur[e];
  int inc = sum;
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(inc, d, 64);
    if (lane >= d) inc += t;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int ex = inc - sum;
  for (int w = 0; w < wave; ++w) ex += wsum[w];
  const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  __syncthreads();                                  // every count is read before it is replaced
  for (int e = e0; e < e1; ++e) {
    const int c = cur[e];
    offsets[e] = ex;
    cur[e] = ex;
    ex += c;
  }
  if (threadIdx.x == 0) {
    offsets[E] = total;                             // rows with a valid expert id
    if (bad) *bad = (int64_t)F - total;             // entries whose id is outside [0, E)
  }
  __syncthreads();
  for (int f0 = 0; f0 < F; f0 += kRouteThreads) route_place_round(ids, F, k, E, f0, cur, wc, row_token, row_slot, row_of);
}

// ------------------------------------------------------------------------------ grouped product
constexpr int kBN = 256, kBK = 64;
// Ring slots of the 64-row tiles (kStages - 1 stages in flight). Two slots (34 KB, the epilogue
// staging 35 KB) let four workgroups share a CU, three (51 KB) three, four (68 KB) two; on the
// 4096-token, 512-expert FFN two were the fastest (2:4 up 516 -> 484 us, down 278 -> 253 us;
// dense 2-6%). With the buffer-resource loads (fewer registers, four workgroups per CU for every
// form) three slots were measured again, alternated with two on one box: FFN dense 564-580 ->
// 594-610 us, 2:4 453-456 -> 477-479 us. 256-row tiles for the experts with many rows, beside
// 64-row tiles for the rest, were slower throughout (the second launch has too few tiles to fill
// the chip).
template <int BM>
constexpr int moe_stages() { return 2; }
constexpr int kThreads = 256;
constexpr int kEpiNone = 0, kEpiSilu = 1;

// silu(g) = g / (1 + exp(-g)) on the hardware's base-2 exponential and reciprocal
// (exp(-g) = 2^(-g log2 e)); relative error a few 1e-7 for |g| of a few units, ~1e-6 at |g| = 20,
// far inside half a bf16 ulp of H (2^-9). Large -g: 2^(..) overflows to inf and the reciprocal
// gives 0, so silu -> -0; large g: 2^(..) underflows to 0 and silu -> g.
__device__ __forceinline__ float silu_f32(float g) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.44269504088896341f);
  return g * __builtin_amdgcn_rcpf(1.0f + e);
}

// One LDS ring slot (bytes): activations [BM][128 B] (chunk swizzle), weights of the 256 tile
// columns (dense codes [256][32 B] with half swizzle, or 2:4 vals [256][16 B] + meta
// [256][8 B]), scales [256][4 B].
template <int WF, int BM>
struct MSlot {
  static constexpr int kX = 0;
  static constexpr int kW = BM * kBK * 2;
  static constexpr int kMeta = WF == kDense ? 0 : kW + kBN * 16;
  static constexpr int kSc = WF == kDense ? kW + kBN * 32 : kMeta + kBN * 8;
  static constexpr int kBytes = kSc + kBN * 4;
  static constexpr int kXLoads = BM / 32;                                    // per wave per stage
  static constexpr int kLoads = kXLoads + (WF == kDense ? 2 : 1 + 2) + 1;
};
// epilogue staging: row blocks of 32 x 64 f32 per wave, or the BM x 128 up tile
constexpr int kStageStrideNone = 68, kStageStrideSilu = 132;
template <int WF, int BM>
constexpr int moe_lds_bytes() {
  constexpr int ring = moe_stages<BM>() * MSlot<WF, BM>::kBytes;
  constexpr int a = 4 * 32 * kStageStrideNone * 4, b = BM * kStageStrideSilu * 4;
  return ring > a ? (ring > b ? ring : b) : (a > b ? a : b);
}

// Item index of workgroup b of `total`: XCD b % 8 takes the contiguous run of items
// [x * per + min(x, extra), ...) in dispatch order.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_contiguous(int b, int total) {
  const int per = total / kXcds, extra = total % kXcds;
  const int x = b % kXcds, idx = b / kXcds;
  return x * per + min(x, extra) + idx;
}

// Rows [a, b) of expert e, clamped into [0, R] so that inconsistent offsets cannot address
// rows outside Y.
__device__ __forceinline__ void expert_part(const int32_t* off, int e, int R, int& a, int& b) {
  a = min(max(off[e], 0), R);
  b = min(max(off[e + 1], a), R);
}

// Expert, first row and row count of linear tile bx (all threads of the block take part:
// every thread sums the tiles of E / 256 experts, a block scan finds the owner). False when
// bx is past the last tile (uniformly for the block).
template <int BM>
__device__ bool find_tile(const int32_t* __restrict__ off, int E, int R, int bx, int& e_out, int& r0_out,
                          int& cnt_out) {
  __shared__ int sm[8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (E + kThreads - 1) / kThreads;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  int t = 0;
  for (int e = e0; e < e1; ++e) {
    int a, b;
    expert_part(off, e, R, a, b);
    t += (b - a + BM - 1) / BM;
  }
  int inc = t;
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(inc, d, 64);
    if (lane >= d) inc += v;
  }
  if (lane == 63) sm[wave] = inc;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += sm[w];
  const int total = sm[0] + sm[1] + sm[2] + sm[3];
  const int excl = before + inc - t;
  if (bx >= total) return false;
  if (bx >= excl && bx < excl + t) {
    int acc = excl;
    for (int e = e0; e < e1; ++e) {
      int a, b;
      expert_part(off, e, R, a, b);
      const int nt = (b - a + BM - 1) / BM;
      if (bx < acc + nt) {
        const int r0 = a + BM * (bx - acc);
        sm[4] = e; sm[5] = r0; sm[6] = min(BM, b - r0);
        break;
      }
      acc += nt;
    }
  }
  __syncthreads();
  e_out = sm[4]; r0_out = sm[5]; cnt_out = sm[6];
  return true;
}

// SMF (2:4 weights only): the products run on the sparse matrix cores, v_smfmac_f32_32x32x32_bf16
// with the stored vals/meta as the compressed A operand (weights) and the activations as B, as in
// the square/prefill tiles; the accumulators then hold the transposed tile, which the epilogue
// undoes while staging. Otherwise the weights are expanded to dense codes and multiplied on
// v_mfma_f32_32x32x16_bf16 (activations = A).
template <int WF, int EPI, int BM, bool SMF = false>
__global__ __launch_bounds__(kThreads, 2) void k_moe_gemm(
    const uint16_t* __restrict__ X, int x_rows, int K, const int32_t* __restrict__ row_token,
    const int32_t* __restrict__ off, int E, int R, int N, const uint8_t* __restrict__ w0,
    const uint8_t* __restrict__ w1, const uint8_t* __restrict__ scales, const float* __restrict__ ts,
    void* __restrict__ Y, int y_bf16, int ncols, int ktiled) {
  using L = MSlot<WF, BM>;
  constexpr int kStages = moe_stages<BM>();
  constexpr int MT = BM / 32;   // 32-row blocks per wave
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Work item t = (row tile, column tile), row-tile major. Workgroups are dealt to the eight
  // XCDs round-robin; each XCD takes a contiguous run of items, so the column tiles of a row
  // tile (same gathered activations) and consecutive row tiles of an expert (same weights) meet
  // in one XCD's L2.
  int e, r0, cnt;
  const int t = xcd_contiguous(blockIdx.x, gridDim.x);
  const int tn = t % ncols;
  if (!find_tile<BM>(off, E, R, t / ncols, e, r0, cnt)) return;
  e = __builtin_amdgcn_readfirstlane(e);
  r0 = __builtin_amdgcn_readfirstlane(r0);
  cnt = __builtin_amdgcn_readfirstlane(cnt);
  const int I = N / 2;
  const int r32 = lane & 31, h = lane >> 5;
  const int nst = K / kBK;

  // weight row of tile column tc (0..255); clamped rows are computed and never stored
  auto wrow = [&](int tc) -> int {
    if constexpr (EPI == kEpiSilu) return (tc >> 7) * I + min(128 * tn + (tc & 127), I - 1);
    else return min(kBN * tn + tc, N - 1);
  };

  // Sources of the direct loads: buffer resources at wave-uniform bases (the whole activation
  // matrix; this expert's codes or vals, meta and scales) with one 32-bit byte offset per lane,
  // computed once; a stage moves only the scalar offset. The host admits the tiles only when
  // X and every expert's weight arrays are below 2^31 bytes, so no offset wraps.
  const auto xr = buf_rsrc(X);
  const auto wr = buf_rsrc(w0 + (size_t)e * N * (WF == kDense ? K / 2 : K / 4));
  const auto mr = buf_rsrc(WF == kDense ? w0 : w1 + (size_t)e * N * (K / 8));
  const auto sr = buf_rsrc(scales + (size_t)e * N * (K / 16));
  uint32_t xo[L::kXLoads];
#pragma unroll
  for (int i = 0; i < L::kXLoads; ++i) {
    const int r = 8 * (L::kXLoads * wave + i) + (lane >> 3);
    const int rr = r0 + min(r, cnt - 1);
    int src = row_token ? row_token[rr] : rr;
    src = min(max(src, 0), x_rows - 1);
    const int c = (lane & 7) ^ swz(r);
    xo[i] = (uint32_t)(((size_t)src * K + 8 * c) * 2);
  }
  // Weight offsets. Row-major layout: piece kt of row n at n * row_bytes + kt * piece. 64-k tiled
  // layout: at (kt * N + n) * piece, so a stage's pieces of consecutive rows are contiguous and
  // every load instruction reads whole cache lines.
  const int pw = WF == kDense ? kBK / 2 : kBK / 4, pm = kBK / 8, ps = kBK / 16;   // piece bytes
  const uint32_t wrs = ktiled ? pw : (uint32_t)K * pw / kBK, mrs = ktiled ? pm : (uint32_t)K * pm / kBK,
                 srs = ktiled ? ps : (uint32_t)K * ps / kBK;                      // row strides
  const uint32_t wst = ktiled ? (uint32_t)N * pw : pw, mst = ktiled ? (uint32_t)N * pm : pm,
                 sst = ktiled ? (uint32_t)N * ps : ps;                            // stage strides
  uint32_t wo[2], mo[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if constexpr (WF == kDense) {
      const int tc = 32 * (2 * wave + i) + (lane >> 1);
      const int hl = (lane & 1) ^ ((tc >> 3) & 1);
      wo[i] = (uint32_t)wrow(tc) * wrs + 16u * hl;
      mo[i] = 0u;
    } else {
      wo[i] = i == 0 ? (uint32_t)wrow(64 * wave + lane) * wrs : 0u;
      const int tc = 32 * (2 * wave + i) + (lane >> 1);
      mo[i] = (uint32_t)wrow(tc) * mrs + 4u * (lane & 1);
    }
  }
  const uint32_t so = (uint32_t)wrow(64 * wave + lane) * srs;

  auto issue = [&](int st, char* slot) {
#pragma unroll
    for (int i = 0; i < L::kXLoads; ++i)
      lds_dma16(xr, xo[i], (uint32_t)st * (kBK * 2), slot + L::kX + (L::kXLoads * wave + i) * 1024);
    if constexpr (WF == kDense) {
#pragma unroll
      for (int i = 0; i < 2; ++i) lds_dma16(wr, wo[i], (uint32_t)st * wst, slot + L::kW + (2 * wave + i) * 1024);
    } else {
      lds_dma16(wr, wo[0], (uint32_t)st * wst, slot + L::kW + wave * 1024);
#pragma unroll
      for (int i = 0; i < 2; ++i) lds_dma4(mr, mo[i], (uint32_t)st * mst, slot + L::kMeta + (2 * wave + i) * 256);
    }
    lds_dma4(sr, so, (uint32_t)st * sst, slot + L::kSc + wave * 256);
  };

  f32x16 acc[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.f;

  const int last = nst - 1;
#pragma unroll
  for (int i = 0; i < kStages - 1; ++i) issue(min(i, last), lds + i * L::kBytes);
  // One stage: wait until it has landed, refill the other slot, multiply. Two stages run per trip
  // of the loop below, so that both slot addresses are constants folded into the LDS reads.
  static_assert(kStages == 2, "the stage loop alternates two ring slots");
  auto stage = [&](int st, const char* slot, char* next) __attribute__((always_inline)) {
    wait_vmcnt<0>();            // stage st has landed (the only stage in flight)
    stage_barrier();            // ... for every wave; the other slot is no longer read
    issue(min(st + 1, last), next);
    if constexpr (SMF) {
      static_assert(WF == kSp24, "the sparse matrix cores take 2:4 weights");
      // A: weight rows (tile columns) 64 wave + 32 at + r32; lane half h holds the kept values of
      // 16-blocks 2h and 2h + 1 of the stage (word t: block 2h + t), their positions and scales
      u32x2 v[2];
      uint32_t mw[2], sc[2];
#pragma unroll
      for (int at = 0; at < 2; ++at) {
        const int tc = 64 * wave + 32 * at + r32;
        v[at] = *(const u32x2*)(slot + L::kW + tc * 16 + 8 * h);
        mw[at] = *(const uint32_t*)(slot + L::kMeta + tc * 8 + 4 * h);
        sc[at] = *(const uint32_t*)(slot + L::kSc + tc * 4) >> (16 * h);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        // B: activation row 32 bt + r32, k chunks 2t + h and 4 + 2t + h of the stage
        u32x8 bx[MT];
#pragma unroll
        for (int bt = 0; bt < MT; ++bt) {
          const int r = 32 * bt + r32;
          const u32x4 lo = *(const u32x4*)(slot + L::kX + r * 128 + 16 * ((2 * t + h) ^ swz(r)));
          const u32x4 hi = *(const u32x4*)(slot + L::kX + r * 128 + 16 * ((4 + 2 * t + h) ^ swz(r)));
          bx[bt][0] = lo[0]; bx[bt][1] = lo[1]; bx[bt][2] = lo[2]; bx[bt][3] = lo[3];
          bx[bt][4] = hi[0]; bx[bt][5] = hi[1]; bx[bt][6] = hi[2]; bx[bt][7] = hi[3];
        }
#pragma unroll
        for (int at = 0; at < 2; ++at) {
          const float f = t == 0 ? e4m3_f32_sel<0>(sc[at]) : e4m3_f32_sel<1>(sc[at]);
          const bf16x8 a = as_bf16x8(fp4x8_bf16(v[at][t], f));
          const int idx = (int)((mw[at] >> (16 * t)) & 0xFFFFu);
#pragma unroll
          for (int bt = 0; bt < MT; ++bt)
            acc[bt][at] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a, as_bf16x16(bx[bt]), acc[bt][at], idx, 0, 0);
        }
      }
    } else {
      u32x4 wc[2];
      uint32_t wsc[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int tc = 64 * wave + 32 * nt + r32;
        if constexpr (WF == kDense) {
          wc[nt] = *(const u32x4*)(slot + L::kW + tc * 32 + 16 * (h ^ ((tc >> 3) & 1)));
        } else {
          const u32x2 v = *(const u32x2*)(slot + L::kW + tc * 16 + 8 * h);
          wc[nt][0] = v[0]; wc[nt][1] = v[1];
          wc[nt][2] = *(const uint32_t*)(slot + L::kMeta + tc * 8 + 4 * h);
          wc[nt][3] = 0u;
        }
        wsc[nt] = *(const uint32_t*)(slot + L::kSc + tc * 4) >> (16 * h);
      }
      // activation operands of MFMA step s + 1 are read while step s runs
      u32x4 a[2][MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = 32 * mt + r32;
        a[0][mt] = *(const u32x4*)(slot + L::kX + r * 128 + 16 * ((4 * h) ^ swz(r)));
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (s < 3) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const int r = 32 * mt + r32;
            a[(s + 1) & 1][mt] = *(const u32x4*)(slot + L::kX + r * 128 + 16 * ((4 * h + s + 1) ^ swz(r)));
          }
        }
        bf16x8 b[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const float f = s < 2 ? e4m3_f32_sel<0>(wsc[nt]) : e4m3_f32_sel<1>(wsc[nt]);
          b[nt] = as_bf16x8(fp4x8_bf16(codes_step<WF>(wc[nt], s), f));
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const bf16x8 av = as_bf16x8(a[s & 1][mt]);
          acc[mt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b[0], acc[mt][0], 0, 0, 0);
          acc[mt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b[1], acc[mt][1], 0, 0, 0);
        }
      }
    }
  };
  for (int st = 0; st < nst; st += 2) {
    stage(st, lds, lds + L::kBytes);
    if (st + 1 < nst) stage(st + 1, lds + L::kBytes, lds);
  }
  wait_vmcnt<0>();
  __syncthreads();   // ring slots are free for the epilogue staging

  // dense: lane holds rows 8(i/4) + 4h + i%4 of each 32-row block mt, tile column 64 wave + 32 nt
  // + r32; SMF: the transpose, row r32 of block mt and tile column 64 wave + 32 nt + 8(i/4) + 4h + i%4
  auto erow = [&](int i) { return SMF ? r32 : 8 * (i >> 2) + 4 * h + (i & 3); };
  auto ecol = [&](int nt, int i) { return SMF ? 32 * nt + 8 * (i >> 2) + 4 * h + (i & 3) : 32 * nt + r32; };
  const float sc = ts[e];
  if constexpr (EPI == kEpiNone) {
    const bool vec = (N & 3) == 0;
    float* T = (float*)(lds + wave * (32 * kStageStrideNone * 4));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          T[erow(i) * kStageStrideNone + ecol(nt, i)] = acc[mt][nt][i] * sc;
      __builtin_amdgcn_s_waitcnt(0xC07F);
      const int c4 = lane & 15;
#pragma unroll
      for (int jr = 0; jr < 8; ++jr) {
        const int r = (lane >> 4) + 4 * jr;
        const int row = 32 * mt + r;
        const f32x4 v = *(const f32x4*)(T + r * kStageStrideNone + 4 * c4);
        const int n = kBN * tn + 64 * wave + 4 * c4;
        if (row < cnt) store4(Y, y_bf16, N, r0 + row, n, v, vec);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);
    }
  } else {
    // U [BM rows][128 columns]: the up projection (waves 2, 3), then H in place
    float* U = (float*)lds;
    constexpr int S = kStageStrideSilu;
    if (wave >= 2) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            U[(32 * mt + erow(i)) * S + 64 * (wave - 2) + ecol(nt, i)] = acc[mt][nt][i] * sc;
    }
    __syncthreads();
    if (wave < 2) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float* p = U + (32 * mt + erow(i)) * S + 64 * wave + ecol(nt, i);
            const float g = acc[mt][nt][i] * sc;
            *p = silu_f32(g) * *p;                 // silu(g) * u
          }
    }
    __syncthreads();
    const bool vec = (I & 3) == 0;
#pragma unroll
    for (int i = 0; i < BM * 32 / kThreads; ++i) {
      const int p = threadIdx.x + kThreads * i;
      const int row = p >> 5, c4 = p & 31;
      const int jc = 128 * tn + 4 * c4;
      const f32x4 v = *(const f32x4*)(U + row * S + 4 * c4);
      if (row < cnt && jc < I) store4(Y, y_bf16, I, r0 + row, jc, v, vec);
    }
  }
}

// ------------------------------------------------------------------------------ weight streaming
// Decode-sized routings (a few routed rows per touched expert): every touched expert's weights
// must still be read once, so the work is cut along the weight rows and along K until every CU
// has loads in flight. A work item is (expert e, group g of 32 weight rows, chunk of up to 32
// routed rows of e) and runs on one workgroup of KS waves; wave w takes the w-th share of the
// 64-wide K chunks (KS > 1 only when there are too few items to keep every CU's loads in flight), reads its 32 rows straight into registers (a ring of kSwRing chunks in
// flight) and multiplies them on the matrix cores with the weights as the 32-row A operand:
//  - dense: v_mfma_f32_32x32x16_bf16; lane (n = l % 32, h = l / 32) holds codes k = 32h..32h+31
//    of each 64-k chunk (16 contiguous bytes) and feeds k = 32h + 8s + j to MFMA step s;
//  - 2:4: v_smfmac_f32_32x32x32_bf16 with the stored vals/meta as the compressed A operand and
//    its index operand (the two 16-k halves of step t are the 16-blocks 2h + t of the chunk).
// The activations are the B operand (routed row m = l % 32; rows past the chunk read a zero
// block). Weights are decoded with their E4M3 scale folded in (exact in bf16), so any k order
// inside a chunk is valid as long as both operands use it. With KS > 1 the waves' partial sums
// meet in LDS; wave 0 applies the tensor scale and the epilogue. Items run expert-major, weight group
// next, routed-row chunk fastest, so workgroups that share weight rows run side by side.
// For the SiLU-gate form the 32 rows of group g are gate rows 16g..16g+15 and up rows
// I + 16g..I + 16g + 15; D row n of lane m holds gate row n and up row n + 16 at i and i + 8.
constexpr int kSwRows = 32, kSwM = 32;
constexpr int kSwRing = 4;
__device__ __attribute__((aligned(16))) uint32_t g_sw_zero[16];   // 64 zero bytes

template <int WF>
struct SwChunk {
  u32x4 w;        // dense: 32 codes; 2:4: vals words 0, 1 and the meta word in w[2]
  uint32_t sc;    // two E4M3 scale bytes (16-blocks 2h, 2h + 1 of the chunk)
  u32x4 x[4];     // activation pieces (dense: k = 32h + 8s; 2:4: 16t + 8h and 32 + 16t + 8h)
};

template <int WF, int EPI, int KS, int NCH>
__global__ __launch_bounds__(KS * 64) __attribute__((amdgpu_waves_per_eu(2))) void k_moe_stream(
    const uint16_t* __restrict__ X, int x_rows, int K, const int32_t* __restrict__ row_token,
    const int32_t* __restrict__ off, int E, int R, int N, const uint8_t* __restrict__ w0,
    const uint8_t* __restrict__ w1, const uint8_t* __restrict__ scales, const float* __restrict__ ts,
    void* __restrict__ Y, int y_bf16, int ktiled) {
  // LDS: clamped offsets co[E + 1], first item of each expert pre[E + 1], partial sums
  extern __shared__ int lds_i[];
  const int stride = (E + 4) & ~3;
  int* co = lds_i;
  int* pre = lds_i + stride;
  float* red = (float*)(lds_i + 2 * stride);               // [KS - 1][16][64]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = N / kSwRows;        // weight-row groups per expert
  // offsets clamped into [0, R] (one independent load per entry); the rows of expert e are
  // [co[e], max(co[e + 1], co[e]))
  for (int i = threadIdx.x; i <= E; i += KS * 64) co[i] = min(max(off[i], 0), R);
  __syncthreads();
  if (wave == 0) {                  // item counts per expert and their exclusive prefix
    const int per = (E + 63) / 64;
    const int e0 = min(E, lane * per), e1 = min(E, e0 + per);
    int t = 0;
    for (int e = e0; e < e1; ++e) t += G * ((max(co[e + 1] - co[e], 0) + kSwM - 1) / kSwM);
    int inc = t;
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(inc, d, 64);
      if (lane >= d) inc += v;
    }
    int acc = inc - t;
    for (int e = e0; e < e1; ++e) {
      pre[e] = acc;
      acc += G * ((max(co[e + 1] - co[e], 0) + kSwM - 1) / kSwM);
    }
    if (lane == 63) pre[E] = inc;
  }
  __syncthreads();
  const int total = pre[E];
  const int n = lane & 31, h = lane >> 5;
  // NCH > 0: K / 64 known at compile time, so the chunk loop unrolls completely (no ring
  // registers carried around a loop back-edge, whose moves would wait for the loads in flight)
  const int nch = NCH > 0 ? NCH : K / 64;
  const int c_lo = nch * wave / KS, c_hi = nch * (wave + 1) / KS;   // this wave's chunks
  const size_t rowA = WF == kDense ? K / 2 : K / 4;        // main bytes per weight row
  for (int it = blockIdx.x; it < total; it += gridDim.x) {
    int lo = 0, hi = E;                                      // last e with pre[e] <= it
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pre[mid] <= it) lo = mid; else hi = mid;
    }
    const int e = __builtin_amdgcn_readfirstlane(lo);
    const int o0 = co[e], o1 = max(co[e + 1], o0);
    const int mcs = (o1 - o0 + kSwM - 1) / kSwM;
    const int local = it - pre[e];
    const int g = local / mcs, mc = local % mcs;
    const int r0 = o0 + kSwM * mc, cnt = min(kSwM, o1 - r0);
    // this lane's weight row (A row n) and activation row (B column n)
    const int wrow = EPI == kEpiSilu ? (n < 16 ? 16 * g + n : N / 2 + 16 * g + n - 16) : kSwRows * g + n;
    const size_t er = (size_t)e * N + wrow;                 // row in the [E * N] row space
    const uint8_t* pa;                                      // main weights of chunk 0
    const uint8_t* pm = nullptr;                            // meta of chunk 0
    const uint8_t* ps;                                      // scales of chunk 0
    size_t sa, sm = 0, ss;                                  // byte steps per chunk
    if (!ktiled) {
      pa = w0 + er * rowA + (WF == kDense ? 16 : 8) * h; sa = WF == kDense ? 32 : 16;
      if (WF == kSp24) { pm = w1 + er * (K / 8) + 4 * h; sm = 8; }
      ps = scales + er * (K / 16) + 2 * h; ss = 4;
    } else {                                                // piece (e, c, n) at ((e * nch + c) * N + n) * P
      const size_t base = (size_t)e * nch * N + wrow;
      pa = w0 + base * (WF == kDense ? 32 : 16) + (WF == kDense ? 16 : 8) * h; sa = (size_t)N * (WF == kDense ? 32 : 16);
      if (WF == kSp24) { pm = w1 + base * 8 + 4 * h; sm = (size_t)N * 8; }
      ps = scales + base * 4 + 2 * h; ss = (size_t)N * 4;
    }
    const bool xok = n < cnt;
    int tok = r0 + n;
    if (xok && row_token) tok = min(max(row_token[r0 + n], 0), x_rows - 1);
    const uint16_t* xrow = xok ? X + (size_t)tok * K : (const uint16_t*)g_sw_zero;

    auto load = [&](int c) -> SwChunk<WF> {
      SwChunk<WF> o;
      const bool in = c < c_hi;
      const int cc = in ? c : c_lo;                          // past the share: its first chunk again, times zero
      if constexpr (WF == kDense) {
        o.w = *(const u32x4*)(pa + cc * sa);
      } else {
        const u32x2 v = *(const u32x2*)(pa + cc * sa);
        o.w[0] = v[0]; o.w[1] = v[1]; o.w[2] = *(const uint32_t*)(pm + cc * sm); o.w[3] = 0u;
      }
      o.sc = *(const uint16_t*)(ps + cc * ss);
      const bool live = xok && in;
      const uint16_t* xp = live ? xrow + 64 * c : (const uint16_t*)g_sw_zero;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kx = WF == kDense ? 32 * h + 8 * j : 32 * (j >> 1) + 16 * (j & 1) + 8 * h;
        o.x[j] = *(const u32x4*)(xp + (live ? kx : 0));
      }
      return o;
    };

    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    if (c_lo < c_hi) {
      SwChunk<WF> ring[kSwRing];
#pragma unroll
      for (int u = 0; u < kSwRing; ++u) ring[u] = load(c_lo + u);
#pragma unroll
      for (int c = c_lo; c < c_hi; c += kSwRing) {
#pragma unroll
        for (int u = 0; u < kSwRing; ++u) {
          const SwChunk<WF> cur = ring[u];
          ring[u] = load(c + u + kSwRing);
          // the refill goes out here, a ring length ahead of its use: without this fence the
          // scheduler sinks it next to the arithmetic and the wait for it drains the ring
          __builtin_amdgcn_sched_barrier(0);
          const float f0 = e4m3_f32_sel<0>(cur.sc), f1 = e4m3_f32_sel<1>(cur.sc);
          if constexpr (WF == kDense) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const u32x4 a = fp4x8_bf16(cur.w[s], s < 2 ? f0 : f1);
              acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(cur.x[s]), acc, 0, 0, 0);
            }
          } else {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const u32x4 a = fp4x8_bf16(cur.w[t], t == 0 ? f0 : f1);
              u32x8 b;
              b[0] = cur.x[t][0]; b[1] = cur.x[t][1]; b[2] = cur.x[t][2]; b[3] = cur.x[t][3];
              b[4] = cur.x[2 + t][0]; b[5] = cur.x[2 + t][1]; b[6] = cur.x[2 + t][2]; b[7] = cur.x[2 + t][3];
              const int idx = (int)((cur.w[2] >> (16 * t)) & 0xFFFFu);
              acc = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(as_bf16x8(a), as_bf16x16(b), acc, idx, 0, 0);
            }
          }
        }
      }
    }
    // the K shares meet in LDS; wave 0 holds D[8(i/4) + 4h + i%4][n] for routed row r0 + n
    if (KS > 1) {
      if (wave != 0)
#pragma unroll
        for (int i = 0; i < 16; ++i) red[((wave - 1) * 16 + i) * 64 + lane] = acc[i];
      __syncthreads();
    }
    if (wave == 0) {
#pragma unroll
      for (int w = 1; w < KS; ++w)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] += red[((w - 1) * 16 + i) * 64 + lane];
      if (n < cnt) {
        const float sc = ts[e];
        if constexpr (EPI == kEpiSilu) {
          const int I = N / 2;
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            f32x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float gt = acc[4 * b + i] * sc, up = acc[8 + 4 * b + i] * sc;
              v[i] = silu_f32(gt) * up;                // silu(g) * u
            }
            store4(Y, y_bf16, I, r0 + n, 16 * g + 8 * b + 4 * h, v, (I & 3) == 0);
          }
        } else {
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            f32x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = acc[4 * b + i] * sc;
            store4(Y, y_bf16, N, r0 + n, kSwRows * g + 8 * b + 4 * h, v, (N & 3) == 0);
          }
        }
      }
    }
    if (KS > 1) __syncthreads();                            // red is reused by the next item
  }
}

// ------------------------------------------------------------------------------ weight layout
// 64-k tiled copy of one weight array: dst[e][kt][n][0:P] = src[e][n][kt P : (kt + 1) P], one
// 4-byte word per thread (P is 4, 8, 16 or 32 bytes; row_bytes = (K / 64) P).
__global__ __launch_bounds__(256) void k_pack_ktiles(const uint32_t* __restrict__ src, int64_t E, int64_t N,
                                                     int64_t row_words, int64_t piece_words,
                                                     uint32_t* __restrict__ dst) {
  const int64_t per_e = N * row_words, total = E * per_e;
  for (int64_t o = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; o < total; o += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = o / per_e, rem = o - e * per_e;
    const int64_t kt = rem / (N * piece_words), rem2 = rem - kt * (N * piece_words);
    const int64_t n = rem2 / piece_words, b = rem2 - n * piece_words;
    dst[o] = src[e * per_e + n * row_words + kt * piece_words + b];
  }
}

// ------------------------------------------------------------------------------ combine
// out[t, :] = sum_j w[t, j] * Yd[row_of[t, j], :], j in slot order. Work item (t, c) covers the
// 1024 columns [1024 c, 1024 c + 1024) of token t, four per thread; blocks stride over the
// T * ceil(D / 1024) items. The slots are taken eight at a time: their rows and weights first,
// then the eight row loads together, then the adds in slot order, so a token's k rows are
// fetched in k / 8 round trips rather than k.
constexpr int kCombineCols = 1024, kCombineBatch = 8;

template <bool BF16>
__device__ __forceinline__ f32x4 combine_load(const void* Yd, int r, int D, int d0, bool full) {
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  if (BF16) {
    const uint16_t* y = (const uint16_t*)Yd + (size_t)r * D + d0;
    if (full) {
      const uint2 p = *(const uint2*)y;
      v[0] = __uint_as_float(p.x << 16); v[1] = __uint_as_float(p.x & 0xFFFF0000u);
      v[2] = __uint_as_float(p.y << 16); v[3] = __uint_as_float(p.y & 0xFFFF0000u);
    } else {
      for (int i = 0; i < 4; ++i)
        if (d0 + i < D) v[i] = __uint_as_float((uint32_t)y[i] << 16);
    }
  } else {
    const float* y = (const float*)Yd + (size_t)r * D + d0;
    if (full) v = *(const f32x4*)y;
    else
      for (int i = 0; i < 4; ++i)
        if (d0 + i < D) v[i] = y[i];
  }
  return v;
}

template <bool BF16>
__device__ __forceinline__ void combine_cols(const void* __restrict__ Yd, int R, const int32_t* __restrict__ row_of,
                                             const float* __restrict__ w, int k, int D, float* __restrict__ out,
                                             int64_t t, int d0) {
  const bool full = d0 + 3 < D && (D & 3) == 0;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < k; j0 += kCombineBatch) {
    int r[kCombineBatch];
    float wt[kCombineBatch];
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      const int jj = j0 + u;
      r[u] = jj < k ? row_of[(size_t)t * k + jj] : -1;
      wt[u] = jj < k ? w[(size_t)t * k + jj] : 0.f;
      if (r[u] >= R) r[u] = -1;
    }
    f32x4 v[kCombineBatch];
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u)
      v[u] = r[u] >= 0 ? combine_load<BF16>(Yd, r[u], D, d0, full) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u)
      if (r[u] >= 0)
        for (int i = 0; i < 4; ++i) acc[i] += wt[u] * v[u][i];
  }
  if (full) *(f32x4*)(out + (size_t)t * D + d0) = acc;
  else
    for (int i = 0; i < 4; ++i)
      if (d0 + i < D) out[(size_t)t * D + d0 + i] = acc[i];
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_moe_combine(const void* __restrict__ Yd, int R,
                                                     const int32_t* __restrict__ row_of,
                                                     const float* __restrict__ w, int k, int D,
                                                     float* __restrict__ out, int64_t T) {
  const int64_t chunks = (D + kCombineCols - 1) / kCombineCols;
  for (int64_t item = blockIdx.x; item < T * chunks; item += gridDim.x) {
    const int64_t t = item / chunks;
    const int d0 = (int)(item - t * chunks) * kCombineCols + 4 * threadIdx.x;
    if (d0 < D) combine_cols<BF16>(Yd, R, row_of, w, k, D, out, t, d0);
  }
}

template <int WF, int EPI, int BM, bool SMF = false>
hipError_t launch_moe_gemm_t(const MoeGemmArgs& a, hipStream_t s) {
  constexpr int bytes = moe_lds_bytes<WF, BM>();
  static_assert(2 * bytes <= 160 * 1024, "LDS budget: 64-row tiles run at least two workgroups per CU");
  hipError_t e = hipFuncSetAttribute((const void*)k_moe_gemm<WF, EPI, BM, SMF>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  // upper bound of the tile count: R / BM + min(E, R) (each expert's last tile may be partial)
  const long tiles = (a.R + BM - 1) / BM + (a.E < a.R ? a.E : a.R);
  if (tiles == 0) return hipSuccess;
  const int ntiles = EPI == kEpiSilu ? (int)((a.N / 2 + 127) / 128) : (int)((a.N + kBN - 1) / kBN);
  if (tiles * ntiles > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_moe_gemm<WF, EPI, BM, SMF>), dim3((unsigned)(tiles * ntiles)), dim3(kThreads), bytes, s,
                     a.X, (int)a.x_rows, (int)a.K, a.row_token, a.offsets, a.E, (int)a.R, (int)a.N, a.w0, a.w1,
                     a.scales, a.ts, a.Y, a.y_bf16, ntiles, a.ktiled);
  return hipGetLastError();
}

template <int WF, int EPI>
hipError_t launch_moe_gemm_both(const MoeGemmArgs& a, hipStream_t s) {
  if constexpr (WF == kSp24)
    if (a.smfmac) return launch_moe_gemm_t<WF, EPI, 64, true>(a, s);
  return launch_moe_gemm_t<WF, EPI, 64>(a, s);
}

template <int WF, int EPI, int NCH>
hipError_t launch_moe_stream_n(const MoeGemmArgs& a, hipStream_t s) {
  const int G = (int)(a.N / kSwRows);
  // items <= G * (touched experts + R / 32) <= G * (min(E, R) + R / 32); extra workgroups exit
  // after the item scan, and a workgroup loops over items when the grid is capped
  const long touched = a.E < a.R ? a.E : a.R;
  const long items = (long)G * (touched + a.R / kSwM);
  if (items == 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<long>(items, 4096);
  const size_t stride = (size_t)((a.E + 4) & ~3);
  // Few items and a long K: split K over four waves per item so that enough loads are in flight
  if ((long)G * touched < 2048 && a.K / 64 >= 16) {
    const size_t lds = 2 * stride * sizeof(int) + 3 * 16 * 64 * sizeof(float);
    hipLaunchKernelGGL((k_moe_stream<WF, EPI, 4, NCH>), dim3(grid), dim3(4 * 64), lds, s, a.X, (int)a.x_rows,
                       (int)a.K, a.row_token, a.offsets, a.E, (int)a.R, (int)a.N, a.w0, a.w1, a.scales, a.ts, a.Y,
                       a.y_bf16, a.ktiled);
  } else {
    const size_t lds = 2 * stride * sizeof(int);
    hipLaunchKernelGGL((k_moe_stream<WF, EPI, 1, NCH>), dim3(grid), dim3(64), lds, s, a.X, (int)a.x_rows, (int)a.K,
                       a.row_token, a.offsets, a.E, (int)a.R, (int)a.N, a.w0, a.w1, a.scales, a.ts, a.Y, a.y_bf16,
                       a.ktiled);
  }
  return hipGetLastError();
}

// the expert shapes of the grouped FFN (D = 2048 and I = 512: 32 and 8 chunks) get a fully
// unrolled chunk loop; other K run the generic loop
template <int WF, int EPI>
hipError_t launch_moe_stream_t(const MoeGemmArgs& a, hipStream_t s) {
  if (a.K == 2048) return launch_moe_stream_n<WF, EPI, 32>(a, s);
  if (a.K == 512) return launch_moe_stream_n<WF, EPI, 8>(a, s);
  return launch_moe_stream_n<WF, EPI, 0>(a, s);
}

}  // namespace

size_t moe_route_workspace(int64_t F, int E) {
  if (F == 0) return 0;
  const size_t B = (size_t)((F + kRouteChunk - 1) / kRouteChunk);
  return (B + 1) * (size_t)E * sizeof(int32_t);      // histogram [B][E], then totals [E]
}

hipError_t launch_moe_route(const int32_t* ids, int64_t T, int k, int E, int32_t* offsets, int32_t* row_token,
                            int32_t* row_slot, int32_t* row_of, int64_t* bad, void* ws, hipStream_t s) {
  const int F = (int)(T * k);
  const int B = (F + kRouteChunk - 1) / kRouteChunk;
  if (B == 0) {   // nothing to place: every offset and the bad count are zero
    hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(1024), 0, s, (const int32_t*)nullptr, E, 0, offsets, bad);
    return hipGetLastError();
  }
  if (F <= kRouteSmallMax) {
    hipLaunchKernelGGL(k_route_small, dim3(1), dim3(kRouteThreads), 5 * E * sizeof(int32_t), s, ids, F, k, E, offsets,
                       bad, row_token, row_slot, row_of);
    return hipGetLastError();
  }
  int32_t* hist = (int32_t*)ws;
  int32_t* tot = hist + (size_t)B * E;
  hipLaunchKernelGGL(k_route_hist, dim3(B), dim3(kRouteThreads), E * sizeof(int32_t), s, ids, F, E, hist);
  hipLaunchKernelGGL(k_route_colscan, dim3((E + kRouteThreads / 64 - 1) / (kRouteThreads / 64)), dim3(kRouteThreads), 0,
                     s, hist, B, E, tot);
  hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(1024), 0, s, (const int32_t*)tot, E, F, offsets, bad);
  hipLaunchKernelGGL(k_route_scatter, dim3(B), dim3(kRouteThreads), 5 * E * sizeof(int32_t), s, ids, F, k, E,
                     (const int32_t*)hist, (const int32_t*)offsets, row_token, row_slot, row_of);
  return hipGetLastError();
}

hipError_t launch_moe_stream(const MoeGemmArgs& a, hipStream_t s) {
  if (a.sparse) return a.silu ? launch_moe_stream_t<kSp24, kEpiSilu>(a, s) : launch_moe_stream_t<kSp24, kEpiNone>(a, s);
  return a.silu ? launch_moe_stream_t<kDense, kEpiSilu>(a, s) : launch_moe_stream_t<kDense, kEpiNone>(a, s);
}

hipError_t launch_moe_gemm(const MoeGemmArgs& a, hipStream_t s) {
  if (a.sparse) return a.silu ? launch_moe_gemm_both<kSp24, kEpiSilu>(a, s) : launch_moe_gemm_both<kSp24, kEpiNone>(a, s);
  return a.silu ? launch_moe_gemm_both<kDense, kEpiSilu>(a, s) : launch_moe_gemm_both<kDense, kEpiNone>(a, s);
}

hipError_t launch_moe_pack_ktiles(const uint8_t* src, int64_t E, int64_t N, int64_t row_bytes, int64_t piece,
                                  uint8_t* dst, hipStream_t s) {
  const int64_t words = E * N * (row_bytes / 4);
  if (words == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((words + 255) / 256, 16384);
  hipLaunchKernelGGL(k_pack_ktiles, dim3((unsigned)blocks), dim3(256), 0, s, (const uint32_t*)src, E, N, row_bytes / 4,
                     piece / 4, (uint32_t*)dst);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const void* Yd, int yd_bf16, int64_t R, const int32_t* row_of, const float* w,
                              int64_t T, int k, int64_t D, float* out, hipStream_t s) {
  const int64_t items = T * ((D + kCombineCols - 1) / kCombineCols);
  const dim3 grid((unsigned)std::min<int64_t>(items, 1 << 20));
  if (yd_bf16)
    hipLaunchKernelGGL(k_moe_combine<true>, grid, dim3(256), 0, s, Yd, (int)R, row_of, w, k, (int)D, out, T);
  else
    hipLaunchKernelGGL(k_moe_combine<false>, grid, dim3(256), 0, s, Yd, (int)R, row_of, w, k, (int)D, out, T);
  return hipGetLastError();
}

}  // namespace ssn
