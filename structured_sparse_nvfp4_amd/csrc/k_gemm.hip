// Prefill-shaped and square products (M > 16): 256x256 output tiles on the matrix cores (and
// 128x256 tiles for a half-empty last round of them).
//
// The square and prefill shapes are compute-bound ("NVFP4 Without FP4 Hardware", ai-muninn.com,
// section on prefill: unpacking is extra work on top of the dense product), so the design keeps
// the matrix cores fed and spends as little vector-ALU time per weight as possible:
//  - every operand of a 64-wide K stage (activation tile [256][64] bf16 and the 4-bit weights
//    of the 256 output columns with their scales) is copied HBM -> LDS by the direct-to-LDS
//    loads, three stages in flight; the kernel waits for them with explicit vmcnt counts, and
//    no register load is left in the loop for the compiler to wait on conservatively;
//  - 16-byte chunks are XOR-swizzled so that matrix-operand reads are free of bank conflicts;
//  - every wave decodes its own weights from LDS into matrix operands in registers: a weight is
//    decoded once per output tile and never written back.
//
// Dense and 2:4-expanded products (v_mfma_f32_32x32x16_bf16, weights = A, activations = B, so
//   each 32 x 32 block is a block of Y^T and a lane ends with four consecutive outputs of a row):
//   wave w owns all TM rows x columns [64w, 64w + 64) of the tile: TM / 32 x 2 blocks of 32 x 32.
//   Lane l (r = l % 32, h = l / 32) feeds k = 8h..8h+7 of each 16-wide MFMA step. The kernel
//   maps MFMA step s of a 64-wide stage to k = 32h + 8s + j, so one lane's weights for a whole
//   stage are 16 contiguous code bytes (32 codes, two E4M3 scale blocks).
// 2:4 products on the sparse matrix cores (v_smfmac_f32_32x32x32_bf16, weights = compressed A,
//   activations = B, blocks of Y^T as above): wave (wn, wm) owns 128 weight rows x 128
//   activation rows (4 x 4 blocks). The two 16-wide halves of MFMA step t take the
//   16-blocks 2H + t of the stage (H = 0, 1), so each lane's compressed weights for a stage are
//   8 contiguous vals bytes, 4 meta bytes and 2 scale bytes. The compressed layout of this
//   library is the SMFMAC A operand and index operand as stored ("NVFP4 vs 2:4 sparse",
//   robertz.co, section "What 2:4 actually is": two kept values plus a 2-bit index each).
//
// K must be a multiple of 64 (whole stages; every per-row weight piece is then aligned).
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "device_once.hpp"
#include "launch.hpp"
#include "pipeline.hpp"
#include "tile.hpp"

namespace ssn {
namespace {

constexpr int kTM = 256, kTN = 256, kTK = 64;   // output tile and K-stage
constexpr int kStages = 3;                       // stages resident in LDS
constexpr int kThreads = 256;
// One LDS ring slot (bytes) of a tile with TM activation rows and 256 weight rows (tile-local).
//   X      [TM][128 B]   activation k-chunk c of row r at physical chunk c ^ swz(r)
//   dense: codes [256][32 B]  half h of row r at physical half h ^ ((r >> 3) & 1)
//   2:4:   vals  [256][16 B], meta [256][8 B]
//   scales [256][4 B]   (the four 16-blocks of the stage)
template <int WF, int TM = kTM>
struct Slot {
  static constexpr int kX = 0;
  static constexpr int kW = TM * kTK * 2;
  static constexpr int kMeta = WF == kDense ? 0 : kW + kTN * 16;
  static constexpr int kSc = WF == kDense ? kW + kTN * 32 : kMeta + kTN * 8;
  static constexpr int kBytes = kSc + kTN * 4;
  // direct loads per wave per stage: activations TM / 32, weights (dense 2 / 2:4 1 + 2), scales 1
  static constexpr int kXLoads = TM / 32;
  static constexpr int kLoads = WF == kDense ? kXLoads + 2 + 1 : kXLoads + 1 + 2 + 1;
};

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

// ---- one K stage of operands -> LDS slot. Per-lane byte offsets are computed once; each
// stage only moves the wave-uniform base pointers, so the loads take a scalar base plus a
// 32-bit vector offset. Rows beyond M or N are clamped to the last row (their results are not
// stored). Every boundary issues the same loads (a stage past the end re-reads the last one
// into a free slot), so the loads a wait must cover are a fixed count.
template <int WF, int TM = kTM>
struct StageSrc {
  const char* xb;   // activations of rows m0.. at k = 0
  const char* wb;   // codes (dense) or vals (2:4) of rows n0.. at k = 0
  const char* mb;   // meta of rows n0.. (2:4)
  const char* sb;   // scales of rows n0..
  uint32_t xo[TM / 32], wo[2], mo[2], so;
};

template <int WF, int TM = kTM>
__device__ __forceinline__ StageSrc<WF, TM> stage_src(const uint16_t* X, const uint8_t* w0, const uint8_t* w1,
                                                  const uint8_t* scales, int M, int N, int K, int m0, int n0,
                                                  int wave, int lane) {
  StageSrc<WF, TM> o;
  o.xb = (const char*)(X + (size_t)m0 * K);
  o.wb = (const char*)w0 + (size_t)n0 * (WF == kDense ? K / 2 : K / 4);
  o.mb = WF == kDense ? nullptr : (const char*)w1 + (size_t)n0 * (K / 8);
  o.sb = (const char*)scales + (size_t)n0 * (K / 16);
  // activations: load i of the wave writes row 8 (TM / 32 wave + i) + l / 8, physical chunk l % 8
#pragma unroll
  for (int i = 0; i < TM / 32; ++i) {
    const int r = 8 * (TM / 32 * wave + i) + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    o.xo[i] = (uint32_t)((min(m0 + r, M - 1) - m0) * K + 8 * c) * 2u;
  }
  if constexpr (WF == kDense) {
    // codes: load i writes row 32 (2 wave + i) + l / 2, physical half l % 2
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 32 * (2 * wave + i) + (lane >> 1);
      const int hl = (lane & 1) ^ ((r >> 3) & 1);
      o.wo[i] = (uint32_t)(min(n0 + r, N - 1) - n0) * (uint32_t)(K / 2) + 16u * hl;
      o.mo[i] = 0u;
    }
  } else {
    // vals: one load of row 64 wave + l (16 B); meta: load i writes row 32 (2 wave + i) + l / 2
    o.wo[0] = (uint32_t)(min(n0 + 64 * wave + lane, N - 1) - n0) * (uint32_t)(K / 4);
    o.wo[1] = 0u;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 32 * (2 * wave + i) + (lane >> 1);
      o.mo[i] = (uint32_t)(min(n0 + r, N - 1) - n0) * (uint32_t)(K / 8) + 4u * (lane & 1);
    }
  }
  o.so = (uint32_t)(min(n0 + 64 * wave + lane, N - 1) - n0) * (uint32_t)(K / 16);
  return o;
}

template <int WF, int TM = kTM>
__device__ __forceinline__ void issue_stage(const StageSrc<WF, TM>& g, int st, char* slot, int wave) {
  using L = Slot<WF, TM>;
  const auto xr = buf_rsrc(g.xb), wr = buf_rsrc(g.wb), sr = buf_rsrc(g.sb);
#pragma unroll
  for (int i = 0; i < TM / 32; ++i) lds_dma16(xr, g.xo[i], st * (kTK * 2), slot + L::kX + (TM / 32 * wave + i) * 1024);
  if constexpr (WF == kDense) {
#pragma unroll
    for (int i = 0; i < 2; ++i) lds_dma16(wr, g.wo[i], st * (kTK / 2), slot + L::kW + (2 * wave + i) * 1024);
  } else {
    const auto mr = buf_rsrc(g.mb);
    lds_dma16(wr, g.wo[0], st * (kTK / 4), slot + L::kW + wave * 1024);
#pragma unroll
    for (int i = 0; i < 2; ++i) lds_dma4(mr, g.mo[i], st * (kTK / 8), slot + L::kMeta + (2 * wave + i) * 256);
  }
  lds_dma4(sr, g.so, st * (kTK / 16), slot + L::kSc + wave * 256);
}

// Load `idx` of a stage (scales, then the weight loads, then the activation loads): the loads of
// a stage can be issued in four parts spread over the MFMA steps instead of in one burst.
template <int WF, int TM>
__device__ __forceinline__ void issue_one(const StageSrc<WF, TM>& g, int st, char* slot, int wave, int idx) {
  using L = Slot<WF, TM>;
  constexpr int nW = WF == kDense ? 2 : 3;
  if (idx == 0) {
    lds_dma4(buf_rsrc(g.sb), g.so, st * (kTK / 16), slot + L::kSc + wave * 256);
  } else if (idx <= nW) {
    const int i = idx - 1;
    if constexpr (WF == kDense) {
      lds_dma16(buf_rsrc(g.wb), g.wo[i], st * (kTK / 2), slot + L::kW + (2 * wave + i) * 1024);
    } else {
      if (i == 0) lds_dma16(buf_rsrc(g.wb), g.wo[0], st * (kTK / 4), slot + L::kW + wave * 1024);
      else lds_dma4(buf_rsrc(g.mb), g.mo[i - 1], st * (kTK / 8), slot + L::kMeta + (2 * wave + i - 1) * 256);
    }
  } else {
    const int i = idx - 1 - nW;
    lds_dma16(buf_rsrc(g.xb), g.xo[i], st * (kTK * 2), slot + L::kX + (TM / 32 * wave + i) * 1024);
  }
}

template <int WF, int TM>
constexpr int part_loads(int part) {
  constexpr int n = Slot<WF, TM>::kLoads, per = (n + 3) / 4;
  return part * per >= n ? 0 : ((part + 1) * per > n ? n - part * per : per);
}

template <int WF, int TM, int PART>
__device__ __forceinline__ void issue_part(const StageSrc<WF, TM>& g, int st, char* slot, int wave) {
  constexpr int per = (Slot<WF, TM>::kLoads + 3) / 4;
#pragma unroll
  for (int idx = PART * per; idx < (PART + 1) * per && idx < Slot<WF, TM>::kLoads; ++idx) issue_one<WF, TM>(g, st, slot, wave, idx);
}

// One lane's weights for one stage: dense 32 codes, or 2:4 (vals word 0, vals word 1, meta)
template <int WF, int TM = kTM>
__device__ __forceinline__ u32x4 lds_w(const char* slot, int r, int h) {
  using L = Slot<WF, TM>;
  if constexpr (WF == kDense) {
    return *(const u32x4*)(slot + L::kW + r * 32 + 16 * (h ^ ((r >> 3) & 1)));
  } else {
    const u32x2 v = *(const u32x2*)(slot + L::kW + r * 16 + 8 * h);
    u32x4 o;
    o[0] = v[0]; o[1] = v[1]; o[2] = *(const uint32_t*)(slot + L::kMeta + r * 8 + 4 * h); o[3] = 0u;
    return o;
  }
}

// ---------------------------------------------------------------------------------------------
// Dense (or 2:4 expanded to dense) x activations on v_mfma_f32_32x32x16_bf16.
// WGM x (4 / WGM) waves: wave (wm, wn) owns activation rows [TM/WGM * wm, +TM/WGM) and
// weight rows [64 WGM * wn, +64 WGM) of the tile, MB x NB blocks of 32 x 32. With WGM = 2 each
// activation operand read from LDS feeds four MFMAs instead of two (half the LDS read traffic
// of WGM = 1), and each weight is decoded by two waves instead of one.
// Tile `tile` of the first `total` tiles in the tile order of an M x N product (Y row stride ldy).
template <int WF, int WGM, int TM, bool YB>
__device__ __forceinline__ void mfma_tile(const uint16_t* __restrict__ X, int M, int N, int K,
                                          const uint8_t* __restrict__ w0, const uint8_t* __restrict__ w1,
                                          const uint8_t* __restrict__ scales, const float* __restrict__ ts,
                                          void* __restrict__ Y, int ldy, int tile, int total, char* lds) {
  using L = Slot<WF, TM>;
  constexpr int MB = TM / 32 / WGM, NB = 2 * WGM;       // 32 x 32 blocks per wave along M and N
  constexpr int VS = NB == 2 ? 3 : 5, VB = NB == 2 ? 3 : 6;   // decode instructions per MFMA slot
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave % (4 / WGM), wm = wave / (4 / WGM);
  const int tiles_m = (M + TM - 1) / TM, tiles_n = (N + kTN - 1) / kTN;
  int tm, tn;
  tile_of(tile, total, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * TM, n0 = tn * kTN;
  const int r32 = lane & 31, h = lane >> 5;
  const int nst = K / kTK, last = nst - 1;
  const int am = 32 * MB * wm, bn0 = 32 * NB * wn;  // first activation / weight row of the wave
  const float st_scale = *ts;   // loaded here: its latency is hidden by the K loop, not the epilogue

  f32x16 acc[MB][NB];
#pragma unroll
  for (int mt = 0; mt < MB; ++mt)
#pragma unroll
    for (int nt = 0; nt < NB; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.f;

  // Software pipeline over K stages (ring of three LDS slots). Stage st's loads are issued at
  // the boundary of stage st - 3 and waited for at the boundary of stage st - 1. The boundary
  // (wait, barrier, next loads, first operands of the next stage) sits before the last MFMA
  // step of a stage, so that step's MFMAs cover it.
  const StageSrc<WF, TM> src = stage_src<WF, TM>(X, w0, w1, scales, M, N, K, m0, n0, wave, lane);
  issue_stage<WF, TM>(src, 0, lds, wave);
  issue_stage<WF, TM>(src, min(1, last), lds + L::kBytes, wave);
  issue_part<WF, TM, 0>(src, min(2, last), lds + 2 * L::kBytes, wave);

  u32x4 wc[NB];         // this stage's weights (per column block) and their scale pair
  uint32_t wsc[NB];
  u32x4 abuf[2][MB];    // activation operands, double-buffered across MFMA steps
  bf16x8 bcur[NB];      // decoded weight operands of the current step

  // the scale word is kept as loaded (all four 16-blocks of the stage) and this lane's pair is
  // picked in the decode: a shift here would make the wave wait for the LDS read before the
  // MFMAs that follow a stage boundary
  auto load_w_regs = [&](const char* slot, u32x4 (&c)[NB], uint32_t (&sc)[NB]) {
#pragma unroll
    for (int nt = 0; nt < NB; ++nt) {
      const int r = bn0 + 32 * nt + r32;
      c[nt] = lds_w<WF, TM>(slot, r, h);
      sc[nt] = *(const uint32_t*)(slot + L::kSc + r * 4);
    }
  };
  auto decode = [&](const u32x4 (&c)[NB], const uint32_t (&sc)[NB], int s, bf16x8 (&b)[NB]) {
#pragma unroll
    for (int nt = 0; nt < NB; ++nt) {
      const uint32_t pair = sc[nt] >> (16 * h);   // 16-blocks 2h, 2h + 1
      const float f = s < 2 ? e4m3_f32_sel<0>(pair) : e4m3_f32_sel<1>(pair);
      b[nt] = as_bf16x8(fp4x8_bf16(codes_step<WF>(c[nt], s), f));
    }
  };
  // Byte offset in a slot of the activation piece of MFMA step s for row block mt: row
  // am + 32 mt + r32, chunk (4h + s) ^ swz(row). With am a multiple of 64 the swizzle depends on
  // mt only through mt & 1, so eight per-lane offsets (s, mt & 1) plus the constant 4096 mt
  // address every read (the constant folds into the instruction's offset field).
  static_assert(WGM == 1 || WGM == 2, "am = 32 MB wm must be a multiple of 64");
  uint32_t xoff[4][2];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int p = 0; p < 2; ++p) xoff[s][p] = (uint32_t)((am + r32) * 128 + 16 * ((4 * h + s) ^ swz(r32 + 32 * p)));
  auto read_a = [&](const char* slot, int s, u32x4 (&a)[MB]) {
#pragma unroll
    for (int mt = 0; mt < MB; ++mt) a[mt] = *(const u32x4*)(slot + 4096 * mt + xoff[s][mt & 1]);
  };
  auto mfmas = [&](const u32x4 (&a)[MB], const bf16x8 (&b)[NB]) {
#pragma unroll
    for (int mt = 0; mt < MB; ++mt) {
      const bf16x8 av = as_bf16x8(a[mt]);
#pragma unroll
      for (int nt = 0; nt < NB; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[nt], av, acc[mt][nt], 0, 0, 0);
    }
  };

  wait_vmcnt<L::kLoads + part_loads<WF, TM>(0)>();
  stage_barrier();
  load_w_regs(lds, wc, wsc);
  read_a(lds, 0, abuf[0]);
  decode(wc, wsc, 0, bcur);

  auto stage = [&](auto slot_c, int st) {
    constexpr int S = decltype(slot_c)::value;
    const char* slot = lds + S * L::kBytes;
    const char* next = lds + ((S + 1) % kStages) * L::kBytes;
    char* fill = lds + ((S + 2) % kStages) * L::kBytes;   // stage st + 2: its first part is in flight
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      // stage st + 2's loads, issued in four parts over the MFMA steps instead of one burst at
      // the boundary (the load address/command queues were filling)
      if (s == 0) issue_part<WF, TM, 1>(src, min(st + 2, last), fill, wave);
      else if (s == 1) issue_part<WF, TM, 2>(src, min(st + 2, last), fill, wave);
      else issue_part<WF, TM, 3>(src, min(st + 2, last), fill, wave);
      read_a(slot, s + 1, abuf[(s + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);         // operand reads go out first, a whole step ahead
      bf16x8 bn[NB];
      decode(wc, wsc, s + 1, bn);
      mfmas(abuf[s & 1], bcur);
      interleave_mfma_valu<1, MB * NB - 1, VS>();
#pragma unroll
      for (int nt = 0; nt < NB; ++nt) bcur[nt] = bn[nt];
    }
    // boundary: this wave's reads of slot S are done (their values are in registers) ...
    __builtin_amdgcn_sched_barrier(0);           // the MFMAs above stay above the barrier
    __builtin_amdgcn_s_waitcnt(0xC07F);          // lgkmcnt(0)
    wait_vmcnt<L::kLoads>();                     // ... and stage st + 1 has landed
    stage_barrier();
    issue_part<WF, TM, 0>(src, min(st + 3, last), lds + S * L::kBytes, wave);
    u32x4 wn_[NB];
    uint32_t wsn[NB];
    bf16x8 bn[NB];
    load_w_regs(next, wn_, wsn);
    __builtin_amdgcn_sched_barrier(0);           // the weights go out first: the decode below waits only for them
    read_a(next, 0, abuf[0]);
    __builtin_amdgcn_sched_barrier(0);
    decode(wn_, wsn, 0, bn);
    mfmas(abuf[1], bcur);                        // last MFMA step of stage st
    interleave_mfma_valu<4, MB * NB - 4, VB>();  // the first MFMAs cover the operand reads
#pragma unroll
    for (int nt = 0; nt < NB; ++nt) { wc[nt] = wn_[nt]; wsc[nt] = wsn[nt]; bcur[nt] = bn[nt]; }
  };
  for (int st = 0; st < nst; st += 3) {
    stage(std::integral_constant<int, 0>{}, st);
    if (st + 1 < nst) stage(std::integral_constant<int, 1>{}, st + 1);
    if (st + 2 < nst) stage(std::integral_constant<int, 2>{}, st + 2);
  }
  wait_vmcnt<0>();   // the duplicate stages past the end have landed before the wave exits

  // epilogue: the blocks are Y^T (weights = A, activations = B), so lane (r32, h) holds
  // Y[m][n .. n + 3] for m = 32 mt + r32 and n = 32 nt + 8 g + 4 h (plus the wave's offsets) in
  // acc[mt][nt][4g .. 4g + 3]. Each 32-row block of the wave (32 rows x 32 NB columns) is staged
  // in LDS and leaves as row-contiguous pieces: bf16 output is rounded first and staged as
  // 16-byte pieces of 8 values (piece c of row r at position c ^ (r & 7)), so a read of eight
  // lanes covers one 128-byte row and every lane stores 16 bytes; f32 output is staged as
  // 16-byte pieces of 4 values (piece q at q ^ (r & 7)).
  __syncthreads();                                  // every wave is done with the ring slots
  // the lane index again, from the lane mask count: a value the compiler cannot take from the
  // prologue, so it is not kept in a register (or spilled) across the K loop
  const int el = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int er32 = el & 31, eh = el >> 5;
  if constexpr (YB) {                               // bf16 output (y_bf16 != 0)
    constexpr int kPR = 4 * NB;                     // 16-byte pieces (8 bf16) per staged row
    char* T = lds + wave * (32 * kPR * 16);
    const bool vec = (ldy & 7) == 0 && ((uintptr_t)Y & 15) == 0;
#pragma unroll
    for (int mt = 0; mt < MB; ++mt) {
#pragma unroll
      for (int nt = 0; nt < NB; ++nt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16& a = acc[mt][nt];
          u32x2 w;
          w[0] = pk_bf16_rne(a[4 * g] * st_scale, a[4 * g + 1] * st_scale);
          w[1] = pk_bf16_rne(a[4 * g + 2] * st_scale, a[4 * g + 3] * st_scale);
          const int c = 4 * nt + g;
          *(u32x2*)(T + er32 * (16 * kPR) + 16 * (c ^ (er32 & 7)) + 8 * eh) = w;
        }
      __builtin_amdgcn_s_waitcnt(0xC07F);           // lgkmcnt(0): this wave's stores to T are done
      const int c = el % kPR;
#pragma unroll
      for (int j = 0; j < 32 * kPR / 64; ++j) {
        const int r = el / kPR + (64 / kPR) * j;
        const u32x4 v = *(const u32x4*)(T + r * (16 * kPR) + 16 * (c ^ (r & 7)));
        const int m = m0 + am + 32 * mt + r;
        if (m < M) store8_bf16_ld(Y, ldy, N, m, n0 + bn0 + 8 * c, v, vec);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);           // reads of T done before the next block overwrites it
    }
  } else {
    constexpr int kPR = 8 * NB;                     // 16-byte pieces (4 f32) per staged row
    float* T = (float*)(lds + wave * (32 * kPR * 16));
    const bool vec = (ldy & 3) == 0 && ((uintptr_t)Y & 15) == 0;
#pragma unroll
    for (int mt = 0; mt < MB; ++mt) {
#pragma unroll
      for (int nt = 0; nt < NB; ++nt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = acc[mt][nt][4 * g + i];
          const int q = 8 * nt + 2 * g + eh;
          *(f32x4*)(T + er32 * (4 * kPR) + 4 * (q ^ (er32 & 7))) = v;
        }
      __builtin_amdgcn_s_waitcnt(0xC07F);
      const int p = el % kPR;
#pragma unroll
      for (int j = 0; j < 32 * kPR / 64; ++j) {
        const int r = el / kPR + (64 / kPR) * j;
        const f32x4 v = *(const f32x4*)(T + r * (4 * kPR) + 4 * (p ^ (r & 7))) * st_scale;
        const int m = m0 + am + 32 * mt + r;
        if (m < M) store4_ld(Y, 0, ldy, N, m, n0 + bn0 + 4 * p, v, vec);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);
    }
  }
}

// The first `nbig` workgroups take the 256 x 256 tiles of the product in tile order. When the
// last round of those would leave more than half of the CUs idle, the tiles of that round (the
// bottom-right rectangle from activation row row0 and weight row col0) are taken instead by the
// workgroups after them as twice as many 128 x 256 tiles: dispatched last, they go to the CUs
// that finish first.
template <int WF, bool YB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_gemm_mfma(const uint16_t* __restrict__ X, int M, int N, int K, const uint8_t* __restrict__ w0,
                 const uint8_t* __restrict__ w1, const uint8_t* __restrict__ scales, const float* __restrict__ ts,
                 void* __restrict__ Y, int nbig, int row0, int col0) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  if ((int)blockIdx.x < nbig) {
    mfma_tile<WF, 1, kTM, YB>(X, M, N, K, w0, w1, scales, ts, Y, N, blockIdx.x, nbig, lds);
  } else {
    const size_t wrow = WF == kDense ? K / 2 : K / 4;
    mfma_tile<WF, 1, kTM / 2, YB>(X + (size_t)row0 * K, M - row0, N - col0, K, w0 + (size_t)col0 * wrow,
                                  WF == kDense ? w1 : w1 + (size_t)col0 * (K / 8), scales + (size_t)col0 * (K / 16),
                                  ts, (char*)Y + ((size_t)row0 * N + col0) * (YB ? 2 : 4), N, blockIdx.x - nbig,
                                  gridDim.x - nbig, lds);
  }
}

// ---------------------------------------------------------------------------------------------
// 2:4 weights on the sparse matrix cores: Y^T tile = W (compressed A) x X^T (B).
template <bool YB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_gemm_smfmac(const uint16_t* __restrict__ X, int M, int N, int K, const uint8_t* __restrict__ vals,
                   const uint8_t* __restrict__ meta, const uint8_t* __restrict__ scales,
                   const float* __restrict__ ts, void* __restrict__ Y, int y_bf16) {
  using L = Slot<kSp24>;
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave & 1, wm = wave >> 1;
  const int tiles_m = (M + kTM - 1) / kTM, tiles_n = (N + kTN - 1) / kTN;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * kTM, n0 = tn * kTN;
  const int r32 = lane & 31, q = lane >> 5;
  const int nst = K / kTK, last = nst - 1;
  const float st_scale = *ts;   // loaded here: its latency is hidden by the K loop, not the epilogue

  f32x16 acc[4][4];
#pragma unroll
  for (int at = 0; at < 4; ++at)
#pragma unroll
    for (int bt = 0; bt < 4; ++bt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[at][bt][i] = 0.f;

  const StageSrc<kSp24> src = stage_src<kSp24>(X, vals, meta, scales, M, N, K, m0, n0, wave, lane);
  issue_stage<kSp24>(src, 0, lds, wave);
  issue_stage<kSp24>(src, min(1, last), lds + L::kBytes, wave);
  issue_stage<kSp24>(src, min(2, last), lds + 2 * L::kBytes, wave);

  u32x4 wa[4];          // this stage's compressed weights (vals, vals, meta) per row block
  uint32_t wsc[4];
  u32x8 bx[4];          // activation operands of the current MFMA step
  bf16x8 acur[4];       // decoded kept weights of the current step

  auto load_w_regs = [&](const char* slot, u32x4 (&c)[4], uint32_t (&sc)[4]) {
#pragma unroll
    for (int at = 0; at < 4; ++at) {
      const int r = 128 * wn + 32 * at + r32;
      c[at] = lds_w<kSp24>(slot, r, q);
      sc[at] = *(const uint32_t*)(slot + L::kSc + r * 4) >> (16 * q);   // 16-blocks 2q, 2q + 1
    }
  };
  // B (activations) of MFMA step t: col r32 of block bt; k = 16t + 8q + j (j < 8) and
  // 32 + 16t + 8q + j - 8 (j >= 8)
  // per-lane byte offsets of those pieces: row 128 wm + 32 bt + r32, chunk c ^ swz(row), where
  // the swizzle depends on bt only through bt & 1 (the constant 4096 bt folds into the
  // instruction's offset field)
  uint32_t xoff[2][2][2];   // [t][lo / hi][bt & 1]
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int p = 0; p < 2; ++p)
        xoff[t][u][p] = (uint32_t)((128 * wm + r32) * 128 + 16 * ((4 * u + 2 * t + q) ^ swz(r32 + 32 * p)));
  auto read_b = [&](const char* slot, int t, u32x8 (&b)[4]) {
#pragma unroll
    for (int bt = 0; bt < 4; ++bt) {
      const u32x4 lo = *(const u32x4*)(slot + 4096 * bt + xoff[t][0][bt & 1]);
      const u32x4 hi = *(const u32x4*)(slot + 4096 * bt + xoff[t][1][bt & 1]);
      b[bt][0] = lo[0]; b[bt][1] = lo[1]; b[bt][2] = lo[2]; b[bt][3] = lo[3];
      b[bt][4] = hi[0]; b[bt][5] = hi[1]; b[bt][6] = hi[2]; b[bt][7] = hi[3];
    }
  };
  // A (weights): the 8 kept values of 16-block 2q + t
  auto decode = [&](const u32x4 (&c)[4], const uint32_t (&sc)[4], int t, bf16x8 (&a)[4]) {
#pragma unroll
    for (int at = 0; at < 4; ++at) {
      const float f = t == 0 ? e4m3_f32_sel<0>(sc[at]) : e4m3_f32_sel<1>(sc[at]);
      a[at] = as_bf16x8(fp4x8_bf16(c[at][t], f));
    }
  };
  auto mfmas = [&](const bf16x8 (&a)[4], const u32x4 (&c)[4], int t, const u32x8 (&b)[4]) {
#pragma unroll
    for (int at = 0; at < 4; ++at) {
      const int idx = (int)((c[at][2] >> (16 * t)) & 0xFFFFu);   // positions of the 8 kept values
#pragma unroll
      for (int bt = 0; bt < 4; ++bt)
        acc[at][bt] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a[at], as_bf16x16(b[bt]), acc[at][bt], idx, 0, 0);
    }
  };

  wait_vmcnt<2 * L::kLoads>();
  stage_barrier();
  load_w_regs(lds, wa, wsc);
  read_b(lds, 0, bx);
  decode(wa, wsc, 0, acur);

  auto stage = [&](auto slot_c, int st) {
    constexpr int S = decltype(slot_c)::value;
    const char* slot = lds + S * L::kBytes;
    const char* next = lds + ((S + 1) % kStages) * L::kBytes;
    u32x8 b1[4];
    bf16x8 a1[4];
    read_b(slot, 1, b1);
    __builtin_amdgcn_sched_barrier(0);
    decode(wa, wsc, 1, a1);
    mfmas(acur, wa, 0, bx);
    interleave_mfma_valu<1, 15, 5>();
    __builtin_amdgcn_sched_barrier(0);           // the MFMAs above stay above the barrier
    __builtin_amdgcn_s_waitcnt(0xC07F);          // lgkmcnt(0): reads of slot S are in registers
    wait_vmcnt<L::kLoads>();                     // stage st + 1 has landed
    stage_barrier();
    issue_stage<kSp24>(src, min(st + 3, last), lds + S * L::kBytes, wave);
    u32x4 wn[4];
    uint32_t wsn[4];
    load_w_regs(next, wn, wsn);
    __builtin_amdgcn_sched_barrier(0);
    read_b(next, 0, bx);
    __builtin_amdgcn_sched_barrier(0);
    decode(wn, wsn, 0, acur);
    mfmas(a1, wa, 1, b1);                        // second MFMA step of stage st
    interleave_mfma_valu<4, 12, 6>();
#pragma unroll
    for (int at = 0; at < 4; ++at) { wa[at] = wn[at]; wsc[at] = wsn[at]; }
  };
  for (int st = 0; st < nst; st += 3) {
    stage(std::integral_constant<int, 0>{}, st);
    if (st + 1 < nst) stage(std::integral_constant<int, 1>{}, st + 1);
    if (st + 2 < nst) stage(std::integral_constant<int, 2>{}, st + 2);
  }
  wait_vmcnt<0>();

  // epilogue: lane holds weight rows 8(i/4) + 4q + i%4 of each block, activation row r32, i.e.
  // Y[m][n .. n + 3] for n = 32 at + 8 g + 4 q. Each activation row block of the wave (32 rows x
  // 128 columns) is staged in LDS and leaves as row-contiguous pieces: bf16 output is rounded
  // first and staged as 16-byte pieces of 8 values (piece c of row r at position c ^ (r & 7)),
  // f32 output as pieces of 4 values in padded rows.
  __syncthreads();
  if constexpr (YB) {
    char* T = lds + wave * (32 * 256);
    const bool vec = (N & 7) == 0;
#pragma unroll
    for (int bt = 0; bt < 4; ++bt) {
#pragma unroll
      for (int at = 0; at < 4; ++at)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16& a = acc[at][bt];
          u32x2 w;
          w[0] = pk_bf16_rne(a[4 * g] * st_scale, a[4 * g + 1] * st_scale);
          w[1] = pk_bf16_rne(a[4 * g + 2] * st_scale, a[4 * g + 3] * st_scale);
          const int c = 4 * at + g;
          *(u32x2*)(T + r32 * 256 + 16 * (c ^ (r32 & 7)) + 8 * q) = w;
        }
      __builtin_amdgcn_s_waitcnt(0xC07F);
      const int c = lane & 15;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = (lane >> 4) + 4 * j;
        const u32x4 v = *(const u32x4*)(T + r * 256 + 16 * (c ^ (r & 7)));
        const int m = m0 + 128 * wm + 32 * bt + r;
        if (m < M) store8_bf16(Y, N, m, n0 + 128 * wn + 8 * c, v, vec);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);
    }
  } else {
    const bool vec = (N & 3) == 0;
    constexpr int kTS = 132;
    float* T = (float*)(lds + wave * (32 * kTS * 4));
#pragma unroll
    for (int bt = 0; bt < 4; ++bt) {
#pragma unroll
      for (int at = 0; at < 4; ++at)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = acc[at][bt][4 * g + i] * st_scale;
          *(f32x4*)(T + r32 * kTS + 32 * at + 8 * g + 4 * q) = v;
        }
      __builtin_amdgcn_s_waitcnt(0xC07F);
      const int c4 = lane & 31;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = (lane >> 5) + 2 * j;
        const f32x4 v = *(const f32x4*)(T + r * kTS + 4 * c4);
        const int m = m0 + 128 * wm + 32 * bt + r, n = n0 + 128 * wn + 4 * c4;
        if (m < M) store4(Y, 0, N, m, n, v, vec);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);
    }
  }
}



template <int WF, bool YB>
hipError_t launch_mfma_tiles(const GemmArgs& a, hipStream_t s) {
  const int bytes = kStages * Slot<WF, kTM>::kBytes;   // the 128-row tiles need less
  const void* fn = (const void*)k_gemm_mfma<WF, YB>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  const int64_t tiles_m = (a.M + kTM - 1) / kTM, tiles_n = (a.N + kTN - 1) / kTN, tiles = tiles_m * tiles_n;
  const int64_t cu = cu_count(), rem = tiles % cu;
  int64_t nbig = tiles, row0 = 0, col0 = 0, grid = tiles;
  // with whole kGroupM-row groups, the last rem tiles of the order are the last kGroupM tile
  // rows x the last rem / kGroupM tile columns
  if (tiles > cu && rem > 0 && 2 * rem <= cu && tiles_m % kGroupM == 0 && rem % kGroupM == 0 &&
      rem <= kGroupM * tiles_n) {
    nbig = tiles - rem;
    row0 = (tiles_m - kGroupM) * kTM;
    col0 = (tiles_n - rem / kGroupM) * kTN;
    grid = nbig + ((a.M - row0 + kTM / 2 - 1) / (kTM / 2)) * (rem / kGroupM);
  }
  hipLaunchKernelGGL((k_gemm_mfma<WF, YB>), dim3((unsigned)grid), dim3(kThreads), bytes, s, a.X, (int)a.M, (int)a.N,
                     (int)a.K, a.w0, a.w1, a.scales, a.ts, a.Y, (int)nbig, (int)row0, (int)col0);
  return hipGetLastError();
}

template <bool YB>
hipError_t launch_smfmac_tiles(const GemmArgs& a, hipStream_t s) {
  const int bytes = kStages * Slot<kSp24>::kBytes;
  hipError_t e = hipFuncSetAttribute((const void*)k_gemm_smfmac<YB>, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  const unsigned tiles = (unsigned)(((a.M + kTM - 1) / kTM) * ((a.N + kTN - 1) / kTN));
  hipLaunchKernelGGL(k_gemm_smfmac<YB>, dim3(tiles), dim3(kThreads), bytes, s, a.X, (int)a.M, (int)a.N, (int)a.K,
                     a.w0, a.w1, a.scales, a.ts, a.Y, a.y_bf16);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_dense_mfma(const GemmArgs& a, hipStream_t s) {
  return a.y_bf16 ? launch_mfma_tiles<kDense, true>(a, s) : launch_mfma_tiles<kDense, false>(a, s);
}

hipError_t launch_gemm_sp24_decomp(const GemmArgs& a, hipStream_t s) {
  return a.y_bf16 ? launch_mfma_tiles<kSp24, true>(a, s) : launch_mfma_tiles<kSp24, false>(a, s);
}

hipError_t launch_gemm_sp24_smfmac(const GemmArgs& a, hipStream_t s) {
  return a.y_bf16 ? launch_smfmac_tiles<true>(a, s) : launch_smfmac_tiles<false>(a, s);
}

}  // namespace ssn
