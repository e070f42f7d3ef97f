// Host-side launchers of the gfx950 kernels (internal to the library; the public C ABI is
// declared in include/ssnvfp4.h and implemented in api.hip). Every launcher assumes its
// arguments were validated by the caller and returns the launch status.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssn {

// quantisation / producer side
hipError_t launch_quantize(const void* W, int w_bf16, int64_t N, int64_t K, const float* ts_in,
                           uint8_t* codes, uint8_t* scales, float* ts_out, hipStream_t s);
hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* ts, int64_t N,
                             int64_t K, void* out, int out_bf16, hipStream_t s);
// ts_out nullable: when given, receives s_t = fl32(amax|W| / 2688) gathered during the prune
hipError_t launch_prune(const void* W, int w_bf16, int64_t N, int64_t K, void* out, float* ts_out, hipStream_t s);
// prune -> quantise -> compress in one pass; codes (the pruned tensor's codes) nullable; bad device
hipError_t launch_produce24(const void* W, int w_bf16, int64_t N, int64_t K, const float* ts_in, uint8_t* vals,
                            uint8_t* meta, uint8_t* scales, float* ts_out, uint8_t* codes, int64_t* bad,
                            hipStream_t s);

// 2:4 codec
hipError_t launch_check(const uint8_t* codes, int64_t N, int64_t K, int64_t* bad, int64_t* first,
                        hipStream_t s);
hipError_t launch_compress(const uint8_t* codes, int64_t N, int64_t K, uint8_t* vals, uint8_t* meta,
                           int64_t* bad, hipStream_t s);
hipError_t launch_decompress(const uint8_t* vals, const uint8_t* meta, int64_t N, int64_t K,
                             uint8_t* codes, hipStream_t s);

// products. `w0`/`w1` are (codes, -) for dense and (vals, meta) for 2:4.
struct GemmArgs {
  const uint16_t* X;
  int64_t M, N, K;
  const uint8_t* w0;      // codes [N,K/2] or vals [N,K/4]
  const uint8_t* w1;      // meta [N,K/8] or nullptr
  const uint8_t* scales;  // [N,K/16]
  const float* ts;        // [1]
  void* Y;
  int y_bf16;
};

hipError_t launch_gemv_dense_mfma(const GemmArgs& a, hipStream_t s);     // M <= 16
hipError_t launch_gemv_sp24_smfmac(const GemmArgs& a, hipStream_t s);    // M <= 16, K % 64
hipError_t launch_gemv_sp24_decomp(const GemmArgs& a, hipStream_t s);    // M <= 16
hipError_t launch_gemm_dense_valu(const GemmArgs& a, hipStream_t s);     // any M
hipError_t launch_gemm_sp24_valu(const GemmArgs& a, hipStream_t s);      // any M (skip-and-gather)
hipError_t launch_gemm_dense_mfma(const GemmArgs& a, hipStream_t s);     // 256x256 tiles, any M
hipError_t launch_gemm_sp24_decomp(const GemmArgs& a, hipStream_t s);    // 256x256 tiles, any M
hipError_t launch_gemm_sp24_smfmac(const GemmArgs& a, hipStream_t s);    // 256x256 tiles, any M

// grouped-expert (MoE) path
struct MoeGemmArgs {
  const uint16_t* X;        // activations [x_rows, K] bf16
  int64_t x_rows, K;
  const int32_t* row_token; // [R] source row of each expert-ordered row, or nullptr (identity)
  const int32_t* offsets;   // [E + 1] device
  int E;
  int64_t R, N;             // rows of Y; weight rows per expert (2I for the SiLU-gate form)
  const uint8_t* w0;        // codes [E, N, K/2] or vals [E, N, K/4]
  const uint8_t* w1;        // meta [E, N, K/8] or nullptr
  const uint8_t* scales;    // [E, N, K/16]
  const float* ts;          // [E]
  void* Y;                  // [R, N] (or [R, N/2] for the SiLU-gate form)
  int y_bf16, sparse, silu;
  int ktiled;               // weights (all three arrays) in the 64-k tiled layout [E][K/64][N][piece]
  int smfmac = 0;           // 2:4 tiles on the sparse matrix cores (else expanded to dense)
};

size_t moe_route_workspace(int64_t F, int E);
hipError_t launch_moe_route(const int32_t* ids, int64_t T, int k, int E, int32_t* offsets, int32_t* row_token,
                            int32_t* row_slot, int32_t* row_of, int64_t* bad, void* ws, hipStream_t s);
hipError_t launch_moe_gemm(const MoeGemmArgs& a, hipStream_t s);
// one wave per (expert, 32 weight rows, <= 32 routed rows); N % 32 == 0, K % 64 == 0
hipError_t launch_moe_stream(const MoeGemmArgs& a, hipStream_t s);
hipError_t launch_moe_pack_ktiles(const uint8_t* src, int64_t E, int64_t N, int64_t row_bytes, int64_t piece,
                                  uint8_t* dst, hipStream_t s);
hipError_t launch_moe_combine(const void* Yd, int yd_bf16, int64_t R, const int32_t* row_of, const float* w,
                              int64_t T, int k, int64_t D, float* out, hipStream_t s);

// W4A4 variant (MXFP4 operands on the block-scaled matrix cores)
int64_t mx_tiled_code_bytes(int64_t R, int64_t K);
int64_t mx_tiled_scale_bytes(int64_t R, int64_t K);
hipError_t launch_mx_quantize(const void* V, int v_bf16, int64_t R, int64_t K, int tiled, uint8_t* codes,
                              uint8_t* scales, hipStream_t s);
hipError_t launch_gemm_mx(const uint8_t* xc, const uint8_t* xs, int64_t M, const uint8_t* wc, const uint8_t* ws,
                          int64_t N, int64_t K, void* Y, int y_bf16, hipStream_t s);

// calibration: register-resident matrix ops on random operands (cu_count() * waves_per_simd
// workgroups of 256 threads; sink holds one float per thread)
hipError_t launch_mfma_probe(int kind, int waves_per_simd, int iters, uint32_t seed, float* sink, hipStream_t s);

}  // namespace ssn
