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
hipError_t launch_prune(const void* W, int w_bf16, int64_t N, int64_t K, void* out, hipStream_t s);

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

}  // namespace ssn
