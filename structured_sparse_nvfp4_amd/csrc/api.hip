// C ABI of the library: argument validation, algorithm selection and kernel launches.
// Declarations and the contract of every call are in include/ssnvfp4.h.
#include <stdarg.h>
#include <stdio.h>

#include "../../include/ssnvfp4.h"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() { g_err[0] = 0; return SSN_OK; }

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SSN_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define REQUIRE_PTR(p) \
  do { if (!(p)) return fail(SSN_E_NULL, "%s: argument '%s' is NULL", fn, #p); \
       if (!aligned16(p)) return fail(SSN_E_ALIGN, "%s: argument '%s' is not 16-byte aligned", fn, #p); } while (0)

#define REQUIRE_OPT_PTR(p) \
  do { if ((p) && !aligned16(p)) return fail(SSN_E_ALIGN, "%s: argument '%s' is not 16-byte aligned", fn, #p); } while (0)

// rows (N, M) are indexed with 32-bit ints inside the kernels, tile origins included
constexpr int64_t kMaxRows = ((int64_t)1 << 31) - 1024;

int check_nk(const char* fn, int64_t N, int64_t K) {
  if (N < 0 || K < 0) return fail(SSN_E_SHAPE, "%s: negative size (N=%lld, K=%lld)", fn, (long long)N, (long long)K);
  if (K % 32) return fail(SSN_E_SHAPE, "%s: K=%lld is not a multiple of 32", fn, (long long)K);
  if (N > kMaxRows || K > (int64_t)1 << 30)
    return fail(SSN_E_SHAPE, "%s: size too large (N=%lld, K=%lld)", fn, (long long)N, (long long)K);
  return SSN_OK;
}

int check_dtype(const char* fn, int dt, const char* name) {
  if (dt != SSN_F32 && dt != SSN_BF16) return fail(SSN_E_DTYPE, "%s: unknown %s code %d", fn, name, dt);
  return SSN_OK;
}

hipStream_t as_stream(void* s) { return (hipStream_t)s; }

}  // namespace

extern "C" {

const char* ssn_last_error(void) { return g_err; }
int ssn_version(void) { return 100; }  // 0.1.0

int nvfp4_quantize(const void* W, int w_dtype, int64_t N, int64_t K, const float* tensor_scale_in,
                   uint8_t* codes, uint8_t* scales, float* tensor_scale_out, void* stream) {
  const char* fn = "nvfp4_quantize";
  int st;
  if ((st = check_nk(fn, N, K))) return st;
  if ((st = check_dtype(fn, w_dtype, "w_dtype"))) return st;
  REQUIRE_PTR(tensor_scale_out);
  REQUIRE_OPT_PTR(tensor_scale_in);
  if (N == 0 || K == 0) {
    // an empty tensor still has a well-defined scale: zero (or the given shared scale)
    REQUIRE_PTR(tensor_scale_out);
    return hip_status(ssn::launch_quantize(nullptr, 0, 0, 0, tensor_scale_in, nullptr, nullptr,
                                           tensor_scale_out, as_stream(stream)), fn);
  }
  REQUIRE_PTR(W); REQUIRE_PTR(codes); REQUIRE_PTR(scales);
  return hip_status(ssn::launch_quantize(W, w_dtype == SSN_BF16, N, K, tensor_scale_in, codes, scales,
                                         tensor_scale_out, as_stream(stream)), fn);
}

int nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale, int64_t N,
                     int64_t K, void* out, int out_dtype, void* stream) {
  const char* fn = "nvfp4_dequantize";
  int st;
  if ((st = check_nk(fn, N, K))) return st;
  if ((st = check_dtype(fn, out_dtype, "out_dtype"))) return st;
  if (N == 0 || K == 0) return ok();
  REQUIRE_PTR(codes); REQUIRE_PTR(scales); REQUIRE_PTR(tensor_scale); REQUIRE_PTR(out);
  return hip_status(ssn::launch_dequantize(codes, scales, tensor_scale, N, K, out, out_dtype == SSN_BF16,
                                           as_stream(stream)), fn);
}

int sp24_prune(const void* W, int w_dtype, int64_t N, int64_t K, void* W_out, void* stream) {
  const char* fn = "sp24_prune";
  int st;
  if ((st = check_nk(fn, N, K))) return st;
  if ((st = check_dtype(fn, w_dtype, "w_dtype"))) return st;
  if (N == 0 || K == 0) return ok();
  REQUIRE_PTR(W); REQUIRE_PTR(W_out);
  return hip_status(ssn::launch_prune(W, w_dtype == SSN_BF16, N, K, W_out, as_stream(stream)), fn);
}

int sp24_check(const uint8_t* codes, int64_t N, int64_t K, int64_t* bad_groups, int64_t* first_bad,
               void* stream) {
  const char* fn = "sp24_check";
  int st;
  if ((st = check_nk(fn, N, K))) return st;
  REQUIRE_PTR(bad_groups);
  REQUIRE_OPT_PTR(first_bad);
  if (N * K > 0) REQUIRE_PTR(codes);
  return hip_status(ssn::launch_check(codes, N, K, bad_groups, first_bad, as_stream(stream)), fn);
}

int sp24_compress(const uint8_t* codes, int64_t N, int64_t K, uint8_t* vals, uint8_t* meta,
                  int64_t* bad_groups, void* stream) {
  const char* fn = "sp24_compress";
  int st;
  if ((st = check_nk(fn, N, K))) return st;
  REQUIRE_PTR(bad_groups);
  if (N * K > 0) { REQUIRE_PTR(codes); REQUIRE_PTR(vals); REQUIRE_PTR(meta); }
  return hip_status(ssn::launch_compress(codes, N, K, vals, meta, bad_groups, as_stream(stream)), fn);
}

int sp24_decompress(const uint8_t* vals, const uint8_t* meta, int64_t N, int64_t K, uint8_t* codes,
                    void* stream) {
  const char* fn = "sp24_decompress";
  int st;
  if ((st = check_nk(fn, N, K))) return st;
  if (N == 0 || K == 0) return ok();
  REQUIRE_PTR(vals); REQUIRE_PTR(meta); REQUIRE_PTR(codes);
  return hip_status(ssn::launch_decompress(vals, meta, N, K, codes, as_stream(stream)), fn);
}

}  // extern "C"

namespace {

int gemm_common(const char* fn, const uint16_t* X, int64_t M, int64_t N, int64_t K, const uint8_t* w0,
                const uint8_t* w1, const uint8_t* scales, const float* ts, void* Y, int y_dtype, bool sp24,
                int algo, int* algo_used, void* stream) {
  int st;
  if (M < 0) return fail(SSN_E_SHAPE, "%s: negative M=%lld", fn, (long long)M);
  if (M > kMaxRows) return fail(SSN_E_SHAPE, "%s: M=%lld too large", fn, (long long)M);
  if ((st = check_nk(fn, N, K))) return st;
  if ((st = check_dtype(fn, y_dtype, "y_dtype"))) return st;
  if (algo < SSN_ALGO_AUTO || algo > SSN_ALGO_DECOMPRESS_MFMA || algo == 4)
    return fail(SSN_E_ALGO, "%s: unknown algorithm %d", fn, algo);
  if (!sp24 && (algo == SSN_ALGO_SMFMAC || algo == SSN_ALGO_DECOMPRESS_MFMA))
    return fail(SSN_E_ALGO, "%s: algorithm %d applies to 2:4 weights only", fn, algo);
  if (sp24 && algo == SSN_ALGO_MFMA)
    return fail(SSN_E_ALGO, "%s: use SMFMAC or DECOMPRESS_MFMA for 2:4 weights", fn);
  if (M == 0 || N == 0) { if (algo_used) *algo_used = algo; return ok(); }
  if (K == 0) return fail(SSN_E_SHAPE, "%s: K must be positive when M, N > 0", fn);
  REQUIRE_PTR(X); REQUIRE_PTR(w0); REQUIRE_PTR(scales); REQUIRE_PTR(ts); REQUIRE_PTR(Y);
  if (sp24) REQUIRE_PTR(w1);

  // M <= 16: decode-shaped kernels (weights streamed once); otherwise 256x256 tiles, which
  // take whole 64-wide K stages
  const bool skinny = M <= 16;
  int chosen = algo;
  if (algo == SSN_ALGO_AUTO) {
    if (!skinny && K % 64) chosen = SSN_ALGO_VALU;
    else if (!sp24) chosen = SSN_ALGO_MFMA;
    else chosen = (skinny && K % 64) ? SSN_ALGO_DECOMPRESS_MFMA : SSN_ALGO_SMFMAC;
  }
  // explicit choices that do not apply to this shape are refused, never replaced
  if (chosen == SSN_ALGO_SMFMAC && skinny && K % 64)
    return fail(SSN_E_ALGO, "%s: SMFMAC for M <= 16 needs K %% 64 == 0 (K=%lld)", fn, (long long)K);
  if (chosen != SSN_ALGO_VALU && !skinny && K % 64)
    return fail(SSN_E_ALGO, "%s: matrix-core algorithm %d for M > 16 needs K %% 64 == 0 (K=%lld)", fn, chosen,
                (long long)K);

  ssn::GemmArgs a{X, M, N, K, w0, w1, scales, ts, Y, y_dtype == SSN_BF16};
  hipStream_t s = as_stream(stream);
  hipError_t e = hipSuccess;
  switch (chosen) {
    case SSN_ALGO_VALU: e = sp24 ? ssn::launch_gemm_sp24_valu(a, s) : ssn::launch_gemm_dense_valu(a, s); break;
    case SSN_ALGO_MFMA: e = skinny ? ssn::launch_gemv_dense_mfma(a, s) : ssn::launch_gemm_dense_mfma(a, s); break;
    case SSN_ALGO_SMFMAC: e = skinny ? ssn::launch_gemv_sp24_smfmac(a, s) : ssn::launch_gemm_sp24_smfmac(a, s); break;
    case SSN_ALGO_DECOMPRESS_MFMA:
      e = skinny ? ssn::launch_gemv_sp24_decomp(a, s) : ssn::launch_gemm_sp24_decomp(a, s);
      break;
  }
  if (algo_used) *algo_used = chosen;
  return hip_status(e, fn);
}

}  // namespace

extern "C" {

int gemm_nvfp4_dense(const uint16_t* X, int64_t M, int64_t N, int64_t K, const uint8_t* codes,
                     const uint8_t* scales, const float* tensor_scale, void* Y, int y_dtype, int algo,
                     int* algo_used, void* stream) {
  return gemm_common("gemm_nvfp4_dense", X, M, N, K, codes, nullptr, scales, tensor_scale, Y, y_dtype, false,
                     algo, algo_used, stream);
}

int gemm_nvfp4_sp24(const uint16_t* X, int64_t M, int64_t N, int64_t K, const uint8_t* vals,
                    const uint8_t* meta, const uint8_t* scales, const float* tensor_scale, void* Y,
                    int y_dtype, int algo, int* algo_used, void* stream) {
  return gemm_common("gemm_nvfp4_sp24", X, M, N, K, vals, meta, scales, tensor_scale, Y, y_dtype, true, algo,
                     algo_used, stream);
}

}  // extern "C"
