// C ABI of the library: argument validation, algorithm selection and kernel launches.
// Declarations and the contract of every call are in include/ssnvfp4.h.
#include <stdarg.h>
#include <stdio.h>

#include "../../include/ssnvfp4.h"
#include "device_once.hpp"
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

// scalars and element-wise arrays: the alignment of the element type
#define REQUIRE_ELEM_PTR(p) \
  do { if (!(p)) return fail(SSN_E_NULL, "%s: argument '%s' is NULL", fn, #p); \
       if ((uintptr_t)(p) % alignof(decltype(*(p)))) \
         return fail(SSN_E_ALIGN, "%s: argument '%s' is not aligned to its element type", fn, #p); } while (0)
#define REQUIRE_OPT_ELEM_PTR(p) \
  do { if ((p) && (uintptr_t)(p) % alignof(decltype(*(p)))) \
         return fail(SSN_E_ALIGN, "%s: argument '%s' is not aligned to its element type", fn, #p); } while (0)

// rows (N, M) are indexed with 32-bit ints inside the kernels, tile origins included
constexpr int64_t kMaxRows = ((int64_t)1 << 31) - 1024;
// the 256x256 tiles address their activation panel (256 rows of K bf16) with 32-bit byte offsets
constexpr int64_t kMaxTileK = (int64_t)1 << 21;
// the grouped-expert tiles address X and one expert's weight array with 32-bit byte offsets
constexpr int64_t kMaxTileBytes = (int64_t)1 << 31;

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
  REQUIRE_ELEM_PTR(tensor_scale_out);
  REQUIRE_OPT_ELEM_PTR(tensor_scale_in);
  if (N == 0 || K == 0) {
    // an empty tensor still has a well-defined scale: zero (or the given shared scale)
    return hip_status(ssn::launch_quantize(nullptr, 0, 0, 0, tensor_scale_in, nullptr, nullptr,
                                           tensor_scale_out, as_stream(stream)), fn);
  }
  REQUIRE_PTR(W); REQUIRE_PTR(codes); REQUIRE_PTR(scales);
  return hip_status(ssn::launch_quantize(W, w_dtype == SSN_BF16, N, K, tensor_scale_in, codes, scales,
                                         tensor_scale_out, as_stream(stream)), fn);
}

int nvfp4_sp24_produce(const void* W, int w_dtype, int64_t N, int64_t K, const float* tensor_scale_in,
                       uint8_t* vals, uint8_t* meta, uint8_t* scales, float* tensor_scale_out, uint8_t* codes,
                       int64_t* bad_groups, void* stream) {
  const char* fn = "nvfp4_sp24_produce";
  int st;
  if ((st = check_nk(fn, N, K))) return st;
  if ((st = check_dtype(fn, w_dtype, "w_dtype"))) return st;
  REQUIRE_ELEM_PTR(tensor_scale_out);
  REQUIRE_OPT_ELEM_PTR(tensor_scale_in);
  REQUIRE_ELEM_PTR(bad_groups);
  REQUIRE_OPT_PTR(codes);
  if (N == 0 || K == 0)
    return hip_status(ssn::launch_produce24(nullptr, 0, 0, 0, tensor_scale_in, nullptr, nullptr, nullptr,
                                            tensor_scale_out, nullptr, bad_groups, as_stream(stream)), fn);
  REQUIRE_PTR(W); REQUIRE_PTR(vals); REQUIRE_PTR(meta); REQUIRE_PTR(scales);
  return hip_status(ssn::launch_produce24(W, w_dtype == SSN_BF16, N, K, tensor_scale_in, vals, meta, scales,
                                          tensor_scale_out, codes, bad_groups, as_stream(stream)), fn);
}

int nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale, int64_t N,
                     int64_t K, void* out, int out_dtype, void* stream) {
  const char* fn = "nvfp4_dequantize";
  int st;
  if ((st = check_nk(fn, N, K))) return st;
  if ((st = check_dtype(fn, out_dtype, "out_dtype"))) return st;
  if (N == 0 || K == 0) return ok();
  REQUIRE_PTR(codes); REQUIRE_PTR(scales); REQUIRE_ELEM_PTR(tensor_scale); REQUIRE_PTR(out);
  return hip_status(ssn::launch_dequantize(codes, scales, tensor_scale, N, K, out, out_dtype == SSN_BF16,
                                           as_stream(stream)), fn);
}

int sp24_prune(const void* W, int w_dtype, int64_t N, int64_t K, void* W_out, float* tensor_scale_out,
               void* stream) {
  const char* fn = "sp24_prune";
  int st;
  if ((st = check_nk(fn, N, K))) return st;
  if ((st = check_dtype(fn, w_dtype, "w_dtype"))) return st;
  REQUIRE_OPT_ELEM_PTR(tensor_scale_out);
  if (N == 0 || K == 0) {   // an empty tensor has no maximum: s_t = 0
    if (tensor_scale_out) return hip_status(ssn::launch_prune(nullptr, 0, 0, 0, nullptr, tensor_scale_out,
                                                              as_stream(stream)), fn);
    return ok();
  }
  REQUIRE_PTR(W); REQUIRE_PTR(W_out);
  return hip_status(ssn::launch_prune(W, w_dtype == SSN_BF16, N, K, W_out, tensor_scale_out, as_stream(stream)), fn);
}

int sp24_check(const uint8_t* codes, int64_t N, int64_t K, int64_t* bad_groups, int64_t* first_bad,
               void* stream) {
  const char* fn = "sp24_check";
  int st;
  if ((st = check_nk(fn, N, K))) return st;
  REQUIRE_ELEM_PTR(bad_groups);
  REQUIRE_OPT_ELEM_PTR(first_bad);
  if (N * K > 0) REQUIRE_PTR(codes);
  return hip_status(ssn::launch_check(codes, N, K, bad_groups, first_bad, as_stream(stream)), fn);
}

int sp24_compress(const uint8_t* codes, int64_t N, int64_t K, uint8_t* vals, uint8_t* meta,
                  int64_t* bad_groups, void* stream) {
  const char* fn = "sp24_compress";
  int st;
  if ((st = check_nk(fn, N, K))) return st;
  REQUIRE_ELEM_PTR(bad_groups);
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
  if (algo < SSN_ALGO_AUTO || algo > SSN_ALGO_DECOMPRESS_MFMA)
    return fail(SSN_E_ALGO, "%s: unknown algorithm %d", fn, algo);
  if (!sp24 && (algo == SSN_ALGO_SMFMAC || algo == SSN_ALGO_DECOMPRESS_MFMA || algo == SSN_ALGO_GATHER))
    return fail(SSN_E_ALGO, "%s: algorithm %d applies to 2:4 weights only", fn, algo);
  if (sp24 && algo == SSN_ALGO_MFMA)
    return fail(SSN_E_ALGO, "%s: use SMFMAC or DECOMPRESS_MFMA for 2:4 weights", fn);
  if (M == 0 || N == 0) { if (algo_used) *algo_used = (sp24 && algo == SSN_ALGO_VALU) ? SSN_ALGO_GATHER : algo; return ok(); }
  if (K == 0) return fail(SSN_E_SHAPE, "%s: K must be positive when M, N > 0", fn);
  REQUIRE_PTR(X); REQUIRE_PTR(w0); REQUIRE_PTR(scales); REQUIRE_ELEM_PTR(ts); REQUIRE_PTR(Y);
  if (sp24) REQUIRE_PTR(w1);

  // M <= 16: decode-shaped kernels (weights streamed once); otherwise 256x256 tiles, which
  // take whole 64-wide K stages and address a 256-row activation panel with 32-bit offsets
  const bool skinny = M <= 16;
  const bool tiles_fit = K % 64 == 0 && K <= kMaxTileK;
  const int valu = sp24 ? SSN_ALGO_GATHER : SSN_ALGO_VALU;
  int chosen = algo == SSN_ALGO_VALU ? valu : algo;
  if (algo == SSN_ALGO_AUTO) {
    if (!skinny && !tiles_fit) chosen = valu;
    else if (!sp24) chosen = SSN_ALGO_MFMA;
    else chosen = (skinny && K % 64) ? SSN_ALGO_DECOMPRESS_MFMA : SSN_ALGO_SMFMAC;
  }
  // explicit choices that do not apply to this shape are refused, never replaced
  if (chosen == SSN_ALGO_SMFMAC && skinny && K % 64)
    return fail(SSN_E_ALGO, "%s: SMFMAC for M <= 16 needs K %% 64 == 0 (K=%lld)", fn, (long long)K);
  if (chosen != valu && !skinny && !tiles_fit)
    return fail(SSN_E_ALGO, "%s: matrix-core algorithm %d for M > 16 needs K %% 64 == 0 and K <= %lld (K=%lld)", fn,
                chosen, (long long)kMaxTileK, (long long)K);

  ssn::GemmArgs a{X, M, N, K, w0, w1, scales, ts, Y, y_dtype == SSN_BF16};
  hipStream_t s = as_stream(stream);
  hipError_t e = hipSuccess;
  switch (chosen) {
    case SSN_ALGO_VALU: e = ssn::launch_gemm_dense_valu(a, s); break;
    case SSN_ALGO_GATHER: e = ssn::launch_gemm_sp24_valu(a, s); break;
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

// ---------------------------------------------------------------------------------------------
// grouped-expert path
namespace {

constexpr int kMaxExperts = 2048, kMaxTopK = 64;

int check_route_shape(const char* fn, int64_t T, int k, int E) {
  if (T < 0) return fail(SSN_E_SHAPE, "%s: negative T=%lld", fn, (long long)T);
  if (k < 1 || k > kMaxTopK) return fail(SSN_E_RANGE, "%s: k=%d outside [1, %d]", fn, k, kMaxTopK);
  if (E < 1 || E > kMaxExperts) return fail(SSN_E_RANGE, "%s: E=%d outside [1, %d]", fn, E, kMaxExperts);
  if (T * k >= ((int64_t)1 << 31) - 1024) return fail(SSN_E_SHAPE, "%s: T*k=%lld too large", fn, (long long)(T * k));
  return SSN_OK;
}

int64_t route_ws(int64_t T, int k, int E) { return (int64_t)ssn::moe_route_workspace(T * k, E); }

int64_t align256(int64_t n) { return (n + 255) & ~(int64_t)255; }

}  // namespace

extern "C" {

int64_t moe_route_workspace_bytes(int64_t T, int k, int E) {
  if (check_route_shape("moe_route_workspace_bytes", T, k, E)) return -1;
  return route_ws(T, k, E);
}

int moe_route(const int32_t* topk_ids, int64_t T, int k, int E, int32_t* expert_offsets, int32_t* row_token,
              int32_t* row_slot, int32_t* row_of, int64_t* bad_ids, void* workspace, int64_t workspace_bytes,
              void* stream) {
  const char* fn = "moe_route";
  int st;
  if ((st = check_route_shape(fn, T, k, E))) return st;
  REQUIRE_ELEM_PTR(expert_offsets);
  REQUIRE_OPT_ELEM_PTR(bad_ids);
  const int64_t need = route_ws(T, k, E);
  if (T > 0) {
    REQUIRE_ELEM_PTR(topk_ids); REQUIRE_ELEM_PTR(row_token); REQUIRE_ELEM_PTR(row_slot); REQUIRE_ELEM_PTR(row_of);
    REQUIRE_PTR(workspace);
  }
  if (workspace_bytes < need)
    return fail(SSN_E_RANGE, "%s: workspace of %lld bytes, %lld needed", fn, (long long)workspace_bytes,
                (long long)need);
  return hip_status(ssn::launch_moe_route(topk_ids, T, k, E, expert_offsets, row_token, row_slot, row_of, bad_ids,
                                          workspace, as_stream(stream)), fn);
}

int moe_grouped_gemm_nvfp4(const uint16_t* X, int64_t x_rows, const int32_t* row_token, const int32_t* expert_offsets,
                           int E, int64_t R, int64_t N, int64_t K, int sparse, int w_layout, const uint8_t* w_main,
                           const uint8_t* w_meta, const uint8_t* w_scales, const float* tensor_scales, int epilogue,
                           void* Y, int y_dtype, int algo, int* algo_used, void* stream) {
  const char* fn = "moe_grouped_gemm_nvfp4";
  int st;
  if (E < 1 || E > kMaxExperts) return fail(SSN_E_RANGE, "%s: E=%d outside [1, %d]", fn, E, kMaxExperts);
  if (R < 0 || R > kMaxRows || x_rows < 0 || x_rows > kMaxRows)
    return fail(SSN_E_SHAPE, "%s: bad row counts (R=%lld, x_rows=%lld)", fn, (long long)R, (long long)x_rows);
  if ((st = check_nk(fn, N, K))) return st;
  if ((st = check_dtype(fn, y_dtype, "y_dtype"))) return st;
  if (sparse != 0 && sparse != 1) return fail(SSN_E_RANGE, "%s: sparse=%d must be 0 or 1", fn, sparse);
  if (w_layout != SSN_WLAYOUT_ROWS && w_layout != SSN_WLAYOUT_KTILE64)
    return fail(SSN_E_RANGE, "%s: unknown weight layout %d", fn, w_layout);
  if (epilogue != SSN_EPI_NONE && epilogue != SSN_EPI_SILU_GATE)
    return fail(SSN_E_RANGE, "%s: unknown epilogue %d", fn, epilogue);
  if (epilogue == SSN_EPI_SILU_GATE && N % 2) return fail(SSN_E_SHAPE, "%s: SILU_GATE needs N even (N=%lld)", fn, (long long)N);
  const int tiles = sparse ? SSN_ALGO_SMFMAC : SSN_ALGO_MFMA;
  const bool can_stream = N % 32 == 0;
  // measured crossover (512 experts, D = 2048, I = 512): streaming wins up to ~4 rows per expert
  // for dense weights and ~10 for 2:4 weights
  const int64_t stream_max = (sparse ? 10 : 4) * (int64_t)E;
  // the tiles load X and each expert's weight arrays through buffer resources with 32-bit byte
  // offsets: both must stay below 2^31 bytes (the codes, or the vals, are the largest array)
  const bool tiles_fit = x_rows * K * 2 < kMaxTileBytes && N * (K / (sparse ? 4 : 2)) < kMaxTileBytes;
  const int chosen = algo == SSN_ALGO_AUTO
                         ? (can_stream && (R <= stream_max || !tiles_fit) ? SSN_ALGO_STREAM : tiles)
                         : algo;
  const bool tile_algo = chosen == tiles || (sparse && chosen == SSN_ALGO_DECOMPRESS_MFMA);
  if (!tile_algo && chosen != SSN_ALGO_STREAM)
    return fail(SSN_E_ALGO, "%s: algorithm %d is not available for %s expert weights", fn, algo,
                sparse ? "2:4" : "dense");
  if (chosen == SSN_ALGO_STREAM && !can_stream)
    return fail(SSN_E_ALGO, "%s: STREAM needs N %% 32 == 0 (N=%lld)", fn, (long long)N);
  if (tile_algo && !tiles_fit)
    return fail(algo == SSN_ALGO_AUTO ? SSN_E_SHAPE : SSN_E_ALGO,
                "%s: the tiles need X (x_rows=%lld, K=%lld) and each expert's weights (N=%lld) below 2^31 "
                "bytes%s", fn, (long long)x_rows, (long long)K, (long long)N,
                algo == SSN_ALGO_AUTO ? ", and STREAM needs N % 32 == 0" : "");
  if (algo_used) *algo_used = chosen;
  if (R == 0 || N == 0) return ok();
  if (K == 0 || K % 64) return fail(SSN_E_SHAPE, "%s: K=%lld must be a positive multiple of 64", fn, (long long)K);
  if (x_rows == 0) return fail(SSN_E_SHAPE, "%s: x_rows must be positive when R > 0", fn);
  if (N * (K / 2) * (int64_t)E > ((int64_t)1 << 40)) return fail(SSN_E_SHAPE, "%s: expert weights too large", fn);
  REQUIRE_PTR(X); REQUIRE_OPT_ELEM_PTR(row_token); REQUIRE_ELEM_PTR(expert_offsets); REQUIRE_PTR(w_main);
  REQUIRE_PTR(w_scales); REQUIRE_ELEM_PTR(tensor_scales); REQUIRE_PTR(Y);
  if (sparse) REQUIRE_PTR(w_meta);
  ssn::MoeGemmArgs a{X, x_rows, K, row_token, expert_offsets, E, R, N, w_main, sparse ? w_meta : nullptr, w_scales,
                     tensor_scales, Y, y_dtype == SSN_BF16, sparse, epilogue == SSN_EPI_SILU_GATE,
                     w_layout == SSN_WLAYOUT_KTILE64, chosen == SSN_ALGO_SMFMAC};
  return hip_status(chosen == SSN_ALGO_STREAM ? ssn::launch_moe_stream(a, as_stream(stream))
                                              : ssn::launch_moe_gemm(a, as_stream(stream)), fn);
}

int moe_pack_ktiles(const uint8_t* src, int64_t E, int64_t N, int64_t row_bytes, int64_t piece_bytes, uint8_t* dst,
                    void* stream) {
  const char* fn = "moe_pack_ktiles";
  if (E < 0 || N < 0 || row_bytes < 0 || E > kMaxExperts)
    return fail(SSN_E_SHAPE, "%s: bad sizes (E=%lld, N=%lld, row_bytes=%lld)", fn, (long long)E, (long long)N,
                (long long)row_bytes);
  if (piece_bytes != 4 && piece_bytes != 8 && piece_bytes != 16 && piece_bytes != 32)
    return fail(SSN_E_RANGE, "%s: piece_bytes=%lld must be 4, 8, 16 or 32", fn, (long long)piece_bytes);
  if (row_bytes % piece_bytes) return fail(SSN_E_SHAPE, "%s: row_bytes=%lld is not a multiple of piece_bytes=%lld", fn,
                                           (long long)row_bytes, (long long)piece_bytes);
  if (E * N * row_bytes > ((int64_t)1 << 40)) return fail(SSN_E_SHAPE, "%s: array too large", fn);
  if (E * N * row_bytes == 0) return ok();
  REQUIRE_PTR(src); REQUIRE_PTR(dst);
  if ((const uint8_t*)dst < src + E * N * row_bytes && src < (const uint8_t*)dst + E * N * row_bytes)
    return fail(SSN_E_RANGE, "%s: src and dst overlap", fn);
  return hip_status(ssn::launch_moe_pack_ktiles(src, E, N, row_bytes, piece_bytes, dst, as_stream(stream)), fn);
}

int moe_combine(const void* Yd, int yd_dtype, int64_t R, const int32_t* row_of, const float* topk_weights, int64_t T,
                int k, int64_t D, float* out, void* stream) {
  const char* fn = "moe_combine";
  int st;
  if (T < 0 || D < 0 || R < 0 || R > kMaxRows || T > kMaxRows || D > ((int64_t)1 << 30))
    return fail(SSN_E_SHAPE, "%s: bad sizes (T=%lld, D=%lld, R=%lld)", fn, (long long)T, (long long)D, (long long)R);
  if (k < 1 || k > kMaxTopK) return fail(SSN_E_RANGE, "%s: k=%d outside [1, %d]", fn, k, kMaxTopK);
  if ((st = check_dtype(fn, yd_dtype, "yd_dtype"))) return st;
  if (T == 0 || D == 0) return ok();
  REQUIRE_ELEM_PTR(row_of); REQUIRE_ELEM_PTR(topk_weights); REQUIRE_PTR(out);
  if (R > 0) REQUIRE_PTR(Yd);
  return hip_status(ssn::launch_moe_combine(Yd, yd_dtype == SSN_BF16, R, row_of, topk_weights, T, k, D, out,
                                            as_stream(stream)), fn);
}

int64_t moe_ffn_workspace_bytes(int64_t T, int k, int E, int64_t I, int64_t D) {
  if (check_route_shape("moe_ffn_workspace_bytes", T, k, E) || I < 0 || D < 0) return -1;
  const int64_t F = T * k;
  return align256((E + 1) * 4) + 3 * align256(F * 4) + align256(route_ws(T, k, E)) + align256(F * I * 2) +
         align256(F * D * 4);
}

int moe_nvfp4_ffn(const uint16_t* X, int64_t T, int64_t D, const int32_t* topk_ids, const float* topk_weights, int k,
                  int E, int64_t I, int sparse, int w_layout, const uint8_t* up_main, const uint8_t* up_meta,
                  const uint8_t* up_scales, const float* up_ts, const uint8_t* down_main, const uint8_t* down_meta,
                  const uint8_t* down_scales, const float* down_ts, float* out, int64_t* bad_ids, void* workspace,
                  int64_t workspace_bytes, void* stream) {
  const char* fn = "moe_nvfp4_ffn";
  int st;
  if ((st = check_route_shape(fn, T, k, E))) return st;
  if (I <= 0 || D <= 0 || I % 64 || D % 64)
    return fail(SSN_E_SHAPE, "%s: I=%lld and D=%lld must be positive multiples of 64", fn, (long long)I, (long long)D);
  const int64_t need = moe_ffn_workspace_bytes(T, k, E, I, D);
  if (T > 0) REQUIRE_PTR(workspace);
  if (workspace_bytes < need)
    return fail(SSN_E_RANGE, "%s: workspace of %lld bytes, %lld needed", fn, (long long)workspace_bytes,
                (long long)need);
  if (T == 0) return ok();
  const int64_t F = T * k;
  char* w = (char*)workspace;
  int32_t* offsets = (int32_t*)w; w += align256((E + 1) * 4);
  int32_t* row_token = (int32_t*)w; w += align256(F * 4);
  int32_t* row_slot = (int32_t*)w; w += align256(F * 4);
  int32_t* row_of = (int32_t*)w; w += align256(F * 4);
  void* rws = w; w += align256(route_ws(T, k, E));
  uint16_t* H = (uint16_t*)w; w += align256(F * I * 2);
  float* Yd = (float*)w;
  if ((st = moe_route(topk_ids, T, k, E, offsets, row_token, row_slot, row_of, bad_ids, rws, route_ws(T, k, E), stream)))
    return st;
  if ((st = moe_grouped_gemm_nvfp4(X, T, row_token, offsets, E, F, 2 * I, D, sparse, w_layout, up_main, up_meta,
                                   up_scales, up_ts,
                                   SSN_EPI_SILU_GATE, H, SSN_BF16, SSN_ALGO_AUTO, nullptr, stream)))
    return st;
  if ((st = moe_grouped_gemm_nvfp4(H, F, nullptr, offsets, E, F, D, I, sparse, w_layout, down_main, down_meta,
                                   down_scales,
                                   down_ts, SSN_EPI_NONE, Yd, SSN_F32, SSN_ALGO_AUTO, nullptr, stream)))
    return st;
  return moe_combine(Yd, SSN_F32, F, row_of, topk_weights, T, k, D, out, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------
// W4A4 variant: MXFP4 activations and weights
extern "C" {

int64_t mxfp4_tiled_bytes(int64_t R, int64_t K, int64_t* scale_bytes) {
  if (R < 0 || K < 0 || K % 32 || R > kMaxRows || K > ((int64_t)1 << 30)) return -1;
  if (scale_bytes) *scale_bytes = ssn::mx_tiled_scale_bytes(R, K);
  return ssn::mx_tiled_code_bytes(R, K);
}

int mxfp4_quantize(const void* V, int v_dtype, int64_t R, int64_t K, int layout, uint8_t* codes, uint8_t* scales,
                   void* stream) {
  const char* fn = "mxfp4_quantize";
  int st;
  if ((st = check_nk(fn, R, K))) return st;
  if ((st = check_dtype(fn, v_dtype, "v_dtype"))) return st;
  if (layout != SSN_MX_ROWS && layout != SSN_MX_TILED) return fail(SSN_E_RANGE, "%s: unknown layout %d", fn, layout);
  if (R == 0 || K == 0) return ok();
  REQUIRE_PTR(V); REQUIRE_PTR(codes); REQUIRE_PTR(scales);
  return hip_status(ssn::launch_mx_quantize(V, v_dtype == SSN_BF16, R, K, layout == SSN_MX_TILED, codes, scales,
                                            as_stream(stream)), fn);
}

int gemm_mxfp4(const uint8_t* x_codes, const uint8_t* x_scales, int64_t M, const uint8_t* w_codes,
               const uint8_t* w_scales, int64_t N, int64_t K, void* Y, int y_dtype, int algo, int* algo_used,
               void* stream) {
  const char* fn = "gemm_mxfp4";
  int st;
  if (M < 0 || M > kMaxRows) return fail(SSN_E_SHAPE, "%s: bad M=%lld", fn, (long long)M);
  if ((st = check_nk(fn, N, K))) return st;
  if ((st = check_dtype(fn, y_dtype, "y_dtype"))) return st;
  if (algo != SSN_ALGO_AUTO && algo != SSN_ALGO_MFMA)
    return fail(SSN_E_ALGO, "%s: algorithm %d is not available (the block-scaled matrix cores only)", fn, algo);
  if (algo_used) *algo_used = SSN_ALGO_MFMA;
  if (M == 0 || N == 0) return ok();
  if (K == 0) return fail(SSN_E_SHAPE, "%s: K must be positive when M, N > 0", fn);
  REQUIRE_PTR(x_codes); REQUIRE_PTR(x_scales); REQUIRE_PTR(w_codes); REQUIRE_PTR(w_scales); REQUIRE_PTR(Y);
  return hip_status(ssn::launch_gemm_mx(x_codes, x_scales, M, w_codes, w_scales, N, K, Y, y_dtype == SSN_BF16,
                                        as_stream(stream)), fn);
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------
// Calibration
extern "C" {

int64_t mfma_probe_sink_floats(void) { return (int64_t)ssn::cu_count() * 2 * 256; }

int mfma_probe(int kind, int waves_per_simd, int iters, uint32_t seed, float* sink, double* flops, void* stream) {
  const char* fn = "mfma_probe";
  if (kind != SSN_PROBE_BF16 && kind != SSN_PROBE_FP4) return fail(SSN_E_RANGE, "%s: unknown kind %d", fn, kind);
  if (waves_per_simd != 1 && waves_per_simd != 2)
    return fail(SSN_E_RANGE, "%s: waves_per_simd must be 1 or 2 (got %d)", fn, waves_per_simd);
  if (iters <= 0 || iters > (1 << 24)) return fail(SSN_E_RANGE, "%s: iters=%d outside [1, 2^24]", fn, iters);
  REQUIRE_ELEM_PTR(sink);
  const double per_op = kind == SSN_PROBE_BF16 ? 2.0 * 32 * 32 * 16 : 2.0 * 32 * 32 * 64;
  if (flops) *flops = per_op * (waves_per_simd == 1 ? 16 : 8) * (double)iters * ssn::cu_count() * waves_per_simd * 4;
  return hip_status(ssn::launch_mfma_probe(kind, waves_per_simd, iters, seed, sink, as_stream(stream)), fn);
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------
// Allocation-free whole FFN: its workspace is a static device array, one copy per GPU, held
// until the process ends. Every kernel writes the workspace bytes it later reads (routing
// arrays, H, Yd), so nothing needs clearing between calls; calls that overlap on one GPU share
// the array and race.
namespace {

constexpr int64_t kNoAllocScratchBytes = (int64_t)32 << 20;
static __device__ __attribute__((aligned(256))) uint8_t scratch[kNoAllocScratchBytes];

ssn::PerDeviceOnce g_scratch_once;
void* g_scratch_ptr[ssn::kMaxDevices];

// The device address of this GPU's copy of `scratch` (the host-side name is only a stand-in).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= ssn::kMaxDevices) return hipGetSymbolAddress(out, HIP_SYMBOL(scratch));
  e = ssn::once_per_device(g_scratch_once, [&] { return hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch)); });
  *out = g_scratch_ptr[dev];
  return e;
}

}  // namespace

extern "C" int moe_nvfp4_ffn_noalloc(const uint16_t* X, int64_t T, int64_t D, const int32_t* topk_ids,
                                     const float* topk_weights, int k, int E, int64_t I, int sparse, int w_layout,
                                     const uint8_t* up_main, const uint8_t* up_meta, const uint8_t* up_scales,
                                     const float* up_ts, const uint8_t* down_main, const uint8_t* down_meta,
                                     const uint8_t* down_scales, const float* down_ts, float* out, int64_t* bad_ids,
                                     void* stream) {
  const char* fn = "moe_nvfp4_ffn_noalloc";
  int st;
  if ((st = check_route_shape(fn, T, k, E))) return st;
  if (I <= 0 || D <= 0 || I % 64 || D % 64)
    return fail(SSN_E_SHAPE, "%s: I=%lld and D=%lld must be positive multiples of 64", fn, (long long)I, (long long)D);
  const int64_t need = moe_ffn_workspace_bytes(T, k, E, I, D);
  if (need > kNoAllocScratchBytes)
    return fail(SSN_E_RANGE, "%s: this FFN needs %lld bytes of workspace; the static scratch holds %lld", fn,
                (long long)need, (long long)kNoAllocScratchBytes);
  void* ws = nullptr;
  if ((st = hip_status(scratch_address(&ws), fn))) return st;
  return moe_nvfp4_ffn(X, T, D, topk_ids, topk_weights, k, E, I, sparse, w_layout, up_main, up_meta, up_scales, up_ts,
                       down_main, down_meta, down_scales, down_ts, out, bad_ids, ws, kNoAllocScratchBytes, stream);
}
