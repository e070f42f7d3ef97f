/*
 * ssnvfp4.h — NVFP4 weight-quantised GEMM/GEMV with optional 2:4 structured sparsity,
 * hand-written for AMD Instinct MI355X (gfx950).
 *
 * The problem, as stated on the pages this library follows:
 *  - NVFP4 weights: 4-bit E2M1 values, one FP8 E4M3 scale per 16 consecutive values along the
 *    reduction axis, one FP32 tensor scale ("NVFP4 Without FP4 Hardware", ai-muninn.com, section
 *    "Convert BF16 to NVFP4 yourself"); a scale may be shared by a group of tensors (same page,
 *    section "The shared global scale").
 *  - 2:4 sparsity along the reduction axis K: every group of four has at least two zeros
 *    ("Sparse GPU FLOPS Need the Right Zeros in the Right Places", leviathansystems.co, section
 *    "The operation determines which four entries belong together"), checked per group ("Two
 *    half-zero vectors produce different pattern answers"); stored as the two kept values plus a
 *    2-bit position each ("NVFP4 vs 2:4 sparse", robertz.co, section "What 2:4 actually is").
 *  - Reporting which implementation actually ran (leviathansystems.co page, section "Ask which
 *    sparse implementations were actually selected"): every GEMM call reports its algorithm.
 *
 * Layouts (all row-major, K = reduction axis, contiguous):
 *   W (input to quantise / prune)  f32 or bf16 [N, K]
 *   codes   u8 [N, K/2]   element k=2j in the low nibble of byte j, k=2j+1 in the high nibble
 *   scales  u8 [N, K/16]  E4M3 (OCP "FN": bias 7, 0x7E = 448, no Inf) block scale of K/16 blocks
 *   tensor_scale  f32 [1] s_t; decoded weight = E2M1(code) * E4M3(scale) * s_t
 *   vals    u8 [N, K/4]   2:4 kept codes: byte g = code[4g+i0] | code[4g+i1] << 4, i0 < i1
 *   meta    u8 [N, K/8]   positions: nib(g) = i0 | i1 << 2; byte j = nib(2j) | nib(2j+1) << 4
 *   X       bf16 bit patterns (uint16) [M, K]
 *   Y       f32 or bf16 [M, N];  Y = X . W_hat^T with f32 accumulation
 *
 * Conventions:
 *  - Every pointer is caller-owned DEVICE memory unless marked "host". The library never
 *    allocates or frees memory and keeps no pointer after a call returns. Inputs and outputs
 *    must stay alive until the stream has passed the call's kernels.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream). Calls are
 *    stream-ordered and asynchronous; results are ready when the stream reaches them.
 *  - Every call validates its arguments on the host before launching anything and returns a
 *    status code; it never throws and never silently falls back. On a non-OK return nothing
 *    was launched (except SSN_E_HIP, where a launch itself failed) and ssn_last_error() gives a
 *    thread-local message.
 *  - Sizes: N, M >= 0 (a zero size is a no-op that returns SSN_OK); K % 32 == 0 for the
 *    NVFP4/2:4 calls (so a 32-bit word of meta covers whole groups and rows of every array
 *    are 2-byte aligned). Device pointers to tensors (activations, codes, scales, vals, meta,
 *    outputs) must be 16-byte aligned; pointers to single scalars and to int32/f32 index or
 *    weight arrays (tensor scales, counters, routing arrays, combine weights) only need the
 *    alignment of their element type.
 *  - Data-dependent failures (a group that is not 2:4) are reported in device counters, not
 *    in the return code.
 *  - Calls that write the same output buffers and overlap on one stream or across streams race.
 */
#ifndef SSNVFP4_H
#define SSNVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSN_OK = 0,
  SSN_E_NULL = 1,   /* a required pointer is NULL */
  SSN_E_SHAPE = 2,  /* a size is negative, K % 32 != 0, or sizes are inconsistent */
  SSN_E_ALIGN = 3,  /* a device pointer is not aligned as required */
  SSN_E_DTYPE = 4,  /* unknown dtype code */
  SSN_E_ALGO = 5,   /* unknown algorithm, or an explicit algorithm that does not apply to the shape */
  SSN_E_HIP = 6,    /* a HIP launch or runtime call failed */
  SSN_E_RANGE = 7   /* an argument is outside its documented range (e.g. top-k, expert count) */
} ssn_status;

enum { SSN_F32 = 0, SSN_BF16 = 1 };

/* GEMM algorithms. Each call writes the one it ran to *algo_used (host int, nullable).
 * The matrix-core algorithms run decode-shaped kernels for M <= 16 (weights streamed once
 * through LDS) and 256 x 256 output tiles for larger M; the tiles need K % 64 == 0 and
 * K <= 2^21 (a tile addresses its 256-row activation panel with 32-bit byte offsets). AUTO picks
 * MFMA for dense weights and SMFMAC for 2:4 weights, DECOMPRESS_MFMA when M <= 16 and
 * K % 64 != 0, and the vector-ALU kernels (VALU dense, GATHER 2:4) when M > 16 and the tiles do
 * not apply. */
enum {
  SSN_ALGO_AUTO = 0,             /* let the library choose; the choice is reported */
  SSN_ALGO_VALU = 1,             /* plain vector-ALU kernel, any K % 32 == 0: dense weights, one
                                    FMA per weight; with 2:4 weights it runs the GATHER kernel
                                    and reports GATHER */
  SSN_ALGO_MFMA = 2,             /* dense: bf16 MFMA on weights decoded in registers */
  SSN_ALGO_SMFMAC = 3,           /* 2:4 only: sparse MFMA (v_smfmac) with the compressed weights
                                    as the sparse operand; needs K % 64 == 0 */
  SSN_ALGO_GATHER = 4,           /* 2:4 only: skip-and-gather on the vector ALU: each kept value is
                                    decoded with its scale and multiplied by the activation picked
                                    at its stored position; any K % 32 == 0 */
  SSN_ALGO_DECOMPRESS_MFMA = 5,  /* 2:4 only: expand vals+meta to a dense tile and run the
                                    dense bf16 MFMA (computes on the zeros) */
  SSN_ALGO_STREAM = 6            /* grouped-expert calls only: one wave streams 32 weight rows
                                    of an expert for up to 32 of its routed rows (decode-sized
                                    routings); dense on MFMA, 2:4 on SMFMAC; needs N % 32 == 0 */
};

enum { SSN_EPI_NONE = 0, SSN_EPI_SILU_GATE = 1 };
/* Weight layouts of the grouped-expert calls (see moe_pack_ktiles). */
enum { SSN_WLAYOUT_ROWS = 0, SSN_WLAYOUT_KTILE64 = 1 };

/* Thread-local message describing the last non-OK return on this thread ("" if none). */
const char* ssn_last_error(void);
/* Library version, major * 10000 + minor * 100 + patch. */
int ssn_version(void);

/* ---------------------------------------------------------------------------------------------
 * nvfp4_quantize — NVFP4 quantisation of one tensor ("NVFP4 Without FP4 Hardware",
 * ai-muninn.com, section "Convert BF16 to NVFP4 yourself"; shared scale: section "The shared
 * global scale").
 *   s_t = fl32(amax|W| / 2688) unless tensor_scale_in is given (then s_t = *tensor_scale_in);
 *   per block of 16 along K: S = E4M3 nearest-even of min(amax_block / (6 s_t), 448);
 *   code = sign(w) | E2M1 nearest-even of |w| / (s_t * S), saturating at 6 (a negative value
 *   that rounds to zero gives the FP4 negative zero 0x8); a block with S = 0 stores code 0.
 *   Rounding decisions are exact (taken in float64 on the exact quotients).
 * W: f32 or bf16 (w_dtype) [N, K]; codes [N, K/2]; scales [N, K/16]; tensor_scale_in: f32 [1]
 * or NULL; tensor_scale_out: f32 [1], receives s_t (may equal tensor_scale_in).
 * W must be finite. Errors: NULL, SHAPE (K % 32), ALIGN, DTYPE, HIP.
 * ------------------------------------------------------------------------------------------- */
int nvfp4_quantize(const void* W, int w_dtype, int64_t N, int64_t K, const float* tensor_scale_in,
                   uint8_t* codes, uint8_t* scales, float* tensor_scale_out, void* stream);

/* nvfp4_dequantize — decoded weights out[n,k] = E2M1(code) * E4M3(S) * s_t, written as f32 or
 * bf16 (out_dtype; bf16 is rounded to nearest-even). Same layouts as above. */
int nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                     int64_t N, int64_t K, void* out, int out_dtype, void* stream);

/* ---------------------------------------------------------------------------------------------
 * sp24_prune — magnitude pruning to 2:4 along K: in every group of four keep the two entries
 * of largest |w| (equal magnitudes: the lower index wins) and write +0.0 to the other two.
 * This produces weights that pass sp24_check after quantisation. W, W_out: f32 or bf16
 * [N, K] (same dtype; W_out may equal W for in place). tensor_scale_out: f32 [1] or NULL;
 * when given it receives s_t = fl32(amax|W| / 2688), the NVFP4 tensor scale of nvfp4_quantize
 * ("NVFP4 Without FP4 Hardware", ai-muninn.com, section "The shared global scale"), taken
 * while W is read. The largest entry of every group is kept, so this is the tensor scale of
 * W and of the pruned tensor alike, bit for bit: passed to nvfp4_quantize as tensor_scale_in
 * it spares that call its own pass over the weights. Errors: NULL, SHAPE, ALIGN, DTYPE, HIP.
 * ------------------------------------------------------------------------------------------- */
int sp24_prune(const void* W, int w_dtype, int64_t N, int64_t K, void* W_out, float* tensor_scale_out,
               void* stream);

/* ---------------------------------------------------------------------------------------------
 * sp24_check — per-group 2:4 eligibility of NVFP4 codes ("Sparse GPU FLOPS Need the Right Zeros
 * in the Right Places", leviathansystems.co, sections "The operation determines which four
 * entries belong together" and "Two half-zero vectors produce different pattern answers").
 * A code is zero when its magnitude bits are 0 (0x0 and 0x8). A group passes when it holds at
 * least two zero codes.
 * codes [N, K/2]; bad_groups: int64 [1] = number of failing groups; first_bad: int64 [1]
 * (nullable) = smallest flat index n*(K/4)+g of a failing group, or -1 if none.
 * Errors: NULL, SHAPE, ALIGN, HIP.
 * ------------------------------------------------------------------------------------------- */
int sp24_check(const uint8_t* codes, int64_t N, int64_t K, int64_t* bad_groups, int64_t* first_bad,
               void* stream);

/* ---------------------------------------------------------------------------------------------
 * sp24_compress — 2:4 compression of NVFP4 codes into two kept codes plus two 2-bit positions
 * per group ("NVFP4 vs 2:4 sparse", robertz.co, section "What 2:4 actually is" and its figure:
 * w0 0 0 w3 is stored as w0 w3 with positions 0 and 3).
 * Kept positions: the nonzero codes first, then the lowest-index zero codes, ascending
 * (i0 < i1); kept codes are copied verbatim. A failing group (fewer than two zeros) is written
 * as vals 0x00 and positions (0, 1), and counted in *bad_groups.
 * codes [N, K/2] -> vals [N, K/4], meta [N, K/8]; bad_groups int64 [1].
 * Errors: NULL, SHAPE, ALIGN, HIP.
 * ------------------------------------------------------------------------------------------- */
int sp24_compress(const uint8_t* codes, int64_t N, int64_t K, uint8_t* vals, uint8_t* meta,
                  int64_t* bad_groups, void* stream);

/* ---------------------------------------------------------------------------------------------
 * nvfp4_sp24_produce — the 2:4 weight producer in one pass over W: the result of sp24_prune,
 * then nvfp4_quantize, then sp24_compress, bit for bit ("NVFP4 vs 2:4 sparse", robertz.co,
 * section "Where it is supported in software": the tool that pruned and packed 2:4 checkpoints was
 * withdrawn; "NVFP4 Without FP4 Hardware", ai-muninn.com, sections "Convert BF16 to NVFP4
 * yourself" and "The shared global scale").
 * Pruning keeps the two largest |w| of each group of four along K (ties to the lower index) and
 * sets the others to +0.0; because the largest entry of every block and of the tensor is kept,
 * s_t and the block scales are those of W itself (s_t = *tensor_scale_in when given).
 * W: f32 or bf16 (w_dtype) [N, K], finite; outputs (device, caller-owned): vals [N, K/4],
 * meta [N, K/8], scales [N, K/16], tensor_scale_out f32 [1], codes [N, K/2] (nullable: the
 * pruned tensor's NVFP4 codes, for the dense product on pruned weights), bad_groups int64 [1]
 * (groups with fewer than two zero codes: always 0 after pruning, kept for the compress
 * contract). Errors: NULL, SHAPE (K % 32), ALIGN, DTYPE, HIP.
 * ------------------------------------------------------------------------------------------- */
int nvfp4_sp24_produce(const void* W, int w_dtype, int64_t N, int64_t K, const float* tensor_scale_in,
                       uint8_t* vals, uint8_t* meta, uint8_t* scales, float* tensor_scale_out,
                       uint8_t* codes, int64_t* bad_groups, void* stream);

/* sp24_decompress — inverse of sp24_compress: writes the kept codes at their positions and
 * code 0 elsewhere (if i0 == i1 the second kept code wins). vals [N,K/4], meta [N,K/8] ->
 * codes [N,K/2]. Errors: NULL, SHAPE, ALIGN, HIP. */
int sp24_decompress(const uint8_t* vals, const uint8_t* meta, int64_t N, int64_t K, uint8_t* codes,
                    void* stream);

/* ---------------------------------------------------------------------------------------------
 * gemm_nvfp4_dense — Y = X . W_hat^T with W_hat[n,k] = E2M1(code) * E4M3(S[n,k/16]) * s_t,
 * f32 accumulation; weights are decoded in registers ("NVFP4 Without FP4 Hardware",
 * ai-muninn.com, section "Why NVFP4 helps without FP4 hardware": the 4-bit weights stay 4-bit
 * in memory and are unpacked inside the kernel).
 * X bf16 [M, K]; codes [N, K/2]; scales [N, K/16]; tensor_scale f32 [1]; Y [M, N] of y_dtype
 * (SSN_F32 or SSN_BF16, nearest-even). algo: AUTO, VALU or MFMA. algo_used: host int, nullable.
 * Errors: NULL, SHAPE, ALIGN, DTYPE, ALGO, HIP.
 * ------------------------------------------------------------------------------------------- */
int gemm_nvfp4_dense(const uint16_t* X, int64_t M, int64_t N, int64_t K, const uint8_t* codes,
                     const uint8_t* scales, const float* tensor_scale, void* Y, int y_dtype, int algo,
                     int* algo_used, void* stream);

/* ---------------------------------------------------------------------------------------------
 * gemm_nvfp4_sp24 — the same product from the 2:4-compressed weights: only the two kept
 * values of each group of four contribute, at their stored positions ("NVFP4 vs 2:4 sparse",
 * robertz.co, section "What 2:4 actually is": the pruned lanes are skipped).
 * vals [N, K/4], meta [N, K/8] (positions must satisfy i0 < i1, as sp24_compress writes them),
 * scales [N, K/16] (original K). algo: AUTO, GATHER (skip-and-gather; VALU is accepted for it),
 * SMFMAC (K % 64 == 0), DECOMPRESS_MFMA. Errors: NULL, SHAPE, ALIGN, DTYPE, ALGO, HIP.
 * ------------------------------------------------------------------------------------------- */
int gemm_nvfp4_sp24(const uint16_t* X, int64_t M, int64_t N, int64_t K, const uint8_t* vals,
                    const uint8_t* meta, const uint8_t* scales, const float* tensor_scale, void* Y,
                    int y_dtype, int algo, int* algo_used, void* stream);

/* =============================================================================================
 * Grouped-expert (MoE) path. The pages describe a 512-expert, top-10 mixture whose expert
 * weights are the thing every step reads ("NVFP4 vs 2:4 sparse", robertz.co, sections
 * "Concurrency, not sparsity, is the lever" and "The sparsity that does pay is already
 * running") and note that no grouped 2:4 product exists for it (same page, section "Why it
 * cannot run on this cluster"). Row space: the T*k (token, slot) entries grouped by expert
 * (ascending) and, inside an expert, in flat order f = t*k + j. Limits: 1 <= E <= 2048,
 * 1 <= k <= 64, T*k < 2^31.
 * ============================================================================================= */

/* moe_route_workspace_bytes — device workspace moe_route needs (0 when T*k == 0). */
int64_t moe_route_workspace_bytes(int64_t T, int k, int E);

/* ---------------------------------------------------------------------------------------------
 * moe_route — routing bookkeeping: a stable counting sort of the flat entries by expert id.
 * topk_ids int32 [T, k] (device). Outputs (device, caller-owned): expert_offsets int32 [E+1]
 * (rows of expert e are [offsets[e], offsets[e+1])), row_token int32 [T*k] and row_slot
 * int32 [T*k] (the (t, j) of each row), row_of int32 [T*k] (the row of entry t*k + j, or -1).
 * Entries whose id is outside [0, E) get no row; their count goes to *bad_ids (device int64
 * [1], nullable) and offsets[E] counts the placed rows. workspace: device, at least
 * moe_route_workspace_bytes(T, k, E) bytes. Errors: NULL, SHAPE, ALIGN, RANGE, HIP.
 * ------------------------------------------------------------------------------------------- */
int moe_route(const int32_t* topk_ids, int64_t T, int k, int E, int32_t* expert_offsets,
              int32_t* row_token, int32_t* row_slot, int32_t* row_of, int64_t* bad_ids,
              void* workspace, int64_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------
 * moe_grouped_gemm_nvfp4 — every expert's product in one launch:
 *   Y[r, :] = X[src(r), :] . W_hat_e^T  for r in [offsets[e], offsets[e+1]),
 * src(r) = row_token[r] (gather; nullptr = identity, r itself), W_hat_e as in gemm_nvfp4_dense
 * with the expert's tensor scale tensor_scales[e].
 * X bf16 [x_rows, K]; weights per expert, concatenated over e: dense codes [E, N, K/2], or 2:4
 * (sparse = 1) vals [E, N, K/4] + meta [E, N, K/8]; scales [E, N, K/16]; tensor_scales f32 [E].
 * epilogue SSN_EPI_NONE: Y [R, N] of y_dtype. SSN_EPI_SILU_GATE: weight rows [0, N/2) are the
 * gate and [N/2, N) the up projection (W_up [E, 2, I, K] flattened, one shared tensor scale per
 * expert, "NVFP4 Without FP4 Hardware", ai-muninn.com, section "The shared global scale");
 * Y [R, N/2] = silu(g) * u with silu(g) = g / (1 + exp(-g)), evaluated in f32 and rounded to
 * y_dtype. R: rows of Y (offsets are clamped into [0, R]); source rows are clamped into
 * [0, x_rows). Needs K % 64 == 0 and, for SILU_GATE, N even. w_layout: SSN_WLAYOUT_ROWS (the
 * arrays as above, as nvfp4_quantize / sp24_compress write them) or SSN_WLAYOUT_KTILE64 (all
 * three arrays as moe_pack_ktiles writes them). algo: MFMA (dense), SMFMAC (2:4, the sparse
 * matrix cores with the stored vals/meta as the compressed operand) or DECOMPRESS_MFMA (2:4,
 * expanded to a dense operand in registers) run 64-row x 256-column output tiles; STREAM (dense
 * or 2:4, N % 32 == 0) cuts the work along the weight rows instead, one wave per (expert, 32
 * weight rows, up to 32 routed rows), for routings with few rows per expert ("NVFP4 vs 2:4
 * sparse", robertz.co, section "Where a decode step actually spends itself": the expert weight
 * read is the cost). AUTO picks STREAM when N % 32 == 0 and R <= 4 E (dense) or R <= 10 E (2:4),
 * else the tiles (MFMA dense, SMFMAC 2:4). The tiles address X and one expert's weight arrays
 * with 32-bit byte offsets, so they need x_rows * K * 2 < 2^31 and N * K/2 (dense) or N * K/4
 * (2:4) < 2^31; beyond that AUTO picks STREAM (SHAPE if N % 32 != 0) and an explicit tile
 * algorithm is refused (ALGO).
 * algo_used: host, nullable.
 * Errors: NULL, SHAPE, ALIGN, DTYPE, ALGO, RANGE, HIP.
 * ------------------------------------------------------------------------------------------- */
int moe_grouped_gemm_nvfp4(const uint16_t* X, int64_t x_rows, const int32_t* row_token,
                           const int32_t* expert_offsets, int E, int64_t R, int64_t N, int64_t K,
                           int sparse, int w_layout, const uint8_t* w_main, const uint8_t* w_meta,
                           const uint8_t* w_scales, const float* tensor_scales, int epilogue,
                           void* Y, int y_dtype, int algo, int* algo_used, void* stream);

/* ---------------------------------------------------------------------------------------------
 * moe_pack_ktiles — the 64-k tiled layout of one expert weight array, for the grouped products.
 * Every step of the grouped path reads all expert weights ("NVFP4 vs 2:4 sparse", robertz.co,
 * section "Concurrency, not sparsity, is the lever"); a product tile consumes them 64 k at a
 * time, so this layout stores, per expert, the 64-k pieces of consecutive rows next to each
 * other: dst[e][kt][n][0:P] = src[e][n][kt*P : (kt+1)*P], kt < row_bytes / P. The bytes are
 * unchanged (a permutation). src, dst: device, [E, N, row_bytes], caller-owned, not
 * overlapping. piece_bytes P per 64 k: codes 32, vals 16, meta 8, scales 4 (row_bytes =
 * K/2, K/4, K/8, K/16). Pack all three arrays of a weight set (main, meta, scales) before
 * passing SSN_WLAYOUT_KTILE64. Errors: NULL, SHAPE, ALIGN, RANGE, HIP.
 * ------------------------------------------------------------------------------------------- */
int moe_pack_ktiles(const uint8_t* src, int64_t E, int64_t N, int64_t row_bytes, int64_t piece_bytes,
                    uint8_t* dst, void* stream);

/* ---------------------------------------------------------------------------------------------
 * moe_combine — out[t, :] = sum_j topk_weights[t, j] * Yd[row_of[t*k + j], :], summed in slot
 * order j = 0..k-1 in f32 (rows outside [0, R) are skipped). Yd [R, D] of yd_dtype; row_of
 * int32 [T*k]; topk_weights f32 [T, k]; out f32 [T, D]. Errors: NULL, SHAPE, ALIGN, DTYPE,
 * RANGE, HIP.
 * ------------------------------------------------------------------------------------------- */
int moe_combine(const void* Yd, int yd_dtype, int64_t R, const int32_t* row_of,
                const float* topk_weights, int64_t T, int k, int64_t D, float* out, void* stream);

/* moe_ffn_workspace_bytes — device workspace moe_nvfp4_ffn needs. */
int64_t moe_ffn_workspace_bytes(int64_t T, int k, int E, int64_t I, int64_t D);

/* ---------------------------------------------------------------------------------------------
 * moe_nvfp4_ffn — the whole grouped-expert FFN: route, up (SILU_GATE, H bf16 [T*k, I]),
 * down (Yd f32 [T*k, D]) and combine into out f32 [T, D]. X bf16 [T, D]; topk_ids int32
 * [T, k]; topk_weights f32 [T, k]; up weights [E, 2I, D] (+ meta when sparse), up_ts f32 [E];
 * down weights [E, D, I], down_ts f32 [E]; w_layout (both weight sets) as in
 * moe_grouped_gemm_nvfp4. workspace: device, at least moe_ffn_workspace_bytes(T, k, E, I, D)
 * bytes (holds the routing arrays, H and Yd). bad_ids: as in moe_route. Errors: those of the
 * four calls.
 * ------------------------------------------------------------------------------------------- */
int moe_nvfp4_ffn(const uint16_t* X, int64_t T, int64_t D, const int32_t* topk_ids,
                  const float* topk_weights, int k, int E, int64_t I, int sparse, int w_layout,
                  const uint8_t* up_main, const uint8_t* up_meta, const uint8_t* up_scales,
                  const float* up_ts, const uint8_t* down_main, const uint8_t* down_meta,
                  const uint8_t* down_scales, const float* down_ts, float* out, int64_t* bad_ids,
                  void* workspace, int64_t workspace_bytes, void* stream);

/* =============================================================================================
 * W4A4 variant: activations quantised as well ("Trying to beat the bandwidth", NVIDIA developer
 * forum: block-scaled FP4 x FP4 is the FP4 tensor cores' performance unlock, W4A16 has to
 * dequantise first; "NVFP4 Without FP4 Hardware", ai-muninn.com, section "Convert BF16 to NVFP4
 * yourself": W4A4 checkpoints carry activation scales). gfx950's block-scaled matrix cores take
 * E2M1 operands with one E8M0 (power-of-two) scale per 32 values along K, the OCP MX format, so
 * both operands of this variant are MXFP4:
 *   codes: E2M1 nibbles as for NVFP4 (element k = 2j in the low nibble of byte j);
 *   scales: one E8M0 byte per 32 consecutive values along K, value 2^(b - 127);
 *   quantisation of a block: e = floor(log2(amax)) - 2 clamped to [-127, 127] (-127 for an
 *   all-zero block); code = sign | E2M1 nearest-even of |v| / 2^e, saturating at 6.
 * Layouts (SSN_MX_ROWS: codes [R, K/2], scales [R, K/32] row-major; SSN_MX_TILED: the order the
 * matrix cores read, rows padded to a multiple of 32 and K to a multiple of 256 with zero codes
 * and scale byte 0):
 *   codes  [R32/32][K256/64][64][16 B]: entry l of piece (rb, ks) holds row 32 rb + l % 32,
 *          k = 64 ks + 32 (l / 32) .. + 31;
 *   scales [R32/32][K256/256][64][4 B]: byte s of entry l of piece (rb, kg) is the scale of row
 *          32 rb + l % 32 for k = 256 kg + 64 s + 32 (l / 32) .. + 31.
 * ============================================================================================= */
enum { SSN_MX_ROWS = 0, SSN_MX_TILED = 1 };

/* mxfp4_tiled_bytes — bytes of the SSN_MX_TILED codes array for [R, K] (return value) and of its
 * scales array (*scale_bytes, host, nullable); -1 for invalid sizes (K % 32 != 0, negative). */
int64_t mxfp4_tiled_bytes(int64_t R, int64_t K, int64_t* scale_bytes);

/* ---------------------------------------------------------------------------------------------
 * mxfp4_quantize — MXFP4 quantisation of V [R, K] (f32 or bf16, v_dtype; finite) into codes and
 * scales of the given layout (SSN_MX_ROWS: [R, K/2] and [R, K/32]; SSN_MX_TILED: the sizes
 * mxfp4_tiled_bytes gives, padding written as zeros). Rounding decisions are exact.
 * Errors: NULL, SHAPE (K % 32), ALIGN, DTYPE, RANGE (layout), HIP.
 * ------------------------------------------------------------------------------------------- */
int mxfp4_quantize(const void* V, int v_dtype, int64_t R, int64_t K, int layout, uint8_t* codes,
                   uint8_t* scales, void* stream);

/* ---------------------------------------------------------------------------------------------
 * gemm_mxfp4 — the W4A4 product Y = X_hat . W_hat^T on the block-scaled FP4 matrix cores
 * (v_mfma_scale_f32_32x32x64_f8f6f4), f32 accumulation: X_hat from x_codes / x_scales (M rows),
 * W_hat from w_codes / w_scales (N rows), both in the SSN_MX_TILED layout of [M, K] and [N, K];
 * Y [M, N] of y_dtype (SSN_F32 or SSN_BF16, nearest-even). algo: AUTO or MFMA (reported in
 * *algo_used, host, nullable). Errors: NULL, SHAPE, ALIGN, DTYPE, ALGO, HIP.
 * ------------------------------------------------------------------------------------------- */
int gemm_mxfp4(const uint8_t* x_codes, const uint8_t* x_scales, int64_t M, const uint8_t* w_codes,
               const uint8_t* w_scales, int64_t N, int64_t K, void* Y, int y_dtype, int algo, int* algo_used,
               void* stream);

/* ---------------------------------------------------------------------------------------------
 * Calibration (measurement only; no product path calls it). The roofline of the compute-bound
 * products is priced against the published matrix-core peaks, which assume the full clock.
 * mfma_probe measures what the GPU sustains instead: every wave issues back-to-back matrix ops
 * on register-resident operands whose bits are random (drawn once per lane from a hash of the
 * lane, the workgroup and `seed`), so the rate is set by the power limit that real data meets,
 * not by memory: the ceiling a product kernel of the same instruction can approach at best.
 * ------------------------------------------------------------------------------------------- */
enum { SSN_PROBE_BF16 = 0, SSN_PROBE_FP4 = 1 };

/* Floats the sink of mfma_probe needs (device memory, 4-byte aligned): one per launched thread
 * of the largest launch. */
int64_t mfma_probe_sink_floats(void);

/*
 * mfma_probe — launch cu_count * waves_per_simd workgroups of 256 threads (waves_per_simd waves on
 * each SIMD), each wave issuing `iters` rounds of 16 (one wave per SIMD) or 8 (two) independent
 * v_mfma_f32_32x32x16_bf16 (kind SSN_PROBE_BF16) or v_mfma_scale_f32_32x32x64_f8f6f4 on E2M1
 * codes with unit scales (SSN_PROBE_FP4). `sink` (mfma_probe_sink_floats() floats) receives one
 * value per thread so the work is kept; `*flops` (optional, host) receives the launch's
 * floating-point operations. The caller times the launch on `stream`. Errors: kind,
 * waves_per_simd (1 or 2) or iters outside [1, 2^24]: SSN_E_RANGE; sink NULL: SSN_E_NULL.
 */
int mfma_probe(int kind, int waves_per_simd, int iters, uint32_t seed, float* sink, double* flops, void* stream);

/* ---------------------------------------------------------------------------------------------
 * moe_nvfp4_ffn_noalloc — moe_nvfp4_ffn without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation). Arguments and results are those of moe_nvfp4_ffn. The workspace is a
 * static device array of the library, one copy per GPU, 32 MiB, held until the process ends;
 * a routing whose moe_ffn_workspace_bytes(T, k, E, I, D) exceeds it is refused with
 * SSN_E_RANGE before anything is launched (decode-sized routings need a few MiB: 32 tokens x
 * top-10 at D = 2048, I = 512 need 3 MiB). The call allocates nothing. Every call on a GPU
 * uses that GPU's one array: calls that overlap on one GPU (two streams, or two host threads)
 * race and must be ordered by the caller. Errors: those of moe_nvfp4_ffn, and RANGE.
 * ------------------------------------------------------------------------------------------- */
int moe_nvfp4_ffn_noalloc(const uint16_t* X, int64_t T, int64_t D, const int32_t* topk_ids,
                          const float* topk_weights, int k, int E, int64_t I, int sparse, int w_layout,
                          const uint8_t* up_main, const uint8_t* up_meta, const uint8_t* up_scales,
                          const float* up_ts, const uint8_t* down_main, const uint8_t* down_meta,
                          const uint8_t* down_scales, const float* down_ts, float* out, int64_t* bad_ids,
                          void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SSNVFP4_H */
