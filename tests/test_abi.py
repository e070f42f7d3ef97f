"""C-ABI checks that need no GPU: the library loads, exports every entry point the header
declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

import structured_sparse_nvfp4_amd as ssn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssnvfp4.h")

pytestmark = pytest.mark.skipif(not os.path.exists(ssn.LIB_PATH), reason="library not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_calls():
    names = declared_functions()
    for want in ["nvfp4_quantize", "nvfp4_dequantize", "sp24_prune", "sp24_check", "sp24_compress",
                 "sp24_decompress", "gemm_nvfp4_dense", "gemm_nvfp4_sp24", "ssn_last_error", "ssn_version"]:
        assert want in names


def test_every_declared_symbol_is_exported():
    L = ctypes.CDLL(ssn.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name
    assert set(declared_functions()) <= set(ssn._SIGS), "binding misses a declared call"


def test_version():
    assert ssn.lib().ssn_version() >= 100


def _bad(ptr=0x1000):
    return ctypes.c_void_p(ptr)


def test_validation_paths_return_codes_without_launching():
    L = ssn.lib()
    p, n = _bad(), None
    # K not a multiple of 32
    assert L.sp24_check(p, 4, 48, p, p, n) == ssn.SSN_E_SHAPE
    assert b"multiple of 32" in L.ssn_last_error()
    assert L.sp24_compress(p, 4, 16, p, p, p, n) == ssn.SSN_E_SHAPE
    assert L.nvfp4_quantize(p, 0, 4, 40, n, p, p, p, n) == ssn.SSN_E_SHAPE
    # negative sizes
    assert L.sp24_decompress(p, p, -1, 32, p, n) == ssn.SSN_E_SHAPE
    assert L.gemm_nvfp4_dense(p, -2, 4, 32, p, p, p, p, 0, 0, n, n) == ssn.SSN_E_SHAPE
    # NULL and misaligned pointers
    assert L.sp24_check(p, 4, 64, n, n, n) == ssn.SSN_E_NULL
    assert b"bad_groups" in L.ssn_last_error()
    assert L.sp24_compress(_bad(0x1008), 4, 64, p, p, p, n) == ssn.SSN_E_ALIGN
    # sp24_prune: the tensor scale output is optional, but a given one must be f32-aligned
    assert L.sp24_prune(p, 0, 4, 48, p, n, n) == ssn.SSN_E_SHAPE
    assert L.sp24_prune(p, 0, 4, 64, p, _bad(0x1002), n) == ssn.SSN_E_ALIGN
    assert b"tensor_scale_out" in L.ssn_last_error()
    assert L.sp24_prune(n, 0, 4, 64, p, n, n) == ssn.SSN_E_NULL
    assert L.nvfp4_quantize(p, 0, 4, 64, n, p, p, n, n) == ssn.SSN_E_NULL
    assert L.gemm_nvfp4_dense(p, 2, 4, 64, n, p, p, p, 0, 0, n, n) == ssn.SSN_E_NULL
    # dtype and algorithm codes
    assert L.nvfp4_quantize(p, 7, 4, 64, n, p, p, p, n) == ssn.SSN_E_DTYPE
    assert L.gemm_nvfp4_dense(p, 2, 4, 64, p, p, p, p, 3, 0, n, n) == ssn.SSN_E_DTYPE
    assert L.gemm_nvfp4_dense(p, 2, 4, 64, p, p, p, p, 0, 99, n, n) == ssn.SSN_E_ALGO
    assert L.gemm_nvfp4_dense(p, 2, 4, 64, p, p, p, p, 0, ssn.ALGO_SMFMAC, n, n) == ssn.SSN_E_ALGO
    assert L.gemm_nvfp4_sp24(p, 2, 4, 64, p, p, p, p, p, 0, ssn.ALGO_MFMA, n, n) == ssn.SSN_E_ALGO
    # an explicit algorithm that does not fit the shape is refused, not replaced
    used = ctypes.c_int(-1)
    assert L.gemm_nvfp4_sp24(p, 2, 4, 96, p, p, p, p, p, 0, ssn.ALGO_SMFMAC, ctypes.byref(used), n) == ssn.SSN_E_ALGO
    assert b"K % 64" in L.ssn_last_error()
    for algo, fn in ((ssn.ALGO_MFMA, "dense"), (ssn.ALGO_DECOMPRESS_MFMA, "sp24"), (ssn.ALGO_SMFMAC, "sp24")):
        if fn == "dense":
            st = L.gemm_nvfp4_dense(p, 17, 4, 96, p, p, p, p, 0, algo, ctypes.byref(used), n)
        else:
            st = L.gemm_nvfp4_sp24(p, 17, 4, 96, p, p, p, p, p, 0, algo, ctypes.byref(used), n)
        assert st == ssn.SSN_E_ALGO and b"K % 64" in L.ssn_last_error()


def test_empty_problem_is_a_noop():
    L = ssn.lib()
    used = ctypes.c_int(-1)
    assert L.gemm_nvfp4_dense(None, 0, 4, 64, None, None, None, None, 0, 0, ctypes.byref(used), None) == ssn.SSN_OK
    assert L.gemm_nvfp4_sp24(None, 3, 0, 64, None, None, None, None, None, 0, 0, None, None) == ssn.SSN_OK
    assert L.sp24_decompress(None, None, 0, 64, None, None) == ssn.SSN_OK
    assert L.ssn_last_error() == b""


def test_moe_validation_without_launch():
    L = ssn.lib()
    p = ctypes.c_void_p(16)
    n = None
    p2 = ctypes.c_void_p(1 << 20)   # a second, non-overlapping fake device address
    assert L.moe_route_workspace_bytes(10, 0, 8) == -1
    assert L.moe_route_workspace_bytes(10, 2, 4096) == -1
    assert L.moe_route_workspace_bytes(0, 2, 8) == 0
    # top-k and expert count outside their ranges
    assert L.moe_route(p, 10, 0, 8, p, p, p, p, n, p, 1 << 20, n) == ssn.SSN_E_RANGE
    assert L.moe_route(p, 10, 2, 0, p, p, p, p, n, p, 1 << 20, n) == ssn.SSN_E_RANGE
    # too small a workspace is refused before any launch
    need = L.moe_route_workspace_bytes(5000, 10, 512)
    assert need > 0
    assert L.moe_route(p, 5000, 10, 512, p, p, p, p, n, p, need - 1, n) == ssn.SSN_E_RANGE
    assert b"workspace" in L.ssn_last_error()
    # grouped product: odd N with the SiLU gate, K not a multiple of 64, unknown epilogue and algorithms
    used = ctypes.c_int(-1)
    assert L.moe_grouped_gemm_nvfp4(p, 8, p, p, 4, 8, 33, 64, 0, 0, p, n, p, p, 1, p, 1, 0, n, n) == ssn.SSN_E_SHAPE
    assert L.moe_grouped_gemm_nvfp4(p, 8, p, p, 4, 8, 32, 96, 0, 0, p, n, p, p, 0, p, 0, 0, n, n) == ssn.SSN_E_SHAPE
    assert L.moe_grouped_gemm_nvfp4(p, 8, p, p, 4, 8, 32, 64, 0, 0, p, n, p, p, 5, p, 0, 0, n, n) == ssn.SSN_E_RANGE
    assert L.moe_grouped_gemm_nvfp4(p, 8, p, p, 4, 8, 32, 64, 0, 0, p, n, p, p, 0, p, 0, ssn.ALGO_SMFMAC,
                                    ctypes.byref(used), n) == ssn.SSN_E_ALGO
    assert L.moe_grouped_gemm_nvfp4(p, 8, p, p, 4, 8, 32, 64, 1, 0, p, n, p, p, 0, p, 0, 0, n, n) == ssn.SSN_E_NULL
    assert L.moe_grouped_gemm_nvfp4(p, 8, n, p, 9999, 8, 32, 64, 0, 0, p, n, p, p, 0, p, 0, 0, n, n) == ssn.SSN_E_RANGE
    # empty problems are no-ops
    assert L.moe_grouped_gemm_nvfp4(n, 0, n, n, 4, 0, 32, 64, 0, 0, n, n, n, n, 0, n, 0, 0, ctypes.byref(used), n) == ssn.SSN_OK
    assert used.value == ssn.ALGO_STREAM       # AUTO: few rows per expert and N % 32 == 0
    assert L.moe_grouped_gemm_nvfp4(n, 0, n, n, 4, 0, 40, 64, 0, 0, n, n, n, n, 0, n, 0, 0, ctypes.byref(used), n) == ssn.SSN_OK
    assert used.value == ssn.ALGO_MFMA         # N % 32 != 0: the tiles
    assert L.moe_grouped_gemm_nvfp4(n, 0, n, n, 4, 0, 40, 64, 0, 0, n, n, n, n, 0, n, 0, ssn.ALGO_STREAM,
                                    ctypes.byref(used), n) == ssn.SSN_E_ALGO
    assert L.moe_grouped_gemm_nvfp4(n, 0, n, n, 4, 0, 32, 64, 1, 0, n, n, n, n, 0, n, 0, ssn.ALGO_STREAM,
                                    ctypes.byref(used), n) == ssn.SSN_OK and used.value == ssn.ALGO_STREAM
    # unknown weight layout
    assert L.moe_grouped_gemm_nvfp4(p, 8, p, p, 4, 8, 32, 64, 0, 7, p, n, p, p, 0, p, 0, 0, n, n) == ssn.SSN_E_RANGE
    # the tiles address X and one expert's weights with 32-bit byte offsets: X of 2^31 bytes
    # (x_rows = 2^20, K = 1024) or an expert's codes / vals of 2^31 bytes are refused for an
    # explicit tile algorithm, and for AUTO when STREAM cannot take the shape (N % 32 != 0)
    for sparse, algo in ((0, ssn.ALGO_MFMA), (1, ssn.ALGO_SMFMAC), (1, ssn.ALGO_DECOMPRESS_MFMA)):
        assert L.moe_grouped_gemm_nvfp4(p, 1 << 20, p, p, 4, 64, 64, 1024, sparse, 0, p, p, p, p, 0, p, 0, algo,
                                        ctypes.byref(used), n) == ssn.SSN_E_ALGO
        assert b"below 2^31 bytes" in L.ssn_last_error()
    assert L.moe_grouped_gemm_nvfp4(p, (1 << 20) - 1, n, p, 4, 0, 64, 1024, 0, 0, n, n, n, n, 0, n, 0,
                                    ssn.ALGO_MFMA, ctypes.byref(used), n) == ssn.SSN_OK   # just below: admitted
    assert L.moe_grouped_gemm_nvfp4(p, 8, p, p, 4, 64, 1 << 20, 4096, 0, 0, p, n, p, p, 0, p, 0, ssn.ALGO_MFMA,
                                    ctypes.byref(used), n) == ssn.SSN_E_ALGO            # N * K/2 = 2^31
    assert L.moe_grouped_gemm_nvfp4(p, 8, p, p, 4, 64, 1 << 21, 4096, 1, 0, p, p, p, p, 0, p, 0, ssn.ALGO_SMFMAC,
                                    ctypes.byref(used), n) == ssn.SSN_E_ALGO            # N * K/4 = 2^31
    assert L.moe_grouped_gemm_nvfp4(p, 1 << 20, p, p, 4, 64, 40, 1024, 0, 0, p, n, p, p, 0, p, 0, 0,
                                    ctypes.byref(used), n) == ssn.SSN_E_SHAPE           # AUTO, N % 32 != 0
    assert b"STREAM needs N % 32 == 0" in L.ssn_last_error()
    # 64-k tiling of a weight array: piece sizes, divisibility, overlap, NULL, empty
    assert L.moe_pack_ktiles(p, 2, 8, 32, 12, p2, n) == ssn.SSN_E_RANGE
    assert L.moe_pack_ktiles(p, 2, 8, 48, 32, p2, n) == ssn.SSN_E_SHAPE
    assert L.moe_pack_ktiles(p, 2, 8, 32, 32, p, n) == ssn.SSN_E_RANGE
    assert L.moe_pack_ktiles(n, 2, 8, 32, 32, p2, n) == ssn.SSN_E_NULL
    assert L.moe_pack_ktiles(n, 0, 8, 32, 32, n, n) == ssn.SSN_OK
    assert L.moe_combine(n, 0, 0, n, n, 0, 4, 16, n, n) == ssn.SSN_OK
    assert L.moe_combine(p, 7, 4, p, p, 2, 2, 16, p, n) == ssn.SSN_E_DTYPE
    assert L.moe_ffn_workspace_bytes(4096, 10, 512, 512, 2048) > 4096 * 10 * 2048 * 4


def _declared_params():
    """name -> list of parameter declarations, parsed from the header."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(([^)]*)\)\s*;", text, flags=re.M):
        params = [p.strip() for p in m.group(2).split(",") if p.strip() and p.strip() != "void"]
        out[m.group(1)] = params
    return out


def test_binding_signatures_match_the_header():
    # every call (including those whose arguments differ from the problem statement's sketch:
    # moe_route's row_of / bad_ids / workspace, the grouped product's x_rows / R / w_layout /
    # algo_used, moe_combine's row_of, the whole-FFN call) is bound with the header's argument count
    decl = _declared_params()
    assert decl, "no declarations parsed"
    for name, params in decl.items():
        assert len(ssn._SIGS[name][0]) == len(params), name


def test_algorithm_codes_match_the_header():
    text = open(HEADER).read()
    codes = {k: int(v) for k, v in re.findall(r"SSN_ALGO_(\w+)\s*=\s*(\d+)", text)}
    assert codes == {"AUTO": 0, "VALU": 1, "MFMA": 2, "SMFMAC": 3, "GATHER": 4, "DECOMPRESS_MFMA": 5, "STREAM": 6}
    for name, v in codes.items():
        assert getattr(ssn, f"ALGO_{name}") == v


def test_gather_algorithm_and_tile_k_limit():
    L = ssn.lib()
    p, n = _bad(), None
    used = ctypes.c_int(-1)
    # skip-and-gather is a 2:4 algorithm; the vector-ALU request on 2:4 weights reports it
    assert L.gemm_nvfp4_dense(p, 2, 4, 64, p, p, p, p, 0, ssn.ALGO_GATHER, n, n) == ssn.SSN_E_ALGO
    assert b"2:4 weights only" in L.ssn_last_error()
    assert L.gemm_nvfp4_sp24(n, 0, 4, 64, n, n, n, n, n, 0, ssn.ALGO_GATHER, ctypes.byref(used), n) == ssn.SSN_OK
    assert used.value == ssn.ALGO_GATHER
    assert L.gemm_nvfp4_sp24(n, 0, 4, 64, n, n, n, n, n, 0, ssn.ALGO_VALU, ctypes.byref(used), n) == ssn.SSN_OK
    assert used.value == ssn.ALGO_GATHER
    # the 256 x 256 tiles address their activation panel with 32-bit offsets: K beyond 2^21 is
    # refused for an explicit matrix-core choice at M > 16 (AUTO takes the vector-ALU kernels)
    big_k = (1 << 21) + 64
    assert L.gemm_nvfp4_dense(p, 17, 4, big_k, p, p, p, p, 0, ssn.ALGO_MFMA, n, n) == ssn.SSN_E_ALGO
    assert b"K <= 2097152" in L.ssn_last_error()
    for algo in (ssn.ALGO_SMFMAC, ssn.ALGO_DECOMPRESS_MFMA):
        assert L.gemm_nvfp4_sp24(p, 17, 4, big_k, p, p, p, p, p, 0, algo, n, n) == ssn.SSN_E_ALGO
    assert L.gemm_nvfp4_dense(n, 0, 4, big_k, n, n, n, n, 0, ssn.ALGO_MFMA, n, n) == ssn.SSN_OK


def test_mfma_probe_validation_without_launch():
    # the calibration call rejects its ranges before anything is launched
    L = ssn.lib()
    p, n = ctypes.c_void_p(4096), None
    assert L.mfma_probe(2, 1, 16, 0, p, n, n) == ssn.SSN_E_RANGE
    assert L.mfma_probe(ssn.PROBE_BF16, 3, 16, 0, p, n, n) == ssn.SSN_E_RANGE
    assert L.mfma_probe(ssn.PROBE_FP4, 1, 0, 0, p, n, n) == ssn.SSN_E_RANGE
    assert L.mfma_probe(ssn.PROBE_FP4, 2, (1 << 24) + 1, 0, p, n, n) == ssn.SSN_E_RANGE
    assert L.mfma_probe(ssn.PROBE_BF16, 1, 16, 0, None, n, n) == ssn.SSN_E_NULL
    assert L.mfma_probe(ssn.PROBE_BF16, 1, 16, 0, ctypes.c_void_p(4098), n, n) == ssn.SSN_E_ALIGN
