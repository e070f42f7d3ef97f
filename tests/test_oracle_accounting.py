"""Pins for the byte / bit / roofline / Amdahl arithmetic against the pages' printed numbers."""
import json
import os

import pytest

from oracle import accounting as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _g(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_ridge_and_ceilings():
    g = _g("roofline.json")
    r = A.ridge(g["peak_tflops"] * 1e12, g["bandwidth_gbs"] * 1e9)
    assert round(r) == g["ridge_flop_per_byte"]
    assert round(100 * A.roof_fraction(g["decode_intensity"], g["ridge_flop_per_byte"]), 1) == g["decode_ceiling_pct"]
    assert round(100 * A.roof_fraction(g["mixed_intensity"], g["ridge_flop_per_byte"]), 1) == g["mixed_ceiling_pct"]


def test_storage_bits():
    g = _g("storage.json")
    assert A.bits_per_weight_dense() == g["dense_bits"]
    assert A.bits_per_weight_dense() / 8 == g["dense_bytes"]
    # the page's estimate prices one scale per 16 kept values (= 32 original weights)
    page = A.bits_per_weight_sp24(scale_block_original=32)
    assert page == g["sp24_bits_page"]
    assert round(100 * A.saving(A.bits_per_weight_dense(), page)) == g["saving_pct_page"]
    # values + index alone exceed half of dense, which is why the saving is not a half
    assert g["sp24_value_bits"] + g["sp24_index_bits"] > g["dense_bits"] / 2
    # the layout stored here keeps one scale per 16 original weights: 3.5 bits
    assert A.bits_per_weight_sp24() == 3.5
    b = A.sp24_bytes(128, 256)
    d = A.dense_bytes(128, 256)
    assert (b["vals"] + b["meta"] + b["scales"]) * 8 / (128 * 256) == 3.5
    assert (d["codes"] + d["scales"]) * 8 / (128 * 256) == 4.5


def test_amdahl():
    g = _g("amdahl.json")
    assert g["total_ms"] - g["affected_ms"] + g["affected_ms"] / g["region_speedup"] == g["new_total_ms"]
    assert round(A.amdahl(g["total_ms"], g["affected_ms"], g["region_speedup"]), 2) == g["ratio"]


def test_output_head_size():
    g = _g("output_head.json")
    assert round(g["bf16_gib"] * A.bits_per_weight_dense() / 16, 2) == g["nvfp4_gib"]


def test_gemm_flops():
    assert A.gemm_flops(4096, 4096, 4096) == 137438953472
    assert A.gemm_flops(1, 13824, 5120) == 141557760
    with pytest.raises(TypeError):
        A.gemm_flops(1, 2)
