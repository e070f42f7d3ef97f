"""Byte, bit and roofline arithmetic for NVFP4 and 2:4 weights (oracle).

* Storage: "NVFP4 vs 2:4 sparse" (robertz.co), section "The byte saving is about a quarter,
  not a half" and its figure: dense NVFP4 spends 4 value bits plus an 8-bit scale per 16
  weights (4.5 bits, 0.5625 bytes); 2:4 halves the value bits and adds a 2-bit index per kept
  value. The page prices the scale at about 0.25 bit (one scale per 16 *kept* values) and lands
  near 3.25 bits; with one scale per 16 *original* K values, as stored here, it is 3.5 bits.
* Byte counts of a quantised tensor: "NVFP4 Without FP4 Hardware" (ai-muninn.com), table of
  section "Bit-exact check against lyf's ModelOpt output": packed bytes = numel / 2, block-scale
  bytes = numel / 16, global scale 4 bytes.
* Roofline: robertz.co page, section "The roofline is the whole argument": ridge point = peak
  FLOP/s / bandwidth; below it a kernel is bound by memory.
* Amdahl: "Sparse GPU FLOPS Need the Right Zeros in the Right Places" (leviathansystems.co),
  section "A twofold arithmetic opportunity is not a twofold application result".
"""
from __future__ import annotations


def dense_bytes(N: int, K: int) -> dict:
    numel = N * K
    return dict(codes=numel // 2, scales=numel // 16, tensor_scale=4)


def sp24_bytes(N: int, K: int) -> dict:
    numel = N * K
    return dict(vals=numel // 4, meta=numel // 8, scales=numel // 16, tensor_scale=4)


def bits_per_weight_dense(scale_block: int = 16) -> float:
    return 4.0 + 8.0 / scale_block


def bits_per_weight_sp24(scale_block_original: int = 16) -> float:
    """Per original weight: 4 value bits and 2 index bits for half of them, plus the scales."""
    return 0.5 * 4.0 + 0.5 * 2.0 + 8.0 / scale_block_original


def saving(dense_bits: float, sparse_bits: float) -> float:
    return 1.0 - sparse_bits / dense_bits


def gemm_flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


def ridge(peak_flops: float, bandwidth: float) -> float:
    return peak_flops / bandwidth


def roof_fraction(intensity: float, ridge_point: float) -> float:
    """Largest fraction of peak compute reachable at a given arithmetic intensity."""
    return min(1.0, intensity / ridge_point)


def amdahl(total: float, affected: float, speedup: float) -> float:
    """Overall speed ratio when ``affected`` of ``total`` time runs ``speedup`` times faster."""
    return total / (total - affected + affected / speedup)
