"""GPU parity of gemm_nvfp4_dense / gemm_nvfp4_sp24 against the float64 oracle, within
|err| <= 2e-3 * sum_k |x_k w_k| per element (+ half a bf16 ulp for bf16 outputs)."""
import numpy as np
import pytest
import torch

import structured_sparse_nvfp4_amd as ssn
import synth
from oracle import gemm, quant, sp24
from tests.gpu_util import assert_within_bound, dev, host, x_dev, y_host

pytestmark = pytest.mark.gpu

DENSE_ALGOS = [ssn.ALGO_AUTO, ssn.ALGO_MFMA, ssn.ALGO_VALU]
SP24_ALGOS = [ssn.ALGO_AUTO, ssn.ALGO_SMFMAC, ssn.ALGO_DECOMPRESS_MFMA, ssn.ALGO_GATHER, ssn.ALGO_VALU]


def _problem(M, N, K, seed, prune):
    x = synth.activations(M, K, seed=seed)
    w = synth.weights(N, K, seed=seed)
    if prune:
        w = sp24.prune24(w)
    c, s, st = quant.quantize(w)
    return x, c, s, st


# the small configuration: X [16, 512], W [256, 512], plus ragged and multi-slice shapes; the
# M > 16 shapes run the 256 x 256 tiles: several tiles in M and N, ragged edges, K tails of 32
DENSE_CASES = [(16, 256, 512), (1, 256, 512), (3, 37, 96), (8, 100, 160), (16, 64, 1024), (5, 48, 4096),
               (17, 40, 64), (40, 33, 128), (300, 520, 640), (257, 300, 96), (513, 257, 1056),
               (64, 1000, 2048), (257, 300, 128), (513, 257, 1088),
               (3, 17000, 512),                   # ragged last row group of the decode slabs
               (3, 24608, 512), (8, 24608, 512),  # more row groups than workgroups a CU holds at once
               # K % 256 == 0 but K % 512 != 0 (the decode slabs' partial last stage), M <= 8 and 9..16
               (1, 100, 768), (8, 300, 1280), (5, 1000, 768), (12, 64, 768),
               # few row groups per CU, every activation-row count of the post-scale slab
               (2, 3000, 1024), (3, 40, 512), (4, 500, 2048), (6, 1000, 1536), (7, 333, 3072),
               # M = 9..16, K % 512 == 0: the 16-row post-scale slab (waves load a second
               # activation row), ragged row groups and more row groups than the grid
               (9, 1000, 1024), (10, 33, 1536), (13, 300, 2048), (15, 17000, 512), (16, 24608, 512)]


@pytest.mark.parametrize("M,N,K", DENSE_CASES)
@pytest.mark.parametrize("algo", DENSE_ALGOS)
@pytest.mark.parametrize("prune", [False, True])
def test_dense(M, N, K, algo, prune):
    if algo == ssn.ALGO_MFMA and M > 16 and K % 64:
        pytest.skip("the 256x256 tiles need K % 64 == 0 (refusal is tested on the CPU)")
    x, c, s, st = _problem(M, N, K, seed=M * 7 + N + K, prune=prune)
    Y, B = gemm.gemm_dense(x, c, s, st)
    g, used = ssn.gemm_nvfp4_dense(x_dev(x), dev(c), dev(s), dev(np.array([st], np.float32)), algo=algo)
    assert used != ssn.ALGO_AUTO and (algo == ssn.ALGO_AUTO or used == algo)
    assert_within_bound(y_host(g), Y, B, what=f"dense algo={used}")


SP24_CASES = [(16, 256, 512), (1, 256, 512), (3, 37, 96), (8, 100, 320), (16, 64, 1024), (4, 48, 4096),
              (17, 40, 64), (40, 33, 128), (300, 520, 640), (257, 300, 96), (513, 257, 1056),
              (64, 1000, 2048), (257, 300, 128), (513, 257, 1088),
              # M <= 8, K % 512 == 0 (full-width-load decode kernel): ragged row groups, every M
              (8, 100, 512), (5, 1000, 1536), (2, 17000, 512), (7, 33, 1024),
              # M = 1: two to six 512-wide stages, ragged row groups
              (1, 1000, 1024), (1, 17000, 2048), (1, 33, 3072),
              # K % 256 == 0 but K % 512 != 0: the slab kernels' partial last stage (8- and 16-wave forms)
              (1, 100, 768), (8, 300, 1280), (5, 1000, 768), (12, 64, 768),
              # few row groups per CU, every activation-row count of the 2:4 slab
              (2, 3000, 1024), (3, 40, 512), (4, 500, 2048), (6, 1000, 1536),
              # M = 9..16, K % 512 == 0: the 16-row 2:4 slab (waves load a second activation row)
              (9, 1000, 1024), (10, 33, 1536), (13, 300, 2048), (15, 17000, 512), (16, 24608, 512)]


@pytest.mark.parametrize("M,N,K", SP24_CASES)
@pytest.mark.parametrize("algo", SP24_ALGOS)
def test_sp24(M, N, K, algo):
    if K % 64 and (algo == ssn.ALGO_SMFMAC or (algo == ssn.ALGO_DECOMPRESS_MFMA and M > 16)):
        pytest.skip("SMFMAC and the 256x256 tiles need K % 64 == 0 (refusal is tested on the CPU)")
    x, c, s, st = _problem(M, N, K, seed=M * 5 + N + K, prune=True)
    vals, meta, bad = sp24.compress(c)
    assert bad == 0
    Y, B = gemm.gemm_sp24(x, vals, meta, s, st)
    g, used = ssn.gemm_nvfp4_sp24(x_dev(x), dev(vals), dev(meta), dev(s), dev(np.array([st], np.float32)),
                                  algo=algo)
    want = ssn.ALGO_GATHER if algo == ssn.ALGO_VALU else algo     # the vector-ALU 2:4 form is skip-and-gather
    assert used != ssn.ALGO_AUTO and (algo == ssn.ALGO_AUTO or used == want)
    assert_within_bound(y_host(g), Y, B, what=f"sp24 algo={used}")


# The decode slabs launch at most 16 workgroups per CU, each taking ceil(N / workgroups)
# consecutive rows in 32-row groups: N = 140000 on 256 CUs gives 4096 workgroups of 35 rows, a
# full group and then a 3-row one. The problem repeats a 4999-row block (rows are independent,
# so the oracle's result repeats with it); a workgroup that took a wrong group would read rows
# that differ from the right ones.
_BASE_ROWS, _MANY_ROWS = 4999, 140000


def _tiled_rows(a, axis):
    reps = -(-_MANY_ROWS // _BASE_ROWS)
    t = np.concatenate([a] * reps, axis=axis)
    return np.ascontiguousarray(np.take(t, np.arange(_MANY_ROWS), axis=axis))


@pytest.mark.parametrize("M", [1, 3, 11])
@pytest.mark.parametrize("sparse", [False, True])
def test_decode_several_row_groups_per_workgroup(M, sparse):
    K = 1024
    x, c, s, st = _problem(M, _BASE_ROWS, K, seed=40 + M, prune=sparse)
    ts = dev(np.array([st], np.float32))
    if sparse:
        vals, meta, _ = sp24.compress(c)
        Y, B = gemm.gemm_sp24(x, vals, meta, s, st)
        g, used = ssn.gemm_nvfp4_sp24(x_dev(x), dev(_tiled_rows(vals, 0)), dev(_tiled_rows(meta, 0)),
                                      dev(_tiled_rows(s, 0)), ts, algo=ssn.ALGO_SMFMAC)
    else:
        Y, B = gemm.gemm_dense(x, c, s, st)
        g, used = ssn.gemm_nvfp4_dense(x_dev(x), dev(_tiled_rows(c, 0)), dev(_tiled_rows(s, 0)), ts,
                                       algo=ssn.ALGO_MFMA)
    assert_within_bound(y_host(g), _tiled_rows(Y, 1), _tiled_rows(B, 1), what=f"M={M} sparse={sparse}")


@pytest.mark.parametrize("M,N,K", [(8, 96, 512), (270, 300, 320)])
@pytest.mark.parametrize("sparse", [False, True])
def test_bf16_output(sparse, M, N, K):
    x, c, s, st = _problem(M, N, K, seed=21, prune=sparse)
    ts = dev(np.array([st], np.float32))
    if sparse:
        vals, meta, _ = sp24.compress(c)
        Y, B = gemm.gemm_sp24(x, vals, meta, s, st)
        g, _ = ssn.gemm_nvfp4_sp24(x_dev(x), dev(vals), dev(meta), dev(s), ts, y_dtype=torch.bfloat16)
    else:
        Y, B = gemm.gemm_dense(x, c, s, st)
        g, _ = ssn.gemm_nvfp4_dense(x_dev(x), dev(c), dev(s), ts, y_dtype=torch.bfloat16)
    assert_within_bound(y_host(g), Y, B, out="bf16", what="bf16 output")


@pytest.mark.parametrize("algo", [ssn.ALGO_MFMA, ssn.ALGO_VALU])
def test_one_hot_rows_extract_weights_dense(algo):
    # X rows are unit vectors e_k: each output is one decoded weight times the tensor scale,
    # exact up to the single f32 rounding of the scale product; this pins the operand layouts.
    N, K = 48, 512
    ks = np.array([0, 7, 8, 31, 32, 63, 100, 127, 128, 200, 255, 256, 300, 383, 384, 511])
    x = np.zeros((16, K), np.float32)
    x[np.arange(16), ks] = 1.0
    xb = synth.f32_to_bf16_bits(x)
    _, c, s, st = _problem(1, N, K, seed=4, prune=False)
    g, _ = ssn.gemm_nvfp4_dense(x_dev(xb), dev(c), dev(s), dev(np.array([st], np.float32)), algo=algo)
    want = quant.dequantize(c, s, st)[:, ks].T.astype(np.float32)
    assert np.array_equal(y_host(g).astype(np.float32), want)


@pytest.mark.parametrize("rows", [16, 8])
@pytest.mark.parametrize("algo", [ssn.ALGO_SMFMAC, ssn.ALGO_DECOMPRESS_MFMA, ssn.ALGO_GATHER])
def test_one_hot_rows_extract_weights_sp24(algo, rows):
    N, K = 48, 512
    ks_all = np.array([0, 1, 2, 3, 17, 63, 64, 100, 127, 128, 200, 255, 256, 301, 383, 510])
    _, c, s, st = _problem(1, N, K, seed=5, prune=True)
    vals, meta, _ = sp24.compress(c)
    for ks in (ks_all[:rows], ks_all[rows:]):
        if ks.size == 0:
            continue
        x = np.zeros((ks.size, K), np.float32)
        x[np.arange(ks.size), ks] = 1.0
        xb = synth.f32_to_bf16_bits(x)
        g, _ = ssn.gemm_nvfp4_sp24(x_dev(xb), dev(vals), dev(meta), dev(s), dev(np.array([st], np.float32)), algo=algo)
        want = quant.dequantize(sp24.decompress(vals, meta), s, st)[:, ks].T.astype(np.float32)
        assert np.array_equal(y_host(g).astype(np.float32), want)


def _one_hot_tiled(M, K, seed):
    # row m of X is the unit vector e_{k(m)}; k(m) sweeps every position of a 64-wide stage and
    # both K stages, so each (row block, lane half, MFMA step) operand slot is exercised
    ks = (np.arange(M) * 37 + 5) % K
    x = np.zeros((M, K), np.float32)
    x[np.arange(M), ks] = 1.0
    return synth.f32_to_bf16_bits(x), ks


@pytest.mark.parametrize("algo", [ssn.ALGO_MFMA])
def test_one_hot_rows_extract_weights_dense_tiled(algo):
    M, N, K = 300, 290, 192
    xb, ks = _one_hot_tiled(M, K, 0)
    _, c, s, st = _problem(1, N, K, seed=6, prune=False)
    g, used = ssn.gemm_nvfp4_dense(x_dev(xb), dev(c), dev(s), dev(np.array([st], np.float32)), algo=algo)
    want = quant.dequantize(c, s, st)[:, ks].T.astype(np.float32)
    assert used == algo and np.array_equal(y_host(g).astype(np.float32), want)


@pytest.mark.parametrize("algo", [ssn.ALGO_SMFMAC, ssn.ALGO_DECOMPRESS_MFMA])
def test_one_hot_rows_extract_weights_sp24_tiled(algo):
    M, N, K = 300, 290, 192
    xb, ks = _one_hot_tiled(M, K, 1)
    _, c, s, st = _problem(1, N, K, seed=7, prune=True)
    vals, meta, _ = sp24.compress(c)
    g, used = ssn.gemm_nvfp4_sp24(x_dev(xb), dev(vals), dev(meta), dev(s), dev(np.array([st], np.float32)),
                                  algo=algo)
    want = quant.dequantize(sp24.decompress(vals, meta), s, st)[:, ks].T.astype(np.float32)
    assert used == algo and np.array_equal(y_host(g).astype(np.float32), want)


def test_empty_and_degenerate():
    ts = dev(np.array([1.0], np.float32))
    c = torch.zeros((4, 16), dtype=torch.uint8, device="cuda")
    s = torch.zeros((4, 2), dtype=torch.uint8, device="cuda")
    x = torch.zeros((0, 32), dtype=torch.bfloat16, device="cuda")
    y, used = ssn.gemm_nvfp4_dense(x, c, s, ts)
    assert y.shape == (0, 4)
    # all-zero weights give exact zeros
    x1 = torch.ones((2, 32), dtype=torch.bfloat16, device="cuda")
    y, _ = ssn.gemm_nvfp4_dense(x1, c, s, ts)
    assert torch.count_nonzero(y).item() == 0


# 16 x 17 tiles of 256 x 256 = one round of 256 plus 16: the last 16 tiles of the order (the last
# four tile rows x the last four tile columns) run as a second launch of 128 x 256 tiles, whose
# output rows are strided by the full N; ragged M and N put partial tiles in that second launch
@pytest.mark.parametrize("M,N", [(4096, 4352), (4000, 4300)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("sparse", [False, True])
def test_tiles_with_split_tail(M, N, out, sparse):
    K = 192
    x, c, s, st = _problem(M, N, K, seed=M + N + (1 if sparse else 0), prune=sparse)
    ts = dev(np.array([st], np.float32))
    ydt = torch.bfloat16 if out == "bf16" else torch.float32
    if sparse:
        vals, meta, _ = sp24.compress(c)
        Y, B = gemm.gemm_sp24(x, vals, meta, s, st)
        g, used = ssn.gemm_nvfp4_sp24(x_dev(x), dev(vals), dev(meta), dev(s), ts, y_dtype=ydt,
                                      algo=ssn.ALGO_DECOMPRESS_MFMA)
        assert used == ssn.ALGO_DECOMPRESS_MFMA
    else:
        Y, B = gemm.gemm_dense(x, c, s, st)
        g, used = ssn.gemm_nvfp4_dense(x_dev(x), dev(c), dev(s), ts, y_dtype=ydt, algo=ssn.ALGO_MFMA)
        assert used == ssn.ALGO_MFMA
    assert_within_bound(y_host(g), Y, B, out=out, what=f"split tail {M}x{N} {out}")


# A one-hot row of X picks one decoded weight, so every bf16 output is the exact product
# E2M1 * E4M3 * s_t (at most 15 significant bits, exact in f32) rounded once. With s_t = 1 + 2^-8
# the products of power-of-two weights sit exactly halfway between two bf16 values with an even
# lower neighbour and the rest above halfway; with 1 + 2^-7 there are ties whose lower neighbour is
# odd, exact values and values below halfway. Comparing bit for bit pins round-to-nearest-even in
# the bf16 epilogue of every product form.
ROUND_CASES = [("dense", ssn.ALGO_MFMA, 300), ("dense", ssn.ALGO_MFMA, 16), ("dense", ssn.ALGO_MFMA, 4),
               ("dense", ssn.ALGO_MFMA, 1), ("sp24", ssn.ALGO_SMFMAC, 300), ("sp24", ssn.ALGO_DECOMPRESS_MFMA, 300),
               ("sp24", ssn.ALGO_SMFMAC, 8), ("sp24", ssn.ALGO_SMFMAC, 1)]


@pytest.mark.parametrize("form,algo,M", ROUND_CASES)
@pytest.mark.parametrize("ts_val", [1.0 + 2.0 ** -8, 1.0 + 2.0 ** -7])
def test_bf16_output_rounds_to_nearest_even(form, algo, M, ts_val):
    N, K = 290, 512
    xb, ks = _one_hot_tiled(M, K, 3)
    _, c, s, _ = _problem(1, N, K, seed=8, prune=form == "sp24")
    ts = dev(np.array([ts_val], np.float32))
    if form == "sp24":
        vals, meta, _ = sp24.compress(c)
        g, used = ssn.gemm_nvfp4_sp24(x_dev(xb), dev(vals), dev(meta), dev(s), ts, y_dtype=torch.bfloat16, algo=algo)
        w = quant.dequantize(sp24.decompress(vals, meta), s, ts_val)
    else:
        g, used = ssn.gemm_nvfp4_dense(x_dev(xb), dev(c), dev(s), ts, y_dtype=torch.bfloat16, algo=algo)
        w = quant.dequantize(c, s, ts_val)
    assert used == algo
    exact = w[:, ks].T
    f = exact.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), exact)
    assert ((f.view(np.uint32) & 0xFFFF) == 0x8000).any()          # the case holds exact ties
    # a weight coded -0 gives a sum of signed zeros, which is +0; compare zeros by value
    got, want = host(g), synth.f32_to_bf16_bits(f)
    got, want = np.where(got == 0x8000, 0, got), np.where(want == 0x8000, 0, want)
    assert np.array_equal(got, want)
