"""GPU parity of the W4A4 variant against the oracle: MXFP4 quantisation bit-exact (row and
tiled layouts, f32 and bf16 inputs, ties, zeros, signs, tiny and huge values), the tiled layout
against its definition, and the FP4 x FP4 product within 2e-3 * sum |x_hat w_hat| (+ half a
bf16 ulp for bf16 outputs) on ragged shapes, one-hot rows, and the prefill shape at full size
(sampled outputs and one whole interior 256 x 256 tile)."""
import numpy as np
import pytest
import torch

import structured_sparse_nvfp4_amd as ssn
import synth
from oracle import formats, mx
from tests.gpu_util import assert_within_bound, dev, host, x_dev

pytestmark = pytest.mark.gpu


def _untile(codes, scales, R, K):
    """The row layout from the tiled one, by the layout's definition."""
    R32, K256 = (R + 31) // 32 * 32, (K + 255) // 256 * 256
    c = codes.reshape(R32 // 32, K256 // 64, 2, 32, 16)          # [rb][ks][half][row][16 B]
    c = c.transpose(0, 3, 1, 2, 4).reshape(R32, K256 // 2)       # row, then k = 64 ks + 32 half + ...
    s = scales.reshape(R32 // 32, K256 // 256, 2, 32, 4)         # [rb][kg][half][row][step]
    s = s.transpose(0, 3, 1, 4, 2).reshape(R32, K256 // 32)      # row, then block = 8 kg + 2 step + half
    return c, s


def _values(R, K, seed, kind):
    rng = np.random.default_rng(seed)
    v = (rng.standard_normal((R, K)) * np.exp(rng.uniform(-6, 6, (R, 1)))).astype(np.float32)
    if kind == "special":
        v[:, :32] = 0.0                                      # an all-zero block
        if K >= 96:
            v[0, 32:64] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, 7, 8] + [0] * 23, np.float32)  # ties, saturation
            v[0, 64:96] = -v[0, 32:64]
        if R > 1 and K >= 96:
            v[1, 32:64] = np.float32(1e-39) * np.arange(32)  # float32 subnormals
            v[1, 64:96] = np.float32(3e38) * ((np.arange(32) % 3) - 1)
    return v


@pytest.mark.parametrize("R,K", [(1, 32), (5, 96), (33, 256), (64, 512), (257, 1056), (70, 5120)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind", ["normal", "special"])
def test_quantize_bit_exact_both_layouts(R, K, dtype, kind):
    v = _values(R, K, R * 31 + K, kind)
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(v)
        V = x_dev(bits)
        want_c, want_s = mx.quantize_bf16(bits)
    else:
        V = dev(v)
        want_c, want_s = mx.quantize(v)
    c, s = ssn.mxfp4_quantize(V, layout=ssn.MX_ROWS)
    assert np.array_equal(host(c), want_c) and np.array_equal(host(s), want_s)
    tc, ts = ssn.mxfp4_quantize(V, layout=ssn.MX_TILED)
    uc, us = _untile(host(tc), host(ts), R, K)
    assert np.array_equal(uc[:R, :K // 2], want_c) and np.array_equal(us[:R, :K // 32], want_s)
    assert not uc[R:].any() and not uc[:, K // 2:].any() and not us[R:].any() and not us[:, K // 32:].any()


def _w4a4_problem(M, N, K, seed):
    x = synth.activations(M, K, seed=seed)
    w = synth.weights(N, K, seed=seed)
    xc, xs = mx.quantize_bf16(x)
    wc, ws = mx.quantize(w)
    return x, w, (xc, xs, wc, ws)


def _gpu_operands(x, w):
    X = x_dev(x)
    W = dev(w)
    a = ssn.mxfp4_quantize(X)
    b = ssn.mxfp4_quantize(W)
    return a, b


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (16, 256, 512), (3, 37, 96), (40, 33, 128), (300, 520, 640),
                                   (257, 300, 96), (513, 257, 1056), (64, 1000, 2048), (256, 256, 256),
                                   (260, 513, 768)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_w4a4_product(M, N, K, out):
    x, w, (xc, xs, wc, ws) = _w4a4_problem(M, N, K, seed=M + 3 * N + K)
    Y, B = mx.gemm_w4a4(xc, xs, wc, ws)
    (gxc, gxs), (gwc, gws) = _gpu_operands(x, w)
    ydt = torch.bfloat16 if out == "bf16" else torch.float32
    y, used = ssn.gemm_mxfp4(gxc, gxs, M, gwc, gws, N, K, y_dtype=ydt)
    assert used == ssn.ALGO_MFMA
    assert_within_bound(y.float().cpu().numpy().astype(np.float64), Y, B, out=out, what=f"w4a4 {M}x{N}x{K}")


def test_w4a4_one_hot_rows_extract_weights():
    # X rows are unit vectors e_k (1 = 4 x 2^-2 exactly): each output is one decoded weight,
    # exact; k sweeps both K halves of a step, every step of a stage and several stages
    M, N, K = 64, 70, 768
    ks = (np.arange(M) * 37 + 5) % K
    xf = np.zeros((M, K), np.float32)
    xf[np.arange(M), ks] = 1.0
    w = synth.weights(N, K, seed=9)
    wc, ws = mx.quantize(w)
    a = ssn.mxfp4_quantize(dev(xf))
    b = ssn.mxfp4_quantize(dev(w))
    y, _ = ssn.gemm_mxfp4(a[0], a[1], M, b[0], b[1], N, K)
    want = mx.dequantize(wc, ws)[:, ks].T.astype(np.float32)
    assert np.array_equal(y.cpu().numpy(), want)


def test_w4a4_empty_and_zero():
    a = ssn.mxfp4_quantize(torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda"))
    b = ssn.mxfp4_quantize(torch.zeros((5, 64), dtype=torch.float32, device="cuda"))
    y, _ = ssn.gemm_mxfp4(a[0], a[1], 0, b[0], b[1], 5, 64)
    assert y.shape == (0, 5)
    a = ssn.mxfp4_quantize(torch.ones((3, 64), dtype=torch.bfloat16, device="cuda"))
    y, _ = ssn.gemm_mxfp4(a[0], a[1], 3, b[0], b[1], 5, 64)
    assert torch.count_nonzero(y).item() == 0


@pytest.fixture(scope="module")
def prefill_w4a4():
    M, N, K = 8192, 27648, 5120
    x = synth.activations(M, K)
    w = synth.weight_rows_with_outliers(N, K, 0, N, p=0.01, mult=20.0)
    (gxc, gxs), (gwc, gws) = _gpu_operands(x, w)
    y, used = ssn.gemm_mxfp4(gxc, gxs, M, gwc, gws, N, K, y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    d = dict(x=x, w=w, y=y, M=M, N=N, K=K)
    yield d
    d.clear()
    torch.cuda.empty_cache()


def test_w4a4_prefill_sampled_and_whole_tile(prefill_w4a4):
    d = prefill_w4a4
    ms = np.array([0, 1, 255, 256, 4097, 8191])
    ns = np.array([0, 1, 255, 256, 13824, 27647])
    for rows, cols in ((ms, ns), (np.arange(256 * 17, 256 * 18), np.arange(256 * 61, 256 * 62))):
        xc, xs = mx.quantize_bf16(d["x"][rows])
        wc, ws = mx.quantize(d["w"][cols])
        Y, B = mx.gemm_w4a4(xc, xs, wc, ws)
        got = d["y"][torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()].float().cpu().numpy()
        assert_within_bound(got.astype(np.float64), Y, B, out="bf16", what="w4a4 prefill")
    assert bool(torch.isfinite(d["y"]).all())


def test_w4a4_distance_to_w4a16_within_the_activation_error(prefill_w4a4):
    # the W4A4 result differs from the product on unquantised bf16 activations (same MXFP4
    # weights) by at most the activations' quantisation error carried through |w_hat|
    d = prefill_w4a4
    rows, cols = np.array([3, 5000]), np.array([7, 20001])
    x = formats.bf16_decode(d["x"][rows])
    xc, xs = mx.quantize_bf16(d["x"][rows])
    wc, ws = mx.quantize(d["w"][cols])
    Y16 = x @ mx.dequantize(wc, ws).T
    Y4, B = mx.gemm_w4a4(xc, xs, wc, ws)
    D = mx.activation_error(x, xc, xs, wc, ws)
    got = d["y"][torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()].float().cpu().numpy()
    tol = 2e-3 * B + 0.5 * formats.bf16_ulp(np.abs(Y4) + 2e-3 * B) + D
    assert np.all(np.abs(got - Y16) <= tol)
