"""GPU parity of the producer-side calls against the oracle, bit-exact: nvfp4_quantize,
nvfp4_dequantize, sp24_prune, sp24_check, sp24_compress, sp24_decompress."""
import numpy as np
import pytest
import torch

import structured_sparse_nvfp4_amd as ssn
import synth
from oracle import formats, quant, sp24
from tests.gpu_util import dev, host

pytestmark = pytest.mark.gpu

SHAPES = [(256, 512), (37, 96), (1, 32), (129, 160), (64, 5120)]


def _w(N, K, seed):
    return synth.weights(N, K, seed=seed)


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_bit_exact(N, K, dtype):
    w = _w(N, K, seed=N + K)
    w[0, :8] = [-1e-9, 1e-9, -0.0, 0.0, 1e-30, -1e-30, 0.3, -0.3] if K >= 8 else w[0, :8]
    if dtype == "bf16":
        wb = synth.f32_to_bf16_bits(w)
        w_or = synth.bf16_bits_to_f32(wb)
        W = dev(wb.view(np.int16)).view(torch.bfloat16)
    else:
        w_or = w
        W = dev(w)
    c, s, st = quant.quantize(w_or)
    gc, gs, gt = ssn.nvfp4_quantize(W)
    assert host(gt)[0] == st
    assert np.array_equal(host(gs), s)
    assert np.array_equal(host(gc), c)


def test_quantize_ties_and_shared_scale():
    # exact E2M1 midpoints relative to the block scale; shared tensor scale given by the caller
    st = np.float32(1.0 / 2688.0)
    unit = np.float64(st) * 448.0
    r = np.array([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.2, 0.3, 2.9, 3.1, 4.9, 5.1, 1.0, 0.5] * 2)
    w = np.stack([(r * unit), -(r * unit), (r * unit * 0.37)]).astype(np.float32)
    c, s, _ = quant.quantize(w, tensor_scale_in=st)
    gc, gs, gt = ssn.nvfp4_quantize(dev(w), tensor_scale_in=dev(np.array([st], np.float32)))
    assert host(gt)[0] == st
    assert np.array_equal(host(gs), s) and np.array_equal(host(gc), c)
    # the output scale may be the input scale itself
    t = dev(np.array([st], np.float32))
    gc, gs, gt = ssn.nvfp4_quantize(dev(w), tensor_scale_in=t, tensor_scale_out=t)
    assert host(t)[0] == st
    assert np.array_equal(host(gs), s) and np.array_equal(host(gc), c)


def test_quantize_zero_and_subnormal_scales():
    w = np.zeros((4, 64), np.float32)
    w[1, :16] = 1.0
    w[1, 16:32] = 1e-6          # block scale underflows toward the E4M3 subnormals / zero
    w[2, 32:48] = 3e-4
    w[3, 48:] = -2e-5
    c, s, st = quant.quantize(w)
    gc, gs, gt = ssn.nvfp4_quantize(dev(w))
    assert host(gt)[0] == st and np.array_equal(host(gs), s) and np.array_equal(host(gc), c)
    z = np.zeros((3, 32), np.float32)
    gc, gs, gt = ssn.nvfp4_quantize(dev(z))
    assert host(gt)[0] == 0 and not host(gc).any() and not host(gs).any()


@pytest.mark.parametrize("N,K", SHAPES[:3])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_dequantize_bit_exact(N, K, out):
    c, s, st = quant.quantize(_w(N, K, seed=3))
    ref = quant.dequantize(c, s, st)
    o = ssn.nvfp4_dequantize(dev(c), dev(s), dev(np.array([st], np.float32)),
                             out_dtype=torch.float32 if out == "f32" else torch.bfloat16)
    if out == "f32":
        assert np.array_equal(host(o), ref.astype(np.float32))
    else:
        got = formats.bf16_decode(host(o))
        assert np.array_equal(got, formats.bf16_round(ref))


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prune_bit_exact(N, K, dtype):
    w = _w(N, K, seed=11)
    w[0, :8] = [1.0, -1.0, 1.0, 0.5, 0.0, -0.0, 0.0, 0.0]        # ties and zeros
    if dtype == "bf16":
        wb = synth.f32_to_bf16_bits(w)
        ref = synth.f32_to_bf16_bits(sp24.prune24(synth.bf16_bits_to_f32(wb)))
        got = host(ssn.sp24_prune(dev(wb.view(np.int16)).view(torch.bfloat16))).view(np.uint16)
        assert np.array_equal(got, ref)
    else:
        ref = sp24.prune24(w)
        got = host(ssn.sp24_prune(dev(w)))
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("N,K", SHAPES + [(0, 64), (3000, 4096)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prune_tensor_scale(N, K, dtype):
    """The tensor scale sp24_prune gathers while it reads W is the oracle's s_t of W and of the
    pruned tensor alike, bit for bit (3000 x 4096 needs more groups than the prune's blocks
    take in one stride; its largest entry sits in the last group). nvfp4_quantize given that
    scale writes the oracle's codes."""
    w = _w(N, K, seed=21)
    if N * K:
        w[-1, -1] = 7.5
    if dtype == "bf16":
        wb = synth.f32_to_bf16_bits(w)
        w = synth.bf16_bits_to_f32(wb)
        W = dev(wb.view(np.int16)).view(torch.bfloat16)
    else:
        W = dev(w)
    ts = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    Wp = ssn.sp24_prune(W, tensor_scale_out=ts)
    st = quant.tensor_scale(w)
    assert host(ts).view(np.uint32)[0] == np.float32(st).view(np.uint32)
    assert np.float32(quant.tensor_scale(sp24.prune24(w))).view(np.uint32) == np.float32(st).view(np.uint32)
    if N * K and N * K <= 256 * 512:
        for src, ref in ((W, w), (Wp, sp24.prune24(w))):
            codes, scales, ts2 = ssn.nvfp4_quantize(src, tensor_scale_in=ts)
            rc, rs, _ = quant.quantize(ref, tensor_scale_in=st)
            assert np.array_equal(host(codes), rc) and np.array_equal(host(scales), rs)
            assert host(ts2).view(np.uint32)[0] == np.float32(st).view(np.uint32)


def _codes_with_failures(N, K, seed, p_fail=0.01):
    """Oracle codes of a pruned tensor with a few groups broken (extra nonzero codes)."""
    c, _, _ = quant.quantize(sp24.prune24(_w(N, K, seed)))
    nib = quant.unpack_nibbles(c)
    rng = np.random.default_rng(seed)
    brk = rng.random((N, K // 4)) < p_fail
    for n, g in zip(*np.nonzero(brk)):
        nib[n, 4 * g:4 * g + 4] = rng.integers(1, 16, 4)
    return quant.pack_nibbles(nib)


@pytest.mark.parametrize("N,K", SHAPES)
def test_check_bit_exact(N, K):
    for codes in (_codes_with_failures(N, K, 5), quant.quantize(sp24.prune24(_w(N, K, 6)))[0],
                  np.random.default_rng(7).integers(0, 256, (N, K // 2), dtype=np.uint8)):
        bad, first = sp24.check(codes)
        gb, gf = ssn.sp24_check(dev(codes))
        assert int(host(gb)[0]) == bad and int(host(gf)[0]) == first


@pytest.mark.parametrize("N,K", SHAPES)
def test_compress_decompress_bit_exact(N, K):
    for codes in (_codes_with_failures(N, K, 8, p_fail=0.05),
                  np.random.default_rng(9).integers(0, 256, (N, K // 2), dtype=np.uint8)):
        vals, meta, bad = sp24.compress(codes)
        gv, gm, gb = ssn.sp24_compress(dev(codes))
        assert int(host(gb)[0]) == bad
        assert np.array_equal(host(gv), vals) and np.array_equal(host(gm), meta)
        back = sp24.decompress(vals, meta)
        assert np.array_equal(host(ssn.sp24_decompress(dev(vals), dev(meta))), back)


def test_compress_raises_on_failing_groups():
    codes = quant.pack_nibbles(np.array([[2, 4, 5, 0, 6, 0, 0, 0] * 4], np.uint8))
    with pytest.raises(ValueError):
        ssn.sp24_compress(dev(codes), raise_if_bad=True)


def test_toy_vectors_on_gpu():
    # the pages' toy vectors, as codes with a unit-ish scale (see the oracle pins)
    a = quant.pack_nibbles(np.array([[2, 0, 4, 0, 5, 0, 6, 0] * 4], np.uint8))
    b = quant.pack_nibbles(np.array([[2, 4, 5, 0, 6, 0, 0, 0] * 4], np.uint8))
    ga, fa = ssn.sp24_check(dev(a))
    gb, fb = ssn.sp24_check(dev(b))
    assert (int(host(ga)[0]), int(host(fa)[0])) == (0, -1)
    assert (int(host(gb)[0]), int(host(fb)[0])) == (4, 0)
