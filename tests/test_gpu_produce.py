"""GPU parity of the fused 2:4 producer nvfp4_sp24_produce against the oracle's prune, quantise
and compress in turn (bit-exact), and against the library's own unfused chain at the decode
size (13824 x 5120)."""
import numpy as np
import pytest
import torch

import structured_sparse_nvfp4_amd as ssn
import synth
from oracle import quant, sp24
from tests.gpu_util import dev, host

pytestmark = pytest.mark.gpu

SHAPES = [(256, 512), (37, 96), (1, 32), (129, 160), (64, 5120)]


def _special_rows(w):
    """Rows that stress the rules: magnitude ties inside a group, kept values that round to
    (negative) zero next to larger ones, an all-zero block, sign patterns."""
    K = w.shape[1]
    if w.shape[0] < 4 or K < 32:
        return w
    w = w.copy()
    w[0, :16] = [0.5, -0.5, 0.5, -0.5, 1e-9, 0.0, 0.3, -1e-9, 0.0, 0.0, 0.0, 0.0, -0.2, 0.2, 0.2, -0.2]
    w[1, :16] = 0.0                                            # block scale 0
    w[2, :16] = [-1e-12, 0.0, 0.7, 0.0, 0.0, -1e-12, 0.0, 0.7, 1.0, 1.0, 1.0, 1.0, -3.0, 2e-9, -2e-9, 0.0]
    w[3, 16:32] = -np.abs(w[3, 16:32])
    return w


def _expected(w_or, st_in=None):
    wp = sp24.prune24(w_or)
    c, s, st = quant.quantize(wp, tensor_scale_in=st_in)
    v, m, nb = sp24.compress(c)
    return c, s, st, v, m, nb


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("want_codes", [False, True])
def test_produce_matches_oracle(N, K, dtype, want_codes):
    w = _special_rows(synth.weights(N, K, seed=3 * N + K))
    if dtype == "bf16":
        wb = synth.f32_to_bf16_bits(w)
        w_or = synth.bf16_bits_to_f32(wb)
        W = dev(wb.view(np.int16)).view(torch.bfloat16)
    else:
        w_or, W = w, dev(w)
    c, s, st, v, m, nb = _expected(w_or)
    assert nb == 0
    gv, gm, gs, gt, gb, gc = ssn.nvfp4_sp24_produce(W, want_codes=want_codes)
    assert host(gt)[0] == st and int(host(gb)[0]) == 0
    assert np.array_equal(host(gs), s)
    assert np.array_equal(host(gv), v) and np.array_equal(host(gm), m)
    if want_codes:
        assert np.array_equal(host(gc), c)


def test_produce_shared_scale():
    w = _special_rows(synth.weights(48, 256, seed=77))
    st_in = np.float32(quant.tensor_scale(w) * 0.75)          # a group scale smaller than this tensor's own
    c, s, st, v, m, _ = _expected(w, st_in)
    gv, gm, gs, gt, gb, gc = ssn.nvfp4_sp24_produce(dev(w), tensor_scale_in=dev(np.array([st_in], np.float32)),
                                                    want_codes=True)
    assert host(gt)[0] == st_in
    assert np.array_equal(host(gs), s) and np.array_equal(host(gc), c)
    assert np.array_equal(host(gv), v) and np.array_equal(host(gm), m)


def test_produce_empty():
    gv, gm, gs, gt, gb, gc = ssn.nvfp4_sp24_produce(torch.zeros((0, 64), dtype=torch.float32, device="cuda"))
    assert host(gt)[0] == 0.0 and int(host(gb)[0]) == 0
    _, _, qt = ssn.nvfp4_quantize(torch.zeros((0, 64), dtype=torch.float32, device="cuda"))
    assert host(qt)[0] == 0.0


def test_produce_equals_unfused_chain_decode_size():
    N, K = 13824, 5120
    W = dev(synth.weights(N, K))
    Wp = ssn.sp24_prune(W)
    pc, ps, pts = ssn.nvfp4_quantize(Wp)
    vals, meta, bad = ssn.sp24_compress(pc)
    gv, gm, gs, gt, gb, gc = ssn.nvfp4_sp24_produce(W, want_codes=True)
    torch.cuda.synchronize()
    assert torch.equal(gt, pts) and int(gb.item()) == 0 and int(bad.item()) == 0
    assert torch.equal(gs, ps) and torch.equal(gc, pc)
    assert torch.equal(gv, vals) and torch.equal(gm, meta)
