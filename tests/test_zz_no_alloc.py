"""The allocation-free grouped-expert FFN (moe_nvfp4_ffn_noalloc, workspace in the library's
static per-GPU array) against the workspace form (moe_nvfp4_ffn) and the oracle: two calls in a
row, the second with a smaller routing, for dense and 2:4 weights; a routing too large for the
static array is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import structured_sparse_nvfp4_amd as ssn
import synth
from oracle import moe, quant, sp24
from tests.gpu_util import dev, host, x_dev, y_host

pytestmark = pytest.mark.gpu

E, D, I, K_TOP = 24, 256, 128, 4


def _weights(sparse):
    def one(w):
        if sparse:
            w = sp24.prune24(w)
        c, s, st = quant.quantize(w)
        if sparse:
            v, m, nb = sp24.compress(c)
            assert nb == 0
            return ("sp24", v, m, s, st)
        return ("dense", c, s, st)
    qu = [one(synth.expert_up(e, I, D, seed=3)) for e in range(E)]
    qd = [one(synth.expert_down(e, I, D, seed=3)) for e in range(E)]

    def stack(qs):
        main = dev(np.stack([q[1] for q in qs]))
        meta = dev(np.stack([q[2] for q in qs])) if sparse else None
        sc = dev(np.stack([q[-2] for q in qs]))
        ts = dev(np.array([q[-1] for q in qs], np.float32))
        return main, meta, sc, ts
    return qu, qd, stack(qu), stack(qd)


@pytest.mark.parametrize("sparse", [False, True])
def test_noalloc_matches_the_workspace_call_twice(sparse):
    qu, qd, up, down = _weights(sparse)
    for T, seed in ((96, 41), (7, 42)):            # the second call is smaller than the first
        x = synth.activations(T, D, seed=seed)
        ids, w = synth.routing(T, E, K_TOP, 1.1, seed=seed)
        X, dids, dw = x_dev(x), dev(ids), dev(w)
        ref, ref_bad = ssn.moe_nvfp4_ffn(X, dids, dw, E, up, down)
        out = torch.full((T, D), float("nan"), dtype=torch.float32, device="cuda")
        bad = torch.full((1,), -7, dtype=torch.int64, device="cuda")
        ssn.moe_nvfp4_ffn_noalloc(X, dids, dw, E, up, down, out, bad)
        got, want = y_host(out), y_host(ref)
        assert int(host(bad)[0]) == int(host(ref_bad)[0]) == 0
        assert np.array_equal(got, want)           # same kernels on the same inputs
        oref, tol, _ = moe.moe_ffn(x, ids, w, lambda e: qu[e], lambda e: qd[e], E, I)
        assert np.all(np.abs(got - oref) <= tol)


def test_noalloc_refuses_a_routing_beyond_its_scratch():
    L = ssn.lib()
    p = ctypes.c_void_p(16)
    # 4096 tokens x top-10 at D = 2048, I = 512 need about 380 MB of workspace
    st = L.moe_nvfp4_ffn_noalloc(p, 4096, 2048, p, p, 10, 512, 512, 0, 0, p, None, p, p, p, None, p, p, p, None, None)
    assert st == ssn.SSN_E_RANGE and b"static scratch" in L.ssn_last_error()
