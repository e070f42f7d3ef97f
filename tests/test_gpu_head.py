"""An output-head-shaped product (vocabulary-sized N = 131072, K = 5120; M = 1 and 9 rows): the
GPU producer chain and the decode products at full size, checked against the oracle on sampled
weight rows (outputs the oracle computes one by one)."""
import numpy as np
import pytest
import torch

import structured_sparse_nvfp4_amd as ssn
import synth
from oracle import gemm, quant, sp24
from tests.gpu_util import assert_within_bound, dev, host, x_dev, y_host

pytestmark = pytest.mark.gpu

N, K = 131072, 5120
SAMPLE = np.array([0, 31, 32, 255, 256, 65535, 65536, 100003, 131039, 131040, 131071])


@pytest.fixture(scope="module")
def head():
    w = synth.weights(N, K)
    W = dev(w)
    codes, scales, ts = ssn.nvfp4_quantize(W)
    Wp = ssn.sp24_prune(W)
    pc, ps, pts = ssn.nvfp4_quantize(Wp)
    vals, meta, bad = ssn.sp24_compress(pc)
    del W, Wp, pc
    torch.cuda.synchronize()
    st = quant.tensor_scale(w)
    stp = quant.tensor_scale(sp24.prune24(w))
    ws = w[SAMPLE].copy()
    del w
    return dict(ws=ws, codes=codes, scales=scales, ts=ts, ps=ps, pts=pts, vals=vals, meta=meta, bad=bad, st=st, stp=stp)


@pytest.mark.parametrize("M", [1, 9])
def test_head_products_sampled_rows(head, M):
    x = synth.activations(M, K, seed=41)
    assert host(head["ts"])[0] == head["st"] and host(head["pts"])[0] == head["stp"]
    assert int(host(head["bad"])[0]) == 0
    c, s, _ = quant.quantize(head["ws"], tensor_scale_in=head["st"])
    assert np.array_equal(host(head["codes"])[SAMPLE], c) and np.array_equal(host(head["scales"])[SAMPLE], s)
    yd, _ = ssn.gemm_nvfp4_dense(x_dev(x), head["codes"], head["scales"], head["ts"])
    Y, Bd = gemm.gemm_dense(x, c, s, head["st"])
    assert_within_bound(y_host(yd)[:, SAMPLE], Y, Bd, what="dense")
    pc, psc, _ = quant.quantize(sp24.prune24(head["ws"]), tensor_scale_in=head["stp"])
    v, m, nb = sp24.compress(pc)
    assert nb == 0
    assert np.array_equal(host(head["vals"])[SAMPLE], v) and np.array_equal(host(head["meta"])[SAMPLE], m)
    ys, _ = ssn.gemm_nvfp4_sp24(x_dev(x), head["vals"], head["meta"], head["ps"], head["pts"])
    Ys, Bs = gemm.gemm_sp24(x, v, m, psc, head["stp"])
    assert_within_bound(y_host(ys)[:, SAMPLE], Ys, Bs, what="sp24")
