"""The decode workload at full size (X [8, 5120] bf16, W [13824, 5120]), run as the benchmark
runs it (GPU prune -> quantise -> check -> compress -> GEMV at M = 1, 4, 8), checked against the
oracle: quantised and compressed weights on a sample of rows, every output of the GEMVs (the
oracle quantises all weight rows itself), and properties that hold at any size."""
import numpy as np
import pytest
import torch

import structured_sparse_nvfp4_amd as ssn
import synth
from oracle import gemm, quant, sp24
from tests.gpu_util import assert_within_bound, dev, host, x_dev, y_host

pytestmark = pytest.mark.gpu

N, K, MMAX = 13824, 5120, 8
SAMPLE = np.array([0, 1, 15, 16, 255, 256, 4097, 6911, 6912, 9000, 13807, 13808, 13822, 13823])


@pytest.fixture(scope="module")
def full():
    w = synth.weights(N, K)
    x = synth.activations(MMAX, K)
    W = dev(w)
    codes, scales, ts = ssn.nvfp4_quantize(W)
    Wp = ssn.sp24_prune(W)
    pc, ps, pts = ssn.nvfp4_quantize(Wp)
    bad, first = ssn.sp24_check(pc)
    vals, meta, cbad = ssn.sp24_compress(pc)
    torch.cuda.synchronize()
    st = quant.tensor_scale(w)
    wp = sp24.prune24(w[SAMPLE])
    stp = quant.tensor_scale(sp24.prune24(w))
    return dict(w=w, x=x, W=W, codes=codes, scales=scales, ts=ts, pc=pc, ps=ps, pts=pts, bad=bad, first=first,
                vals=vals, meta=meta, cbad=cbad, st=st, stp=stp, wp=wp)


def test_quantize_sampled_rows(full):
    c, s, _ = quant.quantize(full["w"][SAMPLE], tensor_scale_in=full["st"])
    assert host(full["ts"])[0] == full["st"]
    assert np.array_equal(host(full["codes"])[SAMPLE], c)
    assert np.array_equal(host(full["scales"])[SAMPLE], s)


def test_prune_quantize_compress_sampled_rows(full):
    assert host(full["pts"])[0] == full["stp"]
    c, s, _ = quant.quantize(full["wp"], tensor_scale_in=full["stp"])
    assert np.array_equal(host(full["pc"])[SAMPLE], c) and np.array_equal(host(full["ps"])[SAMPLE], s)
    v, m, bad = sp24.compress(c)
    assert bad == 0
    assert np.array_equal(host(full["vals"])[SAMPLE], v) and np.array_equal(host(full["meta"])[SAMPLE], m)


def test_check_and_compress_properties(full):
    # pruned-then-quantised weights pass everywhere; unpruned ones fail in many groups
    assert int(host(full["bad"])[0]) == 0 and int(host(full["first"])[0]) == -1
    assert int(host(full["cbad"])[0]) == 0
    ub, uf = ssn.sp24_check(full["codes"])
    nb = int(host(ub)[0])
    assert nb > 0 and 0 <= int(host(uf)[0]) < N * K // 4
    # sampled-row count equals the oracle's on those rows' own codes
    c, _, _ = quant.quantize(full["w"][SAMPLE[:4]], tensor_scale_in=full["st"])
    assert int(host(ssn.sp24_check(dev(c))[0])[0]) == sp24.check(c)[0]
    back = ssn.sp24_decompress(full["vals"], full["meta"])
    assert torch.equal(back.cpu() & 0x77, full["pc"].cpu() & 0x77)   # magnitudes survive the round trip


@pytest.fixture(scope="module")
def oracle_all(full):
    """The oracle's products of all 8 activation rows with every weight row (dense and 2:4),
    quantised by the oracle in chunks with the tensor scale of the whole W."""
    w, x = full["w"], full["x"]
    Yd, Bd, Ys, Bs = [], [], [], []
    for r0 in range(0, N, 2048):
        c, s, _ = quant.quantize(w[r0:r0 + 2048], tensor_scale_in=full["st"])
        Y, B = gemm.gemm_dense(x, c, s, full["st"])
        Yd.append(Y); Bd.append(B)
        pc, ps, _ = quant.quantize(sp24.prune24(w[r0:r0 + 2048]), tensor_scale_in=full["stp"])
        v, m, nb = sp24.compress(pc)
        assert nb == 0
        Y, B = gemm.gemm_sp24(x, v, m, ps, full["stp"])
        Ys.append(Y); Bs.append(B)
    return dict(Yd=np.concatenate(Yd, 1), Bd=np.concatenate(Bd, 1), Ys=np.concatenate(Ys, 1), Bs=np.concatenate(Bs, 1))


@pytest.mark.parametrize("M", [1, 4, 8])
def test_gemv_dense_all_outputs(full, oracle_all, M):
    x = full["x"][:M]
    y, used = ssn.gemm_nvfp4_dense(x_dev(x), full["codes"], full["scales"], full["ts"])
    assert_within_bound(y_host(y), oracle_all["Yd"][:M], oracle_all["Bd"][:M], what=f"dense M={M} algo={used}")


@pytest.mark.parametrize("M", [1, 4, 8])
@pytest.mark.parametrize("algo", [ssn.ALGO_SMFMAC, ssn.ALGO_DECOMPRESS_MFMA, ssn.ALGO_GATHER])
def test_gemv_sp24_all_outputs(full, oracle_all, M, algo):
    x = full["x"][:M]
    y, used = ssn.gemm_nvfp4_sp24(x_dev(x), full["vals"], full["meta"], full["ps"], full["pts"], algo=algo)
    assert used == algo
    assert_within_bound(y_host(y), oracle_all["Ys"][:M], oracle_all["Bs"][:M], what=f"sp24 M={M} algo={used}")
