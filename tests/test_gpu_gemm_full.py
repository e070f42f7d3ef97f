"""The square (4096 x 4096 x 4096, f32 out) and prefill (X [8192, 5120], W [27648, 5120] with 1%
of entries x20 before pruning, bf16 out) products at full size, launched as the benchmark
launches them, checked against the oracle on sampled outputs (rows and columns that straddle
tile edges), on one whole output row, one whole output column and one whole interior 256 x 256
tile (at the prefill shape also a whole tile of the last half-round, which runs as 128-row
tiles; the oracle quantises every weight row itself, in chunks), and by properties that hold at
any size."""
import numpy as np
import pytest
import torch

import structured_sparse_nvfp4_amd as ssn
import synth
from oracle import gemm, quant, sp24
from tests.gpu_util import assert_within_bound, dev, host, x_dev

pytestmark = pytest.mark.gpu


def _sample(n, extra):
    s = {0, 1, 31, 32, 255, 256, 257, n // 2, n - 257, n - 256, n - 1} | set(extra)
    return np.array(sorted(i for i in s if 0 <= i < n))


def _setup(M, N, K, w):
    x = synth.activations(M, K)
    W = dev(w)
    codes, scales, ts = ssn.nvfp4_quantize(W)
    Wp = ssn.sp24_prune(W)
    pc, ps, pts = ssn.nvfp4_quantize(Wp)
    vals, meta, bad = ssn.sp24_compress(pc)
    del W, Wp, pc
    torch.cuda.synchronize()
    return dict(x=x, X=x_dev(x), codes=codes, scales=scales, ts=ts, vals=vals, meta=meta, ps=ps, pts=pts,
                bad=bad, st=quant.tensor_scale(w), w=w)


@pytest.fixture(scope="module")
def square():
    M = N = K = 4096
    d = _setup(M, N, K, synth.weights(N, K))
    d.update(M=M, N=N, K=K, ms=_sample(M, [1000, 3001]), ns=_sample(N, [777, 2222]), out="f32",
             whole_row=2345, whole_col=1234, tile=(7, 9))
    yield d
    d.clear()
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def prefill():
    M, N, K = 8192, 27648, 5120
    w = synth.weight_rows_with_outliers(N, K, 0, N, p=0.01, mult=20.0)
    d = _setup(M, N, K, w)
    # 3456 tiles on 256 CUs: the last half-round (tile rows 28..31 x tile columns 76..107) runs as
    # 128 x 256 tiles in the dense and expanded forms; tile (31, 100) is checked whole as well
    d.update(M=M, N=N, K=K, ms=_sample(M, [5000]), ns=_sample(N, [13824, 20000]), out="bf16",
             whole_row=5001, whole_col=20001, tile=(17, 61), tail_tile=(31, 100))
    yield d
    d.clear()
    torch.cuda.empty_cache()


def _check(d, sparse, algo):
    x, ms, ns = d["x"], d["ms"], d["ns"]
    ydt = torch.bfloat16 if d["out"] == "bf16" else torch.float32
    # pruning keeps the largest magnitude of every group, so the pruned tensor's amax (and scale)
    # equals the unpruned one's
    assert host(d["ts"])[0] == d["st"] and host(d["pts"])[0] == d["st"]
    if sparse:
        assert int(host(d["bad"])[0]) == 0
        y, used = ssn.gemm_nvfp4_sp24(d["X"], d["vals"], d["meta"], d["ps"], d["pts"], y_dtype=ydt, algo=algo)
        c, s, _ = quant.quantize(sp24.prune24(d["w"][ns]), tensor_scale_in=d["st"])
        v, m, nb = sp24.compress(c)
        assert nb == 0
        Y, B = gemm.gemm_sp24(x[ms], v, m, s, d["st"])
    else:
        y, used = ssn.gemm_nvfp4_dense(d["X"], d["codes"], d["scales"], d["ts"], y_dtype=ydt, algo=algo)
        c, s, _ = quant.quantize(d["w"][ns], tensor_scale_in=d["st"])
        Y, B = gemm.gemm_dense(x[ms], c, s, d["st"])
    assert used == algo
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all())
    got = y[torch.from_numpy(ms).cuda()][:, torch.from_numpy(ns).cuda()].float().cpu().numpy().astype(np.float64)
    assert_within_bound(got, Y, B, out=d["out"], what=f"{'sp24' if sparse else 'dense'} algo={used}")
    return y


@pytest.mark.parametrize("sparse,algo", [(False, ssn.ALGO_MFMA), (True, ssn.ALGO_SMFMAC),
                                         (True, ssn.ALGO_DECOMPRESS_MFMA)])
def test_square(square, sparse, algo):
    _check(square, sparse, algo)


CHUNK = 2048


def _oracle_weights(d):
    """The oracle's dense and 2:4 weights for every row of W (chunked), with the tensor scale of
    the whole W."""
    if "oq" not in d:
        w, st, N = d["w"], d["st"], d["N"]
        cs, ss, vs, ms_, ps_ = [], [], [], [], []
        for r0 in range(0, N, CHUNK):
            c, s, _ = quant.quantize(w[r0:r0 + CHUNK], tensor_scale_in=st)
            pc, ps, _ = quant.quantize(sp24.prune24(w[r0:r0 + CHUNK]), tensor_scale_in=st)
            v, m, nb = sp24.compress(pc)
            assert nb == 0
            cs.append(c); ss.append(s); vs.append(v); ms_.append(m); ps_.append(ps)
        d["oq"] = dict(c=np.concatenate(cs), s=np.concatenate(ss), v=np.concatenate(vs), m=np.concatenate(ms_),
                       ps=np.concatenate(ps_))
    return d["oq"]


def _oracle_block(d, rows, cols, sparse):
    """Oracle product and bound base for activation rows `rows` x weight rows `cols` (chunked)."""
    oq = _oracle_weights(d)
    Ys, Bs = [], []
    for c0 in range(0, len(cols), CHUNK):
        cc = cols[c0:c0 + CHUNK]
        if sparse:
            Y, B = gemm.gemm_sp24(d["x"][rows], oq["v"][cc], oq["m"][cc], oq["ps"][cc], d["st"])
        else:
            Y, B = gemm.gemm_dense(d["x"][rows], oq["c"][cc], oq["s"][cc], d["st"])
        Ys.append(Y); Bs.append(B)
    return np.concatenate(Ys, axis=1), np.concatenate(Bs, axis=1)


def _whole(d, sparse, algo):
    """A whole output row, a whole output column and a whole interior 256 x 256 tile."""
    ydt = torch.bfloat16 if d["out"] == "bf16" else torch.float32
    if sparse:
        y, used = ssn.gemm_nvfp4_sp24(d["X"], d["vals"], d["meta"], d["ps"], d["pts"], y_dtype=ydt, algo=algo)
    else:
        y, used = ssn.gemm_nvfp4_dense(d["X"], d["codes"], d["scales"], d["ts"], y_dtype=ydt, algo=algo)
    assert used == algo
    M, N = d["M"], d["N"]
    m_row, n_col = d["whole_row"], d["whole_col"]
    tm, tn = d["tile"]
    blocks = [("row", np.array([m_row]), np.arange(N)), ("column", np.arange(M), np.array([n_col])),
              ("tile", np.arange(256 * tm, 256 * tm + 256), np.arange(256 * tn, 256 * tn + 256))]
    if "tail_tile" in d:
        um, un = d["tail_tile"]
        blocks.append(("tail tile", np.arange(256 * um, 256 * um + 256), np.arange(256 * un, 256 * un + 256)))
    for what, rows, cols in blocks:
        Y, B = _oracle_block(d, rows, cols, sparse)
        got = y[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()].float().cpu().numpy().astype(np.float64)
        assert_within_bound(got, Y, B, out=d["out"], what=f"{'sp24' if sparse else 'dense'} algo={used} whole {what}")


@pytest.mark.parametrize("sparse,algo", [(False, ssn.ALGO_MFMA), (True, ssn.ALGO_SMFMAC),
                                         (True, ssn.ALGO_DECOMPRESS_MFMA)])
def test_square_whole_row_column_tile(square, sparse, algo):
    _whole(square, sparse, algo)


@pytest.mark.parametrize("sparse,algo", [(False, ssn.ALGO_MFMA), (True, ssn.ALGO_SMFMAC)])
def test_prefill_whole_row_column_tile(prefill, sparse, algo):
    _whole(prefill, sparse, algo)


@pytest.mark.parametrize("sparse,algo", [(False, ssn.ALGO_MFMA), (True, ssn.ALGO_SMFMAC),
                                         (True, ssn.ALGO_DECOMPRESS_MFMA)])
def test_prefill(prefill, sparse, algo):
    _check(prefill, sparse, algo)


def test_square_sparse_variants_agree(square):
    # the two 2:4 matrix-core paths sum the same exact products in different orders
    d = square
    a, _ = ssn.gemm_nvfp4_sp24(d["X"], d["vals"], d["meta"], d["ps"], d["pts"], algo=ssn.ALGO_SMFMAC)
    b, _ = ssn.gemm_nvfp4_sp24(d["X"], d["vals"], d["meta"], d["ps"], d["pts"], algo=ssn.ALGO_DECOMPRESS_MFMA)
    torch.cuda.synchronize()
    scale = float(a.abs().max())
    assert float((a - b).abs().max()) <= 1e-3 * scale
