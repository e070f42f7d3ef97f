"""Stage-by-stage parity of the grouped-expert FFN at its full size: 4096 tokens, 512 experts,
top-10 of Zipf(1.1) popularity, D = 2048, I = 512 ("NVFP4 vs 2:4 sparse", robertz.co, section
"Concurrency, not sparsity, is the lever"), dense and 2:4 weights, launched as the benchmark
launches it (64-k tiled weights, AUTO algorithms).

* routing: every row exact;
* up projection with the SiLU gate: every row of the three largest experts (3687, 2795 and 2110
  rows) and of a median one, plus 64 random rows, within the oracle's H bound;
* down projection and combine: computed by the oracle from the GPU's own H for 64 tokens whose
  rows lie in interior tiles of the largest experts, at the plain product bound;
* the one-call FFN gives the staged calls' output bit for bit."""
import functools

import numpy as np
import pytest
import torch

import structured_sparse_nvfp4_amd as ssn
import synth
from oracle import moe, quant, sp24
from tests.gpu_util import dev, host, x_dev, y_host
from tests.test_gpu_moe import _full_gpu_weights

pytestmark = pytest.mark.gpu

T, E, K_TOP, D, I = 4096, 512, 10, 2048, 512


def _oracle_weights(gen, e, sparse):
    w = gen(e)
    if sparse:
        w = sp24.prune24(w)
    c, s, st = quant.quantize(w)
    if sparse:
        v, m, nb = sp24.compress(c)
        assert nb == 0
        return ("sp24", v, m, s, st)
    return ("dense", c, s, st)


@pytest.fixture(scope="module", params=[False, True], ids=["dense", "sp24"])
def staged(request):
    sparse = request.param
    x = synth.activations(T, D)
    ids, wts = synth.routing(T, E, K_TOP, 1.1)
    up, down = _full_gpu_weights(E, I, D, sparse)
    up, down = ssn.moe_pack_weights(up), ssn.moe_pack_weights(down)
    kt = ssn.WLAYOUT_KTILE64
    X, dids, dw = x_dev(x), dev(ids), dev(wts)
    R = T * K_TOP
    off, rt, rs, ro, bad = ssn.moe_route(dids, E)
    H, _ = ssn.moe_grouped_gemm_nvfp4(X, rt, off, R, up[0], up[2], up[3], w_meta=up[1], epilogue=ssn.EPI_SILU_GATE,
                                      y_dtype=torch.bfloat16, w_layout=kt)
    Yd, _ = ssn.moe_grouped_gemm_nvfp4(H, None, off, R, down[0], down[2], down[3], w_meta=down[1], w_layout=kt)
    out = ssn.moe_combine(Yd, ro, dw)
    ffn, ffn_bad = ssn.moe_nvfp4_ffn(X, dids, dw, E, up, down, w_layout=kt)
    torch.cuda.synchronize()
    d = dict(sparse=sparse, x=x, ids=ids, wts=wts, off=host(off).astype(np.int64), rt=host(rt).astype(np.int64),
             rs=host(rs).astype(np.int64), bad=int(host(bad)[0]), H=y_host(H), out=y_host(out), ffn=y_host(ffn),
             ffn_bad=int(host(ffn_bad)[0]))
    del up, down, H, Yd, out, ffn
    torch.cuda.empty_cache()
    yield d
    d.clear()


@functools.lru_cache(maxsize=256)
def _up_q(e, sparse):
    return _oracle_weights(lambda i: synth.expert_up(i, I, D), e, sparse)


@functools.lru_cache(maxsize=256)
def _down_q(e, sparse):
    return _oracle_weights(lambda i: synth.expert_down(i, I, D), e, sparse)


def test_routing_exact(staged):
    counts, offsets, row_token, row_slot = moe.route(staged["ids"], E)
    assert staged["bad"] == 0 and staged["ffn_bad"] == 0
    assert np.array_equal(staged["off"], offsets)
    assert np.array_equal(staged["rt"], row_token) and np.array_equal(staged["rs"], row_slot)


def _check_h_rows(staged, e, rows):
    """H rows `rows` (routing rows of expert e) within the oracle's H bound."""
    st = moe.up_stage(staged["x"][staged["rt"][rows]], _up_q(e, staged["sparse"]), I)
    err = np.abs(staged["H"][rows] - st["H"])
    bound = moe.h_bound(st)
    assert np.all(err <= bound), f"expert {e}: {int((err > bound).sum())} H values outside the bound"


def test_h_all_rows_of_the_largest_and_a_median_expert(staged):
    counts = np.diff(staged["off"])
    order = np.argsort(-counts, kind="stable")
    median = int(np.argsort(counts, kind="stable")[E // 2])
    for e in [int(order[0]), int(order[1]), int(order[2]), median]:
        rows = np.arange(staged["off"][e], staged["off"][e + 1])
        assert rows.size > 0
        _check_h_rows(staged, e, rows)
    assert counts[order[0]] > 3000       # a single expert spans dozens of 64-row tiles


def test_h_random_rows(staged):
    rng = np.random.default_rng(77)
    rows = np.sort(rng.choice(T * K_TOP, 64, replace=False))
    expert_of = np.searchsorted(staged["off"], rows, side="right") - 1
    for e in np.unique(expert_of):
        _check_h_rows(staged, int(e), rows[expert_of == e])


def test_down_and_combine_from_the_gpu_h(staged):
    ids = staged["ids"]
    counts = np.diff(staged["off"])
    top = set(np.argsort(-counts, kind="stable")[:64].tolist())
    cand = np.array([t for t in range(T) if set(ids[t].tolist()) <= top])
    tokens = cand[np.linspace(0, cand.size - 1, 64).astype(int)]
    sel = np.nonzero(np.isin(staged["rt"], tokens))[0]
    assert sel.size == tokens.size * K_TOP
    expert_of = np.searchsorted(staged["off"], sel, side="right") - 1
    # rows inside interior tiles of the two largest experts are among them
    for e in np.argsort(-counts, kind="stable")[:2]:
        local = sel[expert_of == e] - staged["off"][e]
        assert np.any((local >= 64) & (local < counts[e] - 64))
    ref, tol = moe.ffn_from_h(staged["H"][sel], staged["rt"][sel], staged["rs"][sel], sel, expert_of, staged["wts"],
                              lambda e: _down_q(e, staged["sparse"]), tokens)
    err = np.abs(staged["out"][tokens] - ref)
    assert np.all(err <= tol), f"{int((err > tol).sum())} outputs outside the bound; max excess {float((err - tol).max())}"


def test_one_call_ffn_equals_the_staged_calls(staged):
    assert np.array_equal(staged["ffn"], staged["out"])
    assert np.all(np.isfinite(staged["out"]))
