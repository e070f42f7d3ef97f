"""Pins for the oracle's grouped-expert FFN: routing identities (brute force), SiLU special
values, and reduction of the MoE to single-expert products."""
import math

import numpy as np

import synth
from oracle import formats, gemm, moe, quant, sp24


def test_route_brute_force():
    rng = np.random.default_rng(0)
    T, k, E = 50, 3, 7
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    counts, offsets, rt, rs = moe.route(ids, E)
    assert counts.sum() == T * k and offsets[0] == 0 and offsets[-1] == T * k
    assert np.all(np.diff(offsets) == counts)
    rows = []
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if ids[t, j] == e:
                    rows.append((t, j))
    assert list(zip(rt.tolist(), rs.tolist())) == rows


def test_synthetic_routing_properties():
    ids, w = synth.routing(256, 64, 10, 1.1, seed=0)
    assert ids.shape == (256, 10) and w.shape == (256, 10)
    assert all(len(set(r)) == 10 for r in ids.tolist())       # distinct experts per token
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6) and np.all(w > 0)
    assert np.all(np.diff(w, axis=1) <= 1e-7)                  # weights follow the score order
    counts = np.bincount(ids.ravel(), minlength=64)
    assert counts.max() > 4 * np.median(counts)               # Zipf skew


def test_silu_values():
    assert moe.silu(np.array([0.0]))[0] == 0.0
    assert moe.silu(np.array([1.0]))[0] == 1.0 / (1.0 + math.exp(-1.0))
    assert moe.silu(np.array([50.0]))[0] == 50.0
    assert abs(moe.silu(np.array([-50.0]))[0]) < 1e-18
    g = np.linspace(-10, 10, 200001)
    slope = np.diff(moe.silu(g)) / np.diff(g)
    assert slope.max() <= moe.SILU_SLOPE_MAX and slope.max() > 1.09


def _experts(E, I, D, sparse):
    up, down = [], []
    for e in range(E):
        wu, wd = synth.expert_up(e, I, D), synth.expert_down(e, I, D)
        if sparse:
            wu, wd = sp24.prune24(wu), sp24.prune24(wd)
        cu, su, tu = quant.quantize(wu)
        cd, sd, td = quant.quantize(wd)
        if sparse:
            vu, mu, _ = sp24.compress(cu)
            vd, md, _ = sp24.compress(cd)
            up.append(("sp24", vu, mu, su, tu))
            down.append(("sp24", vd, md, sd, td))
        else:
            up.append(("dense", cu, su, tu))
            down.append(("dense", cd, sd, td))
    return up, down


def test_single_expert_reduces_to_products():
    T, D, I, E = 6, 64, 32, 3
    x = synth.activations(T, D, seed=1)
    up, down = _experts(E, I, D, sparse=False)
    ids = np.full((T, 1), 2, np.int32)
    w = np.ones((T, 1), np.float32)
    out, tol, _ = moe.moe_ffn(x, ids, w, lambda e: up[e], lambda e: down[e], E, I)
    _, cu, su, tu = up[2]
    g, _ = gemm.gemm_dense(x, cu[:I], su[:I], tu)
    u, _ = gemm.gemm_dense(x, cu[I:], su[I:], tu)
    H = formats.bf16_round(g / (1 + np.exp(-g)) * u)
    _, cd, sd, td = down[2]
    y, _ = gemm.gemm_dense(moe.f64_to_bf16_bits(H), cd, sd, td)
    assert np.allclose(out, y, rtol=0, atol=1e-15)
    assert np.all(tol > 0)


def test_combine_is_weighted_sum_and_token_subset():
    T, D, I, E, k = 10, 64, 32, 4, 2
    x = synth.activations(T, D, seed=2)
    up, down = _experts(E, I, D, sparse=True)
    ids = np.array([[t % E, (t + 1) % E] for t in range(T)], np.int32)
    w = np.tile(np.array([[0.25, 0.75]], np.float32), (T, 1))
    out, tol, _ = moe.moe_ffn(x, ids, w, lambda e: up[e], lambda e: down[e], E, I)
    # each token by hand from the single-expert path
    for t in range(T):
        acc = np.zeros(D)
        for j in range(k):
            e = ids[t, j]
            st = moe.up_stage(x[t:t + 1], up[e], I)
            yd, _ = moe.down_stage(st["H"], down[e])
            acc += float(w[t, j]) * yd[0]
        assert np.allclose(out[t], acc, rtol=0, atol=1e-15)
    sub, tsub, _ = moe.moe_ffn(x, ids, w, lambda e: up[e], lambda e: down[e], E, I, tokens=[3, 7])
    assert np.array_equal(sub, out[[3, 7]]) and np.array_equal(tsub, tol[[3, 7]])


def test_h_bound_covers_bf16_rounding():
    st = dict(g=np.array([[1.0]]), u=np.array([[2.0]]), Bg=np.array([[0.0]]), Bu=np.array([[0.0]]))
    st["h"] = moe.silu(st["g"]) * st["u"]
    b = moe.h_bound(st)
    assert b[0, 0] >= formats.bf16_ulp(st["h"])[0, 0]
