"""GPU parity of the grouped-expert path against the oracle: routing bookkeeping bit-exact,
grouped products row by row within the product bound, H = bf16(silu(g) * u) within the oracle's
H bound, the weighted combine, the whole FFN on a reduced configuration, and the full
configuration (4096 tokens, 512 experts, top-10, D = 2048, I = 512) on sampled tokens."""
import numpy as np
import pytest
import torch

import structured_sparse_nvfp4_amd as ssn
import synth
from oracle import gemm, moe, quant, sp24
from tests.gpu_util import assert_within_bound, dev, host, x_dev, y_host

pytestmark = pytest.mark.gpu


def _route_expect(ids, E):
    """Oracle routing over the entries whose id is in range (others get no row)."""
    flat = ids.reshape(-1)
    ok = (flat >= 0) & (flat < E)
    k = ids.shape[1]
    valid_f = np.nonzero(ok)[0]
    sub = flat[valid_f].reshape(-1, 1)
    counts, offsets, rt_sub, _ = moe.route(sub, E)     # k = 1: row i <-> valid entry i
    f_of_row = valid_f[rt_sub]
    row_of = np.full(flat.size, -1, np.int64)
    row_of[f_of_row] = np.arange(f_of_row.size)
    return offsets, f_of_row // k, f_of_row % k, row_of, int((~ok).sum())


def _check_route(ids, E):
    off, rt, rs, ro, bad = ssn.moe_route(dev(ids.astype(np.int32)), E)
    eo, ert, ers, ero, ebad = _route_expect(ids, E)
    F = ids.size
    assert np.array_equal(host(off).astype(np.int64), eo)
    n = int(eo[-1])
    assert np.array_equal(host(rt)[:n].astype(np.int64), ert)
    assert np.array_equal(host(rs)[:n].astype(np.int64), ers)
    assert np.array_equal(host(ro).astype(np.int64), ero)
    assert int(host(bad)[0]) == ebad
    if ebad == 0:   # with every id valid this is exactly the oracle's routing
        _, o2, rt2, rs2 = moe.route(ids, E)
        assert np.array_equal(host(rt).astype(np.int64), rt2) and np.array_equal(host(rs).astype(np.int64), rs2)
    assert F == ids.shape[0] * ids.shape[1]


@pytest.mark.parametrize("T,E,k", [(50, 7, 3), (300, 64, 10), (1, 5, 2), (2000, 512, 10), (4096, 512, 10),
                                   (256, 1, 4), (102, 2048, 10), (103, 2048, 10), (32, 512, 10)])
def test_route_matches_oracle(T, E, k):
    if k <= E and T > 1:
        ids, _ = synth.routing(T, E, k, 1.1, seed=T + E)
    else:
        ids = np.random.default_rng(T).integers(0, E, size=(T, k)).astype(np.int32)
    _check_route(ids, E)


@pytest.mark.parametrize("T", [700, 60])   # the multi-kernel routing (F > 1024) and the one-block one
def test_route_repeated_ids_and_invalid_ids(T):
    rng = np.random.default_rng(5)
    ids = rng.integers(-2, 9, size=(T, 4)).astype(np.int32)   # repeats, and ids outside [0, 7)
    _check_route(ids, 7)


def test_route_empty():
    off, rt, rs, ro, bad = ssn.moe_route(torch.zeros((0, 4), dtype=torch.int32, device="cuda"), 16)
    assert np.array_equal(host(off), np.zeros(17, np.int32)) and int(host(bad)[0]) == 0


# ------------------------------------------------------------------------------ grouped products
def _quant_experts(ws, sparse):
    """List of per-expert float32 weights -> oracle tuples and stacked device tensors."""
    qs, mains, metas, scs, tss = [], [], [], [], []
    for w in ws:
        if sparse:
            w = sp24.prune24(w)
        c, s, st = quant.quantize(w)
        if sparse:
            v, m, nb = sp24.compress(c)
            assert nb == 0
            qs.append(("sp24", v, m, s, st)); mains.append(v); metas.append(m)
        else:
            qs.append(("dense", c, s, st)); mains.append(c)
        scs.append(s); tss.append(st)
    dm = dev(np.stack(mains))
    dmeta = dev(np.stack(metas)) if sparse else None
    return qs, dm, dmeta, dev(np.stack(scs)), dev(np.array(tss, np.float32))


def _product(x, q, rows=None):
    if q[0] == "dense":
        return gemm.gemm_dense(x, q[1], q[2], q[3], rows=rows)
    return gemm.gemm_sp24(x, q[1], q[2], q[3], q[4], rows=rows)


def _ktiles(a, piece):
    """The 64-k tiled layout by its definition: dst[e][kt][n] = src[e][n][kt*P:(kt+1)*P]."""
    E, N, rb = a.shape
    return np.ascontiguousarray(a.reshape(E, N, rb // piece, piece).transpose(0, 2, 1, 3)).reshape(E, N, rb)


@pytest.mark.parametrize("piece", [4, 8, 16, 32])
def test_pack_ktiles_matches_definition(piece):
    rng = np.random.default_rng(piece)
    for E, N, rb in [(1, 1, piece), (3, 37, 8 * piece), (5, 256, 32 * piece)]:
        a = rng.integers(0, 256, size=(E, N, rb), dtype=np.uint8)
        got = host(ssn.moe_pack_ktiles(dev(a), piece))
        assert np.array_equal(got, _ktiles(a, piece))


def _tile_algo(algo, sparse):
    """The algorithm a parametrised grouped-product test asks for (AUTO for the default tiles)."""
    if algo == "stream":
        return ssn.ALGO_STREAM, ssn.ALGO_STREAM
    if algo == "tiles_expand":
        return ssn.ALGO_DECOMPRESS_MFMA, ssn.ALGO_DECOMPRESS_MFMA
    return ssn.ALGO_AUTO, (ssn.ALGO_SMFMAC if sparse else ssn.ALGO_MFMA)


@pytest.mark.parametrize("algo", ["tiles", "tiles_expand", "stream"])
@pytest.mark.parametrize("layout", [ssn.WLAYOUT_ROWS, ssn.WLAYOUT_KTILE64])
@pytest.mark.parametrize("sparse", [False, True])
@pytest.mark.parametrize("gather", [True, False])
def test_grouped_product_rows(sparse, gather, layout, algo):
    if algo == "tiles_expand" and not sparse:
        pytest.skip("the expanded-dense tiles are a 2:4 algorithm")
    T, E, k, N, K = 90, 6, 3, 320, 192
    x = synth.activations(T, K, seed=11)
    ids = np.random.default_rng(3).integers(0, E, size=(T, k)).astype(np.int32)
    ids[:, 0] = 2                                   # one expert with > 64 rows (two row tiles)
    ws = [synth.weights(N, K, seed=100 + e) for e in range(E)]
    qs, dm, dmeta, dsc, dts = _quant_experts(ws, sparse)
    off, rt, rs, ro, _ = ssn.moe_route(dev(ids), E)
    R = T * k
    offs = host(off).astype(np.int64)
    rts = host(rt).astype(np.int64)
    if gather:
        X, rtok, src = x_dev(x), rt, rts
    else:                                           # identity rows: X already in expert order
        X, rtok, src = x_dev(x[rts]), None, np.arange(R)
        x = x[rts]
    if layout == ssn.WLAYOUT_KTILE64:
        dm, dmeta, dsc, dts = ssn.moe_pack_weights((dm, dmeta, dsc, dts))
    ask, want = _tile_algo(algo, sparse)
    y, used = ssn.moe_grouped_gemm_nvfp4(X, rtok, off, R, dm, dsc, dts, w_meta=dmeta, w_layout=layout, algo=ask)
    assert used == want
    yh = y_host(y)
    for e in range(E):
        r0, r1 = offs[e], offs[e + 1]
        if r1 == r0:
            continue
        Y, B = _product(x[src[r0:r1]], qs[e])
        assert_within_bound(yh[r0:r1], Y, B, what=f"expert {e}")


@pytest.mark.parametrize("algo", ["tiles", "tiles_expand", "stream"])
@pytest.mark.parametrize("layout", [ssn.WLAYOUT_ROWS, ssn.WLAYOUT_KTILE64])
@pytest.mark.parametrize("sparse", [False, True])
def test_grouped_silu_gate(sparse, layout, algo):
    if algo == "tiles_expand" and not sparse:
        pytest.skip("the expanded-dense tiles are a 2:4 algorithm")
    T, E, k, D, I = 70, 5, 2, 128, 160
    x = synth.activations(T, D, seed=12)
    ids = np.random.default_rng(4).integers(0, E, size=(T, k)).astype(np.int32)
    ws = [synth.expert_up(e, I, D, seed=7) for e in range(E)]
    qs, dm, dmeta, dsc, dts = _quant_experts(ws, sparse)
    off, rt, _, _, _ = ssn.moe_route(dev(ids), E)
    R = T * k
    if layout == ssn.WLAYOUT_KTILE64:
        dm, dmeta, dsc, dts = ssn.moe_pack_weights((dm, dmeta, dsc, dts))
    ask, want = _tile_algo(algo, sparse)
    H, used = ssn.moe_grouped_gemm_nvfp4(x_dev(x), rt, off, R, dm, dsc, dts, w_meta=dmeta,
                                         epilogue=ssn.EPI_SILU_GATE, y_dtype=torch.bfloat16, w_layout=layout, algo=ask)
    assert used == want
    Hh = y_host(H)
    offs, rts = host(off).astype(np.int64), host(rt).astype(np.int64)
    for e in range(E):
        r0, r1 = offs[e], offs[e + 1]
        if r1 == r0:
            continue
        st = moe.up_stage(x[rts[r0:r1]], qs[e], I)
        err = np.abs(Hh[r0:r1] - st["H"])
        bound = moe.h_bound(st)
        assert np.all(err <= bound), f"expert {e}: max excess {float((err - bound).max())}"


@pytest.mark.parametrize("sparse", [False, True])
def test_stream_k_split_and_edges(sparse):
    """Few items and a long K (the four-wave K split), an expert with more than 32 routed rows
    (several routed-row chunks), and K not a multiple of the chunk ring."""
    E, D, I = 6, 1088, 96                          # up: K = 1088 (17 chunks), N = 192
    x = synth.activations(40, D, seed=21)
    ids = np.array([[1, 4]] * 3 + [[4, 2]] * 37, np.int32)   # expert 4: 40 rows, 1: 3, 2: 37
    ws = [synth.expert_up(e, I, D, seed=8) for e in range(E)]
    qs, dm, dmeta, dsc, dts = _quant_experts(ws, sparse)
    off, rt, _, _, _ = ssn.moe_route(dev(ids), E)
    R = ids.size
    H, used = ssn.moe_grouped_gemm_nvfp4(x_dev(x), rt, off, R, dm, dsc, dts, w_meta=dmeta,
                                         epilogue=ssn.EPI_SILU_GATE, y_dtype=torch.float32, algo=ssn.ALGO_STREAM)
    assert used == ssn.ALGO_STREAM
    Hh = y_host(H)
    offs, rts = host(off).astype(np.int64), host(rt).astype(np.int64)
    for e in range(E):
        r0, r1 = offs[e], offs[e + 1]
        if r1 == r0:
            continue
        st = moe.up_stage(x[rts[r0:r1]], qs[e], I)
        # f32 output: compare the unrounded silu(g) * u with the GEMM bound propagated through silu
        err = np.abs(Hh[r0:r1] - st["h"])
        bound = moe.h_bound(st)
        assert np.all(err <= bound), f"expert {e}: max excess {float((err - bound).max())}"


def test_stream_rejects_unaligned_n():
    E, K, N = 2, 64, 48                            # N % 32 != 0
    X = torch.zeros((4, K), dtype=torch.bfloat16, device="cuda")
    off = torch.tensor([0, 2, 4], dtype=torch.int32, device="cuda")
    w = torch.zeros((E, N, K // 2), dtype=torch.uint8, device="cuda")
    sc = torch.zeros((E, N, K // 16), dtype=torch.uint8, device="cuda")
    ts = torch.ones(E, dtype=torch.float32, device="cuda")
    with pytest.raises(ssn.SsnError):
        ssn.moe_grouped_gemm_nvfp4(X, None, off, 4, w, sc, ts, algo=ssn.ALGO_STREAM)
    _, used = ssn.moe_grouped_gemm_nvfp4(X, None, off, 4, w, sc, ts)   # AUTO: the tiles
    assert used == ssn.ALGO_MFMA


def test_combine_weighted_sum():
    T, k, D, E = 64, 4, 200, 9
    ids = np.random.default_rng(8).integers(0, E, size=(T, k)).astype(np.int32)
    w = np.random.default_rng(9).random((T, k)).astype(np.float32)
    off, rt, rs, ro, _ = ssn.moe_route(dev(ids), E)
    Yd = np.random.default_rng(10).standard_normal((T * k, D)).astype(np.float32)
    out = ssn.moe_combine(dev(Yd), ro, dev(w))
    rows = host(ro).astype(np.int64).reshape(T, k)
    want = np.einsum("tj,tjd->td", w.astype(np.float64), Yd.astype(np.float64)[rows])
    got = host(out).astype(np.float64)
    assert np.all(np.abs(got - want) <= 1e-6 * np.einsum("tj,tjd->td", np.abs(w), np.abs(Yd)[rows]) + 1e-30)


@pytest.mark.parametrize("T,k,D,bf16", [(3, 10, 2500, False), (5, 17, 2049, False), (2, 10, 2050, True),
                                        (1, 64, 1024, True), (70, 3, 6, False)])
def test_combine_slots_columns_and_skipped_rows(T, k, D, bf16):
    """Slot counts across the eight-slot batches, column counts across 1024-column items with
    ragged and non-multiple-of-4 tails, bf16 rows, and rows outside [0, R) skipped. Against
    the fp64 sum: an f32 sum of k products (fused or not) is within (k + 1) * 2^-24 of the sum
    of their magnitudes."""
    rng = np.random.default_rng(T * 1000 + k)
    R = T * k
    Yd = rng.standard_normal((R, D)).astype(np.float32)
    if bf16:   # values exactly representable in bf16
        Yd = (Yd.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    w = rng.random((T, k)).astype(np.float32)
    rows = rng.permutation(R).astype(np.int32)
    rows[rng.random(R) < 0.2] = -1
    rows[rng.random(R) < 0.05] = R + 3
    yd = dev(Yd).to(torch.bfloat16) if bf16 else dev(Yd)
    out = host(ssn.moe_combine(yd, dev(rows), dev(w)))
    want = np.zeros((T, D))
    mag = np.zeros((T, D))
    r2 = rows.reshape(T, k)
    for t in range(T):
        for j in range(k):
            if 0 <= r2[t, j] < R:
                want[t] += float(w[t, j]) * Yd[r2[t, j]].astype(np.float64)
                mag[t] += abs(float(w[t, j])) * np.abs(Yd[r2[t, j]]).astype(np.float64)
    assert np.all(np.abs(out.astype(np.float64) - want) <= (k + 1) * 2.0 ** -24 * mag)


# ------------------------------------------------------------------------------ whole FFN
def _ffn_weights(E, I, D, sparse):
    ups = [synth.expert_up(e, I, D) for e in range(E)]
    downs = [synth.expert_down(e, I, D) for e in range(E)]
    qu, um, umeta, usc, uts = _quant_experts(ups, sparse)
    qd, dm, dmeta, dsc, dts = _quant_experts(downs, sparse)
    return qu, qd, (um, umeta, usc, uts), (dm, dmeta, dsc, dts)


@pytest.mark.parametrize("layout", [ssn.WLAYOUT_ROWS, ssn.WLAYOUT_KTILE64])
@pytest.mark.parametrize("sparse", [False, True])
def test_ffn_reduced_config(sparse, layout):
    T, E, k, D, I = 256, 16, 4, 256, 128
    x = synth.activations(T, D, seed=13)
    ids, w = synth.routing(T, E, k, 1.1, seed=14)
    qu, qd, up, down = _ffn_weights(E, I, D, sparse)
    if layout == ssn.WLAYOUT_KTILE64:
        up, down = ssn.moe_pack_weights(up), ssn.moe_pack_weights(down)
    out, bad = ssn.moe_nvfp4_ffn(x_dev(x), dev(ids), dev(w), E, up, down, w_layout=layout)
    ref, tol, _ = moe.moe_ffn(x, ids, w, lambda e: qu[e], lambda e: qd[e], E, I)
    assert int(host(bad)[0]) == 0
    err = np.abs(y_host(out) - ref)
    assert np.all(err <= tol), f"max excess {float((err - tol).max())}"


# every token routed to the same k experts: those experts hold all T rows (ragged last tiles),
# every other expert is empty (the first and last expert among them); T = 300 takes the tiled
# products, T = 8 the streaming kernel
@pytest.mark.parametrize("T", [300, 8])
@pytest.mark.parametrize("layout", [ssn.WLAYOUT_ROWS, ssn.WLAYOUT_KTILE64])
@pytest.mark.parametrize("sparse", [False, True])
def test_ffn_all_tokens_on_the_same_experts(sparse, layout, T):
    E, k, D, I = 64, 4, 256, 128
    x = synth.activations(T, D, seed=15)
    chosen = np.array([3, 7, 8, 62], np.int32)
    ids = np.tile(chosen, (T, 1))
    w = synth.rng(16).random((T, k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    qu, qd, up, down = _ffn_weights(E, I, D, sparse)
    if layout == ssn.WLAYOUT_KTILE64:
        up, down = ssn.moe_pack_weights(up), ssn.moe_pack_weights(down)
    out, bad = ssn.moe_nvfp4_ffn(x_dev(x), dev(ids), dev(w), E, up, down, w_layout=layout)
    ref, tol, _ = moe.moe_ffn(x, ids, w, lambda e: qu[e], lambda e: qd[e], E, I)
    assert int(host(bad)[0]) == 0
    err = np.abs(y_host(out) - ref)
    assert np.all(err <= tol), f"max excess {float((err - tol).max())}"


def _full_gpu_weights(E, I, D, sparse):
    """All experts quantised (and pruned/compressed) on the GPU from the synthetic weights."""
    def build(gen, rows, cols):
        c = torch.empty((E, rows, cols // (4 if sparse else 2)), dtype=torch.uint8, device="cuda")
        m = torch.empty((E, rows, cols // 8), dtype=torch.uint8, device="cuda") if sparse else None
        s = torch.empty((E, rows, cols // 16), dtype=torch.uint8, device="cuda")
        ts = torch.empty(E, dtype=torch.float32, device="cuda")
        for e in range(E):
            W = torch.from_numpy(gen(e)).cuda()
            if sparse:
                W = ssn.sp24_prune(W)
                codes, _, _ = ssn.nvfp4_quantize(W, scales=s[e], tensor_scale_out=ts[e:e + 1])
                ssn.sp24_compress(codes, vals=c[e], meta=m[e])
            else:
                ssn.nvfp4_quantize(W, codes=c[e], scales=s[e], tensor_scale_out=ts[e:e + 1])
        return c, m, s, ts
    up = build(lambda e: synth.expert_up(e, I, D), 2 * I, D)
    down = build(lambda e: synth.expert_down(e, I, D), D, I)
    return up, down


@pytest.mark.parametrize("layout", [ssn.WLAYOUT_ROWS, ssn.WLAYOUT_KTILE64])
@pytest.mark.parametrize("sparse", [False, True])
def test_ffn_full_config_sampled_tokens(sparse, layout):
    T, E, k, D, I = 4096, 512, 10, 2048, 512
    x = synth.activations(T, D)
    ids, w = synth.routing(T, E, k, 1.1)
    up, down = _full_gpu_weights(E, I, D, sparse)
    if layout == ssn.WLAYOUT_KTILE64:
        up, down = ssn.moe_pack_weights(up), ssn.moe_pack_weights(down)
    out, bad = ssn.moe_nvfp4_ffn(x_dev(x), dev(ids), dev(w), E, up, down, w_layout=layout)
    tokens = np.array([0, 4095])

    def q(gen, e):
        wt = gen(e)
        if sparse:
            wt = sp24.prune24(wt)
        c, s, st = quant.quantize(wt)
        if sparse:
            v, m, _ = sp24.compress(c)
            return ("sp24", v, m, s, st)
        return ("dense", c, s, st)

    cache = {}

    def qu(e):
        if ("u", e) not in cache:
            cache[("u", e)] = q(lambda i: synth.expert_up(i, I, D), e)
        return cache[("u", e)]

    def qd(e):
        if ("d", e) not in cache:
            cache[("d", e)] = q(lambda i: synth.expert_down(i, I, D), e)
        return cache[("d", e)]

    ref, tol, _ = moe.moe_ffn(x, ids, w, qu, qd, E, I, tokens=tokens)
    assert int(host(bad)[0]) == 0
    got = y_host(out)[tokens]
    err = np.abs(got - ref)
    assert np.all(err <= tol), f"max excess {float((err - tol).max())}"
    assert bool(torch.isfinite(out).all())


@pytest.mark.parametrize("layout", [ssn.WLAYOUT_ROWS, ssn.WLAYOUT_KTILE64])
@pytest.mark.parametrize("sparse", [False, True])
def test_ffn_full_config_decode_tokens(sparse, layout):
    """Decode-sized routing on the full expert set (512 experts, top-10, D = 2048, I = 512): two
    tokens, every output checked. AUTO runs the routing in one block and both projections on the
    weight-streaming kernel (the up projection with its K split over four waves)."""
    T, E, k, D, I = 2, 512, 10, 2048, 512
    x = synth.activations(T, D, seed=31)
    ids, w = synth.routing(T, E, k, 1.1, seed=32)
    up, down = _full_gpu_weights(E, I, D, sparse)
    if layout == ssn.WLAYOUT_KTILE64:
        up, down = ssn.moe_pack_weights(up), ssn.moe_pack_weights(down)
    out, bad = ssn.moe_nvfp4_ffn(x_dev(x), dev(ids), dev(w), E, up, down, w_layout=layout)

    def q(gen, e):
        wt = gen(e)
        if sparse:
            wt = sp24.prune24(wt)
        c, s, st = quant.quantize(wt)
        if sparse:
            v, m, _ = sp24.compress(c)
            return ("sp24", v, m, s, st)
        return ("dense", c, s, st)

    ref, tol, _ = moe.moe_ffn(x, ids, w, lambda e: q(lambda i: synth.expert_up(i, I, D), e),
                              lambda e: q(lambda i: synth.expert_down(i, I, D), e), E, I)
    assert int(host(bad)[0]) == 0
    err = np.abs(y_host(out) - ref)
    assert np.all(err <= tol), f"max excess {float((err - tol).max())}"
