"""Pins for the oracle's grouped-expert tolerances: the H bound (silu(g) * u from products that
each carry the 2e-3 * sum |x w| bound, evaluated in f32 and rounded to bf16), the down-product
bound on a perturbed input, the f32 combine bound, and their composition in ``moe_ffn``.

Each bound is checked from both sides against an emulated GPU whose every stage errs as far as
its own contract allows (worst-case corners found by brute force, f32 arithmetic done in f32):
soundness (the emulation never leaves the bound) and tightness (the worst case reaches a fixed
fraction of the bound, so a bound made twice too loose, or one with a term dropped, fails)."""
import itertools

import numpy as np

import synth
from oracle import formats, gemm, moe, quant, sp24

REL = gemm.REL_TOL


def _f32_h(g, u):
    """bf16(silu(g) * u) with every operation in float32, as a kernel evaluates it."""
    g32, u32 = np.asarray(g, np.float32), np.asarray(u, np.float32)
    s = g32 / (np.float32(1.0) + np.exp(-g32))
    return formats.bf16_round((s * u32).astype(np.float32).astype(np.float64))


def _cases(rng, n, g_lo, g_hi, b_lo, b_hi):
    g = rng.uniform(g_lo, g_hi, n)
    u = rng.choice([-1.0, 1.0], n) * rng.uniform(0.3, 2.5, n)
    st = dict(g=g[:, None], u=u[:, None], Bg=rng.uniform(b_lo, b_hi, n)[:, None],
              Bu=rng.uniform(b_lo, b_hi, n)[:, None])
    st["h"] = moe.silu(st["g"]) * st["u"]
    st["H"] = formats.bf16_round(st["h"])
    return st


def _worst_h_error(st, rng, interior=24):
    """max |H_gpu - H| over the four corners of the (g', u') box and random interior points."""
    dg, du = REL * st["Bg"], REL * st["Bu"]
    n = st["g"].shape[0]
    sg = np.concatenate([np.array([[-1, -1, 1, 1]] * n, float), rng.uniform(-1, 1, (n, interior))], axis=1)
    su = np.concatenate([np.array([[-1, 1, -1, 1]] * n, float), rng.uniform(-1, 1, (n, interior))], axis=1)
    Hg = _f32_h(st["g"] + sg * dg, st["u"] + su * du)
    return np.abs(Hg - st["H"]).max(axis=1, keepdims=True)


def test_h_bound_is_sound_over_the_error_box():
    rng = np.random.default_rng(0)
    for g_lo, g_hi, b_lo, b_hi in [(-8, 8, 0, 40), (-30, 30, 0, 5), (-3, 3, 0, 0.01), (1, 4, 10, 60)]:
        st = _cases(rng, 3000, g_lo, g_hi, b_lo, b_hi)
        err = _worst_h_error(st, rng)
        assert np.all(err <= moe.h_bound(st))


def test_h_bound_is_tight_where_silu_is_steepest():
    # near g = 2.4 silu' reaches its maximum, so the corners attain the propagated terms: halving
    # the bound (or dropping either product term) must fail there
    rng = np.random.default_rng(1)
    st = _cases(rng, 2000, 2.3, 2.5, 20, 60)
    ratio = _worst_h_error(st, rng, interior=0) / moe.h_bound(st)
    assert ratio.min() >= 0.7 and ratio.max() <= 1.0


def test_h_bound_each_term_is_needed():
    rng = np.random.default_rng(2)
    # only the gate product errs: the dg term alone must cover it
    st = _cases(rng, 2000, 2.3, 2.5, 20, 60)
    st["Bu"][:] = 0.0
    err = _worst_h_error(st, rng, interior=0)
    dg = REL * st["Bg"]
    no_dg = moe.h_bound(st) - moe.SILU_SLOPE_MAX * dg * np.abs(st["u"])
    assert np.all(err <= moe.h_bound(st)) and np.any(err > no_dg)
    # only the up product errs: the |silu(g)| du term
    st = _cases(rng, 2000, 2.3, 2.5, 20, 60)
    st["Bg"][:] = 0.0
    err = _worst_h_error(st, rng, interior=0)
    no_du = moe.h_bound(st) - np.abs(moe.silu(st["g"])) * REL * st["Bu"]
    assert np.all(err <= moe.h_bound(st)) and np.any(err > no_du)


def test_h_bound_covers_a_full_bf16_ulp_when_both_sides_round():
    # exact products (Bg = Bu = 0): float32 evaluation lands on the other side of a bf16 rounding
    # midpoint now and then, a whole ulp away from the float64 result; the bound must allow it
    rng = np.random.default_rng(3)
    n = 1_000_000
    st = dict(g=rng.uniform(-6, 6, (n, 1)), u=rng.uniform(-3, 3, (n, 1)), Bg=np.zeros((n, 1)), Bu=np.zeros((n, 1)))
    st["h"] = moe.silu(st["g"]) * st["u"]
    H = formats.bf16_round(st["h"])
    err = np.abs(_f32_h(st["g"], st["u"]) - H)
    b = moe.h_bound(st)
    flips = err > 0
    assert flips.sum() >= 10                                  # such cases exist
    assert np.all(err <= b)
    ulp = formats.bf16_ulp(np.abs(st["h"]))
    assert np.all(err[flips] >= ulp[flips])                   # each is a full ulp: half the ulp term fails
    assert np.any(err[flips] > (b - 0.5 * formats.bf16_ulp(np.abs(st["h"]) + b))[flips])


def _expert_down(sparse, D=8, I=8, seed=0):
    w = synth.expert_down(seed, I, D)
    w = w * np.float32(50.0)                                     # larger than ~N(0, 0.02): not relevant here
    if sparse:
        w = sp24.prune24(w)
    c, s, st = quant.quantize(w)
    if sparse:
        v, m, _ = sp24.compress(c)
        return ("sp24", v, m, s, st), quant.dequantize(sp24.decompress(v, m), s, st)
    return ("dense", c, s, st), quant.dequantize(c, s, st)


def test_down_bound_exact_input_is_the_product_bound():
    # with the GPU's own H as input (dH = 0) the down bound is the plain per-element product
    # bound 2e-3 * sum_i |H_i w_i|, computed independently by the product oracles
    rng = np.random.default_rng(4)
    for sparse in (False, True):
        q, _ = _expert_down(sparse, D=48, I=64, seed=1)
        H = formats.bf16_round(rng.standard_normal((7, 64)))
        got = moe.down_bound(H, np.zeros_like(H), q)
        bits = moe.f64_to_bf16_bits(H)
        B = gemm.gemm_sp24(bits, q[1], q[2], q[3], q[4])[1] if sparse else gemm.gemm_dense(bits, q[1], q[2], q[3])[1]
        assert np.allclose(got, REL * B, rtol=1e-12, atol=0)


def test_down_bound_brute_force_over_input_corners():
    # every H' with |H' - H| <= dH elementwise, at all 2^I corners, followed by a product that
    # errs by its full bound on H': the worst case stays inside down_bound and reaches it up to
    # the cross term (the two worst cases pick different corners)
    rng = np.random.default_rng(5)
    I = 16
    signs = np.array(list(itertools.product((-1.0, 1.0), repeat=I)))          # [2^I, I]
    for sparse in (False, True):
        q, w = _expert_down(sparse, D=8, I=I, seed=2)
        H = formats.bf16_round(rng.standard_normal((3, I)))
        dH = np.abs(rng.standard_normal((3, I))) * 0.05
        bound = moe.down_bound(H, dH, q)
        for m in range(H.shape[0]):
            Hp = H[m] + signs * dH[m]                                        # [2^I, I]
            dev = np.abs((Hp - H[m]) @ w.T) + REL * (np.abs(Hp) @ np.abs(w).T)
            worst = dev.max(axis=0)
            assert np.all(worst <= bound[m] * (1 + 1e-12))
            cross = 2 * REL * (dH[m] @ np.abs(w).T)
            assert np.all(worst >= bound[m] - cross - 1e-15)


def test_combine_bound_f32_rounding_and_row_errors():
    rng = np.random.default_rng(6)
    k, D, T = 10, 64, 400
    yd = rng.standard_normal((T * k, D)) * np.exp(rng.uniform(-3, 3, (T * k, 1)))
    r = rng.random(T * k).astype(np.float32).astype(np.float64)
    tok = np.repeat(np.arange(T), k)
    exact = np.zeros((T, D))
    np.add.at(exact, tok, r[:, None] * yd)

    def f32_combine(y):
        acc = np.zeros((T, D), np.float32)
        yy = y.astype(np.float32).reshape(T, k, D)
        rr = r.astype(np.float32).reshape(T, k)
        for j in range(k):
            acc = (acc + rr[:, j, None] * yy[:, j]).astype(np.float32)
        return acc.astype(np.float64)

    # exact rows: only the f32 rounding of the combine (yd itself rounded to f32 is part of it)
    tol = np.zeros((T, D))
    np.add.at(tol, tok, moe.combine_bound(yd, np.zeros_like(yd), r, k))
    err = np.abs(f32_combine(yd) - exact)
    assert np.all(err <= tol) and np.any(err > 0)             # the rounding term is needed
    # rows off by their full allowance in the direction of r: the row term is attained
    dyd = np.abs(yd) * 1e-2
    tol = np.zeros((T, D))
    np.add.at(tol, tok, moe.combine_bound(yd, dyd, r, k))
    err = np.abs(f32_combine(yd + dyd) - exact)
    assert np.all(err <= tol) and np.all(err >= 0.98 * tol)


def _ffn_weights(E, I, D):
    up, down = [], []
    for e in range(E):
        cu, su, tu = quant.quantize(synth.expert_up(e, I, D))
        cd, sd, td = quant.quantize(synth.expert_down(e, I, D))
        up.append(("dense", cu, su, tu))
        down.append(("dense", cd, sd, td))
    return up, down


def test_moe_ffn_bound_contains_an_adversarial_pipeline():
    """Every stage errs as far as its own contract allows, in the direction that moves output
    column 0 upwards: g and u at the corner of their product bounds that raises each H element
    whose down weight for column 0 is positive (lowers it otherwise), H from f32 silu(g) * u
    rounded to bf16, the down product off by its full bound on that H, the combine in f32.
    The result stays inside moe_ffn's bound everywhere and reaches a fixed share of it in
    column 0."""
    T, D, I, E, k = 12, 64, 32, 3, 2
    x = synth.activations(T, D, seed=9)
    up, down = _ffn_weights(E, I, D)
    ids = np.array([[t % E, (t + 1) % E] for t in range(T)], np.int32)
    wts = np.tile(np.array([[0.625, 0.375]], np.float32), (T, 1))
    out, tol, (_, offsets, row_token, row_slot) = moe.moe_ffn(x, ids, wts, lambda e: up[e], lambda e: down[e], E, I)
    rows_out = np.zeros((T, D))
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        rt, rs = row_token[r0:r1], row_slot[r0:r1]
        st = moe.up_stage(x[rt], up[e], I)
        wd = quant.dequantize(down[e][1], down[e][2], down[e][3])            # [D, I]
        want_up = np.sign(wd[0])[None, :]                                    # raise H where w[0, i] > 0
        dg, du = REL * st["Bg"], REL * st["Bu"]
        best = None
        for sg, su in itertools.product((-1.0, 1.0), repeat=2):
            Hc = _f32_h(st["g"] + sg * dg, st["u"] + su * du)
            score = want_up * (Hc - st["H"])
            if best is None:
                best, bscore = Hc, score
            else:
                take = score > bscore
                best, bscore = np.where(take, Hc, best), np.where(take, score, bscore)
        Hp = best
        yd = Hp @ wd.T + REL * (np.abs(Hp) @ np.abs(wd).T)                    # product errs upwards
        r = wts[rt, rs].astype(np.float32)
        contrib = (r[:, None] * yd.astype(np.float32)).astype(np.float32)
        for i, t in enumerate(rt):
            rows_out[t] = (rows_out[t].astype(np.float32) + contrib[i]).astype(np.float64)
    err = np.abs(rows_out - out)
    assert np.all(err <= tol)
    assert (err[:, 0] / tol[:, 0]).min() >= 0.3


def test_ffn_from_h_is_the_down_and_combine_of_moe_ffn():
    # with the oracle's own H, the stage-by-stage form gives moe_ffn's output, and its bound is
    # the product bound alone (no H term), so it is tighter
    T, D, I, E, k = 9, 64, 32, 4, 2
    x = synth.activations(T, D, seed=10)
    up, down = _ffn_weights(E, I, D)
    ids = np.array([[t % E, (t + 2) % E] for t in range(T)], np.int32)
    wts = np.tile(np.array([[0.5, 0.5]], np.float32), (T, 1))
    out, tol, (_, offsets, row_token, row_slot) = moe.moe_ffn(x, ids, wts, lambda e: up[e], lambda e: down[e], E, I)
    R = T * k
    H = np.zeros((R, I))
    eo = np.zeros(R, np.int64)
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        H[r0:r1] = moe.up_stage(x[row_token[r0:r1]], up[e], I)["H"]
        eo[r0:r1] = e
    toks = np.array([0, 4, 8])
    sel = np.nonzero(np.isin(row_token, toks))[0]
    o2, t2 = moe.ffn_from_h(H[sel], row_token[sel], row_slot[sel], sel, eo[sel], wts, lambda e: down[e], toks)
    assert np.allclose(o2, out[toks], rtol=0, atol=1e-12)
    assert np.all(t2 < tol[toks]) and np.all(t2 > 0)
