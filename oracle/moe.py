"""Grouped-expert (MoE) SiLU-gated FFN with NVFP4 expert weights (oracle).

The pages give the shape of the problem, not a formula: a 512-expert mixture where each token
is routed to 10 experts ("NVFP4 vs 2:4 sparse", robertz.co, sections "Concurrency, not
sparsity, is the lever" and "The sparsity that does pay is already running"), whose expert
weights are NVFP4 and whose gate/up projections share one global scale ("NVFP4 Without FP4
Hardware", ai-muninn.com, section "The shared global scale"); the same robertz.co page, section
"Why it cannot run on this cluster", notes that no 2:4 grouped GEMM exists for such a model.
The plain reading taken here, for every expert e:

* g = X_e . W_gate,e^T and u = X_e . W_up,e^T, where X_e are the rows of the tokens routed to e
  and W_up,e = [W_gate,e; W_up,e] is one [2I, D] NVFP4 tensor (one shared tensor scale);
* H = bf16(silu(g) * u) with silu(g) = g / (1 + exp(-g)) — H is stored in bf16;
* Yd = H . W_down,e^T with W_down,e an NVFP4 [D, I] tensor;
* out[t] = sum_j r[t, j] * Yd[row(t, j)] over the token's selected experts, with the router's
  combine weights r.

Routing bookkeeping: rows are grouped by expert (ascending); inside an expert, rows follow the
flat (token, slot) order t * k + j. ``expert_offsets[e]`` is the first row of expert e.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_round, bf16_ulp, bf16_decode
from .gemm import REL_TOL, gemm_dense, gemm_sp24
from .quant import dequantize
from .sp24 import decompress

SILU_SLOPE_MAX = 1.0999  # max |d silu / dg| (attained near g = 2.4)
F32_U = 2.0 ** -24       # unit roundoff of float32
F32_EVAL_REL = 1e-6      # relative error allowed for evaluating silu(g) * u in float32


def route(topk_ids: np.ndarray, E: int):
    """(counts [E], expert_offsets [E+1], row_token [T*k], row_slot [T*k])."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    counts = np.bincount(flat, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    order = np.argsort(flat, kind="stable")       # by expert, then by flat index
    return counts, offsets, (order // k).astype(np.int64), (order % k).astype(np.int64)


def silu(g: np.ndarray) -> np.ndarray:
    return g / (1.0 + np.exp(-g))


def _product(x_bits, wq, rows=None):
    """wq = ('dense', codes, scales, s_t) or ('sp24', vals, meta, scales, s_t)."""
    if wq[0] == "dense":
        return gemm_dense(x_bits, wq[1], wq[2], wq[3], rows=rows)
    return gemm_sp24(x_bits, wq[1], wq[2], wq[3], wq[4], rows=rows)


def up_stage(x_bits: np.ndarray, up_q, I: int):
    """Gate/up products of one expert on its rows x_bits [r, D].

    Returns dict with g, u (float64 [r, I]), their bound bases Bg, Bu, h = silu(g) * u and
    H = bf16(h) (float64 holding bf16 values)."""
    g, Bg = _product(x_bits, up_q, rows=np.arange(0, I))
    u, Bu = _product(x_bits, up_q, rows=np.arange(I, 2 * I))
    h = silu(g) * u
    return dict(g=g, u=u, Bg=Bg, Bu=Bu, h=h, H=bf16_round(h))


def h_bound(st: dict) -> np.ndarray:
    """Allowed |H_gpu - H| when the GPU's g and u each carry the product bound and H_gpu is
    bf16(silu(g) * u) evaluated in f32.

    With |g' - g| <= dg and |u' - u| <= du (dg = 2e-3 * Bg, du = 2e-3 * Bu):
    silu(g') u' - silu(g) u = (silu(g') - silu(g)) u' + silu(g) (u' - u), so
    |h' - h| <= L dg (|u| + du) + |silu(g)| du with L = max |silu'| (the L dg du slack term is
    kept); the f32 evaluation adds a few f32 ulps of h (1e-6 relative); both sides then round
    to bf16, at most half an ulp each.
    """
    dg = REL_TOL * st["Bg"]
    du = REL_TOL * st["Bu"]
    sg = np.abs(silu(st["g"]))
    dh = SILU_SLOPE_MAX * dg * (np.abs(st["u"]) + du) + (sg + SILU_SLOPE_MAX * dg) * du
    dh = dh + F32_EVAL_REL * np.abs(st["h"])             # float32 evaluation of silu(g) * u
    return dh + bf16_ulp(np.abs(st["h"]) + dh)            # both sides round to bf16


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of values that are already bf16 (float64 holding bf16 values)."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def down_stage(H: np.ndarray, down_q):
    """Yd = H . W_down^T for one expert (H float64 holding bf16 values, [r, I]); returns (Yd, B)."""
    return _product(f64_to_bf16_bits(H), down_q)


def down_bound(H: np.ndarray, dH: np.ndarray, down_q) -> np.ndarray:
    """Allowed |Yd_gpu - Yd| of one expert's down product Yd = H . W_down^T when the GPU's
    input H_gpu differs from H by at most dH per element (dH = 0: the GPU's own H is the input).

    Yd_gpu - Yd = (H_gpu - H) . W^T + (the product error on H_gpu), so the bound is
    sum_i dH_i |w_i| + 2e-3 * sum_i |H_gpu,i| |w_i| with |H_gpu| <= |H| + dH.
    """
    absw = _abs_product(np.abs(H), down_q)
    errw = _abs_product(dH, down_q)
    return errw + REL_TOL * (absw + errw)


def combine_bound(yd: np.ndarray, dyd: np.ndarray, r: np.ndarray, k: int) -> np.ndarray:
    """Per-row contributions to the allowed |out_gpu - out| of the weighted combine.

    The GPU's rows carry |Yd_gpu - Yd| <= dyd; the combine sums its k products r_j * Yd_gpu,j
    in f32, whose rounding is at most (k + 1) f32 unit roundoffs of sum_j |r_j Yd_gpu,j|.
    Returns |r| * (dyd + (k + 1) 2^-24 (|yd| + dyd)); summing it over a token's rows gives
    that token's bound."""
    ar = np.abs(r)[:, None]
    return ar * dyd + (k + 1) * F32_U * ar * (np.abs(yd) + dyd)


def moe_ffn(x_bits: np.ndarray, topk_ids: np.ndarray, topk_w: np.ndarray, up_q, down_q, E: int,
            I: int, tokens=None):
    """End-to-end MoE output (float64 [T', D]) for ``tokens`` (default all) and its parity bound.

    up_q[e] / down_q[e] give the quantised weights of expert e (see ``_product``); they are
    only read for experts that the selected tokens use. The bound composes the three stage
    bounds: H within ``h_bound``, the down product within ``down_bound`` of that H error, and
    the combine within ``combine_bound``. Returns (out, bound, route tuple).
    """
    counts, offsets, row_token, row_slot = route(topk_ids, E)
    T, k = topk_ids.shape
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    want = np.zeros(T, dtype=bool)
    want[toks] = True
    D = None
    out = tol = None
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        rt, rs = row_token[r0:r1], row_slot[r0:r1]
        sel = want[rt]
        if not sel.any():
            continue
        rt, rs = rt[sel], rs[sel]
        st = up_stage(x_bits[rt], up_q(e), I)
        dH = h_bound(st)
        yd, _ = down_stage(st["H"], down_q(e))
        dyd = down_bound(st["H"], dH, down_q(e))
        if out is None:
            D = yd.shape[1]
            out, tol = np.zeros((T, D)), np.zeros((T, D))
        r = topk_w[rt, rs].astype(np.float64)
        np.add.at(out, rt, r[:, None] * yd)
        np.add.at(tol, rt, combine_bound(yd, dyd, r, k))
    if out is None:
        D = bf16_decode(x_bits[:1]).shape[1]
        out, tol = np.zeros((T, D)), np.zeros((T, D))
    return out[toks], tol[toks], (counts, offsets, row_token, row_slot)


def ffn_from_h(H: np.ndarray, row_token: np.ndarray, row_slot: np.ndarray, rows: np.ndarray,
               expert_of_row: np.ndarray, topk_w: np.ndarray, down_q, tokens: np.ndarray):
    """Down product and combine computed from a given H (the GPU's), for ``tokens``.

    H: float64 holding bf16 values [n_rows, I], the H of routing rows ``rows`` (expert of each
    in ``expert_of_row``; (token, slot) of each in row_token / row_slot). Every row of every
    selected token must be present. Returns (out [len(tokens), D], bound) where the bound is
    the product bound on the given H (``down_bound`` with dH = 0) composed with the combine.
    """
    tokens = np.asarray(tokens)
    pos = {int(t): i for i, t in enumerate(tokens)}
    k = int(topk_w.shape[1])
    out = tol = None
    for e in np.unique(expert_of_row):
        sel = np.nonzero(expert_of_row == e)[0]
        Hs = H[sel]
        yd, _ = down_stage(Hs, down_q(int(e)))
        dyd = down_bound(Hs, np.zeros_like(Hs), down_q(int(e)))
        if out is None:
            out, tol = np.zeros((tokens.size, yd.shape[1])), np.zeros((tokens.size, yd.shape[1]))
        rt, rs = row_token[sel], row_slot[sel]
        r = topk_w[rt, rs].astype(np.float64)
        idx = np.array([pos[int(t)] for t in rt])
        np.add.at(out, idx, r[:, None] * yd)
        np.add.at(tol, idx, combine_bound(yd, dyd, r, k))
    return out, tol


def _abs_product(a: np.ndarray, wq) -> np.ndarray:
    """sum_i a[:, i] * |w_hat[n, i]| for a >= 0 (float64), any weight form."""
    if wq[0] == "dense":
        w = dequantize(wq[1], wq[2], wq[3])
    else:
        w = dequantize(decompress(wq[1], wq[2]), wq[3], wq[4])
    return a @ np.abs(w).T
