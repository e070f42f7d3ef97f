"""Seeded synthetic inputs for the NVFP4 / 2:4 weight-GEMM workloads.

This module is shared by the CPU oracle and the GPU path as the single source of
inputs. It draws random numbers and nothing else: it holds none of the method's
arithmetic (no quantisation, no pruning, no 2:4 logic, no products).

Every tensor has its own counter-addressed PCG64 stream,
``numpy.random.default_rng([seed, stream_id, index...])``, so any one tensor (or one
expert's weights, or one 256-row block of a large weight) can be redrawn on its own
without replaying the draws before it.

Workloads (sizes follow the statement of the problem; all values are synthetic):

* ``tiny``    X [16, 512] bf16 ~ N(0,1); W [256, 512] f32 ~ N(0, 0.02).
* ``decode``  X [8, 5120] bf16 (rows [:M] for M in {1, 4, 8}); W [13824, 5120].
* ``square``  X [4096, 4096]; W [4096, 4096].
* ``moe``     X [4096, 2048]; 512 experts; W_up [512, 2, 512, 2048] (index 0 = gate,
              1 = up); W_down [512, 2048, 512]; top-10 routing with Zipf(1.1) expert
              popularity.
* ``prefill`` X [8192, 5120]; W [27648, 5120] with a Bernoulli(1%) mask of x20
              outliers; bf16 output.
"""
from __future__ import annotations

import numpy as np

SEED = 0
W_STD = 0.02
ROW_BLOCK = 256  # rows per independently-seeded block of a weight matrix

# stream ids
_S_X, _S_W, _S_OUTLIER, _S_WUP, _S_WDOWN, _S_ROUTE = 1, 2, 3, 10, 11, 20

WORKLOADS = {
    "tiny": dict(M=16, N=256, K=512, out="f32"),
    "decode": dict(M=8, Ms=(1, 4, 8), N=13824, K=5120, out="f32"),
    "square": dict(M=4096, N=4096, K=4096, out="f32"),
    "moe": dict(T=4096, E=512, D=2048, I=512, topk=10, zipf_s=1.1, out="f32"),
    "prefill": dict(M=8192, N=27648, K=5120, outlier_p=0.01, outlier_mult=20.0, out="bf16"),
}


def rng(*key: int, seed: int = SEED) -> np.random.Generator:
    return np.random.default_rng([seed, *key])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); return the uint16 bit patterns.

    This is how the synthetic activations are delivered (bf16 storage); it is input
    preparation, not part of the method.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def activations(M: int, K: int, seed: int = SEED, stream: int = _S_X) -> np.ndarray:
    """X ~ N(0, 1), delivered as bf16 bit patterns, shape [M, K] uint16."""
    x = rng(stream, M, K, seed=seed).standard_normal((M, K), dtype=np.float32)
    return f32_to_bf16_bits(x)


def weight_rows(N: int, K: int, row0: int, row1: int, seed: int = SEED, stream: int = _S_W,
                std: float = W_STD) -> np.ndarray:
    """Rows [row0, row1) of W ~ N(0, std^2), float32 [row1-row0, K].

    Rows are drawn in independently seeded blocks of ``ROW_BLOCK`` rows, so a slice can be
    produced without drawing the whole matrix.
    """
    out = np.empty((row1 - row0, K), dtype=np.float32)
    b0, b1 = row0 // ROW_BLOCK, (row1 + ROW_BLOCK - 1) // ROW_BLOCK
    for b in range(b0, b1):
        lo, hi = b * ROW_BLOCK, min(N, (b + 1) * ROW_BLOCK)
        blk = rng(stream, N, K, b, seed=seed).standard_normal((hi - lo, K), dtype=np.float32)
        blk *= np.float32(std)
        s0, s1 = max(lo, row0), min(hi, row1)
        out[s0 - row0:s1 - row0] = blk[s0 - lo:s1 - lo]
    return out


def weights(N: int, K: int, seed: int = SEED, stream: int = _S_W, std: float = W_STD) -> np.ndarray:
    return weight_rows(N, K, 0, N, seed=seed, stream=stream, std=std)


def outlier_mask_rows(N: int, K: int, row0: int, row1: int, p: float, seed: int = SEED) -> np.ndarray:
    """Bernoulli(p) mask over W's entries (rows [row0, row1)), drawn per ROW_BLOCK block."""
    out = np.empty((row1 - row0, K), dtype=bool)
    b0, b1 = row0 // ROW_BLOCK, (row1 + ROW_BLOCK - 1) // ROW_BLOCK
    for b in range(b0, b1):
        lo, hi = b * ROW_BLOCK, min(N, (b + 1) * ROW_BLOCK)
        blk = rng(_S_OUTLIER, N, K, b, seed=seed).random((hi - lo, K), dtype=np.float32) < p
        s0, s1 = max(lo, row0), min(hi, row1)
        out[s0 - row0:s1 - row0] = blk[s0 - lo:s1 - lo]
    return out


def weight_rows_with_outliers(N: int, K: int, row0: int, row1: int, p: float, mult: float,
                              seed: int = SEED) -> np.ndarray:
    """W rows with a Bernoulli(p) subset of entries multiplied by ``mult`` (before any pruning)."""
    w = weight_rows(N, K, row0, row1, seed=seed)
    m = outlier_mask_rows(N, K, row0, row1, p, seed=seed)
    w[m] *= np.float32(mult)
    return w


def expert_up(e: int, I: int, D: int, seed: int = SEED) -> np.ndarray:
    """W_up of expert e, float32 [2*I, D]: rows [0, I) are the gate projection, [I, 2I) the up projection."""
    return rng(_S_WUP, e, I, D, seed=seed).standard_normal((2 * I, D), dtype=np.float32) * np.float32(W_STD)


def expert_down(e: int, I: int, D: int, seed: int = SEED) -> np.ndarray:
    """W_down of expert e, float32 [D, I]."""
    return rng(_S_WDOWN, e, I, D, seed=seed).standard_normal((D, I), dtype=np.float32) * np.float32(W_STD)


def routing(T: int, E: int, topk: int, zipf_s: float, seed: int = SEED):
    """Synthetic router output: top-k expert ids and combine weights per token.

    Expert popularity follows Zipf(s): the expert at popularity rank r (1-based) has
    weight r^-s; ranks are assigned to experts by a seeded permutation. Each token draws
    ``topk`` distinct experts without replacement in proportion to popularity, using the
    Gumbel-top-k trick (top-k of log p + Gumbel noise). Combine weights are the softmax of
    the selected perturbed scores. Returns (ids int32 [T, topk], weights float32 [T, topk]),
    ids in descending score order.
    """
    g = rng(_S_ROUTE, T, E, topk, seed=seed)
    perm = g.permutation(E)
    logp = np.empty(E, dtype=np.float64)
    logp[perm] = -zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))
    scores = logp[None, :] + g.gumbel(size=(T, E))
    ids = np.argsort(-scores, axis=1, kind="stable")[:, :topk]
    sel = np.take_along_axis(scores, ids, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    w = z / z.sum(axis=1, keepdims=True)
    return ids.astype(np.int32), w.astype(np.float32)
