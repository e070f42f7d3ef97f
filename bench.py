"""Benchmark of the NVFP4 / 2:4 weight-GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode|square|prefill|tiny]

Prints ONE JSON line. A step is one pass of the whole hot path over one batch of synthetic
input at the chosen workload. For the default decode workload (X [M, 5120] bf16 for
M in {1, 4, 8}; W [13824, 5120] float32 ~ N(0, 0.02)) a step is:

    nvfp4_quantize(W)                        dense NVFP4 weights
    sp24_prune(W) -> nvfp4_quantize          2:4-pruned NVFP4 weights
    sp24_check, sp24_compress                2:4 eligibility and compression
    gemm_nvfp4_dense  at M = 1, 4, 8         decode GEMVs on dense weights
    gemm_nvfp4_sp24   at M = 1, 4, 8         decode GEMVs on compressed weights

Inputs are resident in HBM before timing starts. The GEMVs read weight copies that were
written several steps earlier (a ring of copies larger than the 256 MB Infinity Cache), so
they are measured from HBM, not from cache. Every kernel is bracketed by HIP events on the
stream it runs on; ``value`` is the algorithmic bytes of the whole step divided by the step
time. ``roofline`` describes the kernel with the largest share of the step time.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4 GEMM TFLOP/s & HBM GB/s, 2:4 vs dense, % of MI355X roofline"
HBM_PEAK_GBPS = 8000.0          # MI355X published HBM3E bandwidth
BF16_PEAK_TFLOPS = 2500.0       # MI355X published dense bf16 matrix peak
RING = 16                       # weight copies rotated by the GEMVs (16 x 40 MB > 2 x 256 MB cache)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="decode", choices=["decode"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=6912, help="weight rows of the oracle sample")
    return p.parse_args()


# ------------------------------------------------------------------------------------------
# algorithmic bytes (minimum HBM traffic of each call) and flops
def bytes_quantize(N, K, w_bytes=4):
    return N * K * w_bytes + N * K // 2 + N * K // 16 + 4


def bytes_prune(N, K, w_bytes=4):
    return 2 * N * K * w_bytes


def bytes_check(N, K):
    return N * K // 2


def bytes_compress(N, K):
    return N * K // 2 + N * K // 4 + N * K // 8


def bytes_gemv_dense(M, N, K, y_bytes=4):
    return N * K // 2 + N * K // 16 + M * K * 2 + M * N * y_bytes


def bytes_gemv_sp24(M, N, K, y_bytes=4):
    return N * K // 4 + N * K // 8 + N * K // 16 + M * K * 2 + M * N * y_bytes


class Timer:
    """Per-name HIP event pairs recorded on the current stream, which is also the stream the
    prepared calls launch on. Events are created up front so recording costs one call each."""

    def __init__(self, torch, pool=4096):
        self.torch = torch
        self.free = [torch.cuda.Event(enable_timing=True) for _ in range(pool)]
        self.ev = {}

    def __call__(self, name, fn):
        a, b = self.free.pop(), self.free.pop()
        a.record()
        fn()
        b.record()
        self.ev.setdefault(name, []).append((a, b))

    def mean_ms(self, name):
        pairs = self.ev[name]
        return sum(a.elapsed_time(b) for a, b in pairs) / len(pairs)

    def reset(self):
        for pairs in self.ev.values():
            for a, b in pairs:
                self.free += [a, b]
        self.ev = {}


def hbm_probe(torch, ssn):
    """Measured bandwidth on this GPU: a 2 GiB device copy and a 2 GiB streaming read
    (sp24_check over 2 GiB of codes reads every byte once and writes two counters)."""
    n = 1 << 31
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(0x11)
    codes = src.view(1 << 16, n >> 16)
    for _ in range(2):
        dst.copy_(src)
        ssn.sp24_check(codes)
    torch.cuda.synchronize()
    res = {}
    for name, fn, nbytes in (("copy", lambda: dst.copy_(src), 2 * n), ("read", lambda: ssn.sp24_check(codes), n)):
        ts = []
        for _ in range(10):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(); fn(); b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b))
        ts.sort()
        res[f"{name}_GBps"] = round(nbytes / (ts[len(ts) // 2] * 1e-3) / 1e9, 1)
    del src, dst, codes
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------------------------------
def run_decode(args, torch, ssn, synth):
    N, K, Ms = 13824, 5120, (1, 4, 8)
    dev = "cuda"
    x = synth.activations(max(Ms), K)
    w = synth.weights(N, K)
    X = torch.from_numpy(x.view("int16")).view(torch.bfloat16).to(dev)
    W = torch.from_numpy(w).to(dev)
    Wp = torch.empty_like(W)
    u8 = dict(dtype=torch.uint8, device=dev)
    dense = [dict(codes=torch.empty((N, K // 2), **u8), scales=torch.empty((N, K // 16), **u8),
                  ts=torch.empty(1, dtype=torch.float32, device=dev)) for _ in range(RING)]
    sparse = [dict(codes=torch.empty((N, K // 2), **u8), scales=torch.empty((N, K // 16), **u8),
                   ts=torch.empty(1, dtype=torch.float32, device=dev), vals=torch.empty((N, K // 4), **u8),
                   meta=torch.empty((N, K // 8), **u8), bad=torch.empty(1, dtype=torch.int64, device=dev),
                   first=torch.empty(1, dtype=torch.int64, device=dev)) for _ in range(RING)]
    Yd = {M: torch.empty((M, N), dtype=torch.float32, device=dev) for M in Ms}
    Ys = {M: torch.empty((M, N), dtype=torch.float32, device=dev) for M in Ms}
    Xm = {M: X[:M].contiguous() for M in Ms}
    T = Timer(torch)
    # every call of the step, marshalled once per ring slot
    calls = []
    for j in range(RING):
        d, sp = dense[j], sparse[j]
        rd, rs = dense[(j + RING // 2) % RING], sparse[(j + RING // 2) % RING]
        c = [("quantize", ssn.nvfp4_quantize(W, codes=d["codes"], scales=d["scales"], tensor_scale_out=d["ts"],
                                             prepare=True)[0]),
             ("prune", ssn.sp24_prune(W, out=Wp, prepare=True)[0]),
             ("quantize_pruned", ssn.nvfp4_quantize(Wp, codes=sp["codes"], scales=sp["scales"],
                                                    tensor_scale_out=sp["ts"], prepare=True)[0]),
             ("check", ssn.sp24_check(sp["codes"], bad_groups=sp["bad"], first_bad=sp["first"], prepare=True)[0]),
             ("compress", ssn.sp24_compress(sp["codes"], vals=sp["vals"], meta=sp["meta"], bad_groups=sp["bad"],
                                            prepare=True)[0])]
        for M in Ms:
            c.append((f"gemv_dense_M{M}", ssn.gemm_nvfp4_dense(Xm[M], rd["codes"], rd["scales"], rd["ts"], Y=Yd[M],
                                                               prepare=True)))
        for M in Ms:
            c.append((f"gemv_sp24_M{M}", ssn.gemm_nvfp4_sp24(Xm[M], rs["vals"], rs["meta"], rs["scales"], rs["ts"],
                                                             Y=Ys[M], prepare=True)))
        calls.append(c)
    used = {}

    def step(i):
        for name, call in calls[i % RING]:
            if isinstance(call, tuple):            # GEMMs return (prepared, (Y, algo_used))
                T(name, call[0])
                used[name] = call[1][1]
            else:
                T(name, call)

    # fill every ring slot once so the GEMVs always read valid weights
    for i in range(RING):
        step(i)
    torch.cuda.synchronize()
    T.reset()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    T.reset()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps

    kb = {"quantize": bytes_quantize(N, K), "prune": bytes_prune(N, K), "quantize_pruned": bytes_quantize(N, K),
          "check": bytes_check(N, K), "compress": bytes_compress(N, K)}
    for M in Ms:
        kb[f"gemv_dense_M{M}"] = bytes_gemv_dense(M, N, K)
        kb[f"gemv_sp24_M{M}"] = bytes_gemv_sp24(M, N, K)
    kernels = {}
    for name, b in kb.items():
        ms = T.mean_ms(name)
        e = {"us": round(ms * 1e3, 2), "alg_bytes": b, "GBps": round(b / (ms * 1e-3) / 1e9, 1),
             "hbm_frac": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
        if name.startswith("gemv"):
            M = int(name.split("_M")[1])
            flops = 2 * M * N * K
            e["tflops_dense_equiv"] = round(flops / (ms * 1e-3) / 1e12, 3)
            if "sp24" in name:
                e["tflops_actual"] = round(flops / 2 / (ms * 1e-3) / 1e12, 3)
            e["algo"] = ssn.ALGO_NAMES.get(used[name].value, "?")
        kernels[name] = e
    for M in Ms:
        kernels[f"gemv_sp24_M{M}"]["speedup_vs_dense"] = round(
            kernels[f"gemv_dense_M{M}"]["us"] / kernels[f"gemv_sp24_M{M}"]["us"], 3)
    step_bytes = sum(kb.values())
    dominant = max(kernels, key=lambda k: kernels[k]["us"])
    dk = kernels[dominant]
    roof = {"kernel": dominant, "bound": "hbm", "achieved": dk["GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(dk["GBps"] / HBM_PEAK_GBPS, 4), "traffic": None}
    result = {
        "value": round(step_bytes / (ms_step * 1e-3) / 1e9, 1), "unit": "GB/s", "ms_per_step": round(ms_step, 4),
        "dtype": "bf16",
        "config": {"workload": "decode: X bf16 [M in {1,4,8}, 5120] ~N(0,1); W f32 [13824, 5120] ~N(0,0.02); "
                               "NVFP4 dense and 2:4-pruned+compressed; quantize, prune, check, compress, 6 GEMVs",
                   "M": list(Ms), "N": N, "K": K, "weight_ring": RING, "step_alg_bytes": step_bytes},
        "roofline": roof, "kernels": kernels,
    }
    return result, (w, x)


def cpu_baseline_decode(w, x, rows):
    """The oracle (unchanged) on the host: the decode step's calls over a sample of weight rows."""
    import numpy as np
    from oracle import gemm, quant, sp24
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    N, K = w.shape
    rows = min(rows, N)
    ws = w[:rows]
    t0 = time.perf_counter()
    st = quant.tensor_scale(w)
    c, s, _ = quant.quantize(ws, tensor_scale_in=st)
    wp = sp24.prune24(ws)
    stp = quant.tensor_scale(wp)
    pc, ps, _ = quant.quantize(wp, tensor_scale_in=stp)
    sp24.check(pc)
    v, m, _ = sp24.compress(pc)
    for M in (1, 4, 8):
        gemm.gemm_dense(x[:M], c, s, st)
    for M in (1, 4, 8):
        gemm.gemm_sp24(x[:M], v, m, ps, stp)
    sec = time.perf_counter() - t0
    b = (2 * bytes_quantize(rows, K) + bytes_prune(rows, K) + bytes_check(rows, K) + bytes_compress(rows, K)
         + sum(bytes_gemv_dense(M, rows, K) + bytes_gemv_sp24(M, rows, K) for M in (1, 4, 8)))
    return {"value": round(b / sec / 1e9, 3), "unit": "GB/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"the decode step's calls on weight rows [0, {rows}) of {N} (K={K}), M in {{1,4,8}}; "
                      f"{sec:.1f} s on host cores; NumPy float64 oracle",
            "seconds": round(sec, 2), "host_cores_available": len(os.sched_getaffinity(0))}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path runs on one "
              f"GPU and has no collectives).", file=sys.stderr)
        sys.exit(2)
    import torch
    import structured_sparse_nvfp4_amd as ssn
    import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    ssn.lib()
    hbm = hbm_probe(torch, ssn)
    res, (w, x) = run_decode(args, torch, ssn, synth)
    out = {"metric": METRIC, "value": res["value"], "unit": res["unit"], "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": res["ms_per_step"], "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": res["dtype"], "data": "synthetic", "config": res["config"],
           "roofline": res["roofline"], "hbm_measured": hbm}
    out["kernels"] = res["kernels"]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_decode(w, x, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
