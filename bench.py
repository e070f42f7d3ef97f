"""Benchmark of the NVFP4 / 2:4 weight-GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads decode,square,prefill,head,moe]

Prints ONE JSON line. ``value`` / ``ms_per_step`` / ``roofline`` / ``cpu_baseline`` describe the
decode workload, where a step is one pass of the whole hot path over one batch of synthetic
input (X [M, 5120] bf16 for M in {1, 4, 8}; W [13824, 5120] float32 ~ N(0, 0.02)):

    sp24_prune(W) -> W_pruned, s_t           2:4 prune; s_t = fl32(amax|W| / 2688) taken on the way
    nvfp4_quantize(W, s_t)                   dense NVFP4 weights
    nvfp4_quantize(W_pruned, s_t)            2:4-pruned NVFP4 weights (same s_t: pruning keeps
                                             every group's largest |w|)
    sp24_check, sp24_compress                2:4 eligibility and compression
    gemm_nvfp4_dense  at M = 1, 4, 8         decode GEMVs on dense weights
    gemm_nvfp4_sp24   at M = 1, 4, 8         decode GEMVs on compressed weights

Inputs are resident in HBM before timing starts. The K timed steps run call by call: all K
prunes, then all K quantisations, and so on (every step has its own ring slot of outputs, so
the work is the same as K steps in order); HIP events on the launch stream bracket each batch,
which gives every kernel's average duration over back-to-back launches. The GEMVs read weight
copies written many calls earlier (a ring larger than the 256 MB Infinity Cache), so they read
HBM. ``value`` is the algorithmic bytes of the whole step divided by the step time;
``roofline`` describes the kernel with the largest share of the step.

``workloads`` adds the other shapes, each timed the same way: the square (4096^3, f32 out) and
prefill (8192 x 27648 x 5120, 1% outliers x20, bf16 out) products for dense MFMA, 2:4 SMFMAC
and 2:4 expanded-to-dense MFMA, an output-head-shaped GEMV (N = 131072, K = 5120, M = 1, 8, 9),
and the grouped-expert FFN (4096 tokens, 512 experts, top-10
Zipf(1.1), D = 2048, I = 512) stage by stage, dense and 2:4, plus the same FFN at decode sizes
(1, 4, 16, 32 tokens) against the full expert set, on the weight-streaming grouped kernels.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4 GEMM TFLOP/s & HBM GB/s, 2:4 vs dense, % of MI355X roofline"
HBM_PEAK_GBPS = 8000.0          # MI355X published HBM3E bandwidth
BF16_PEAK_TFLOPS = 2500.0       # MI355X published dense bf16 matrix peak
SPARSE_BF16_PEAK_TFLOPS = 5000.0  # the same with 2:4 structured sparsity (dense-equivalent)
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X published fp32 vector peak
RING = 16                       # weight copies rotated by the GEMVs (16 x 40 MB > 2 x 256 MB cache)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workloads", default="decode,square,prefill,head,moe",
                   help="comma list; decode is always run (it defines the step)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=13824, help="weight rows of the oracle sample")
    return p.parse_args()


# ------------------------------------------------------------------------------------------
# algorithmic bytes (minimum HBM traffic of each call) and flops
def bytes_quantize(N, K, w_bytes=4):
    return N * K * w_bytes + N * K // 2 + N * K // 16 + 4


def bytes_prune(N, K, w_bytes=4):
    return 2 * N * K * w_bytes + 4          # W read, W_pruned written, s_t written


def bytes_check(N, K):
    return N * K // 2


def bytes_compress(N, K):
    return N * K // 2 + N * K // 4 + N * K // 8


def bytes_w_dense(N, K):
    return N * K // 2 + N * K // 16


def bytes_w_sp24(N, K):
    return N * K // 4 + N * K // 8 + N * K // 16


def bytes_gemm(M, N, K, sparse, y_bytes):
    return (bytes_w_sp24(N, K) if sparse else bytes_w_dense(N, K)) + M * K * 2 + M * N * y_bytes


class Batches:
    """Event pairs around batches of back-to-back launches on the current stream (the stream
    the prepared calls launch on)."""

    def __init__(self, torch):
        self.torch = torch
        self.ev = {}

    def run(self, name, fns):
        a = self.torch.cuda.Event(enable_timing=True)
        b = self.torch.cuda.Event(enable_timing=True)
        a.record()
        for f in fns:
            f()
        b.record()
        self.ev[name] = (a, b, len(fns))

    def us(self, name):
        a, b, n = self.ev[name]
        return a.elapsed_time(b) * 1e3 / n


def hbm_probe(torch, ssn):
    """Measured bandwidth on this GPU: a 2 GiB device copy and a 2 GiB streaming read
    (sp24_check over 2 GiB of zero codes reads every byte once; every group passes, so the
    counters are never touched)."""
    n = 1 << 31
    src = torch.zeros(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
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


def traffic_for(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, only if the kernel's
    source is unchanged since the counters were taken (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f).get(kernel)
        if not t:
            return None
        with open(os.path.join(ROOT, t["source"]), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != t["source_sha256"]:
                return None
        return int(t["fetch_bytes"] + t["write_bytes"])
    except (OSError, KeyError, ValueError):
        return None


# ------------------------------------------------------------------------------------------
def run_decode(args, torch, ssn, synth):
    N, K, Ms = 13824, 5120, (1, 4, 8)
    dev = "cuda"
    x = synth.activations(max(Ms), K)
    w = synth.weights(N, K)
    X = torch.from_numpy(x.view("int16")).view(torch.bfloat16).to(dev)
    W = torch.from_numpy(w).to(dev)
    u8 = dict(dtype=torch.uint8, device=dev)
    wps = [torch.empty_like(W) for _ in range(2)]   # pruned copies, alternating
    dense = [dict(codes=torch.empty((N, K // 2), **u8), scales=torch.empty((N, K // 16), **u8),
                  ts=torch.empty(1, dtype=torch.float32, device=dev)) for _ in range(RING)]
    sparse = [dict(codes=torch.empty((N, K // 2), **u8), scales=torch.empty((N, K // 16), **u8),
                   ts=torch.empty(1, dtype=torch.float32, device=dev), vals=torch.empty((N, K // 4), **u8),
                   meta=torch.empty((N, K // 8), **u8), bad=torch.empty(1, dtype=torch.int64, device=dev),
                   first=torch.empty(1, dtype=torch.int64, device=dev)) for _ in range(RING)]
    ts_w = [torch.empty(1, dtype=torch.float32, device=dev) for _ in range(RING)]   # s_t from the prune
    Yd = {M: torch.empty((M, N), dtype=torch.float32, device=dev) for M in Ms}
    Ys = {M: torch.empty((M, N), dtype=torch.float32, device=dev) for M in Ms}
    Xm = {M: X[:M].contiguous() for M in Ms}
    names = ["prune", "quantize", "quantize_pruned", "check", "compress"] + \
            [f"gemv_dense_M{M}" for M in Ms] + [f"gemv_sp24_M{M}" for M in Ms]
    # timed beside the step, not part of it: the fused producer, and the 2:4 GEMVs in the plain
    # skip-and-gather form (vector ALU) for comparison with the SMFMAC ones
    extra = ["producer_fused"] + [f"gemv_sp24_gather_M{M}" for M in Ms]
    prod = [dict(vals=torch.empty((N, K // 4), **u8), meta=torch.empty((N, K // 8), **u8),
                 scales=torch.empty((N, K // 16), **u8), ts=torch.empty(1, dtype=torch.float32, device=dev),
                 bad=torch.empty(1, dtype=torch.int64, device=dev)) for _ in range(2)]
    calls = {n: [] for n in names + extra}
    used = {}
    for j in range(RING):
        d, sp, wp = dense[j], sparse[j], wps[j % 2]
        rd, rs = dense[(j + RING // 2) % RING], sparse[(j + RING // 2) % RING]
        calls["prune"].append(ssn.sp24_prune(W, out=wp, tensor_scale_out=ts_w[j], prepare=True)[0])
        calls["quantize"].append(ssn.nvfp4_quantize(W, tensor_scale_in=ts_w[j], codes=d["codes"], scales=d["scales"],
                                                    tensor_scale_out=d["ts"], prepare=True)[0])
        calls["quantize_pruned"].append(ssn.nvfp4_quantize(wp, tensor_scale_in=ts_w[j], codes=sp["codes"],
                                                           scales=sp["scales"], tensor_scale_out=sp["ts"],
                                                           prepare=True)[0])
        calls["check"].append(ssn.sp24_check(sp["codes"], bad_groups=sp["bad"], first_bad=sp["first"],
                                             prepare=True)[0])
        calls["compress"].append(ssn.sp24_compress(sp["codes"], vals=sp["vals"], meta=sp["meta"],
                                                   bad_groups=sp["bad"], prepare=True)[0])
        pf = prod[j % 2]
        calls["producer_fused"].append(ssn.nvfp4_sp24_produce(W, vals=pf["vals"], meta=pf["meta"], scales=pf["scales"],
                                                              tensor_scale_out=pf["ts"], bad_groups=pf["bad"],
                                                              prepare=True)[0])
        for M in Ms:
            p, (_, u) = ssn.gemm_nvfp4_dense(Xm[M], rd["codes"], rd["scales"], rd["ts"], Y=Yd[M], prepare=True)
            calls[f"gemv_dense_M{M}"].append(p)
            used[f"gemv_dense_M{M}"] = u
            p, (_, u) = ssn.gemm_nvfp4_sp24(Xm[M], rs["vals"], rs["meta"], rs["scales"], rs["ts"], Y=Ys[M],
                                            prepare=True)
            calls[f"gemv_sp24_M{M}"].append(p)
            used[f"gemv_sp24_M{M}"] = u
            p, _ = ssn.gemm_nvfp4_sp24(Xm[M], rs["vals"], rs["meta"], rs["scales"], rs["ts"], Y=Ys[M],
                                       algo=ssn.ALGO_GATHER, prepare=True)
            calls[f"gemv_sp24_gather_M{M}"].append(p)
    B = Batches(torch)

    def steps(count):
        # `count` steps, call by call; step i uses ring slot i % RING
        for n in names:
            B.run(n, [calls[n][i % RING] for i in range(count)])

    steps(RING)                        # every ring slot holds valid weights
    torch.cuda.synchronize()
    steps(args.warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    steps(args.steps)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    for n in extra:
        B.run(n, [calls[n][i % RING] for i in range(2)])
        torch.cuda.synchronize()
        B.run(n, [calls[n][i % RING] for i in range(args.steps)])
    torch.cuda.synchronize()

    kb = {"quantize": bytes_quantize(N, K), "prune": bytes_prune(N, K), "quantize_pruned": bytes_quantize(N, K),
          "check": bytes_check(N, K), "compress": bytes_compress(N, K)}
    for M in Ms:
        kb[f"gemv_dense_M{M}"] = bytes_gemm(M, N, K, False, 4)
        kb[f"gemv_sp24_M{M}"] = bytes_gemm(M, N, K, True, 4)
    kernels = {}
    for name, b in kb.items():
        us = B.us(name)
        e = {"us": round(us, 2), "alg_bytes": b, "GBps": round(b / (us * 1e-6) / 1e9, 1),
             "hbm_frac": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
        if name.startswith("gemv"):
            M = int(name.split("_M")[1])
            flops = 2 * M * N * K
            e["tflops_dense_equiv"] = round(flops / (us * 1e-6) / 1e12, 3)
            if "sp24" in name:
                e["tflops_actual"] = round(flops / 2 / (us * 1e-6) / 1e12, 3)
            e["algo"] = ssn.ALGO_NAMES.get(used[name].value, "?")
        kernels[name] = e
    for M in Ms:
        kernels[f"gemv_sp24_M{M}"]["speedup_vs_dense"] = round(
            kernels[f"gemv_dense_M{M}"]["us"] / kernels[f"gemv_sp24_M{M}"]["us"], 3)
    step_bytes = sum(kb.values())
    pb = N * K * 4 + N * K // 4 + N * K // 8 + N * K // 16 + 4
    pus = B.us("producer_fused")
    chain = sum(kernels[n]["us"] for n in ("prune", "quantize_pruned", "check", "compress"))
    extras = {"producer_fused": {
        "us": round(pus, 2), "alg_bytes": pb, "GBps": round(pb / (pus * 1e-6) / 1e9, 1),
        "hbm_frac": round(pb / (pus * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "unfused_chain_us": round(chain, 2), "speedup_vs_unfused_chain": round(chain / pus, 3),
        "note": "nvfp4_sp24_produce: prune -> quantize -> check -> compress of W in one pass (bit-identical); "
                "not part of the step"}}
    for M in Ms:
        n = f"gemv_sp24_gather_M{M}"
        us = B.us(n)
        b = bytes_gemm(M, N, K, True, 4)
        extras[n] = {"us": round(us, 2), "alg_bytes": b, "GBps": round(b / (us * 1e-6) / 1e9, 1),
                     "hbm_frac": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4), "algo": "valu",
                     "smfmac_speedup_vs_gather": round(us / kernels[f"gemv_sp24_M{M}"]["us"], 3),
                     "note": "2:4 GEMV in the skip-and-gather form (x gathered at the stored positions, "
                             "vector ALU); not part of the step"}
    dominant = max(kernels, key=lambda k: kernels[k]["us"])
    dk = kernels[dominant]
    roof = {"kernel": dominant, "bound": "hbm", "achieved": dk["GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(dk["GBps"] / HBM_PEAK_GBPS, 4), "traffic": traffic_for(dominant)}
    result = {
        "value": round(step_bytes / (ms_step * 1e-3) / 1e9, 1), "unit": "GB/s", "ms_per_step": round(ms_step, 4),
        "dtype": "bf16",
        "config": {"workload": "decode: X bf16 [M in {1,4,8}, 5120] ~N(0,1); W f32 [13824, 5120] ~N(0,0.02); "
                               "NVFP4 dense and 2:4-pruned+compressed; quantize, prune, check, compress, 6 GEMVs",
                   "M": list(Ms), "N": N, "K": K, "weight_ring": RING, "step_alg_bytes": step_bytes},
        "roofline": roof, "kernels": kernels, "extra_kernels": extras,
    }
    return result, (w, x)


# ------------------------------------------------------------------------------------------
def _gpu_weights(ssn, W):
    """Dense and 2:4 NVFP4 forms of W (device float32) made on the GPU."""
    codes, scales, ts = ssn.nvfp4_quantize(W)
    Wp = ssn.sp24_prune(W)
    pc, ps, pts = ssn.nvfp4_quantize(Wp)
    vals, meta, _ = ssn.sp24_compress(pc)
    del Wp, pc
    return (codes, scales, ts), (vals, meta, ps, pts)


def run_gemm_shape(torch, ssn, synth, M, N, K, y_dtype, outliers, reps):
    x = synth.activations(M, K)
    w = synth.weight_rows_with_outliers(N, K, 0, N, 0.01, 20.0) if outliers else synth.weights(N, K)
    X = torch.from_numpy(x.view("int16")).view(torch.bfloat16).cuda()
    W = torch.from_numpy(w).cuda()
    del w, x
    dn, sp = _gpu_weights(ssn, W)
    del W
    Y = torch.empty((M, N), dtype=y_dtype, device="cuda")
    yb = 2 if y_dtype == torch.bfloat16 else 4
    # the skip-and-gather form (vector ALU, x gathered at the stored positions) is the plain
    # comparison point; it is far slower (about a second per prefill call), so it runs one or
    # two timed calls after as many warm-up calls
    variants = [("dense_mfma", False, ssn.ALGO_MFMA), ("sp24_smfmac", True, ssn.ALGO_SMFMAC),
                ("sp24_decompress_mfma", True, ssn.ALGO_DECOMPRESS_MFMA), ("sp24_gather_valu", True, ssn.ALGO_GATHER)]
    vreps = {"sp24_gather_valu": min(reps, 2 if 2.0 * M * N * K < 1e12 else 1)}
    B = Batches(torch)
    preps = {}
    for vname, sparse, algo in variants:
        if sparse:
            p, _ = ssn.gemm_nvfp4_sp24(X, sp[0], sp[1], sp[2], sp[3], y_dtype=y_dtype, algo=algo, Y=Y, prepare=True)
        else:
            p, _ = ssn.gemm_nvfp4_dense(X, dn[0], dn[1], dn[2], y_dtype=y_dtype, algo=algo, Y=Y, prepare=True)
        preps[vname] = p
    for vname in preps:                      # warm-up
        B.run(vname, [preps[vname]] * min(2, vreps.get(vname, 2)))
    torch.cuda.synchronize()
    for vname in preps:
        B.run(vname, [preps[vname]] * vreps.get(vname, reps))
    torch.cuda.synchronize()
    flops = 2.0 * M * N * K
    out = {"shape": {"M": M, "N": N, "K": K, "y": "bf16" if yb == 2 else "f32", "outliers": outliers},
           "flops_dense_equiv": flops}
    for vname, sparse, algo in variants:
        us = B.us(vname)
        b = bytes_gemm(M, N, K, sparse, yb)
        e = {"us": round(us, 1), "tflops_dense_equiv": round(flops / (us * 1e-6) / 1e12, 1),
             "alg_bytes": b, "GBps": round(b / (us * 1e-6) / 1e9, 1)}
        if sparse:
            e["tflops_actual"] = round(flops / 2 / (us * 1e-6) / 1e12, 1)
            e["mfma_frac_actual_vs_bf16_peak"] = round(e["tflops_actual"] / BF16_PEAK_TFLOPS, 4)
            if algo == ssn.ALGO_SMFMAC:
                e["mfma_frac_vs_sparse_peak"] = round(e["tflops_dense_equiv"] / SPARSE_BF16_PEAK_TFLOPS, 4)
            if algo == ssn.ALGO_GATHER:
                e["valu_frac_actual_vs_fp32_peak"] = round(e["tflops_actual"] / FP32_VECTOR_PEAK_TFLOPS, 4)
                e["timed_calls"] = vreps["sp24_gather_valu"]
        else:
            e["mfma_frac"] = round(e["tflops_dense_equiv"] / BF16_PEAK_TFLOPS, 4)
        out[vname] = e
    for vname in ("sp24_smfmac", "sp24_decompress_mfma", "sp24_gather_valu"):
        out[vname]["speedup_vs_dense"] = round(out["dense_mfma"]["us"] / out[vname]["us"], 3)
    del X, Y, dn, sp, preps
    torch.cuda.empty_cache()
    return out


HEAD_N, HEAD_K, HEAD_MS = 131072, 5120, (1, 8, 9)


def run_head(torch, ssn, synth, reps):
    """Output-head-shaped GEMV (vocabulary-sized N = 131072, K = 5120; M = 1, and 8 and 9 rows as
    in speculative verification): weights of 377 MB (dense) / 294 MB (2:4), larger than the
    Infinity Cache; two weight copies alternate so every call reads HBM."""
    N, K = HEAD_N, HEAD_K
    x = synth.activations(max(HEAD_MS), K)
    X = torch.from_numpy(x.view("int16")).view(torch.bfloat16).cuda()
    W = torch.from_numpy(synth.weights(N, K)).cuda()
    dn, sp = _gpu_weights(ssn, W)
    del W
    torch.cuda.empty_cache()
    dns = [dn, tuple(t.clone() for t in dn)]
    sps = [sp, tuple(t.clone() for t in sp)]
    out = {"shape": {"N": N, "K": K, "M": list(HEAD_MS), "y": "f32"}, "weight_copies": 2}
    for M in HEAD_MS:
        Xm = X[:M].contiguous()
        Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        pd, ps, used = [], [], {}
        for d, s_ in zip(dns, sps):
            p, (_, ud) = ssn.gemm_nvfp4_dense(Xm, d[0], d[1], d[2], Y=Y, prepare=True)
            pd.append(p)
            p, (_, us_) = ssn.gemm_nvfp4_sp24(Xm, s_[0], s_[1], s_[2], s_[3], Y=Y, prepare=True)
            ps.append(p)
            used = {"dense": ud, "sp24": us_}
        B = Batches(torch)
        for n, calls in (("dense", pd), ("sp24", ps)):
            B.run(n, calls)
        torch.cuda.synchronize()
        for n, calls in (("dense", pd), ("sp24", ps)):
            B.run(n, calls * reps)
        torch.cuda.synchronize()
        e = {}
        for n in ("dense", "sp24"):
            us = B.us(n)
            b = bytes_gemm(M, N, K, n == "sp24", 4)
            e[n] = {"us": round(us, 1), "alg_bytes": b, "GBps": round(b / (us * 1e-6) / 1e9, 1),
                    "hbm_frac": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                    "tflops_dense_equiv": round(2.0 * M * N * K / (us * 1e-6) / 1e12, 2),
                    "algo": ssn.ALGO_NAMES.get(used[n].value, "?")}
        e["sp24"]["speedup_vs_dense"] = round(e["dense"]["us"] / e["sp24"]["us"], 3)
        out[f"M{M}"] = e
    del dns, sps, dn, sp, X
    torch.cuda.empty_cache()
    return out


def run_moe(torch, ssn, synth, reps):
    import numpy as np
    T, E, k, D, I = 4096, 512, 10, 2048, 512
    ids, wts = synth.routing(T, E, k, 1.1)
    x = synth.activations(T, D)
    X = torch.from_numpy(x.view("int16")).view(torch.bfloat16).cuda()
    dids, dw = torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda()
    g = torch.Generator(device="cuda")
    g.manual_seed(0)

    def build(rows, cols, sparse):
        c = torch.empty((E, rows, cols // (4 if sparse else 2)), dtype=torch.uint8, device="cuda")
        m = torch.empty((E, rows, cols // 8), dtype=torch.uint8, device="cuda") if sparse else None
        s = torch.empty((E, rows, cols // 16), dtype=torch.uint8, device="cuda")
        ts = torch.empty(E, dtype=torch.float32, device="cuda")
        for e in range(E):
            Wf = torch.randn(rows, cols, device="cuda", generator=g) * 0.02
            if sparse:
                Wf = ssn.sp24_prune(Wf)
                codes, _, _ = ssn.nvfp4_quantize(Wf, scales=s[e], tensor_scale_out=ts[e:e + 1])
                ssn.sp24_compress(codes, vals=c[e], meta=m[e])
            else:
                ssn.nvfp4_quantize(Wf, codes=c[e], scales=s[e], tensor_scale_out=ts[e:e + 1])
        return c, m, s, ts

    R = T * k
    flops = 2.0 * R * D * 2 * I + 2.0 * R * I * D
    counts = np.bincount(ids.ravel(), minlength=E)
    out = {"shape": {"T": T, "E": E, "top_k": k, "D": D, "I": I, "rows": R, "zipf_s": 1.1,
                     "experts_touched": int((counts > 0).sum()), "max_rows": int(counts.max()),
                     "median_rows": float(np.median(counts))},
           "flops_dense_equiv": flops,
           "note": "expert weights ~N(0, 0.02) drawn on the GPU (torch generator, seed 0); routing and X from the "
                   "seeded synthetic generators"}
    for sparse in (False, True):
        up_rows, down_rows = build(2 * I, D, sparse), build(D, I, sparse)
        # weight preparation, once: the 64-k tiled layout of the grouped products
        up, down = ssn.moe_pack_weights(up_rows), ssn.moe_pack_weights(down_rows)
        kt = ssn.WLAYOUT_KTILE64
        H = torch.empty((R, I), dtype=torch.bfloat16, device="cuda")
        Yd = torch.empty((R, D), dtype=torch.float32, device="cuda")
        off, rt, rs, ro, bad = ssn.moe_route(dids, E)
        p_route, _ = ssn.moe_route(dids, E, prepare=True)
        p_up, _ = ssn.moe_grouped_gemm_nvfp4(X, rt, off, R, up[0], up[2], up[3], w_meta=up[1],
                                             epilogue=ssn.EPI_SILU_GATE, y_dtype=torch.bfloat16, Y=H, prepare=True,
                                             w_layout=kt)
        p_down, _ = ssn.moe_grouped_gemm_nvfp4(H, None, off, R, down[0], down[2], down[3], w_meta=down[1], Y=Yd,
                                               prepare=True, w_layout=kt)
        p_comb, _ = ssn.moe_combine(Yd, ro, dw, prepare=True)
        p_ffn, _ = ssn.moe_nvfp4_ffn(X, dids, dw, E, up, down, prepare=True, w_layout=kt)
        p_ffn_rows, _ = ssn.moe_nvfp4_ffn(X, dids, dw, E, up_rows, down_rows, prepare=True)
        B = Batches(torch)
        stages = [("route", p_route), ("up_silu_gate", p_up), ("down", p_down), ("combine", p_comb), ("ffn", p_ffn),
                  ("ffn_row_layout", p_ffn_rows)]
        for n, p in stages:
            B.run(n, [p] * 2)
        torch.cuda.synchronize()
        for n, p in stages:
            B.run(n, [p] * reps)
        torch.cuda.synchronize()
        wbytes = sum(t.numel() for t in (up[0], up[1], up[2], down[0], down[1], down[2]) if t is not None)
        ffn_bytes = wbytes + T * D * 2 + 2 * R * I * 2 + T * D * 4
        res = {n: {"us": round(B.us(n), 1)} for n, _ in stages}
        us = res["ffn"]["us"]
        t_roof = max(flops / (2 if sparse else 1) / (BF16_PEAK_TFLOPS * 1e12), ffn_bytes / (HBM_PEAK_GBPS * 1e9))
        res["ffn"].update({"weight_layout": "ktile64", "weight_bytes": wbytes, "alg_bytes": ffn_bytes,
                           "tflops_dense_equiv": round(flops / (us * 1e-6) / 1e12, 1),
                           "GBps_alg": round(ffn_bytes / (us * 1e-6) / 1e9, 1),
                           "t_roof_us": round(t_roof * 1e6, 1), "frac_of_t_roof": round(t_roof / (us * 1e-6), 4)})
        out["sp24" if sparse else "dense"] = res
        del H, Yd, up_rows, down_rows
        torch.cuda.empty_cache()
        out["decode_" + ("sp24" if sparse else "dense")] = run_moe_decode(torch, ssn, synth, x, up, down, sparse,
                                                                          E, k, D, I)
        del up, down
        torch.cuda.empty_cache()
    out["sp24"]["ffn"]["speedup_vs_dense"] = round(out["dense"]["ffn"]["us"] / out["sp24"]["ffn"]["us"], 3)
    for T in MOE_DECODE_TOKENS:
        d, s_ = out["decode_dense"][f"T{T}"], out["decode_sp24"][f"T{T}"]
        s_["ffn_speedup_vs_dense"] = round(d["ffn_us"] / s_["ffn_us"], 3)
    return out


MOE_DECODE_TOKENS = (1, 4, 16, 32)
MOE_RING = 20      # weight copies x routings rotated (20 x 17.7 MB at one token > the 256 MB cache)


def run_moe_decode(torch, ssn, synth, x, up, down, sparse, E, k, D, I):
    """Decode-sized routings (1..32 tokens) on the full expert set: every call reads the touched
    experts' weights. Calls rotate over MOE_RING weight copies and as many routing draws, so
    the weights come from HBM, not from the Infinity Cache of an earlier call."""
    import numpy as np
    ups = [up] + [tuple(t.clone() if t is not None else None for t in up) for _ in range(MOE_RING - 1)]
    downs = [down] + [tuple(t.clone() if t is not None else None for t in down) for _ in range(MOE_RING - 1)]
    kt = ssn.WLAYOUT_KTILE64
    per_expert = sum(t[0].numel() for t in (up[0], up[2], down[0], down[2])) + \
        (sum(t[0].numel() for t in (up[1], down[1])) if sparse else 0)
    res = {"weight_copies": MOE_RING, "weight_layout": "ktile64",
           "note": "stages timed over back-to-back calls, each on its own weight copy and routing draw (seeds "
                   "100..119)"}
    tiles = ssn.ALGO_DECOMPRESS_MFMA if sparse else ssn.ALGO_MFMA
    for T in MOE_DECODE_TOKENS:
        R = T * k
        X = torch.from_numpy(x[:T].view("int16")).view(torch.bfloat16).cuda()
        stages = {n: [] for n in ("route", "up", "down", "combine", "ffn", "up_tiles", "down_tiles")}
        touched, used = [], []
        for j in range(MOE_RING):
            ids, wts = synth.routing(T, E, k, 1.1, seed=100 + j)
            touched.append(len(np.unique(ids)))
            dids, dw = torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda()
            u, d = ups[j], downs[j]
            off, rt, rs, ro, bad = ssn.moe_route(dids, E)
            H = torch.empty((R, I), dtype=torch.bfloat16, device="cuda")
            Yd = torch.empty((R, D), dtype=torch.float32, device="cuda")
            stages["route"].append(ssn.moe_route(dids, E, prepare=True)[0])
            p, (_, a) = ssn.moe_grouped_gemm_nvfp4(X, rt, off, R, u[0], u[2], u[3], w_meta=u[1],
                                                   epilogue=ssn.EPI_SILU_GATE, y_dtype=torch.bfloat16, Y=H,
                                                   prepare=True, w_layout=kt)
            stages["up"].append(p)
            used.append(a)
            p, (_, a) = ssn.moe_grouped_gemm_nvfp4(H, None, off, R, d[0], d[2], d[3], w_meta=d[1], Y=Yd, prepare=True,
                                                   w_layout=kt)
            stages["down"].append(p)
            used.append(a)
            stages["combine"].append(ssn.moe_combine(Yd, ro, dw, prepare=True)[0])
            stages["ffn"].append(ssn.moe_nvfp4_ffn(X, dids, dw, E, u, d, prepare=True, w_layout=kt)[0])
            stages["up_tiles"].append(ssn.moe_grouped_gemm_nvfp4(
                X, rt, off, R, u[0], u[2], u[3], w_meta=u[1], epilogue=ssn.EPI_SILU_GATE, y_dtype=torch.bfloat16,
                Y=torch.empty_like(H), prepare=True, w_layout=kt, algo=tiles)[0])
            stages["down_tiles"].append(ssn.moe_grouped_gemm_nvfp4(
                H, None, off, R, d[0], d[2], d[3], w_meta=d[1], Y=torch.empty_like(Yd), prepare=True, w_layout=kt,
                algo=tiles)[0])
        B = Batches(torch)
        for n, ps in stages.items():
            B.run(n, ps)
        torch.cuda.synchronize()
        for n, ps in stages.items():
            B.run(n, ps + ps)
        torch.cuda.synchronize()
        t = {n: B.us(n) for n in stages}
        wb = float(np.mean(touched)) * per_expert
        e = {"tokens": T, "rows": R, "experts_touched_mean": round(float(np.mean(touched)), 1),
             "weight_bytes_touched": int(wb), "algo": "+".join(sorted({ssn.ALGO_NAMES.get(a.value, "?") for a in used})),
             "route_us": round(t["route"], 1), "up_us": round(t["up"], 1), "down_us": round(t["down"], 1),
             "combine_us": round(t["combine"], 1), "ffn_us": round(t["ffn"], 1),
             "up_tiles_us": round(t["up_tiles"], 1), "down_tiles_us": round(t["down_tiles"], 1),
             "GBps_up_down": round(wb / ((t["up"] + t["down"]) * 1e-6) / 1e9, 1),
             "GBps_ffn": round(wb / (t["ffn"] * 1e-6) / 1e9, 1)}
        e["hbm_frac_up_down"] = round(e["GBps_up_down"] / HBM_PEAK_GBPS, 4)
        e["stream_speedup_vs_tiles"] = round((t["up_tiles"] + t["down_tiles"]) / (t["up"] + t["down"]), 3)
        res[f"T{T}"] = e
    del ups, downs
    return res


# ------------------------------------------------------------------------------------------
def cpu_baseline_decode(w, x, rows):
    """The oracle (unchanged) on the host: the decode step's calls over a sample of weight rows."""
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
         + sum(bytes_gemm(M, rows, K, False, 4) + bytes_gemm(M, rows, K, True, 4) for M in (1, 4, 8)))
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
    wl = set(args.workloads.split(","))
    hbm = hbm_probe(torch, ssn)
    print(f"[bench] hbm probe {hbm}", file=sys.stderr, flush=True)
    res, (w, x) = run_decode(args, torch, ssn, synth)
    print(f"[bench] decode done: {res['ms_per_step']} ms/step", file=sys.stderr, flush=True)
    out = {"metric": METRIC, "value": res["value"], "unit": res["unit"], "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": res["ms_per_step"], "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": res["dtype"], "data": "synthetic", "config": res["config"],
           "roofline": res["roofline"], "hbm_measured": hbm, "mfma_peak_bf16_TFLOPs": BF16_PEAK_TFLOPS,
           "kernels": res["kernels"], "extra_kernels": res["extra_kernels"]}
    work = {}
    if "square" in wl:
        work["square"] = run_gemm_shape(torch, ssn, synth, 4096, 4096, 4096, torch.float32, False, 10)
        print("[bench] square done", file=sys.stderr, flush=True)
    if "prefill" in wl:
        work["prefill"] = run_gemm_shape(torch, ssn, synth, 8192, 27648, 5120, torch.bfloat16, True, 5)
        print("[bench] prefill done", file=sys.stderr, flush=True)
    if "head" in wl:
        work["head"] = run_head(torch, ssn, synth, 10)
        print("[bench] head done", file=sys.stderr, flush=True)
    if "moe" in wl:
        work["moe"] = run_moe(torch, ssn, synth, 5)
        print("[bench] moe done", file=sys.stderr, flush=True)
    out["workloads"] = work
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_decode(w, x, args.cpu_rows)
        print("[bench] cpu baseline done", file=sys.stderr, flush=True)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
