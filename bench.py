"""Benchmark of the NVFP4 / 2:4 weight-GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads decode,square,head,moe,w4a4,refs]

Prints ONE JSON line. The headline (``value``, ``ms_per_step``, ``roofline``) is the prefill
product, the largest of the workloads: X bf16 [8192, 5120] ~ N(0, 1) times dense NVFP4 weights
W [27648, 5120] (~ N(0, 0.02) with 1% of the entries x20 before quantisation), f32 accumulation,
bf16 output, on the matrix cores (gemm_nvfp4_dense, 256 x 256 tiles). One step is one such
product; ``value`` is its dense TFLOP/s (2 M N K per step over the host-clocked step time, K
steps back to back between two synchronisations, inputs resident in HBM). ``roofline`` is
that kernel's TFLOP/s from HIP events on its launch stream (average launch duration over the
timed steps) against the published 2.5 PFLOP/s bf16 matrix peak. The 2:4 forms of the same
product (sparse matrix cores, expanded-to-dense, skip-and-gather) are timed beside it with
their speedup over dense.

Before any timing, every workload checks sampled outputs against the CPU oracle and stops if
one is outside its bound. Each compute-bound workload records the GPU clock, power and
temperature while it runs. Per kernel the bench reports the average over back-to-back launches
(HIP events around the batch) and the median and minimum of at least 20 individually timed
launches.

``workloads`` adds: ``decode`` (the GEMVs at N = 13824, K = 5120, M = 1, 4, 8 on a ring of 16
weight copies, and the weight-preparation calls on three rotating copies of W, each against
8 TB/s and the measured copy bandwidth), ``square`` (4096^3, f32 out), ``head`` (N = 131072,
K = 5120, M = 1, 8, 9), ``moe`` (512 experts, top-10 of Zipf(1.1), D = 2048, I = 512: 4096
tokens stage by stage, and 1-32 tokens on the weight-streaming kernels), ``w4a4`` (the W4A4
variant at the prefill and square shapes: activations quantised to MXFP4 in every step, the FP4 x
FP4 product on the block-scaled matrix cores, against the 10.1 PFLOP/s FP4 peak), ``refs``
(comparison points: the vendor bf16 GEMM at the prefill and square shapes, and a plain streaming
read at the decode GEMV's size).
``cpu_baseline`` is the oracle's dense prefill product on the host cores.

    python bench.py --summarize KIND OUT DIR...

turns rocprofv3 output directories into the text summaries kept under profiles/ (KIND: trace
for --kernel-trace --stats runs; pmc for --pmc runs).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4 GEMM TFLOP/s & HBM GB/s, 2:4 vs dense, % of MI355X roofline"
HBM_PEAK_GBPS = 8000.0            # MI355X published HBM3E bandwidth
BF16_PEAK_TFLOPS = 2500.0         # MI355X published dense bf16 matrix peak
SPARSE_BF16_PEAK_TFLOPS = 5000.0  # the same with 2:4 structured sparsity (dense-equivalent)
FP4_PEAK_TFLOPS = 10100.0         # MI355X published dense fp4 matrix peak
FP32_VECTOR_PEAK_TFLOPS = 157.3   # MI355X published fp32 vector peak
RING = 16                         # weight copies rotated by the GEMVs (16 x 40 MB > 2 x 256 MB cache)
W_COPIES = 3                      # copies of the 283 MB f32 W rotated by the weight-preparation calls
TRIALS = 20                       # individually timed launches per kernel (median, min)
ROUNDS = 5                        # alternated batches of products compared with each other
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "structured_sparse_nvfp4_amd", "csrc")
PREFILL = dict(M=8192, N=27648, K=5120)
DENSE_TILE_KERNEL = "k_gemm_mfma<0, true>"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workloads", default="decode,square,head,moe,w4a4,refs",
                   help="comma list of workloads beside the prefill headline (which always runs)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--summarize", nargs="+", metavar="ARG",
                   help="KIND OUT DIR...: summarise rocprofv3 output (KIND trace or pmc) into OUT")
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


# ------------------------------------------------------------------------------------------
class Timer:
    """HIP events on the current stream (the stream the library's calls launch on): the average
    over a batch of back-to-back launches (or the median of alternated batches), and individually
    timed launches."""

    def __init__(self, torch):
        self.torch = torch
        self.batches = {}
        self.trials = {}
        self.rounded = {}

    def _ev(self):
        return self.torch.cuda.Event(enable_timing=True)

    def batch(self, name, fns):
        a, b = self._ev(), self._ev()
        a.record()
        for f in fns:
            f()
        b.record()
        self.batches[name] = (a, b, len(fns))

    def each(self, name, fns):
        evs = []
        for f in fns:
            a, b = self._ev(), self._ev()
            a.record()
            f()
            b.record()
            evs.append((a, b))
        self.trials[name] = evs

    def rounds(self, groups, n_rounds):
        """Batches of several named call lists alternated round by round (A B A B ...), so that
        clock and power drift between them falls on each alike; us() then gives the median
        round."""
        for _ in range(n_rounds):
            for name, fns in groups:
                a, b = self._ev(), self._ev()
                a.record()
                for f in fns:
                    f()
                b.record()
                self.rounded.setdefault(name, []).append((a, b, len(fns)))

    def us(self, name):
        if name in self.rounded:
            return statistics.median(a.elapsed_time(b) * 1e3 / n for a, b, n in self.rounded[name])
        a, b, n = self.batches[name]
        return a.elapsed_time(b) * 1e3 / n

    def stats(self, name):
        ts = sorted(a.elapsed_time(b) * 1e3 for a, b in self.trials[name])
        return {"median_us": round(statistics.median(ts), 2), "min_us": round(ts[0], 2), "trials": len(ts)}


def _hwmon_read(path, scale):
    try:
        with open(path) as f:
            return round(int(f.read().strip()) / scale, 1)
    except (OSError, ValueError):
        return None


def gpu_state():
    """Current GPU clock, power and temperatures from sysfs (pp_dpm_sclk and the amdgpu hwmon
    files), best effort. No tool is started: a child process of a program that has initialised
    the GPU must not exec another program."""
    out = {}
    v = _sclk_now()
    if v is not None:
        out["sclk_MHz"] = v
    v = _dpm_now("mclk")
    if v is not None:
        out["mclk_MHz"] = v
    for hw in sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*")):
        for name, key in (("power1_average", "power_W"), ("power1_input", "power_W")):
            if key not in out:
                w = _hwmon_read(os.path.join(hw, name), 1e6)
                if w is not None:
                    out[key] = w
        for t in sorted(glob.glob(os.path.join(hw, "temp*_input"))):
            try:
                with open(t.replace("_input", "_label")) as f:
                    label = f.read().strip().lower()
            except OSError:
                label = os.path.basename(t).split("_")[0]
            c = _hwmon_read(t, 1e3)
            if c is not None:
                out[f"temp_{label}_C"] = c
        if out.get("power_W") is not None:
            break
    return out


def _dpm_now(kind="sclk"):
    """Current level (MHz) of a pp_dpm_* clock table in sysfs (the line marked '*')."""
    try:
        for f in glob.glob(f"/sys/class/drm/card*/device/pp_dpm_{kind}"):
            for line in open(f):
                if line.startswith("S:") or line.rstrip().endswith("*"):
                    return int(line.split(":")[1].strip().split("M")[0])
    except (OSError, ValueError, IndexError):
        pass
    return None


def _sclk_now():
    return _dpm_now("sclk")


def state_under_load(torch, fn, seconds=3.0):
    """GPU state while `fn` launches keep the GPU busy for about `seconds`: the clock (sysfs)
    sampled five times, then one reading of power and temperatures (sysfs), all taken while the
    queued launches still run (`still_running` says whether they did); plus idle readings
    before and after."""
    before = gpu_state()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(); fn(); b.record(); b.synchronize()
    # at most 5000 launches (under a profiler every launch is slow), so short kernels queue less
    # than `seconds` of work: the clock is sampled early and over a short window
    n = min(5000, max(1, int(seconds / max(a.elapsed_time(b) * 1e-3, 1e-5))))
    done = torch.cuda.Event()
    for _ in range(n):
        fn()
    done.record()
    time.sleep(0.2)
    sclk = []
    for _ in range(5):
        v = _sclk_now()
        if v is not None:
            sclk.append(v)
        time.sleep(0.05)
    during = gpu_state()
    during["sclk_samples_MHz"] = sclk
    during["still_running"] = not done.query()
    torch.cuda.synchronize()
    return {"before": before, "during": during, "after": gpu_state()}


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
    T = Timer(torch)
    res = {}
    for name, fn, nbytes in (("copy", lambda: dst.copy_(src), 2 * n), ("read", lambda: ssn.sp24_check(codes), n)):
        T.each(name, [fn] * TRIALS)
        torch.cuda.synchronize()
        res[f"{name}_GBps"] = round(nbytes / (T.stats(name)["median_us"] * 1e-6) / 1e9, 1)
    del src, dst, codes
    torch.cuda.empty_cache()
    return res


HOST_ONLY_HEADERS = {"launch.hpp", "device_once.hpp"}   # launcher declarations and host set-up


def _source_hash(kernel_file):
    """SHA-256 of a kernel's source file and of the device headers it includes (headers that
    hold only host-side declarations are left out)."""
    import re
    h = hashlib.sha256()
    path = os.path.join(CSRC, kernel_file)
    with open(path, "rb") as fh:
        text = fh.read()
    h.update(text)
    for inc in sorted(set(re.findall(rb'#include "([\w.]+\.hpp)"', text))):
        if inc.decode() in HOST_ONLY_HEADERS:
            continue
        with open(os.path.join(CSRC, inc.decode()), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_for(key):
    """HBM bytes per launch from the committed counter summary, only while the kernel's sources
    are unchanged since the counters were taken (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f).get(key)
        if not t or _source_hash(t["source"]) != t["source_sha256"]:
            return None
        return int(t["fetch_bytes"] + t["write_bytes"])
    except (OSError, KeyError, ValueError):
        return None


def _bw(b, us, copy_gbps):
    gbps = b / (us * 1e-6) / 1e9
    return {"alg_bytes": b, "GBps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
            "copy_frac": round(gbps / copy_gbps, 4) if copy_gbps else None}


# ------------------------------------------------------------------------------------------
# parity before timing
class ParityError(AssertionError):
    pass


def _assert_bound(got, ref, base, out, what):
    from oracle import gemm
    import numpy as np
    tol = gemm.bound(base, ref, out)
    err = np.abs(got - ref)
    if not np.all(err <= tol):
        i = tuple(np.argwhere(~(err <= tol))[0])
        raise ParityError(f"{what}: outside the parity bound at {i}: gpu={got[i]!r} oracle={ref[i]!r} tol={tol[i]!r}")


def _rows_of(t, rows, cols=None):
    import numpy as np
    torch = sys.modules["torch"]
    sel = t[torch.from_numpy(np.asarray(rows)).to(t.device)]
    if cols is not None:
        sel = sel[:, torch.from_numpy(np.asarray(cols)).to(t.device)]
    return sel.float().cpu().numpy().astype(np.float64)


def check_product(x, w, st, ms, ns, y_dense, y_sp24, out, what):
    """Sampled outputs of the dense and 2:4 products against the oracle (weights of the sampled
    columns quantised by the oracle with the tensor scale of the whole W). y_dense / y_sp24 hold
    the full outputs (sampled here at ms x ns)."""
    from oracle import gemm, quant, sp24
    c, s, _ = quant.quantize(w[ns], tensor_scale_in=st)
    Y, B = gemm.gemm_dense(x[ms], c, s, st)
    _assert_bound(_rows_of(y_dense, ms, ns), Y, B, out, f"{what} dense")
    if y_sp24:
        pc, ps, _ = quant.quantize(sp24.prune24(w[ns]), tensor_scale_in=st)
        v, m, nb = sp24.compress(pc)
        Y, B = gemm.gemm_sp24(x[ms], v, m, ps, st)
        for name, y in y_sp24.items():
            _assert_bound(_rows_of(y, ms, ns), Y, B, out, f"{what} 2:4 {name}")


# ------------------------------------------------------------------------------------------
def _gpu_weights(ssn, W):
    """Dense and 2:4 NVFP4 forms of W (device float32) made on the GPU."""
    codes, scales, ts = ssn.nvfp4_quantize(W)
    Wp = ssn.sp24_prune(W)
    pc, ps, pts = ssn.nvfp4_quantize(Wp)
    vals, meta, _ = ssn.sp24_compress(pc)
    del Wp, pc
    return (codes, scales, ts), (vals, meta, ps, pts)


def _gemm_variants(ssn):
    return [("dense_mfma", False, ssn.ALGO_MFMA), ("sp24_smfmac", True, ssn.ALGO_SMFMAC),
            ("sp24_decompress_mfma", True, ssn.ALGO_DECOMPRESS_MFMA), ("sp24_gather_valu", True, ssn.ALGO_GATHER)]


def run_gemm_shape(torch, ssn, synth, M, N, K, y_dtype, outliers, args, headline=False):
    """Dense and 2:4 products of one shape. With ``headline`` the dense product is also timed as
    the bench's steps (K steps after W warm-up steps, host clock and HIP events)."""
    from oracle import quant
    x = synth.activations(M, K)
    w = synth.weight_rows_with_outliers(N, K, 0, N, 0.01, 20.0) if outliers else synth.weights(N, K)
    st = quant.tensor_scale(w)
    X = torch.from_numpy(x.view("int16")).view(torch.bfloat16).cuda()
    W = torch.from_numpy(w).cuda()
    dn, sp = _gpu_weights(ssn, W)
    del W
    torch.cuda.synchronize()
    if float(dn[2].item()) != float(st) or float(sp[3].item()) != float(st):
        raise ParityError("tensor scale differs from the oracle's")
    out = "bf16" if y_dtype == torch.bfloat16 else "f32"
    yb = 2 if out == "bf16" else 4
    variants = _gemm_variants(ssn)
    Ys = {v: torch.empty((M, N), dtype=y_dtype, device="cuda") for v, _, _ in variants}
    preps, used = {}, {}
    for vname, sparse, algo in variants:
        if sparse:
            p, (_, u) = ssn.gemm_nvfp4_sp24(X, sp[0], sp[1], sp[2], sp[3], y_dtype=y_dtype, algo=algo, Y=Ys[vname],
                                            prepare=True)
        else:
            p, (_, u) = ssn.gemm_nvfp4_dense(X, dn[0], dn[1], dn[2], y_dtype=y_dtype, algo=algo, Y=Ys[vname],
                                             prepare=True)
        preps[vname], used[vname] = p, u
    for vname in preps:                       # one call each, then the parity check on their outputs
        preps[vname]()
    torch.cuda.synchronize()
    ms = sorted({0, 1, 255, 256, M // 2 + 3, M - 1})
    ns = sorted({0, 1, 255, 256, N // 2 + 5, N - 1})
    check_product(x, w, st, ms, ns, Ys["dense_mfma"], {v: Ys[v] for v, s_, _ in variants if s_}, out,
                  f"{M}x{N}x{K}")
    del w
    flops = 2.0 * M * N * K
    res = {"shape": {"M": M, "N": N, "K": K, "y": out, "outliers": outliers}, "flops_dense_equiv": flops,
           "parity": "sampled outputs of every variant within the oracle's bound"}
    T = Timer(torch)
    step = None
    if headline:
        dense = preps["dense_mfma"]
        t_w = time.perf_counter()            # the clock ramps up from idle: warm up for at least 0.5 s
        while time.perf_counter() - t_w < 0.5:
            dense()
            torch.cuda.synchronize()
        for _ in range(args.warmup):
            dense()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        T.batch("steps", [dense] * args.steps)
        torch.cuda.synchronize()
        ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
        step = {"ms_per_step": ms_step, "event_us": T.us("steps")}
    # one timed batch and TRIALS individually timed calls per variant; the skip-and-gather form
    # takes about a second per prefill call, so it gets fewer
    slow = {"sp24_gather_valu": 3 if flops > 1e12 else 5}
    for vname in preps:
        reps = slow.get(vname, TRIALS)
        T.batch(vname + "_warm", [preps[vname]] * min(2, reps))
        torch.cuda.synchronize()
        T.batch(vname, [preps[vname]] * reps)
        T.each(vname, [preps[vname]] * reps)
        torch.cuda.synchronize()
    res["gpu_state"] = state_under_load(torch, preps["dense_mfma"])
    sc = res["gpu_state"]["during"].get("sclk_samples_MHz") or []
    if sc:   # the published peak is at 2.4 GHz; the same matrix rate at the clock measured under load
        mhz = sorted(sc)[len(sc) // 2]
        res["bf16_peak_at_measured_sclk_tflops"] = round(BF16_PEAK_TFLOPS * mhz / 2400.0, 1)
    for vname, sparse, algo in variants:
        us = T.us(vname)
        e = {"us": round(us, 1), **T.stats(vname), "algo": ssn.ALGO_NAMES.get(used[vname].value, "?"),
             "tflops_dense_equiv": round(flops / (us * 1e-6) / 1e12, 1),
             "alg_bytes": bytes_gemm(M, N, K, sparse, yb),
             "GBps": round(bytes_gemm(M, N, K, sparse, yb) / (us * 1e-6) / 1e9, 1)}
        if sparse:
            e["tflops_actual"] = round(flops / 2 / (us * 1e-6) / 1e12, 1)
            e["mfma_frac_actual_vs_bf16_peak"] = round(e["tflops_actual"] / BF16_PEAK_TFLOPS, 4)
            if algo == ssn.ALGO_SMFMAC:
                e["mfma_frac_vs_sparse_peak"] = round(e["tflops_dense_equiv"] / SPARSE_BF16_PEAK_TFLOPS, 4)
            if algo == ssn.ALGO_GATHER:
                e["valu_frac_actual_vs_fp32_peak"] = round(e["tflops_actual"] / FP32_VECTOR_PEAK_TFLOPS, 4)
        else:
            e["mfma_frac"] = round(e["tflops_dense_equiv"] / BF16_PEAK_TFLOPS, 4)
        res[vname] = e
    for vname in ("sp24_smfmac", "sp24_decompress_mfma", "sp24_gather_valu"):
        res[vname]["speedup_vs_dense"] = round(res["dense_mfma"]["us"] / res[vname]["us"], 3)
    if headline:
        del Ys, sp, preps
        res["k_sweep"] = k_sweep(torch, ssn, X, dn, y_dtype)
    torch.cuda.empty_cache()
    return res, step, x


def k_sweep(torch, ssn, X, dn, y_dtype, ks=(1024, 2048, 3072, 5120)):
    """The dense tile on the first k columns of the same activations and weights, for several k:
    a least-squares line through the launch times splits each launch into a part proportional
    to K (the tile's main loop) and a fixed part (tile start, output write). Timing only: the
    products are sub-products of the one checked above."""
    M, K = X.shape
    N = dn[0].shape[0]
    pts = []
    for k in ks:
        if k > K or k % 64:
            continue
        Xk = X[:, :k].contiguous()
        ck, sk = dn[0][:, :k // 2].contiguous(), dn[1][:, :k // 16].contiguous()
        Y = torch.empty((M, N), dtype=y_dtype, device="cuda")
        p, _ = ssn.gemm_nvfp4_dense(Xk, ck, sk, dn[2], y_dtype=y_dtype, algo=ssn.ALGO_MFMA, Y=Y, prepare=True)
        T = Timer(torch)
        T.batch("warm", [p] * 2)
        torch.cuda.synchronize()
        T.batch("k", [p] * TRIALS)
        torch.cuda.synchronize()
        pts.append((k, T.us("k")))
        del Xk, ck, sk, Y, p
    n = len(pts)
    mk = sum(k for k, _ in pts) / n
    mt = sum(t for _, t in pts) / n
    slope = sum((k - mk) * (t - mt) for k, t in pts) / sum((k - mk) ** 2 for k, _ in pts)
    fixed = mt - slope * mk
    torch.cuda.empty_cache()
    return {"points_us": {str(k): round(t, 1) for k, t in pts}, "us_per_k": round(slope, 4),
            "fixed_us": round(fixed, 1), "k_part_tflops": round(2.0 * M * N / (slope * 1e-6) / 1e12, 1),
            "note": f"dense tile at M = {M}, N = {N} on the first k columns; launch time = fixed + us_per_k * K"}


# ------------------------------------------------------------------------------------------
def run_decode(torch, ssn, synth, copy_gbps):
    """Decode GEMVs (N = 13824, K = 5120, M = 1, 4, 8) on a ring of weight copies, and the weight
    preparation calls on rotating copies of W (each call reads a W last read two calls before,
    with 566 MB read in between, more than the 256 MB Infinity Cache)."""
    import numpy as np
    from oracle import gemm, quant, sp24
    N, K, Ms = 13824, 5120, (1, 4, 8)
    x = synth.activations(max(Ms), K)
    w = synth.weights(N, K)
    st = quant.tensor_scale(w)
    X = torch.from_numpy(x.view("int16")).view(torch.bfloat16).cuda()
    Ws = [torch.from_numpy(w).cuda()]
    for _ in range(W_COPIES - 1):
        Ws.append(Ws[0].clone())
    u8 = dict(dtype=torch.uint8, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    i64 = dict(dtype=torch.int64, device="cuda")
    dense = [dict(codes=torch.empty((N, K // 2), **u8), scales=torch.empty((N, K // 16), **u8), ts=torch.empty(1, **f32))
             for _ in range(RING)]
    sparse = [dict(codes=torch.empty((N, K // 2), **u8), scales=torch.empty((N, K // 16), **u8),
                   ts=torch.empty(1, **f32), vals=torch.empty((N, K // 4), **u8), meta=torch.empty((N, K // 8), **u8),
                   bad=torch.empty(1, **i64), first=torch.empty(1, **i64)) for _ in range(RING)]
    wps = [torch.empty_like(Ws[0]) for _ in range(W_COPIES)]
    ts_w = [torch.empty(1, **f32) for _ in range(W_COPIES)]
    # weights of every ring slot: dense from W, 2:4 from the pruned W (GPU calls, checked below)
    for j in range(RING):
        ssn.sp24_prune(Ws[0], out=wps[0], tensor_scale_out=ts_w[0])
        ssn.nvfp4_quantize(Ws[0], codes=dense[j]["codes"], scales=dense[j]["scales"], tensor_scale_out=dense[j]["ts"])
        ssn.nvfp4_quantize(wps[0], tensor_scale_in=ts_w[0], codes=sparse[j]["codes"], scales=sparse[j]["scales"],
                           tensor_scale_out=sparse[j]["ts"])
        ssn.sp24_compress(sparse[j]["codes"], vals=sparse[j]["vals"], meta=sparse[j]["meta"], bad_groups=sparse[j]["bad"])
    Y = {(M, f): torch.empty((M, N), **f32) for M in Ms for f in ("dense", "sp24", "gather")}
    Xm = {M: X[:M].contiguous() for M in Ms}
    calls, used = {}, {}
    for j in range(RING):
        d, s_ = dense[j], sparse[j]
        for M in Ms:
            p, (_, u) = ssn.gemm_nvfp4_dense(Xm[M], d["codes"], d["scales"], d["ts"], Y=Y[(M, "dense")], prepare=True)
            calls.setdefault(f"gemv_dense_M{M}", []).append(p)
            used[f"gemv_dense_M{M}"] = u
            p, (_, u) = ssn.gemm_nvfp4_sp24(Xm[M], s_["vals"], s_["meta"], s_["scales"], s_["ts"], Y=Y[(M, "sp24")],
                                            prepare=True)
            calls.setdefault(f"gemv_sp24_M{M}", []).append(p)
            used[f"gemv_sp24_M{M}"] = u
            p, (_, u) = ssn.gemm_nvfp4_sp24(Xm[M], s_["vals"], s_["meta"], s_["scales"], s_["ts"], Y=Y[(M, "gather")],
                                            algo=ssn.ALGO_GATHER, prepare=True)
            calls.setdefault(f"gemv_sp24_gather_M{M}", []).append(p)
            used[f"gemv_sp24_gather_M{M}"] = u
        calls.setdefault("check", []).append(ssn.sp24_check(s_["codes"], bad_groups=s_["bad"], first_bad=s_["first"],
                                                            prepare=True)[0])
        calls.setdefault("compress", []).append(ssn.sp24_compress(s_["codes"], vals=s_["vals"], meta=s_["meta"],
                                                                  bad_groups=s_["bad"], prepare=True)[0])
    prod = [dict(vals=torch.empty((N, K // 4), **u8), meta=torch.empty((N, K // 8), **u8),
                 scales=torch.empty((N, K // 16), **u8), ts=torch.empty(1, **f32), bad=torch.empty(1, **i64))
            for _ in range(2)]
    qd = [dict(codes=torch.empty((N, K // 2), **u8), scales=torch.empty((N, K // 16), **u8), ts=torch.empty(1, **f32))
          for _ in range(2)]
    for j in range(W_COPIES):
        Wj, wp, q, pf = Ws[j], wps[j], qd[j % 2], prod[j % 2]
        calls.setdefault("prune", []).append(ssn.sp24_prune(Wj, out=wp, tensor_scale_out=ts_w[j], prepare=True)[0])
        calls.setdefault("quantize", []).append(ssn.nvfp4_quantize(Wj, codes=q["codes"], scales=q["scales"],
                                                                   tensor_scale_out=q["ts"], prepare=True)[0])
        calls.setdefault("quantize_given_scale", []).append(ssn.nvfp4_quantize(
            Wj, tensor_scale_in=ts_w[j], codes=q["codes"], scales=q["scales"], tensor_scale_out=q["ts"], prepare=True)[0])
        calls.setdefault("producer_fused", []).append(ssn.nvfp4_sp24_produce(
            Wj, vals=pf["vals"], meta=pf["meta"], scales=pf["scales"], tensor_scale_out=pf["ts"], bad_groups=pf["bad"],
            prepare=True)[0])
    for n in calls:                          # every call once, then parity on what they wrote
        for c in calls[n]:
            c()
    torch.cuda.synchronize()
    rows = np.array([0, 1, 255, 6911, 13823])
    ri = torch.from_numpy(rows).cuda()
    c, s, _ = quant.quantize(w[rows], tensor_scale_in=st)
    for q in (dense[0], qd[0]):
        if not (np.array_equal(q["codes"][ri].cpu().numpy(), c) and np.array_equal(q["scales"][ri].cpu().numpy(), s)):
            raise ParityError("decode: quantised weights differ from the oracle's")
    pc, ps, _ = quant.quantize(sp24.prune24(w[rows]), tensor_scale_in=st)
    v, m, _ = sp24.compress(pc)
    for q in (sparse[0], prod[0]):
        if not (np.array_equal(q["vals"][ri].cpu().numpy(), v) and np.array_equal(q["meta"][ri].cpu().numpy(), m)
                and np.array_equal(q["scales"][ri].cpu().numpy(), ps)):
            raise ParityError("decode: 2:4 compressed weights differ from the oracle's")
    if int(sparse[0]["bad"].item()) != 0 or int(prod[0]["bad"].item()) != 0:
        raise ParityError("decode: pruned weights fail the 2:4 check")
    for M in Ms:
        Yr, Br = gemm.gemm_dense(x[:M], c, s, st)
        _assert_bound(_rows_of(Y[(M, "dense")].t(), rows).T, Yr, Br, "f32", f"decode dense M={M}")
        Yr, Br = gemm.gemm_sp24(x[:M], v, m, ps, st)
        for f in ("sp24", "gather"):
            _assert_bound(_rows_of(Y[(M, f)].t(), rows).T, Yr, Br, "f32", f"decode {f} M={M}")
    T = Timer(torch)
    gemv_groups = {}
    for n, cs in calls.items():
        reps = max(TRIALS, 2 * len(cs))
        seq = [cs[i % len(cs)] for i in range(reps)]
        if n.startswith("gemv_"):
            gemv_groups.setdefault(n.rsplit("_M", 1)[1], []).append((n, seq))
        else:
            T.batch(n, seq)
        T.each(n, seq)
        torch.cuda.synchronize()
    for grp in gemv_groups.values():   # the dense, 2:4 and gather GEMVs of one M, alternated
        T.rounds(grp, ROUNDS)
        torch.cuda.synchronize()
    kb = {"prune": bytes_prune(N, K), "quantize": bytes_quantize(N, K), "quantize_given_scale": bytes_quantize(N, K),
          "check": bytes_check(N, K), "compress": bytes_compress(N, K),
          "producer_fused": N * K * 4 + N * K // 4 + N * K // 8 + N * K // 16 + 4}
    for M in Ms:
        kb[f"gemv_dense_M{M}"] = bytes_gemm(M, N, K, False, 4)
        kb[f"gemv_sp24_M{M}"] = bytes_gemm(M, N, K, True, 4)
        kb[f"gemv_sp24_gather_M{M}"] = bytes_gemm(M, N, K, True, 4)
    kernels = {}
    for name, b in kb.items():
        us = T.us(name)
        e = {"us": round(us, 2), **T.stats(name), **_bw(b, us, copy_gbps)}
        if name.startswith("gemv"):
            M = int(name.split("_M")[1])
            e["tflops_dense_equiv"] = round(2 * M * N * K / (us * 1e-6) / 1e12, 3)
            e["algo"] = ssn.ALGO_NAMES.get(used[name].value, "?")
        kernels[name] = e
    for M in Ms:
        for f in ("sp24", "sp24_gather"):
            kernels[f"gemv_{f}_M{M}"]["speedup_vs_dense"] = round(
                kernels[f"gemv_dense_M{M}"]["us"] / kernels[f"gemv_{f}_M{M}"]["us"], 3)
    kernels["producer_fused"]["unfused_chain_us"] = round(
        sum(kernels[n]["us"] for n in ("prune", "quantize_given_scale", "check", "compress")), 2)
    res = {"shape": {"N": N, "K": K, "M": list(Ms)}, "weight_ring": RING, "w_copies": W_COPIES,
           "parity": "quantised and compressed weights bit-exact and GEMV outputs within bound on sampled rows",
           "kernels": kernels,
           "note": "prune, quantize (own amax pass), quantize_given_scale (the prune's s_t), check, compress and the "
                   "fused producer are weight preparation; the GEMVs are the decode hot path"}
    del Ws, wps, dense, sparse, prod, qd, calls, Y
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------------------------------
HEAD_N, HEAD_K, HEAD_MS = 131072, 5120, (1, 8, 9)


def run_head(torch, ssn, synth, copy_gbps):
    """Output-head-shaped GEMV (vocabulary-sized N = 131072, K = 5120; M = 1, and 8 and 9 rows as
    in speculative verification): weights of 377 MB (dense) / 294 MB (2:4), larger than the
    Infinity Cache; two weight copies alternate so every call reads HBM."""
    import numpy as np
    from oracle import quant
    N, K = HEAD_N, HEAD_K
    x = synth.activations(max(HEAD_MS), K)
    X = torch.from_numpy(x.view("int16")).view(torch.bfloat16).cuda()
    w = synth.weights(N, K)
    st = quant.tensor_scale(w)
    cols = np.array([0, 65537, N - 1])
    ws = w[cols].copy()
    W = torch.from_numpy(w).cuda()
    del w
    dn, sp = _gpu_weights(ssn, W)
    del W
    torch.cuda.empty_cache()
    dns = [dn, tuple(t.clone() for t in dn)]
    sps = [sp, tuple(t.clone() for t in sp)]
    out = {"shape": {"N": N, "K": K, "M": list(HEAD_MS), "y": "f32"}, "weight_copies": 2,
           "parity": "outputs of three weight rows (columns 0, 65537, 131071) within the oracle's bound"}
    dc = torch.from_numpy(cols).cuda()
    for M in HEAD_MS:
        Xm = X[:M].contiguous()
        Yd = torch.empty((M, N), dtype=torch.float32, device="cuda")
        Ys = torch.empty((M, N), dtype=torch.float32, device="cuda")
        pd, ps, used = [], [], {}
        for d, s_ in zip(dns, sps):
            p, (_, ud) = ssn.gemm_nvfp4_dense(Xm, d[0], d[1], d[2], Y=Yd, prepare=True)
            pd.append(p)
            p, (_, us_) = ssn.gemm_nvfp4_sp24(Xm, s_[0], s_[1], s_[2], s_[3], Y=Ys, prepare=True)
            ps.append(p)
            used = {"dense": ud, "sp24": us_}
        pd[0](); ps[0]()
        torch.cuda.synchronize()
        check_product(x[:M], ws, st, np.arange(M), np.arange(3), Yd[:, dc].contiguous(),
                      {"smfmac": Ys[:, dc].contiguous()}, "f32", f"head M={M}")
        T = Timer(torch)
        for n, cs in (("dense", pd), ("sp24", ps)):
            T.batch(n + "_warm", cs)
            torch.cuda.synchronize()
            T.each(n, cs * (TRIALS // 2))
            torch.cuda.synchronize()
        T.rounds((("dense", pd * 4), ("sp24", ps * 4)), ROUNDS)   # alternated
        torch.cuda.synchronize()
        e = {}
        for n in ("dense", "sp24"):
            us = T.us(n)
            e[n] = {"us": round(us, 1), **T.stats(n), **_bw(bytes_gemm(M, N, K, n == "sp24", 4), us, copy_gbps),
                    "tflops_dense_equiv": round(2.0 * M * N * K / (us * 1e-6) / 1e12, 2),
                    "algo": ssn.ALGO_NAMES.get(used[n].value, "?")}
        e["sp24"]["speedup_vs_dense"] = round(e["dense"]["us"] / e["sp24"]["us"], 3)
        out[f"M{M}"] = e
    del dns, sps, dn, sp, X
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------------------------------
def _synth_experts(gen, E, rows, cols):
    """All experts' float32 weights from the seeded generators, drawn on host threads."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    out = np.empty((E, rows, cols), np.float32)

    def one(e):
        out[e] = gen(e)
    with ThreadPoolExecutor(max_workers=min(16, len(os.sched_getaffinity(0)))) as ex:
        list(ex.map(one, range(E)))
    return out


def run_moe(torch, ssn, synth, copy_gbps):
    import numpy as np
    from oracle import moe, quant, sp24
    T, E, k, D, I = 4096, 512, 10, 2048, 512
    ids, wts = synth.routing(T, E, k, 1.1)
    x = synth.activations(T, D)
    X = torch.from_numpy(x.view("int16")).view(torch.bfloat16).cuda()
    dids, dw = torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda()
    up_f = _synth_experts(lambda e: synth.expert_up(e, I, D), E, 2 * I, D)
    down_f = _synth_experts(lambda e: synth.expert_down(e, I, D), E, D, I)

    def build(wf, rows, cols, sparse):
        c = torch.empty((E, rows, cols // (4 if sparse else 2)), dtype=torch.uint8, device="cuda")
        m = torch.empty((E, rows, cols // 8), dtype=torch.uint8, device="cuda") if sparse else None
        s = torch.empty((E, rows, cols // 16), dtype=torch.uint8, device="cuda")
        ts = torch.empty(E, dtype=torch.float32, device="cuda")
        for e in range(E):
            Wf = torch.from_numpy(wf[e]).cuda()
            if sparse:
                Wf = ssn.sp24_prune(Wf)
                codes, _, _ = ssn.nvfp4_quantize(Wf, scales=s[e], tensor_scale_out=ts[e:e + 1])
                ssn.sp24_compress(codes, vals=c[e], meta=m[e])
            else:
                ssn.nvfp4_quantize(Wf, codes=c[e], scales=s[e], tensor_scale_out=ts[e:e + 1])
        return c, m, s, ts

    def oracle_q(wf, e, sparse):
        wt = sp24.prune24(wf[e]) if sparse else wf[e]
        c, s, st = quant.quantize(wt)
        if sparse:
            v, m, _ = sp24.compress(c)
            return ("sp24", v, m, s, st)
        return ("dense", c, s, st)

    R = T * k
    flops = 2.0 * R * D * 2 * I + 2.0 * R * I * D
    counts = np.bincount(ids.ravel(), minlength=E)
    out = {"shape": {"T": T, "E": E, "top_k": k, "D": D, "I": I, "rows": R, "zipf_s": 1.1,
                     "experts_touched": int((counts > 0).sum()), "max_rows": int(counts.max()),
                     "median_rows": float(np.median(counts))},
           "flops_dense_equiv": flops,
           "note": "expert weights, routing and X from the seeded synthetic generators",
           "parity": "routing offsets exact; token 2047 of the whole FFN within the oracle's bound"}
    check_tokens = np.array([2047])
    for sparse in (False, True):
        up_rows, down_rows = build(up_f, 2 * I, D, sparse), build(down_f, D, I, sparse)
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
        p_ffn, (ffn_out, ffn_bad) = ssn.moe_nvfp4_ffn(X, dids, dw, E, up, down, prepare=True, w_layout=kt)
        p_ffn_rows, _ = ssn.moe_nvfp4_ffn(X, dids, dw, E, up_rows, down_rows, prepare=True)
        p_ffn()
        torch.cuda.synchronize()
        # parity before timing: routing offsets exact, two tokens' outputs within the FFN bound
        _, eoff, _, _ = moe.route(ids, E)
        if not np.array_equal(off.cpu().numpy().astype(np.int64), eoff) or int(ffn_bad.item()) != 0:
            raise ParityError("moe: routing differs from the oracle's")
        cache = {}

        def qu(e):
            if ("u", e) not in cache:
                cache[("u", e)] = oracle_q(up_f, e, sparse)
            return cache[("u", e)]

        def qd(e):
            if ("d", e) not in cache:
                cache[("d", e)] = oracle_q(down_f, e, sparse)
            return cache[("d", e)]
        ref, tol, _ = moe.moe_ffn(x, ids, wts, qu, qd, E, I, tokens=check_tokens)
        got = ffn_out[torch.from_numpy(check_tokens).cuda()].cpu().numpy().astype(np.float64)
        if not np.all(np.abs(got - ref) <= tol):
            raise ParityError(f"moe {'2:4' if sparse else 'dense'}: FFN output outside the bound")
        Tm = Timer(torch)
        stages = [("route", p_route), ("up_silu_gate", p_up), ("down", p_down), ("combine", p_comb), ("ffn", p_ffn),
                  ("ffn_row_layout", p_ffn_rows)]
        for n, p in stages:
            Tm.batch(n + "_warm", [p] * 2)
            torch.cuda.synchronize()
            Tm.batch(n, [p] * 5)
            Tm.each(n, [p] * TRIALS)
            torch.cuda.synchronize()
        wbytes = sum(t.numel() for t in (up[0], up[1], up[2], down[0], down[1], down[2]) if t is not None)
        ffn_bytes = wbytes + T * D * 2 + 2 * R * I * 2 + T * D * 4
        res = {n: {"us": round(Tm.us(n), 1), **Tm.stats(n)} for n, _ in stages}
        us = res["ffn"]["us"]
        t_roof = max(flops / (2 if sparse else 1) / (BF16_PEAK_TFLOPS * 1e12), ffn_bytes / (HBM_PEAK_GBPS * 1e9))
        res["ffn"].update({"weight_layout": "ktile64", "weight_bytes": wbytes, "alg_bytes": ffn_bytes,
                           "tflops_dense_equiv": round(flops / (us * 1e-6) / 1e12, 1),
                           "GBps_alg": round(ffn_bytes / (us * 1e-6) / 1e9, 1),
                           "t_roof_us": round(t_roof * 1e6, 1), "frac_of_t_roof": round(t_roof / (us * 1e-6), 4)})
        res["gpu_state"] = state_under_load(torch, p_ffn, seconds=1.0)
        out["sp24" if sparse else "dense"] = res
        del H, Yd, up_rows, down_rows
        torch.cuda.empty_cache()
        out["decode_" + ("sp24" if sparse else "dense")] = run_moe_decode(torch, ssn, synth, x, up, down, sparse,
                                                                          E, k, D, I)
        del up, down
        torch.cuda.empty_cache()
    out["sp24"]["ffn"]["speedup_vs_dense"] = round(out["dense"]["ffn"]["us"] / out["sp24"]["ffn"]["us"], 3)
    for T_ in MOE_DECODE_TOKENS:
        d, s_ = out["decode_dense"][f"T{T_}"], out["decode_sp24"][f"T{T_}"]
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
    tiles = ssn.ALGO_SMFMAC if sparse else ssn.ALGO_MFMA
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
        Tm = Timer(torch)
        for n, ps in stages.items():
            Tm.batch(n + "_warm", ps)
            torch.cuda.synchronize()
            Tm.batch(n, ps + ps)
            torch.cuda.synchronize()
        t = {n: Tm.us(n) for n in stages}
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
def run_w4a4(torch, ssn, synth, M, N, K, outliers, dense_us):
    """The W4A4 variant at one shape: bf16 activations quantised to MXFP4 on the fly
    (mxfp4_quantize, part of every step), weights quantised once (timed too, as preparation),
    and the FP4 x FP4 product on the block-scaled matrix cores, bf16 out."""
    import numpy as np
    from oracle import mx
    x = synth.activations(M, K)
    w = synth.weight_rows_with_outliers(N, K, 0, N, 0.01, 20.0) if outliers else synth.weights(N, K)
    X = torch.from_numpy(x.view("int16")).view(torch.bfloat16).cuda()
    W = torch.from_numpy(w).cuda()
    xc, xs = ssn.mxfp4_quantize(X)
    wc, ws = ssn.mxfp4_quantize(W)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    p_q, _ = ssn.mxfp4_quantize(X, codes=xc, scales=xs, prepare=True)
    p_w, _ = ssn.mxfp4_quantize(W, codes=wc, scales=ws, prepare=True)
    p_g, (_, used) = ssn.gemm_mxfp4(xc, xs, M, wc, ws, N, K, y_dtype=torch.bfloat16, Y=Y, prepare=True)
    p_g()
    torch.cuda.synchronize()
    ms = np.array(sorted({0, 1, 255, 256, M // 2 + 3, M - 1}))
    ns = np.array(sorted({0, 1, 255, 256, N // 2 + 5, N - 1}))
    qxc, qxs = mx.quantize_bf16(x[ms])
    qwc, qws = mx.quantize(w[ns])
    Yr, Br = mx.gemm_w4a4(qxc, qxs, qwc, qws)
    _assert_bound(_rows_of(Y, ms, ns), Yr, Br, "bf16", f"w4a4 {M}x{N}x{K}")
    del w, W
    T = Timer(torch)
    for n, p in (("quantize_x", p_q), ("quantize_w", p_w), ("gemm", p_g)):
        T.batch(n + "_warm", [p] * 2)
        torch.cuda.synchronize()
        T.batch(n, [p] * TRIALS)
        T.each(n, [p] * TRIALS)
        torch.cuda.synchronize()
    flops = 2.0 * M * N * K
    g_us, q_us = T.us("gemm"), T.us("quantize_x")
    qx_bytes = M * K * 2 + M * K // 2 + M * K // 32
    qw_bytes = N * K * 4 + N * K // 2 + N * K // 32
    res = {"shape": {"M": M, "N": N, "K": K, "y": "bf16", "outliers": outliers},
           "format": "MXFP4 activations and weights (E2M1, E8M0 scale per 32 along K), tiled for the matrix cores",
           "parity": "sampled outputs within the oracle's bound",
           "gemm": {"us": round(g_us, 1), **T.stats("gemm"), "algo": ssn.ALGO_NAMES.get(used.value, "?"),
                    "tflops": round(flops / (g_us * 1e-6) / 1e12, 1),
                    "frac_of_fp4_peak": round(flops / (g_us * 1e-6) / 1e12 / FP4_PEAK_TFLOPS, 4)},
           "quantize_x": {"us": round(q_us, 1), **T.stats("quantize_x"), "alg_bytes": qx_bytes,
                          "GBps": round(qx_bytes / (q_us * 1e-6) / 1e9, 1)},
           "quantize_w": {"us": round(T.us("quantize_w"), 1), **T.stats("quantize_w"), "alg_bytes": qw_bytes,
                          "GBps": round(qw_bytes / (T.us("quantize_w") * 1e-6) / 1e9, 1)},
           "step_us": round(g_us + q_us, 1),
           "step_tflops": round(flops / ((g_us + q_us) * 1e-6) / 1e12, 1)}
    if dense_us:
        res["speedup_vs_w4a16_dense"] = round(dense_us / (g_us + q_us), 3)
    res["gpu_state"] = state_under_load(torch, p_g)
    del X, Y, xc, xs, wc, ws
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------------------------------
def run_references(torch, ssn, copy_gbps):
    """Comparison points measured in the same run: the vendor bf16 GEMM (hipBLASLt through
    torch.matmul, bf16 in and out, operands contiguous) at the prefill and square shapes, and
    the plainest streaming read at the decode GEMV's size (sp24_check over 40 MB of zero codes,
    on a ring of copies larger than the Infinity Cache)."""
    out = {}
    for name, (M, N, K) in (("prefill", (8192, 27648, 5120)), ("square", (4096, 4096, 4096))):
        A = torch.randn(M, K, device="cuda").to(torch.bfloat16)
        B = (torch.randn(K, N, device="cuda") * 0.02).to(torch.bfloat16).contiguous()
        C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        fn = lambda: torch.matmul(A, B, out=C)
        T = Timer(torch)
        T.batch("warm", [fn] * 3)
        torch.cuda.synchronize()
        T.batch("mm", [fn] * TRIALS)
        T.each("mm", [fn] * TRIALS)
        torch.cuda.synchronize()
        us = T.us("mm")
        out[f"bf16_gemm_vendor_{name}"] = {"us": round(us, 1), **T.stats("mm"), "shape": [M, N, K],
                                           "tflops": round(2.0 * M * N * K / (us * 1e-6) / 1e12, 1),
                                           "note": "torch.matmul bf16 x bf16 -> bf16 (hipBLASLt)"}
        del A, B, C
    torch.cuda.empty_cache()
    n_bytes = 13824 * 2560                                  # the decode weights' codes (35.4 MB)
    ring = [torch.zeros((13824, 2560), dtype=torch.uint8, device="cuda") for _ in range(24)]
    calls = [ssn.sp24_check(r, prepare=True)[0] for r in ring]
    T = Timer(torch)
    T.batch("warm", calls)
    torch.cuda.synchronize()
    T.batch("read", calls * 2)
    T.each("read", calls)
    torch.cuda.synchronize()
    us = T.us("read")
    out["streaming_read_decode_size"] = {"us": round(us, 2), **T.stats("read"), **_bw(n_bytes, us, copy_gbps),
                                         "note": "sp24_check over 35.4 MB of zero codes, 24 rotating copies"}
    del ring, calls
    src = [torch.zeros(n_bytes, dtype=torch.uint8, device="cuda") for _ in range(12)]
    dst = [torch.empty_like(t) for t in src]
    calls = [(lambda a=a, b=b: b.copy_(a)) for a, b in zip(src, dst)]
    T = Timer(torch)
    T.batch("warm", calls)
    torch.cuda.synchronize()
    T.batch("copy", calls * 2)
    T.each("copy", calls * 2)
    torch.cuda.synchronize()
    us = T.us("copy")
    out["device_copy_decode_size"] = {"us": round(us, 2), **T.stats("copy"),
                                      "GBps_read_plus_write": round(2 * n_bytes / (us * 1e-6) / 1e9, 1),
                                      "note": "torch copy_ of 35.4 MB (read and written), 12 rotating pairs"}
    del src, dst, calls
    torch.cuda.empty_cache()
    out.update(run_mfma_ceiling(torch, ssn))
    return out


def run_mfma_ceiling(torch, ssn):
    """The matrix-core rate this GPU sustains on register-resident random operands (the
    library's calibration launch): the power limit's ceiling for the bf16 products (W4A16 tiles)
    and the FP4 products (W4A4), beside the published peaks the roofline is priced against."""
    out = {}
    sink = torch.empty(ssn.mfma_probe_sink_floats(), dtype=torch.float32, device="cuda")
    for kind, name, peak in ((ssn.PROBE_BF16, "bf16_32x32x16", BF16_PEAK_TFLOPS),
                             (ssn.PROBE_FP4, "fp4_32x32x64", FP4_PEAK_TFLOPS)):
        for wps in (1, 2):
            flops = ssn.mfma_probe(kind, wps, 4096, sink)
            calls = [(lambda s=seed: ssn.mfma_probe(kind, wps, 4096, sink, seed=s)) for seed in range(10)]
            T = Timer(torch)
            T.batch("warm", calls[:3])
            torch.cuda.synchronize()
            T.batch("probe", calls)
            torch.cuda.synchronize()
            us = T.us("probe")
            tf = flops / (us * 1e-6) / 1e12
            out[f"mfma_ceiling_{name}_{wps}wave_per_simd"] = {
                "us_per_launch": round(us, 1), "tflops": round(tf, 1), "frac_of_published_peak": round(tf / peak, 4),
                "note": "register-resident operands with random bits, back-to-back matrix ops, 10 launches"}
    del sink
    return out


# ------------------------------------------------------------------------------------------
def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_prefill(x, cols=PREFILL["N"], chunk=4096):
    """The oracle (unchanged) on the host: the dense prefill product for all 8192 activation
    rows and weight rows [0, cols) (output columns), including the oracle's quantisation of
    those rows, in chunks of weight rows; reported as dense TFLOP/s of that product."""
    import numpy as np
    import synth
    from oracle import gemm, quant
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    M, N, K = PREFILL["M"], PREFILL["N"], PREFILL["K"]
    t0 = time.perf_counter()
    amax = 0.0
    for r0 in range(0, N, 4096):   # the tensor scale needs the whole W's maximum
        blk = synth.weight_rows_with_outliers(N, K, r0, min(N, r0 + 4096), 0.01, 20.0)
        amax = max(amax, float(np.abs(blk).max()))
    t_scale = time.perf_counter() - t0
    st = quant.tensor_scale(np.full((1, 16), amax, np.float32))
    sec = 0.0
    for r0 in range(0, cols, chunk):
        w = synth.weight_rows_with_outliers(N, K, r0, min(cols, r0 + chunk), 0.01, 20.0)
        t1 = time.perf_counter()
        c, s, _ = quant.quantize(w, tensor_scale_in=st)
        gemm.gemm_dense(x, c, s, st)
        sec += time.perf_counter() - t1
    flops = 2.0 * M * cols * K
    stages = oracle_stage_rates()
    return {"value": round(flops / sec / 1e12, 5), "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
            "stages": stages,
            "sample": f"dense prefill product X [{M}, {K}] x weight rows [0, {cols}) of {N} (the oracle's quantisation "
                      f"of those rows with the whole tensor's scale, then its float64 product and bound base, in "
                      f"chunks of {chunk} rows); {sec:.1f} s on host cores; NumPy float64 oracle",
            "seconds": round(sec, 2), "tensor_scale_pass_s": round(t_scale, 2), "cpu_model": cpu_model(),
            "host_cores_available": len(os.sched_getaffinity(0))}


def oracle_stage_rates(rows=2048):
    """The oracle's weight-side stages on rows [0, rows) of the decode weight W [13824, 5120]:
    prune, quantise (given the tensor scale), check and compress, each timed once, as the GB/s
    of the bytes the GPU calls move for the same rows."""
    import numpy as np
    import synth
    from oracle import quant, sp24
    N, K = 13824, 5120
    w = synth.weight_rows(N, K, 0, rows)
    st = quant.tensor_scale(w)
    out = {}
    t = time.perf_counter(); wp = sp24.prune24(w); dt = time.perf_counter() - t
    out["prune"] = {"s": round(dt, 3), "GBps": round(2 * rows * K * 4 / dt / 1e9, 3)}
    t = time.perf_counter(); c, _, _ = quant.quantize(wp, tensor_scale_in=st); dt = time.perf_counter() - t
    out["quantize"] = {"s": round(dt, 3), "GBps": round((rows * K * 4 + rows * K // 2 + rows * K // 16) / dt / 1e9, 3)}
    t = time.perf_counter(); sp24.check(c); dt = time.perf_counter() - t
    out["check"] = {"s": round(dt, 3), "GBps": round(rows * K / 2 / dt / 1e9, 3)}
    t = time.perf_counter(); sp24.compress(c); dt = time.perf_counter() - t
    out["compress"] = {"s": round(dt, 3), "GBps": round((rows * K / 2 + rows * K / 4 + rows * K / 8) / dt / 1e9, 3)}
    out["sample"] = f"weight rows [0, {rows}) of the decode W [{N}, {K}] (no outliers), NumPy oracle, one call each"
    return out


# ------------------------------------------------------------------------------------------
# rocprofv3 output -> profiles/ summaries
def _read_csvs(d, pattern):
    rows = []
    for f in glob.glob(os.path.join(d, "**", pattern), recursive=True):
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _pmc_avg(d, counter):
    """{(kernel, grid): (average value per dispatch, dispatches, largest value)} of one counter."""
    agg = {}
    for r in _read_csvs(d, "*counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        key = (r["Kernel_Name"], int(r.get("Grid_Size", 0) or 0))
        a = agg.setdefault(key, [0.0, 0, 0.0])
        v = float(r["Counter_Value"])
        a[0] += v
        a[1] += 1
        a[2] = max(a[2], v)
    return {k: (v[0] / v[1], v[1], v[2]) for k, v in agg.items()}


COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 1 << 31          # the bandwidth probe's device copy: 2 GiB read and 2 GiB written


def traffic_entry(fetch_dir, write_dir, kernel, grid, source, summary):
    """HBM bytes per launch of `kernel` at `grid` from FETCH_SIZE / WRITE_SIZE runs (KiB per
    dispatch), each scaled by what the same counter reads for the 2 GiB probe copy."""
    fe, wr = _pmc_avg(fetch_dir, "FETCH_SIZE"), _pmc_avg(write_dir, "WRITE_SIZE")

    def copy_cal(tab):
        # the largest single copy dispatch is the 2 GiB probe (the runtime's copy kernel has one
        # grid for every size, so averages per grid mix the probe with smaller copies)
        big = max(v[2] for (k, g), v in tab.items() if k.startswith(COPY_KERNEL))
        return COPY_BYTES / (big * 1024.0)

    def pick(tab):
        m = [v for (k, g), v in tab.items() if k.startswith(kernel) and g == grid]
        if not m:
            raise SystemExit(f"no dispatch of {kernel} with grid {grid}")
        return m[0][0]
    cf, cw = copy_cal(fe), copy_cal(wr)
    return {"kernels": [kernel], "grid": grid, "source": source, "source_sha256": _source_hash(source),
            "fetch_bytes": int(pick(fe) * 1024 * cf), "write_bytes": int(pick(wr) * 1024 * cw),
            "fetch_calibration": round(cf, 4), "write_calibration": round(cw, 4), "summary": summary}


def summarize(kind, out, dirs, cmd_note):
    """KIND trace: kernel_stats.csv of --kernel-trace --stats runs -> markdown table.
    KIND pmc: counter_collection.csv of --pmc runs -> per-kernel, per-grid averages.
    KIND traffic: OUT is profiles/traffic.json; DIRS = KEY KERNEL GRID SOURCE SUMMARY FETCH_DIR
    WRITE_DIR: adds or replaces that entry."""
    if kind == "traffic":
        key, kernel, grid, source, summary, fdir, wdir = dirs
        try:
            with open(out) as f:
                t = json.load(f)
        except OSError:
            t = {}
        t[key] = traffic_entry(fdir, wdir, kernel, int(grid), source, summary)
        with open(out, "w") as f:
            json.dump(t, f, indent=1)
        print(f"{key}: {t[key]}")
        return
    lines = [f"# {os.path.splitext(os.path.basename(out))[0]}", "", "Command(s):", "", "```", cmd_note.strip(), "```", ""]
    if kind == "trace":
        for d in dirs:
            rows = _read_csvs(d, "*kernel_stats.csv")
            lines += [f"From `{os.path.basename(os.path.normpath(d))}` (--stats, per kernel name):", "",
                      "| kernel | calls | average us | min us | max us | share % |", "|---|---|---|---|---|---|"]
            for r in sorted(rows, key=lambda r: -float(r.get("TotalDurationNs", 0))):
                lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                             f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                             f"{float(r['Percentage']):.2f} |")
            lines.append("")
            per = {}
            for r in _read_csvs(d, "*kernel_trace.csv"):
                g = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
                us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                name = r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
                per.setdefault((name[:90], g), []).append(us)
            lines += ["The same dispatches by kernel and grid (work-items); median and mean in us:", "",
                      "| kernel | grid | calls | median us | mean us | min us |", "|---|---|---|---|---|---|"]
            for (k, g), v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
                v = sorted(v)
                lines.append(f"| `{k}` | {g} | {len(v)} | {v[len(v) // 2]:.2f} | {sum(v) / len(v):.2f} | {v[0]:.2f} |")
            lines.append("")
    else:
        agg = {}
        for d in dirs:
            for r in _read_csvs(d, "*counter_collection.csv"):
                key = (r["Kernel_Name"][:90], int(r.get("Grid_Size", 0) or 0), r["Counter_Name"])
                a = agg.setdefault(key, [0.0, 0])
                a[0] += float(r["Counter_Value"])
                a[1] += 1
        counters = sorted({k[2] for k in agg})
        kern = sorted({(k[0], k[1]) for k in agg})
        lines += ["Averages per dispatch (grid = work-items).", "",
                  "| kernel | grid | dispatches | " + " | ".join(counters) + " |",
                  "|---|---|---|" + "---|" * len(counters)]
        for kname, grid in kern:
            vals, nd = [], 0
            for c in counters:
                a = agg.get((kname, grid, c))
                vals.append(f"{a[0] / a[1]:.1f}" if a else "")
                nd = max(nd, a[1] if a else 0)
            lines.append(f"| `{kname}` | {grid} | {nd} | " + " | ".join(vals) + " |")
        lines.append("")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {out}")


# ------------------------------------------------------------------------------------------
def main():
    args = parse()
    if args.summarize:
        kind, out, *dirs = args.summarize
        summarize(kind, out, dirs, os.environ.get("SSN_PROFILE_CMD", ""))
        return
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
    wl = set(w for w in args.workloads.split(",") if w)
    hbm = hbm_probe(torch, ssn)
    print(f"[bench] hbm probe {hbm}", file=sys.stderr, flush=True)
    M, N, K = PREFILL["M"], PREFILL["N"], PREFILL["K"]
    pre, step, x_pre = run_gemm_shape(torch, ssn, synth, M, N, K, torch.bfloat16, True, args, headline=True)
    flops = 2.0 * M * N * K
    ms_step = step["ms_per_step"]
    kus = step["event_us"]
    achieved = flops / (kus * 1e-6) / 1e12
    print(f"[bench] prefill done: {ms_step:.4f} ms/step", file=sys.stderr, flush=True)
    out = {"metric": METRIC, "value": round(flops / (ms_step * 1e-3) / 1e12, 1), "unit": "TFLOP/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "prefill: X bf16 [8192, 5120] ~N(0,1) . W^T, W [27648, 5120] ~N(0,0.02) with 1% "
                                  "outliers x20, dense NVFP4 weights decoded in registers, bf16 matrix cores, f32 "
                                  "accumulate, bf16 out; one step = one product",
                      "M": M, "N": N, "K": K, "weights": "nvfp4 dense", "step_flops": flops},
           "roofline": {"kernel": DENSE_TILE_KERNEL, "bound": "mfma", "achieved": round(achieved, 1),
                        "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                        "traffic": traffic_for("prefill_dense"), "avg_launch_us": round(kus, 2),
                        "flops_per_launch": flops},
           "sp24_vs_dense": {v: pre[v]["speedup_vs_dense"] for v in ("sp24_smfmac", "sp24_decompress_mfma",
                                                                      "sp24_gather_valu")},
           "hbm_measured": hbm}
    work = {"prefill": pre}
    if "decode" in wl:
        work["decode"] = run_decode(torch, ssn, synth, hbm["copy_GBps"])
        print("[bench] decode done", file=sys.stderr, flush=True)
    if "square" in wl:
        work["square"], _, _ = run_gemm_shape(torch, ssn, synth, 4096, 4096, 4096, torch.float32, False, args)
        print("[bench] square done", file=sys.stderr, flush=True)
    if "head" in wl:
        work["head"] = run_head(torch, ssn, synth, hbm["copy_GBps"])
        print("[bench] head done", file=sys.stderr, flush=True)
    if "moe" in wl:
        work["moe"] = run_moe(torch, ssn, synth, hbm["copy_GBps"])
        print("[bench] moe done", file=sys.stderr, flush=True)
    if "refs" in wl:
        work["references"] = run_references(torch, ssn, hbm["copy_GBps"])
        print("[bench] references done", file=sys.stderr, flush=True)
    if "w4a4" in wl:
        work["w4a4"] = {"prefill": run_w4a4(torch, ssn, synth, M, N, K, True, pre["dense_mfma"]["us"])}
        if "square" in work:
            work["w4a4"]["square"] = run_w4a4(torch, ssn, synth, 4096, 4096, 4096, False,
                                              work["square"]["dense_mfma"]["us"])
        print("[bench] w4a4 done", file=sys.stderr, flush=True)
    out["workloads"] = work
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_prefill(x_pre)
        print("[bench] cpu baseline done", file=sys.stderr, flush=True)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
