"""Benchmark of the W4A16 g128 decode GEMV (M=1, K=N=8192) on one MI355X.

One step = one pass of the whole path over the decode workload: quantize_pack
of the fp16 weight matrix (fold, group statistics, scale / zero, codes,
packing), then a burst of GEMV_BURST fused dequantize-GEMVs (decode tokens)
over previously packed sets.  Inputs are resident in HBM before the timed
region.  Weight copies and packed sets are rotated so that every launch
streams from HBM rather than from the 256 MB Infinity Cache.

`value` is the GEMV's effective HBM bandwidth: algorithmic bytes (packed codes
+ fp16 scales + fp16 zeros + x + y) divided by the GEMV kernel's average
duration.  That duration comes from HIP events recorded on the launch stream
around each step's burst of GEMV_BURST back-to-back GEMVs: a pair of timing
events costs about 2 us of its own (the first GEMV after an event also starts
without overlap), so the burst is long enough that this cost stays near 0.1 us
per launch and the figure agrees with the per-kernel durations of a rocprofv3
kernel trace.  The stream is pre-filled with a spin kernel before the timed
steps so host-side launch latency never shows up as GPU idle time inside the
events.  The CPU oracle is timed on a bounded sample
of the same workload (cpu_baseline).

The same run also times the other rows of the path on their own workloads
(`rows`): the LLaMA-2-7B-shaped decode GEMVs with AWQ scales, the fused
projection GEMVs, the group sizes 32 / 64 / 128 / K, the small-batch
GEMM (M = 4, 16, 64; K = 8192, N = 28672), the prefill GEMM (M = 2048,
K = 4096, N = 11008), the AWQ exponent search and GPTQ for the q_proj shape,
and quantize_pack over 32 layers of the LLaMA-2-7B linear
shapes, each as back-to-back launches over rotated weight sets with its
roofline fraction.  The rows keep host copies of sampled outputs; the oracle
checks them (relative L2, byte equality) only inside the cpu_baseline leg,
after all timing, and never with --no-cpu-baseline.

`--write-traffic DIR` turns the rocprofv3 FETCH_SIZE / WRITE_SIZE CSVs of a
bench run and of a `--copy-calibration` run (pmc_fetch, pmc_write,
pmc_copy_fetch, pmc_copy_write under DIR) into profiles/gemv_traffic.json.
`--gemm-only M,N,K` runs five GEMMs of one shape and nothing else, for
rocprofv3 counter runs of a single GEMM kernel.

Usage: python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--no-rows]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD published peak
MFMA_F16_PEAK_TFLOPS = 2516.6  # MI355X dense fp16/bf16 MFMA (no sparsity)
FP64_PEAK_TFLOPS = 78.6        # MI355X fp64 (vector and matrix)
MALL_BYTES = 256 << 20
METRIC = "W4A16 g128 GEMV µs + effective HBM GB/s (% peak) at M=1, K=N=8192"
GEMV_BURST = 64
PREFILL_CYCLES = 40_000_000  # spin kernel that keeps the queue ahead of the host


def gemv_bytes(N, K, bits, G, asym, M=1, act_scale=False):
    """Algorithmic bytes of one dequant-GEMV/GEMM launch."""
    b = N * K * bits // 8 + N * (K // G) * 2 * (1 + int(asym)) + M * K * 2 + M * N * 2
    return b + (4 * K if act_scale else 0)


def quantize_pack_bytes(N, K, bits, G, asym):
    return N * K * 2 + N * K * bits // 8 + N * (K // G) * 2 * (1 + int(asym))


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--extra", default=None, help="write per-config results (JSON lines) to this file")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-rows", action="store_true", help="skip the per-row timings of the other workloads")
    p.add_argument("--write-traffic", default=None, metavar="DIR",
                   help="write profiles/gemv_traffic.json from rocprofv3 counter CSVs in DIR and exit")
    p.add_argument("--copy-mib", type=int, default=256, help="size of the --copy-calibration run used for DIR")
    p.add_argument("--write-trace", default=None, metavar="DIR",
                   help="write profiles/gemv_trace.json from the rocprofv3 kernel_trace.csv under DIR and exit")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB (for HBM counter calibration) and exit")
    p.add_argument("--gemm-only", default=None, metavar="M,N,K",
                   help="only run five fp16 4-bit asymmetric g128 GEMMs of this shape on seeded inputs "
                        "(for rocprofv3 counter runs) and exit")
    return p.parse_args()


class Timer:
    """HIP events recorded on the current (launch) stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def stop(self, e0):
        e1 = self.torch.cuda.Event(enable_timing=True)
        e1.record()
        self.pairs.append((e0, e1))

    def mean_ms(self):
        return float(np.mean([a.elapsed_time(b) for a, b in self.pairs]))


def trace_entry(nb):
    """The committed kernel trace's statistics of the same GEMV (mean, median,
    min per dispatch) and the fraction of peak its mean gives; None when the
    GEMV source changed since the trace."""
    t = measured_trace()
    if t is None:
        return None
    return {"mean_us": t["mean_us"], "median_us": t["median_us"], "min_us": t["min_us"],
            "dispatches": t["dispatches"], "frac_from_mean": round(nb / (t["mean_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "source": "profiles/gemv_trace.json (rocprofv3 --kernel-trace of bench.py)"}


def measured_traffic():
    """HBM bytes per GEMV launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs (scaled by a plain-copy calibration), or None when the
    GEMV source has changed since those counters were taken."""
    path = os.path.join(ROOT, "profiles", "gemv_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if gemv_source_sha() != t.get("kernel_source_sha256"):
        return None
    return int(t["bytes_per_launch"])


GEMV_C2_KERNEL = "gemv_kernel<4, true, woq::F16, false, 4, 4, 2, false>"


def gemv_source_sha():
    import hashlib

    with open(os.path.join(ROOT, "weight_only_quantization_quantize_amd", "csrc", "gemv.hip"), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_trace():
    """Per-dispatch duration statistics of the K = N = 8192 GEMV from the
    committed rocprofv3 kernel trace of a bench run, or None when the GEMV
    source has changed since that trace was taken."""
    path = os.path.join(ROOT, "profiles", "gemv_trace.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    return t if t.get("kernel_source_sha256") == gemv_source_sha() else None


def write_trace(prof_dir):
    """profiles/gemv_trace.json from the kernel_trace.csv of a rocprofv3
    --kernel-trace run of bench.py: durations of the dispatches of the
    K = N = 8192 GEMV instance with its 1024 x 512-thread grid."""
    import csv
    import glob

    files = glob.glob(os.path.join(prof_dir, "**", "*kernel_trace.csv"), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"expected one kernel_trace.csv under {prof_dir}, found {files}")
    durs = []
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            grid = int(r.get("Grid_Size_X", r.get("Grid_Size", 0)))
            if GEMV_C2_KERNEL in r["Kernel_Name"] and grid == 1024 * 512:
                durs.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    if not durs:
        raise SystemExit("no K = N = 8192 GEMV dispatches in the trace")
    d = np.array(durs)
    out = {"kernel": GEMV_C2_KERNEL, "grid": "1024 x 512 threads", "dispatches": int(d.size),
           "mean_us": round(float(d.mean()), 3), "median_us": round(float(np.median(d)), 3),
           "min_us": round(float(d.min()), 3), "max_us": round(float(d.max()), 3),
           "kernel_source_sha256": gemv_source_sha()}
    with open(os.path.join(ROOT, "profiles", "gemv_trace.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def write_traffic(prof_dir, copy_mib):
    """Scale the GEMV's FETCH_SIZE / WRITE_SIZE (KiB per dispatch, median) by
    what the same counters read for a plain device copy of copy_mib MiB."""
    import csv

    def per_kernel(name):
        d = {}
        with open(os.path.join(prof_dir, f"{name}_counter_collection.csv")) as f:
            for r in csv.DictReader(f):
                d.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return d

    def copy_kib(d):
        v = [x for k, xs in d.items() if "copyBuffer" in k for x in xs]
        if len(v) != 1:
            raise SystemExit(f"expected one copy dispatch in the calibration run, found {len(v)}")
        return v[0]

    fetch_scale = copy_mib * 1024 / copy_kib(per_kernel("pmc_copy_fetch"))
    write_scale = copy_mib * 1024 / copy_kib(per_kernel("pmc_copy_write"))
    fetch, write = per_kernel("pmc_fetch"), per_kernel("pmc_write")
    table = []
    for k in sorted(fetch):
        if "woq::" not in k:
            continue
        fk, wk = float(np.median(fetch[k])), float(np.median(write.get(k, [0.0])))
        table.append((k, len(fetch[k]), fk, wk, fk * fetch_scale * 1024, wk * write_scale * 1024))
    gemv = [t for t in table if GEMV_C2_KERNEL in t[0]]
    if len(gemv) != 1:
        raise SystemExit("the K = N = 8192 GEMV kernel is not in the counter CSVs")
    k, _, fk, wk, rb, wb = gemv[0]
    sha = gemv_source_sha()
    out = {
        "kernel": "gemv_kernel<4, true, F16, false, 4, 4, 2, false>",
        "workload": "M=1 K=8192 N=8192 4-bit asym g128",
        "kernel_source_sha256": sha,
        "fetch_size_kib": fk,
        "write_size_kib": wk,
        "fetch_scale": fetch_scale,
        "write_scale": write_scale,
        "bytes_per_launch": int(round(rb + wb)),
        "summary": "profiles/gemv_w4a16_g128_m1_k8192_n8192.md",
    }
    with open(os.path.join(ROOT, "profiles", "gemv_traffic.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(f"fetch scale {fetch_scale:.4f}, write scale {write_scale:.4f}")
    print("| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read MB | scaled write MB |")
    print("|---|---|---|---|---|---|")
    for k, n, fk, wk, rb, wb in table:
        name = k.replace("void ", "").replace("woq::(anonymous namespace)::", "").replace("woq::", "").split("(")[0]
        print(f"| {name} | {n} | {fk:.1f} | {wk:.1f} | "
              f"{rb / 1e6:.3f} | {wb / 1e6:.3f} |")
    print(json.dumps(out))


BURST_CHUNK = 96  # launches enqueued behind one queue prefill


def burst_us(torch, launches, reps=3):
    """Average duration (us) of each launch when the callables in `launches`
    run back to back behind a queue prefill, HIP events on the launch stream;
    the mean over `reps` passes, after one untimed launch (the first launch of
    a kernel also pays for finding its code).  A pass runs the launches in
    order, BURST_CHUNK at a time, each chunk behind its own prefill and
    between its own events, so that the host (about 10 us per call through the
    binding) never falls behind a queue of short kernels: one unbroken burst
    of 800 four-microsecond GEMVs timed the host instead."""
    launches[0]()
    torch.cuda.synchronize()
    total = 0.0
    for _ in range(reps):
        for c0 in range(0, len(launches), BURST_CHUNK):
            torch.cuda.synchronize()
            torch.cuda._sleep(PREFILL_CYCLES // 4)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for f in launches[c0:c0 + BURST_CHUNK]:
                f()
            e1.record()
            torch.cuda.synchronize()
            total += e0.elapsed_time(e1) * 1e3
    return total / (reps * len(launches))


def time_rows(torch, ops, synth, checks):
    """Per-row timings on the other workloads.  Each row also appends to
    `checks` host copies of a sample of its output (and of the inputs that
    define it); the oracle runs on them only in the cpu_baseline leg
    (row_checks), so the timed path never touches it."""
    dev = torch.device("cuda:0")
    rows = {}

    def x_tensor(X, xdtype):
        if xdtype == "f16":
            return torch.from_numpy(X).to(dev)
        return torch.from_numpy(np.ascontiguousarray(X).view(np.int16)).to(dev).view(torch.bfloat16)

    def host_y(Y):
        if Y.dtype == torch.bfloat16:  # bf16 bits -> fp32 (exact) -> fp64
            u = Y.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16
            return u.view(np.float32).astype(np.float64)
        return Y.cpu().numpy().astype(np.float64)

    def record(row, key, lin, Y, s, sel, bits=4, G=128, asym=True, X=None, xdtype=None):
        """Sampled output columns `sel` of a row's result, for the oracle."""
        checks.append(("gemm", row, key, np.ascontiguousarray(lin.W[sel]), lin.X if X is None else X,
                       lin.xdtype if xdtype is None else xdtype, s, host_y(Y)[:, sel], (bits, G, asym)))

    rows["ceilings"] = time_ceilings(torch, dev)

    # Decode GEMVs of the LLaMA-2-7B linears with their AWQ scales, 4-bit and
    # 3-bit asymmetric g128.
    llama = {}
    for bits, row in ((4, "llama7b_decode_gemv_awq"), (3, "llama7b_decode_gemv_awq_3bit")):
        per = {}
        for i in range(7):
            lin = synth.llama7b_linear(i)
            W = torch.from_numpy(lin.W).to(dev)
            s = torch.from_numpy(lin.act_scale).to(dev)
            x = torch.from_numpy(lin.X[0]).to(dev)
            nb = gemv_bytes(lin.N, lin.K, bits, 128, True, act_scale=True)
            R = rotate_count(nb)
            sets = [ops.quantize_pack(W, bits, 128, True, s) for _ in range(R)]
            y = torch.empty(lin.N, dtype=torch.float16, device=dev)
            us = burst_us(torch, [lambda j=j: ops.gemv(x, *sets[j % R], lin.N, lin.K, bits, 128, s, out=y)
                                  for j in range(10 * R)])
            sel = np.arange(0, lin.N, max(1, lin.N // 256))
            per[lin.name] = {"us": round(us, 3), "gbs": round(nb / us / 1e3, 1),
                             "frac_hbm": round(nb / us / 1e3 / HBM_PEAK_GBS, 4), "bytes": nb}
            record(row, lin.name, lin, y[None, :], lin.act_scale, sel, bits=bits)
            del sets, W
        rows[row] = per
        if bits == 4:
            llama = per

    # The decode shape (M = 1, K = N = 8192) with the other quantizers of the
    # workload: 4-bit symmetric, 3-bit asymmetric and symmetric, g128 (the
    # headline 4-bit asymmetric figure is the bench value).
    lin = synth.decode_8k()
    var = {}
    for bits, asym in ((4, False), (3, True), (3, False)):
        ms, vb, y = time_gemv_variant(torch, ops, synth, lin, bits, asym)
        key = f"{bits}bit_{'asym' if asym else 'sym'}"
        var[key] = {"us": round(ms * 1e3, 3), "gbs": round(vb / (ms * 1e-3) / 1e9, 1),
                    "frac_hbm": round(vb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "bytes": vb}
        record("decode_gemv_quantizers_k8192_n8192", key, lin, y[None, :], None, np.arange(0, lin.N, 32),
               bits=bits, asym=asym)
    rows["decode_gemv_quantizers_k8192_n8192"] = var

    # Fused projections: q/k/v (N = 3 x 4096) and gate/up (N = 2 x 11008) share
    # the input and its AWQ scale, so one launch over the stacked rows serves
    # them; compared with the sum of the separate launches above.
    fused = {}
    for name, idx in (("qkv", [0, 1, 2]), ("gate_up", [4, 5])):
        lins = [synth.llama7b_linear(i) for i in idx]
        K = lins[0].K
        s = torch.from_numpy(lins[0].act_scale).to(dev)
        x = torch.from_numpy(lins[0].X[0]).to(dev)
        Ws = [torch.from_numpy(l.W).to(dev) for l in lins]
        N = sum(l.N for l in lins)
        nb = gemv_bytes(N, K, 4, 128, True, act_scale=True)
        R = rotate_count(nb)
        sets = [ops.quantize_pack_fused(Ws, 4, 128, True, s) for _ in range(R)]
        us = burst_us(torch, [lambda j=j: ops.gemv_fused(x, *sets[j % R], K, 4, 128, s) for j in range(10 * R)])
        sep = sum(llama[l.name]["us"] for l in lins)
        fused[name] = {"N": N, "K": K, "us": round(us, 3), "gbs": round(nb / us / 1e3, 1),
                       "frac_hbm": round(nb / us / 1e3 / HBM_PEAK_GBS, 4), "bytes": nb,
                       "separate_us_sum": round(sep, 3), "speedup_vs_separate": round(sep / us, 3)}
        del sets, Ws
    rows["fused_projection_gemv_awq"] = fused

    # Group sizes 32 / 64 / K on the decode shape (M=1, K=N=8192, 4-bit asym).
    lin = synth.decode_8k()
    W = torch.from_numpy(lin.W).to(dev)
    x = torch.from_numpy(lin.X[0]).to(dev)
    gs = {}
    for G in (32, 64, 128, lin.K):
        nb = gemv_bytes(lin.N, lin.K, 4, G, True)
        R = rotate_count(nb)
        sets = [ops.quantize_pack(W, 4, G, True) for _ in range(R)]
        y = torch.empty(lin.N, dtype=torch.float16, device=dev)
        us = burst_us(torch, [lambda j=j: ops.gemv(x, *sets[j % R], lin.N, lin.K, 4, G, out=y) for j in range(10 * R)])
        gs[f"G{G}"] = {"us": round(us, 3), "gbs": round(nb / us / 1e3, 1),
                       "frac_hbm": round(nb / us / 1e3 / HBM_PEAK_GBS, 4), "bytes": nb}
        del sets
    del W
    rows["group_size_gemv_k8192_n8192"] = gs

    # Small-batch GEMM, M = 4 / 16 / 64, K = 8192, N = 28672.
    small = {}
    W, W_np = None, None
    for xdtype in ("f16", "bf16"):
        for M in (4, 16, 64):
            lin = synth.small_batch(M, xdtype, W=W_np)
            W_np = lin.W
            if W is None:
                W = torch.from_numpy(lin.W).to(dev)
                nbw = gemv_bytes(lin.N, lin.K, 4, 128, True, M=0)
                R = rotate_count(nbw)
                sets = [ops.quantize_pack(W, 4, 128, True) for _ in range(R)]
            X = x_tensor(lin.X, xdtype)
            Y = torch.empty(M, lin.N, dtype=X.dtype, device=dev)
            nb = gemv_bytes(lin.N, lin.K, 4, 128, True, M=M)
            us = burst_us(torch, [lambda j=j: ops.gemm(X, *sets[j % R], lin.N, lin.K, 4, 128, out=Y)
                                  for j in range(4 * R)])
            sel = np.arange(0, lin.N, lin.N // 128)
            small[f"M{M}_{xdtype}"] = {"us": round(us, 2), "gbs": round(nb / us / 1e3, 1),
                                    "frac_hbm": round(nb / us / 1e3 / HBM_PEAK_GBS, 4),
                                    "tflops": round(2 * M * lin.N * lin.K / us / 1e6, 1), "bytes": nb}
            record("small_batch_gemm_k8192_n28672", f"M{M}_{xdtype}", lin, Y, None, sel)
    # Crossover from the M = 1 GEMV (dot2 on the VALU) to the MFMA kernels on
    # the same weights: the GEMV per row of X against one GEMM launch.
    cross = {}
    for M in (1, 2, 8, 32):
        lin = synth.small_batch(M, "f16", W=W_np)
        X = x_tensor(lin.X, "f16")
        Y = torch.empty(M, lin.N, dtype=X.dtype, device=dev)
        nb = gemv_bytes(lin.N, lin.K, 4, 128, True, M=M)
        if M == 1:
            us = burst_us(torch, [lambda j=j: ops.gemv(X[0], *sets[j % R], lin.N, lin.K, 4, 128, out=Y[0])
                                  for j in range(4 * R)])
        else:
            us = burst_us(torch, [lambda j=j: ops.gemm(X, *sets[j % R], lin.N, lin.K, 4, 128, out=Y)
                                  for j in range(4 * R)])
        cross[f"M{M}"] = {"us": round(us, 2), "us_per_row": round(us / M, 2),
                          "frac_hbm": round(nb / us / 1e3 / HBM_PEAK_GBS, 4),
                          "kernel": "gemv (VALU dot2)" if M == 1 else "gemm (MFMA)"}
    small["crossover_f16"] = cross
    del sets, W
    rows["small_batch_gemm_k8192_n28672"] = small

    # Prefill GEMM, M = 2048, K = 4096, N = 11008.
    lin = synth.prefill()
    W = torch.from_numpy(lin.W).to(dev)
    sets = [ops.quantize_pack(W, 4, 128, True) for _ in range(4)]
    pre = {}
    for xdtype in ("f16", "bf16"):
        X = torch.from_numpy(lin.X).to(dev)
        if xdtype == "bf16":
            X = X.float().to(torch.bfloat16)
        Y = torch.empty(lin.M, lin.N, dtype=X.dtype, device=dev)
        us = burst_us(torch, [lambda j=j: ops.gemm(X, *sets[j % 4], lin.N, lin.K, 4, 128, out=Y)
                              for j in range(12)])
        fl = 2 * lin.M * lin.N * lin.K
        entry = {"us": round(us, 1), "tflops": round(fl / us / 1e6, 1),
                 "frac_mfma": round(fl / us / 1e6 / MFMA_F16_PEAK_TFLOPS, 4), "flop": fl}
        sel = np.arange(0, lin.N, lin.N // 96)
        if xdtype == "f16":
            record("prefill_gemm_m2048_k4096_n11008", xdtype, lin, Y, None, sel)
        else:
            Xb = X.view(torch.int16).cpu().numpy().view(np.uint16)
            record("prefill_gemm_m2048_k4096_n11008", xdtype, lin, Y, None, sel, X=Xb, xdtype="bf16")
        pre[xdtype] = entry
    del sets, W
    rows["prefill_gemm_m2048_k4096_n11008"] = pre

    # AWQ exponent search (20 exponents) for the q_proj shape on 512
    # calibration tokens with 1% outlier channels: per exponent one scale,
    # quantize_pack, prefill-size GEMM and error reduction.
    lin = synth.llama7b_linear(0)
    ch = lin.extra["channels"]
    Xc = torch.from_numpy(synth.to_f16(synth.activations_f32(synth.CALIBRATION_TOKENS, lin.K, 3200, ch))).to(dev)
    Wq = torch.from_numpy(lin.W).to(dev)
    ops.awq_search(Xc, Wq, 4, 128, True, 20)
    torch.cuda.synchronize()
    us = burst_us(torch, [lambda: ops.awq_search(Xc, Wq, 4, 128, True, 20)], reps=3)
    losses, _, best = ops.awq_search(Xc, Wq, 4, 128, True, 20)
    L = losses.cpu().numpy()
    b = int(best.cpu().numpy()[0])
    T, N, K = synth.CALIBRATION_TOKENS, lin.N, lin.K
    rows["awq_search_q_proj"] = {"T": T, "N": N, "K": K, "n_grid": 20, "ms": round(us / 1e3, 3),
                                 "gemm_flop": 20 * 2 * T * N * K, "best_alpha": b / 20,
                                 "loss_best_over_rtn": float(f"{L[b] / L[0]:.4g}")}
    del Xc, Wq

    # GPTQ of the q_proj shape (N = K = 4096) on 2048 correlated calibration
    # tokens, 4-bit asym g128; the layer objective ||X (W - w_hat)^T||^2 is
    # compared with RTN's (fp32 products on the device, fp64 sums).
    T, N, K = 2048, 4096, 4096
    Xg = torch.from_numpy(synth.correlated_activations(T, K, 6001)).to(dev)
    Wg = torch.from_numpy(synth.weights(N, K, 6002)).to(dev)
    ops.gptq(Xg, Wg, 4, 128, True)
    torch.cuda.synchronize()
    us = burst_us(torch, [lambda: ops.gptq(Xg, Wg, 4, 128, True)], reps=3)

    def layer_loss(q):
        D = Wg.float() - ops.dequantize(q[0], q[1], q[2], N, K, 4, 128)
        return float(((Xg.float() @ D.T).double() ** 2).sum())

    lg, lr = layer_loss(ops.gptq(Xg, Wg, 4, 128, True)), layer_loss(ops.quantize_pack(Wg, 4, 128, True))
    # algorithmic fp64 flops: lower triangle of 2 X^T X, Cholesky, triangular
    # inverse, and the error propagation into later columns
    flop = T * K * (K + 1) + K ** 3 / 3 + K ** 3 / 3 + N * K * K
    rows["gptq_q_proj"] = {"T": T, "N": N, "K": K, "ms": round(us / 1e3, 3), "fp64_flop": flop,
                           "tflops": round(flop / us / 1e6, 2),
                           "frac_fp64": round(flop / us / 1e6 / FP64_PEAK_TFLOPS, 4),
                           "loss_gptq_over_rtn": float(f"{lg / lr:.4g}")}
    del Xg, Wg

    # quantize_pack over 32 layers of the LLaMA-2-7B linear shapes (weights
    # generated on the device, seed 5100 + layer, all 32 layers resident:
    # 13 GB of fp16), 4-bit asym g128: one woq_quantize_pack call per matrix,
    # each layer's 7 back to back; then woq_quantize_pack_many over all 224
    # matrices (32 per launch) into a second set of outputs.
    shapes = [(N, K) for _, N, K in synth.LLAMA7B_LINEARS]
    total_bytes, total_us = 0, 0.0
    g = torch.Generator(device=dev)
    layers = []
    for layer in range(32):
        g.manual_seed(5100 + layer)
        Ws = [(torch.randn(N, K, generator=g, device=dev) * 0.02).half() for N, K in shapes]
        outs = [ops.quantize_pack(w, 4, 128, True) for w in Ws]
        total_us += burst_us(torch, [lambda w=w, o=o: ops.quantize_pack(w, 4, 128, True, out=o)
                                     for w, o in zip(Ws, outs)], reps=1) * len(Ws)
        total_bytes += sum(quantize_pack_bytes(N, K, 4, 128, True) for N, K in shapes)
        if layer == 0:
            checks.append(("quantize_pack", "quantize_pack_32_layers", "sampled_bytes_equal",
                           Ws[0][:256].cpu().numpy(), tuple(t[:256].cpu().numpy() for t in outs[0])))
        layers.append(Ws)
        del outs
    all_W = [w for Ws in layers for w in Ws]
    many_outs = [(torch.empty((w.shape[0], w.shape[1] // 2), dtype=torch.uint8, device=dev),
                  torch.empty((w.shape[0], w.shape[1] // 128), dtype=torch.float16, device=dev),
                  torch.empty((w.shape[0], w.shape[1] // 128), dtype=torch.float16, device=dev)) for w in all_W]
    ops.quantize_pack_many(all_W, 4, 128, True, None, many_outs)  # validated once through the binding
    from weight_only_quantization_quantize_amd import _lib
    lib, stream = _lib.load(), torch.cuda.current_stream().cuda_stream
    descs = (_lib.QMatrix * len(all_W))(*[
        _lib.QMatrix(w.data_ptr(), None, p.data_ptr(), sc.data_ptr(), z.data_ptr(), w.shape[0], w.shape[1])
        for w, (p, sc, z) in zip(all_W, many_outs)])

    def many():
        _lib.check(lib.woq_quantize_pack_many(ctypes.addressof(descs), len(all_W), 4, 128, 1, stream),
                   "woq_quantize_pack_many")

    many_us = burst_us(torch, [many], reps=2)
    checks.append(("quantize_pack", "quantize_pack_32_layers", "many_sampled_bytes_equal",
                   all_W[0][:256].cpu().numpy(), tuple(t[:256].cpu().numpy() for t in many_outs[0])))
    del layers, all_W, many_outs
    rows["quantize_pack_32_layers"] = {
        "ms": round(total_us / 1e3, 3), "bytes": total_bytes, "gbs": round(total_bytes / total_us / 1e3, 1),
        "frac_hbm": round(total_bytes / total_us / 1e3 / HBM_PEAK_GBS, 4),
        "many": {"ms": round(many_us / 1e3, 3), "launches": -(-224 // 32),
                 "gbs": round(total_bytes / many_us / 1e3, 1),
                 "frac_hbm": round(total_bytes / many_us / 1e3 / HBM_PEAK_GBS, 4)}}
    return rows


STREAM_SHAPES = [(b, t, u) for t in (256, 512, 1024) for b in (256, 512, 1024, 2048) for u in (1, 2, 4)]


def time_ceilings(torch, dev):
    """What the chip sustains with no decode at all, measured the same way as
    the quantized kernels (HIP events around back-to-back launches):

    * a read-only stream of the decode GEMV's bytes (35,684,352: codes, scales,
      zeros, x, y at M = 1, K = N = 8192, 4-bit asym g128) over rotated
      buffers, for each launch shape in STREAM_SHAPES (blocks, threads, loads
      in flight per thread);
    * an empty launch back to back (one 64-thread block, and 1024 blocks of
      512 threads, the GEMV's launch shape);
    * fp16 MFMA (v_mfma_f32_32x32x16_f16) on random operands, 512 workgroups
      of 4 waves (two per compute unit), about 5 ms per launch."""
    from weight_only_quantization_quantize_amd import _lib

    lib = _lib.load()
    stream = torch.cuda.current_stream().cuda_stream
    out = {}
    nb = gemv_bytes(8192, 8192, 4, 128, True)
    R = rotate_count(nb)
    bufs = [torch.randint(0, 255, (nb,), dtype=torch.uint8, device=dev) for _ in range(R)]
    sink = torch.empty(2048 * 1024, dtype=torch.int32, device=dev)

    def read(j, b, t, u):
        _lib.check(lib.woq_probe_stream_read(bufs[j % R].data_ptr(), nb, b, t, u, sink.data_ptr(), 0, stream),
                   "woq_probe_stream_read")

    shapes = {}
    for b, t, u in STREAM_SHAPES:
        us = burst_us(torch, [lambda j=j, b=b, t=t, u=u: read(j, b, t, u) for j in range(4 * R)])
        shapes[f"{b}x{t}x{u}"] = round(us, 3)
    best = min(shapes, key=shapes.get)
    out["stream_read_35684352B"] = {
        "bytes": nb, "rotated_buffers": R, "us_by_shape_blocks_x_threads_x_unroll": shapes, "best_shape": best,
        "best_us": shapes[best], "best_gbs": round(nb / shapes[best] / 1e3, 1),
        "best_frac_hbm": round(nb / shapes[best] / 1e3 / HBM_PEAK_GBS, 4),
        "gemv_shape_us": shapes["1024x512x4"]}
    for b, t in ((1, 64), (1024, 512)):
        us = burst_us(torch, [lambda b=b, t=t: _lib.check(lib.woq_probe_empty(b, t, stream), "woq_probe_empty")
                              for _ in range(256)])
        out[f"empty_launch_{b}x{t}"] = {"us": round(us, 3)}
    src = torch.randn(1 << 19, device=dev).to(torch.float16)   # 1 MiB of N(0, 1) fp16 operands
    msink = torch.empty(512 * 256, dtype=torch.float32, device=dev)
    iters = 40000
    launch = lambda: _lib.check(lib.woq_probe_mfma_rate(src.data_ptr(), 512, iters, msink.data_ptr(), 0, stream),
                                "woq_probe_mfma_rate")
    launch()
    us = burst_us(torch, [launch, launch, launch], reps=2)
    fl = 512 * 4 * iters * 4 * 2 * 32 * 32 * 16
    out["mfma_f16_32x32x16_random_operands"] = {
        "us": round(us, 1), "tflops": round(fl / us / 1e6, 1), "frac_mfma": round(fl / us / 1e6 / MFMA_F16_PEAK_TFLOPS, 4)}
    out["mfma_valu_coissue"] = time_mfma_valu(torch, dev, lib, stream)
    del bufs
    return out


def time_mfma_valu(torch, dev, lib, stream):
    """Whether VALU work hides under MFMAs on one SIMD, and the clock it runs at:
    512 workgroups of 4 waves (two per SIMD), 20000 steps of 4 fp16 32x32x16
    MFMAs and/or 16-64 integer VALU operations per wave (committed probe
    woq_probe_mfma_valu).  'clock_ghz' is the shader clock counter's rate
    against the 100 MHz real-time counter, median over workgroups."""
    from weight_only_quantization_quantize_amd import _lib

    src = torch.randn(1 << 19, device=dev).to(torch.float16)
    blocks, iters = 512, 20000
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    clocks = torch.zeros(4 * blocks, dtype=torch.int64, device=dev)
    out = {"blocks": blocks, "waves_per_simd": 2, "iters": iters}
    for nm, nv in ((4, 0), (4, 16), (4, 32), (4, 64), (0, 32), (0, 64)):
        def launch():
            _lib.check(lib.woq_probe_mfma_valu(src.data_ptr(), blocks, iters, nm, nv, sink.data_ptr(),
                                               clocks.data_ptr(), 0, stream), "woq_probe_mfma_valu")
        launch()
        us = burst_us(torch, [launch, launch], reps=2)
        c = clocks.view(-1, 4).cpu().numpy().astype(np.float64)
        ghz = float(np.median((c[:, 1] - c[:, 0]) / np.maximum(c[:, 3] - c[:, 2], 1) * 0.1))
        out[f"mfma{nm}_valu{nv}"] = {"us": round(us, 1), "clock_ghz": round(ghz, 3)}
    t = {k: v["us"] for k, v in out.items() if isinstance(v, dict)}
    for nv in (32, 64):
        mixed, m, v = t[f"mfma4_valu{nv}"], t["mfma4_valu0"], t[f"mfma0_valu{nv}"]
        out[f"valu{nv}_overlap"] = {"mixed_over_max": round(mixed / max(m, v), 3),
                                    "mixed_over_sum": round(mixed / (m + v), 3)}
    return out


def time_gemv_timeline(torch, dev, lib, stream, x, sets, N, y):
    """Per-wave timeline of the K = N = 8192 decode GEMV (the library kernel's
    own instance with timeline stamps, committed probe woq_probe_gemv_timeline):
    a burst of 32 back-to-back launches over the rotated packed sets; medians
    over launches 8..31 of the launch span (first wave start to last wave
    end), the idle gap before the next launch, and per-wave times from the
    launch's first start, in us (100 MHz counter: 0.01 us resolution)."""
    from weight_only_quantization_quantize_amd import _lib

    words = int(lib.woq_probe_gemv_timeline_words(N))
    L, R = 32, len(sets)
    tl = torch.zeros(L, words, dtype=torch.int64, device=dev)

    def launch(j):
        p, s, z = sets[j % R]
        _lib.check(lib.woq_probe_gemv_timeline(x.data_ptr(), p.data_ptr(), s.data_ptr(), z.data_ptr(), N,
                                               y.data_ptr(), tl[j].data_ptr(), words, stream),
                   "woq_probe_gemv_timeline")
    burst_us(torch, [lambda j=j: launch(j) for j in range(L)], reps=1)
    T = tl.view(L, -1, 8).cpu().numpy().astype(np.float64) / 100.0   # us
    span, gap, xr, first, end = [], [], [], [], []
    for j in range(8, L):
        t = T[j]
        t0 = t[:, 0].min()
        span.append(t[:, 4].max() - t0)
        if j + 1 < L:
            gap.append(T[j + 1][:, 0].min() - t[:, 4].max())
        xr.append(np.percentile(t[:, 1] - t[:, 0], [10, 50, 90]))
        first.append(np.percentile(t[:, 2] - t0, [10, 50, 90]))
        end.append(np.percentile(t[:, 4] - t0, [10, 50, 90]))
    med = lambda a: [round(float(v), 2) for v in np.median(np.array(a), axis=0)]
    return {"waves": int(T.shape[1]), "launches": L - 8,
            "span_us": round(float(np.median(span)), 2), "gap_to_next_launch_us": round(float(np.median(gap)), 2),
            "x_staged_after_start_us_p10_p50_p90": med(xr),
            "first_step_done_us_p10_p50_p90": med(first),
            "wave_end_us_p10_p50_p90": med(end)}


def row_checks(checks, rows):
    """The oracle on the samples time_rows kept: relative L2 of each sampled
    GEMV/GEMM output against the fp64 oracle on the same dequantized weights,
    and byte equality of the sampled quantize_pack rows."""
    from oracle import woq_oracle as O

    for c in checks:
        if c[0] == "gemm":
            _, row, key, Wsel, X, xdtype, s, ysel, (bits, G, asym) = c
            _, _, _, q = O.quantize_pack(Wsel, bits, G, asym, s)
            ref = O.gemm(O.activations_f64(X, xdtype), O.dequantize(q), s)
            rows[row][key]["rel_l2_sampled"] = float(f"{O.rel_l2(ysel, ref):.3g}")
        else:
            _, row, key, W0, (p, sc, z) = c
            rp, rs, rz, _ = O.quantize_pack(W0, 4, 128, True)
            rows[row][key] = bool(np.array_equal(p, rp) and np.array_equal(sc.view(np.uint16), rs.view(np.uint16))
                                  and np.array_equal(z.view(np.uint16), rz.view(np.uint16)))


def rotate_count(bytes_per_set, minimum=4):
    return max(minimum, int(np.ceil(2 * MALL_BYTES / bytes_per_set)) + 1)


def time_gemv_variant(torch, ops, synth, lin, bits, asym, iters=100):
    """Average GEMV kernel duration (ms) over rotated packed sets."""
    N, K, G = lin.N, lin.K, 128
    W = torch.from_numpy(lin.W).cuda()
    x = torch.from_numpy(lin.X[0]).cuda()
    nb = gemv_bytes(N, K, bits, G, asym)
    R = rotate_count(nb)
    sets = [ops.quantize_pack(W, bits, G, asym) for _ in range(R)]
    y = torch.empty(N, dtype=torch.float16, device="cuda")
    for i in range(10):
        ops.gemv(x, *sets[i % R], N, K, bits, G, out=y)
    torch.cuda.synchronize()
    torch.cuda._sleep(PREFILL_CYCLES)
    t = Timer(torch)
    e = t.start()
    for i in range(iters):
        ops.gemv(x, *sets[i % R], N, K, bits, G, out=y)
    t.stop(e)
    torch.cuda.synchronize()
    ms = t.mean_ms() / iters
    del sets
    return ms, nb, y


def host_cores():
    """Host threads available to this process: the affinity set, capped by the
    job's OMP_NUM_THREADS share when that is set."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS")
    return min(n, int(cap)) if cap and cap.isdigit() and int(cap) > 0 else n


def cpu_baseline(lin, packed_gpu, bits, G, asym, y_gpu):
    """Time the oracle (as it stands) on the host: one full quantize_pack and
    one unpack + dequantize + fp64 GEMV of the whole decode workload, BLAS on
    every host core this process may use (numpy's element-wise steps run on
    one)."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import woq_oracle as O

    cores = host_cores()
    with threadpool_limits(limits=cores):
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        t0 = time.perf_counter()
        ref_packed, ref_scales, ref_zeros, q = O.quantize_pack(lin.W, bits, G, asym)
        t_quant = time.perf_counter() - t0
        t0 = time.perf_counter()
        codes = O.unpack_v2(ref_packed, bits, lin.K)
        qq = O.Quantized(codes, ref_scales, ref_zeros, bits, G, asym)
        y_ref = O.gemm(lin.X.astype(np.float64), O.dequantize(qq))[0]
        t_gemv = time.perf_counter() - t0
    parity = {
        "packed_equal": bool(np.array_equal(packed_gpu[0], ref_packed)),
        "scales_equal": bool(np.array_equal(packed_gpu[1].view(np.uint16), ref_scales.view(np.uint16))),
        "zeros_equal": bool(ref_zeros is None or np.array_equal(packed_gpu[2].view(np.uint16),
                                                                ref_zeros.view(np.uint16))),
        "gemv_rel_l2": O.rel_l2(y_gpu, y_ref),
    }
    nb = gemv_bytes(lin.N, lin.K, bits, G, asym)
    base = {
        "value": nb / t_gemv / 1e9,
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"one full M=1 K=N={lin.K} GEMV from the packed weights (unpack + dequantize + fp64 matvec, "
                   f"{t_gemv:.2f} s) and one full quantize_pack ({t_quant:.2f} s); numpy, BLAS on {blas_threads} "
                   f"threads ({cores} host cores), element-wise steps on 1"),
        "gemv_s": t_gemv,
        "quantize_pack_s": t_quant,
    }
    return base, parity


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path is not sharded "
              "across GPUs by this library)", file=sys.stderr)
        sys.exit(2)

    if args.write_traffic:
        write_traffic(args.write_traffic, args.copy_mib)
        return
    if args.write_trace:
        write_trace(args.write_trace)
        return

    import torch

    from weight_only_quantization_quantize_amd import _lib, ops, synth

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = args.copy_calibration << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        a.fill_(1)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n}), flush=True)
        return
    if args.gemm_only:
        # W ~ N(0, 0.02), X ~ N(0, 1), drawn on the device from fixed seeds
        M, N, K = (int(v) for v in args.gemm_only.split(","))
        g = torch.Generator(device=dev).manual_seed(7000)
        W = (torch.randn(N, K, generator=g, device=dev) * 0.02).to(torch.float16)
        X = torch.randn(M, K, generator=g, device=dev).to(torch.float16)
        packed, scales, zeros = ops.quantize_pack(W, 4, 128, True)
        Y = torch.empty(M, N, dtype=torch.float16, device=dev)
        for _ in range(5):
            ops.gemm(X, packed, scales, zeros, N, K, 4, 128, out=Y)
        torch.cuda.synchronize()
        print(json.dumps({"gemm_only": [M, N, K], "launches": 5}), flush=True)
        return
    _lib.load()
    torch.cuda.set_device(dev)
    bits, G, asym = 4, 128, True
    lin = synth.decode_8k()
    N, K = lin.N, lin.K

    # Resident inputs: rotated fp16 weight copies and packed sets.
    W0 = torch.from_numpy(lin.W).to(dev)
    nW = 4  # 4 x 134 MB > 2 x MALL
    Ws = [W0] + [W0.clone() for _ in range(nW - 1)]
    x = torch.from_numpy(lin.X[0]).to(dev)
    nb = gemv_bytes(N, K, bits, G, asym)
    R = rotate_count(nb)
    sets = [ops.quantize_pack(W0, bits, G, asym) for _ in range(R)]
    y = torch.empty(N, dtype=torch.float16, device=dev)
    torch.cuda.synchronize()

    tq, tg = Timer(torch), Timer(torch)
    counter = [0]

    def step(i, timed):
        dst = sets[i % R]
        if timed:
            e = tq.start()
        ops.quantize_pack(Ws[i % nW], bits, G, asym, None, out=dst)
        if timed:
            tq.stop(e)
            e = tg.start()
        for _ in range(GEMV_BURST):
            counter[0] += 1
            j = counter[0] % R
            if j == i % R:  # never the set this step's quantize_pack just wrote (cache-resident)
                counter[0] += 1
                j = counter[0] % R
            ops.gemv(x, *sets[j], N, K, bits, G, out=y)
        if timed:
            tg.stop(e)

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    torch.cuda._sleep(PREFILL_CYCLES)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(args.steps):
        step(args.warmup + i, True)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = ev0.elapsed_time(ev1)
    gemv_ms = tg.mean_ms() / GEMV_BURST
    qp_ms = tq.mean_ms()

    achieved = nb / (gemv_ms * 1e-3) / 1e9
    qp_nb = quantize_pack_bytes(N, K, bits, G, asym)
    result = {
        "metric": METRIC,
        "value": round(achieved, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "decode GEMV M=1 K=8192 N=8192, 4-bit asymmetric zero-point RTN, group 128, fp16 "
                        "activations, fp32 accumulate; weights N(0,0.02) with 0.1% N(0,0.5) outliers",
            "M": 1, "K": K, "N": N, "bits": bits, "group_size": G, "asymmetric": asym,
            "rotated_sets": R, "step": f"quantize_pack + {GEMV_BURST} back-to-back gemv",
        },
        "gemv_us": round(gemv_ms * 1e3, 3),
        "gemv_pct_hbm_peak": round(100 * achieved / HBM_PEAK_GBS, 2),
        "quantize_pack_us": round(qp_ms * 1e3, 2),
        "quantize_pack_gbs": round(qp_nb / (qp_ms * 1e-3) / 1e9, 1),
        "wall_s": round(wall, 3),
        "roofline": {
            "bound": "hbm",
            "kernel": "gemv_kernel<4-bit, asymmetric, f16>",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "frac_statistic": f"mean GEMV duration from HIP events on the launch stream around each step's burst "
                              f"of {GEMV_BURST} back-to-back launches (inter-kernel gaps included)",
            "trace": trace_entry(nb),
            "traffic": measured_traffic(),
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "bytes_per_launch": nb,
        },
    }

    checks = []
    if not args.no_rows:
        del Ws, W0
        result["rows"] = time_rows(torch, ops, synth, checks)
        result["rows"]["gemv_timeline_k8192_n8192"] = time_gemv_timeline(
            torch, dev, _lib.load(), torch.cuda.current_stream().cuda_stream, x, sets, N, y)

    if not args.no_cpu_baseline:
        ops.gemv(x, *sets[0], N, K, bits, G, out=y)
        torch.cuda.synchronize()
        host_sets = (sets[0][0].cpu().numpy(), sets[0][1].cpu().numpy(), sets[0][2].cpu().numpy())
        base, parity = cpu_baseline(lin, host_sets, bits, G, asym, y.cpu().numpy().astype(np.float64))
        result["cpu_baseline"] = base
        result["parity"] = parity
        if "rows" in result:
            row_checks(checks, result["rows"])

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
