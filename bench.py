#!/usr/bin/env python3
"""Throughput of the TTQ linear projection on one MI355X.

One step = one full TTQ projection call (activation statistics, on-the-fly
group quantize-dequantize of W D^{1/2}, contraction with X on the matrix
cores) on the 4096 x 4096 attention-projection workload at decode, T = 1:
4-bit, group 128, p = 2, lambda = 1e-3, alpha = 0.5, activations with 1 % of
channels scaled log-uniformly by 10-100x and a new outlier set every call.

Inputs are resident in HBM before the timed region; the weight matrix
rotates over enough distinct copies (> 512 MB) that it is read from HBM, not
from the 256 MB Infinity Cache, as in a real model where every layer has
its own weights.  The JSON line also carries: the roofline of the dominant
kernel (event-timed launches), the oracle timed on the host cores
(cpu_baseline), a plain bf16 GEMM of the same shape (hipBLASLt via torch) for
the pages' overhead ratio rho = 1/d' + 3/T, the same step under a HIP graph,
and the T = 128 case of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("TTQ-linear tokens/s per projection + % HBM/MFMA roofline; "
          "overhead vs bf16 GEMM")
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
ROTATE_BYTES = 640 * 2 ** 20
FORMAT_NAMES = {"asym": "asymmetric", "sym": "symmetric",
                "intzp": "integer zero point", "fp8": "FP8 E4M3"}
KERNEL_SOURCES = {"gemv_t1": "k_gemv.hip", "fused_qdq_mfma": "k_fused.hip",
                  "stats_small": "k_stats.hip", "gemm_mfma": "k_gemm.hip",
                  "quant_what": "k_quant.hip"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--T", type=int, default=1)
    ap.add_argument("--qformat", default="asym",
                    choices=("asym", "sym", "intzp", "fp8"),
                    help="quantizer format of the timed step (fp8: 8-bit "
                         "E4M3 codes; the others 4-bit)")
    ap.add_argument("--no-cpu", action="store_true",
                    help="skip the oracle cpu_baseline leg")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--only-decode", action="store_true",
                    help="time only the one-token decode from stored codes")
    ap.add_argument("--only-segmented", action="store_true",
                    help="time only the continuous-batching call")
    ap.add_argument("--only-pca", action="store_true",
                    help="time only the PCA low-rank factorisation "
                         "(4096 x 4096, r = 64) and print its JSON")
    ap.add_argument("--only-ttq", action="store_true",
                    help="time only the TTQ step (for profiler runs)")
    ap.add_argument("--copy-calib-mb", type=int, default=0,
                    help="after the timed work, run 5 device-to-device copies "
                         "of this many MiB (counter calibration)")
    ap.add_argument("--summarize", nargs=3, metavar=("TRACE", "FETCH", "WRITE"),
                    help="write profiles/ summaries from rocprofv3 output "
                         "directories (kernel trace, FETCH_SIZE, WRITE_SIZE)")
    ap.add_argument("--profile-cmd", default="",
                    help="command lines recorded in the summary")
    return ap.parse_args()


def kernel_src_sha(kernel: str) -> str:
    p = os.path.join(ROOT, "online_activation_aware_ttq_amd", "csrc",
                     KERNEL_SOURCES.get(kernel, "k_fused.hip"))
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def fmt_suffix(qformat: str) -> str:
    return "" if qformat == "asym" else f"_{qformat}"


def traffic_file(kernel: str, T: int, qformat: str = "asym") -> str:
    return os.path.join(ROOT, "profiles",
                        f"traffic_{kernel}_q_proj4096_T{T}{fmt_suffix(qformat)}.json")


def dev_bf16(bits, torch):
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(
        "cuda").view(torch.bfloat16)


def alg_bytes(d, d_out, T, rank=0):
    return 2 * d_out * d + 2 * T * d + 4 * T * d_out + 2 * rank * (d + d_out)


def alg_flops(d, d_out, T, rank=0):
    return 2 * d_out * d * T + 2 * rank * T * (d + d_out)


def format_bits(qformat: str) -> int:
    return 8 if qformat == "fp8" else 4


def measure(T: int, steps: int, warmup: int, torch, ttq, want_graph: bool,
            want_gemm: bool, qformat: str = "asym"):
    import numpy as np
    from workloads import configs as wc

    d = d_out = 4096
    prob = wc.make_c2(T=T)
    prob.bits = format_bits(qformat)
    w_bytes = 2 * d * d_out
    n_w = max(2, -(-ROTATE_BYTES // w_bytes))
    Ws = [dev_bf16(prob.W, torch)]
    for i in range(1, n_w):  # distinct copies of the same seeded W
        Ws.append(Ws[0].clone())
    n_x = 64
    Xs = [dev_bf16(wc.draw_x(1, 1000 + c, 1, T, d, "logu10_100", 41)[0], torch)
          for c in range(n_x)]
    n_y = 8
    Ys = [torch.empty(T, d_out, dtype=torch.float32, device="cuda")
          for _ in range(n_y)]
    kw = dict(p=prob.p, lam=prob.lam, alpha=prob.alpha, bits=prob.bits,
              group=prob.group, qformat=qformat)
    prm = ttq.make_params(d=d, d_out=d_out, T=T, bits=prob.bits,
                          group=prob.group, p=prob.p, lam=prob.lam,
                          alpha=prob.alpha, qformat=qformat)
    ws = torch.empty(ttq.ttq_workspace_bytes(prm), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def step(i):
        ttq.ttq_linear(Ws[i % n_w], Xs[i % n_x], Y=Ys[i % n_y], workspace=ws,
                       stream=stream, **kw)

    def timed(fn, n, w):
        for i in range(w):
            fn(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n  # ms per step

    out = {"T": T, "rotating_w_copies": n_w,
           "rotating_bytes": n_w * w_bytes}
    ms = timed(step, steps, warmup)
    out["ms_per_step"] = ms

    # per-kernel event timing over the same kind of steps
    ttq.timing_reset()
    ttq.timing_enable(True)
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    kt = ttq.timing_query()
    ttq.timing_enable(False)
    ttq.timing_reset()
    out["kernels_ms_avg"] = {k: v[0] / v[1] for k, v in kt.items() if v[1]}
    out["kernels_launches"] = {k: v[1] for k, v in kt.items() if v[1]}

    # hot-cache figure (same W every call) for context
    def step_hot(i):
        ttq.ttq_linear(Ws[0], Xs[i % n_x], Y=Ys[i % n_y], workspace=ws,
                       stream=stream, **kw)
    if want_graph:
        out["ms_per_step_hot_w"] = timed(step_hot, max(50, steps // 4), warmup)

    if want_graph:
        # one graph holding n_w calls (one per W copy), replayed
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(n_w):  # warm-up on the capture stream
                ttq.ttq_linear(Ws[i], Xs[i % n_x], Y=Ys[i % n_y], workspace=ws,
                               stream=s.cuda_stream, **kw)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            cs = torch.cuda.current_stream().cuda_stream
            for i in range(n_w):
                ttq.ttq_linear(Ws[i], Xs[i % n_x], Y=Ys[i % n_y], workspace=ws,
                               stream=cs, **kw)
        reps = max(1, steps // n_w)
        gms = timed(lambda i: g.replay(), reps, 3) / n_w
        out["ms_per_step_graph"] = gms

    if want_gemm:
        # plain bf16 GEMM of the same shape and cache policy (hipBLASLt)
        def gemm(i):
            torch.matmul(Xs[i % n_x], Ws[i % n_w].t())
        out["gemm_bf16_ms"] = timed(gemm, steps, warmup)
    del Ws, Xs, Ys, ws
    torch.cuda.empty_cache()
    return out


FP32_PEAK_TFLOPS = 157.3  # float32 peak, the vector units and the matrix instruction alike


def measure_pca(torch, ttq, reps: int = 10):
    """Low-rank factors by PCA on the same 4096 x 4096 weights shape: r = 64,
    two power iterations, static (context for the low-rank row; not the
    timed step)."""
    import numpy as np
    from workloads.configs import draw_lowrank_w, draw_omega
    d = d_out = 4096
    r, iters = 64, 2
    W = dev_bf16(draw_lowrank_w(1, d_out, d, r), torch)
    Om = torch.from_numpy(draw_omega(2, d, r)).cuda()
    prm = ttq.make_params(d=d, d_out=d_out, T=0, rank=r, bits=4, group=32,
                          p=2.0, lam=0.0, alpha=0.0)
    ws = torch.empty(ttq.ttq_lowrank_pca_workspace_bytes(prm, iters),
                     dtype=torch.uint8, device="cuda")
    f = lambda: ttq.ttq_lowrank_pca(W, Om, iters=iters, workspace=ws)
    for _ in range(2):
        f()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        f()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    ttq.timing_reset()
    ttq.timing_enable(True)
    for _ in range(reps):
        f()
    torch.cuda.synchronize()
    kt = {k: v[0] / reps for k, v in ttq.timing_query().items() if v[1]}
    ttq.timing_enable(False)
    ttq.timing_reset()
    # products with W: M Omega, 2 per power iteration, W^T Q for A (+ Gram
    # and substitution work on the d x r panels, not counted)
    flops_w = (2 + 2 * iters) * 2.0 * d_out * d * r
    sk = kt.get("pca_skinny", float("nan"))
    return {"shape": f"{d_out}x{d}, r={r}, {iters} power iterations",
            "ms": ms, "kernels_ms": kt,
            "skinny_tflops_w_products": flops_w / (sk * 1e-3) / 1e12,
            "skinny_frac_fp32_peak": flops_w / (sk * 1e-3) / 1e12 / FP32_PEAK_TFLOPS}


def measure_decode(torch, ttq, steps: int = 1000):
    """One token against codes stored by ttq_quantize (the same 4096 x 4096
    weights, 4-bit g128): 20 rotating stored copies, as for the main step."""
    from workloads import configs as wc
    d = d_out = 4096
    prob = wc.make_c2(T=16)
    W0 = dev_bf16(prob.W, torch)
    X0 = dev_bf16(prob.X[0], torch)
    kw = dict(bits=4, group=128)
    st = [ttq.ttq_quantize(W0, X0, p=prob.p, lam=prob.lam, alpha=prob.alpha, **kw)
          for _ in range(20)]
    Xs = [dev_bf16(wc.draw_x(1, 3000 + c, 1, 1, d, "logu10_100", 41)[0], torch)
          for c in range(64)]
    Y = torch.empty(1, d_out, dtype=torch.float32, device="cuda")
    prm = ttq.make_params(d=d, d_out=d_out, T=1, bits=4, group=128, p=1.0,
                          lam=0.0, alpha=0.0)
    ws = torch.empty(max(256, ttq.ttq_qmatmul_workspace_bytes(prm)),
                     dtype=torch.uint8, device="cuda")
    f = lambda i: ttq.ttq_qmatmul(*st[i % 20], Xs[i % 64], Y=Y, workspace=ws, **kw)
    for i in range(50):
        f(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        f(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    ttq.timing_reset()
    ttq.timing_enable(True)
    for i in range(steps):
        f(i)
    torch.cuda.synchronize()
    kt = {k: v[0] / v[1] for k, v in ttq.timing_query().items() if v[1]}
    ttq.timing_enable(False)
    ttq.timing_reset()
    # the same calls replayed from a HIP graph (no host work per call)
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        for i in range(20):
            ttq.ttq_qmatmul(*st[i], Xs[i], Y=Y, workspace=ws,
                            stream=cs.cuda_stream, **kw)
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        s = torch.cuda.current_stream().cuda_stream
        for i in range(20):
            ttq.ttq_qmatmul(*st[i], Xs[i], Y=Y, workspace=ws, stream=s, **kw)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // 20)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    gms = e0.elapsed_time(e1) / (reps * 20)
    G = d // 128
    alg = d_out * d // 2 + 8 * d_out * G + 2 * d + 4 * d + 4 * d_out
    k = kt.get("qgemv", float("nan"))
    return {"workload": "4096x4096, 4-bit g128 codes, one token", "ms_per_step": ms,
            "tokens_per_s": 1.0 / (ms * 1e-3), "ms_per_step_graph": gms,
            "tokens_per_s_graph": 1.0 / (gms * 1e-3), "kernel": "qgemv",
            "kernel_ms": k, "alg_bytes": alg,
            "hbm_frac_kernel": alg / (k * 1e-3) / 1e9 / HBM_PEAK_GBS}


def measure_segmented(torch, ttq, reps: int = 50):
    """Continuous batching on the same 4096 x 4096 weights (4-bit g128,
    r = 32): 22 requests of mixed lengths (16 single tokens, 4 of 3..16,
    one of 100, one of 200; 354 tokens) in one packed X, each with its own
    statistics -- one ttq_linear_segmented call against one ttq_linear call
    per request."""
    import numpy as np
    from workloads import configs as wc
    d = d_out = 4096
    prob = wc.make_problem("seg", d=d, d_out=d_out, T=1, bits=4, group=128,
                           rank=32, seed=11)
    lengths = [1] * 16 + [3, 7, 12, 16, 100, 200]
    rng = np.random.default_rng(12)
    lengths = [int(x) for x in rng.permutation(lengths)]
    xs = [wc.draw_x(500 + i, 0, 1, t, d, "logu10_100", 41)[0]
          for i, t in enumerate(lengths)]
    offs = [0] + [int(x) for x in np.cumsum(lengths)]
    W = dev_bf16(prob.W, torch)
    Bm, A = dev_bf16(prob.B, torch), dev_bf16(prob.A, torch)
    X = dev_bf16(np.concatenate(xs), torch)
    Xr = [dev_bf16(x, torch) for x in xs]
    kw = dict(p=prob.p, lam=prob.lam, alpha=prob.alpha, bits=4, group=128)
    Y = torch.empty(offs[-1], d_out, dtype=torch.float32, device="cuda")

    def seg():
        ttq.ttq_linear_segmented(W, X, Bm, A, seg_offsets=offs, Y=Y, **kw)

    def single():
        for i, x in enumerate(Xr):
            ttq.ttq_linear(W, x, Bm, A, Y=Y[offs[i]:offs[i + 1]], **kw)

    out = {"workload": f"4096x4096 4-bit g128 r=32, {len(lengths)} requests, "
                       f"{offs[-1]} tokens (16 x 1, 3, 7, 12, 16, 100, 200)"}
    for name, f in (("segmented", seg), ("one_call_per_request", single)):
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            f()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"ms": ms, "tokens_per_s": offs[-1] / (ms * 1e-3)}
    return out


def cpu_baseline(T: int, seconds: float, qformat: str = "asym"):
    """The oracle as it stands, on the host cores, on a bounded sample."""
    import numpy as np
    import oracle
    from workloads import configs as wc
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    prob = wc.make_c2(T=T)
    prob.bits = format_bits(qformat)
    calls = 0
    t0 = time.perf_counter()
    while True:
        X = wc.draw_x(1, 5000 + calls, 1, T, prob.d, "logu10_100", 41)[0]
        oracle.ttq_linear(prob.W, X, bits=prob.bits, group=prob.group,
                          p=prob.p, lam=prob.lam, alpha=prob.alpha,
                          qformat=qformat)
        calls += 1
        el = time.perf_counter() - t0
        if (el >= seconds and calls >= 3) or el >= 3 * seconds:
            break
    return {"value": calls * T / el, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{calls} full calls of the same workload (T={T}, "
                      f"d=d'=4096), X redrawn per call, {el:.1f} s wall, "
                      f"host cpu_count={os.cpu_count()}"}


def _read_csv(d, suffix):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)
    rows = []
    for f in files:
        rows += list(csv.DictReader(open(f)))
    return rows


def summarize(a):
    """profiles/: kernel-trace summary of the dominant kernel and the HBM
    traffic per launch from FETCH_SIZE / WRITE_SIZE, each scaled by what the
    same counter reads for a device-to-device copy of known size."""
    trace, fetch, write = a.summarize
    stats = _read_csv(trace, "kernel_stats.csv")
    T = a.T
    key = {1: "gemv", 128: "k_fused"}.get(T, "k_fused")
    kname = {1: "gemv_t1"}.get(T, "fused_qdq_mfma")
    calib_bytes = a.copy_calib_mb * 2 ** 20

    def per_dispatch(rows, counter, match):
        vals = [float(r["Counter_Value"]) for r in rows
                if r["Counter_Name"] == counter and match(r["Kernel_Name"])]
        return vals

    fr = _read_csv(fetch, "counter_collection.csv")
    wr = _read_csv(write, "counter_collection.csv")
    k_f = per_dispatch(fr, "FETCH_SIZE", lambda n: key in n)
    k_w = per_dispatch(wr, "WRITE_SIZE", lambda n: key in n)

    def calib(rows, counter):
        cp = [r for r in rows if r["Counter_Name"] == counter
              and "copyBuffer" in r["Kernel_Name"]]
        cp.sort(key=lambda r: int(r["Dispatch_Id"]))
        vals = [float(r["Counter_Value"]) for r in cp[-5:]]
        return sum(vals) / len(vals) if vals else float("nan")

    c_f, c_w = calib(fr, "FETCH_SIZE"), calib(wr, "WRITE_SIZE")
    sf = calib_bytes / (c_f * 1024) if c_f == c_f and c_f > 0 else float("nan")
    sw = calib_bytes / (c_w * 1024) if c_w == c_w and c_w > 0 else float("nan")
    f_kib = sum(k_f) / len(k_f)
    w_kib = sum(k_w) / len(k_w)
    traffic = f_kib * 1024 * sf + w_kib * 1024 * sw
    d = d_out = 4096
    ab = alg_bytes(d, d_out, T)
    fs = fmt_suffix(a.qformat)
    rec = {"kernel": kname, "workload": f"q_proj 4096x4096 T={T}",
           "qformat": a.qformat,
           "kernel_src_sha": kernel_src_sha(kname),
           "fetch_kib_per_launch": f_kib, "write_kib_per_launch": w_kib,
           "copy_calib_bytes": calib_bytes,
           "copy_fetch_kib": c_f, "copy_write_kib": c_w,
           "fetch_scale": sf, "write_scale": sw,
           "bytes_per_launch": traffic, "alg_bytes_per_launch": ab,
           "traffic_over_alg": traffic / ab,
           "launches_counted": [len(k_f), len(k_w)]}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    json.dump(rec, open(traffic_file(kname, T, a.qformat), "w"), indent=1)
    lines = [f"# {kname}: 4096x4096 q_proj, T={T} ({format_bits(a.qformat)}-bit "
             f"g128 {FORMAT_NAMES[a.qformat]}, p=2)", "",
             "Commands (from the repository root):", "", "```"]
    lines += [c for c in a.profile_cmd.split(";;") if c] + ["```", "",
              "## rocprofv3 --kernel-trace --stats (kernel_stats.csv)", "",
              "| kernel | calls | avg ns | min ns | max ns |",
              "|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| {r['Name'][:70]} | {r['Calls']} | "
                     f"{float(r['AverageNs']):.0f} | {r['MinNs']} | {r['MaxNs']} |")
    lines += ["", "## HBM traffic (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)", "",
              f"- kernel FETCH_SIZE {f_kib:.0f} KiB/launch, WRITE_SIZE {w_kib:.1f} KiB/launch"
              f" (averaged over {len(k_f)} / {len(k_w)} launches)",
              f"- calibration: device-to-device copy of {calib_bytes} bytes reads "
              f"FETCH_SIZE {c_f:.0f} KiB and WRITE_SIZE {c_w:.0f} KiB; scale "
              f"factors {sf:.4f} (fetch) and {sw:.4f} (write)",
              f"- traffic = {traffic / 1e6:.3f} MB/launch against "
              f"{ab / 1e6:.3f} MB algorithmic (ratio {traffic / ab:.3f})", ""]
    md = os.path.join(ROOT, "profiles", f"{kname}_q_proj4096_T{T}{fs}.md")
    open(md, "w").write("\n".join(lines))
    print(json.dumps(rec))


def traffic_entry(kernel: str, T: int, qformat: str = "asym"):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel source has changed since it was taken."""
    try:
        rec = json.load(open(traffic_file(kernel, T, qformat)))
    except Exception:
        return None
    if rec.get("kernel_src_sha") != kernel_src_sha(kernel):
        return None
    return rec.get("bytes_per_launch")


def copy_calibration(mb: int, torch):
    n = mb * 2 ** 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()


def main():
    a = parse()
    if a.summarize:
        summarize(a)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the TTQ projection is built and "
              "timed on a single MI355X (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    import online_activation_aware_ttq_amd as ttq

    torch.cuda.init()
    if a.only_pca:
        print(json.dumps({"lowrank_pca": measure_pca(torch, ttq, reps=a.steps)}),
              flush=True)
        return
    if a.only_decode:
        r = measure_decode(torch, ttq, a.steps)
        if a.copy_calib_mb:
            copy_calibration(a.copy_calib_mb, torch)
        print(json.dumps({"decode_from_codes": r}), flush=True)
        return
    if a.only_segmented:
        print(json.dumps({"continuous_batching": measure_segmented(torch, ttq, a.steps)}),
              flush=True)
        return
    main_m = measure(a.T, a.steps, a.warmup, torch, ttq,
                     want_graph=not a.only_ttq, want_gemm=not a.only_ttq,
                     qformat=a.qformat)
    if a.copy_calib_mb:
        copy_calibration(a.copy_calib_mb, torch)
    sec = None
    if not a.only_ttq and a.T != 128:
        sec = measure(128, max(100, a.steps // 4), a.warmup, torch, ttq,
                      want_graph=False, want_gemm=True, qformat=a.qformat)
    # the other quantizer formats on the same step (context lines)
    fmts = {}
    if not a.only_ttq:
        for f in ("asym", "sym", "intzp", "fp8"):
            if f == a.qformat:
                continue
            m = measure(a.T, max(200, a.steps // 4), a.warmup, torch, ttq,
                        want_graph=False, want_gemm=False, qformat=f)
            kms = max(m["kernels_ms_avg"].values())
            fmts[f] = {"bits": format_bits(f), "ms_per_step": m["ms_per_step"],
                       "tokens_per_s": a.T / (m["ms_per_step"] * 1e-3),
                       "dominant_kernel_ms": kms,
                       "hbm_frac_kernel": alg_bytes(4096, 4096, a.T) / (kms * 1e-3)
                       / 1e9 / HBM_PEAK_GBS}

    d = d_out = 4096
    T = a.T
    ms = main_m["ms_per_step"]
    value = T / (ms * 1e-3)
    # dominant kernel: the largest share of the step's kernel time
    kt = main_m["kernels_ms_avg"]
    launches = main_m["kernels_launches"]
    kname = max(kt, key=lambda k: kt[k] * launches[k])
    k_ms = kt[kname]
    ab = alg_bytes(d, d_out, T)
    af = alg_flops(d, d_out, T)
    hbm_bound = ab / HBM_PEAK_GBS > af / (BF16_PEAK_TFLOPS * 1e3)
    if hbm_bound:
        achieved = ab / (k_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS}
    else:
        achieved = af / (k_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved,
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / BF16_PEAK_TFLOPS}
    roof["traffic"] = traffic_entry(kname, T, a.qformat)
    roof.update(kernel=kname, kernel_ms=k_ms, alg_bytes=ab, alg_flops=af)

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"attention q_proj d=d'=4096 T={T}, "
                        f"{format_bits(a.qformat)}-bit g128 "
                        f"{FORMAT_NAMES[a.qformat]}, p=2, lambda=1e-3, "
                        "alpha=0.5, 1% outlier channels x10-100 redrawn per call",
            "d": d, "d_out": d_out, "T": T, "bits": format_bits(a.qformat),
            "group": 128, "qformat": a.qformat,
            "rank": 0, "parallelism": "single GPU",
            "weights": f"{main_m['rotating_w_copies']} rotating copies "
                       f"({main_m['rotating_bytes'] / 1e6:.0f} MB, above the "
                       "256 MB Infinity Cache)",
        },
        "roofline": roof,
        "step_all_kernels_ms": main_m["kernels_ms_avg"],
        "hbm_frac_whole_step": ab / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "ms_per_step_hot_w": main_m.get("ms_per_step_hot_w"),
        "ms_per_step_graph": main_m.get("ms_per_step_graph"),
    }
    if "gemm_bf16_ms" in main_m:
        g = main_m["gemm_bf16_ms"]
        line["gemm_bf16"] = {"ms": g, "tokens_per_s": T / (g * 1e-3),
                             "impl": "torch.matmul (hipBLASLt), same shape "
                                     "and cache rotation"}
        line["rho_measured"] = ms / g - 1.0
        line["rho_pages"] = 1.0 / d_out + 3.0 / T
    if sec is not None:
        s_ms = sec["ms_per_step"]
        k2 = max(sec["kernels_ms_avg"].values())
        line["secondary_T128"] = {
            "tokens_per_s": 128 / (s_ms * 1e-3), "ms_per_step": s_ms,
            "fused_kernel_ms": k2,
            "hbm_frac_kernel": alg_bytes(d, d_out, 128) / (k2 * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "mfma_frac_kernel": alg_flops(d, d_out, 128) / (k2 * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "gemm_bf16_ms": sec.get("gemm_bf16_ms"),
            "rho_measured": s_ms / sec["gemm_bf16_ms"] - 1.0 if sec.get("gemm_bf16_ms") else None,
            "rho_pages": 1.0 / d_out + 3.0 / 128,
            "kernels_ms_avg": sec["kernels_ms_avg"],
        }
    if fmts:
        line["other_formats"] = fmts
    if not a.only_ttq:
        line["decode_from_codes"] = measure_decode(torch, ttq)
        line["continuous_batching"] = measure_segmented(torch, ttq)
        line["lowrank_pca"] = measure_pca(torch, ttq)
    if not a.no_cpu and not a.only_ttq:
        line["cpu_baseline"] = cpu_baseline(T, a.cpu_seconds, a.qformat)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
