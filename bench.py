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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fused_c2_T1.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--T", type=int, default=1)
    ap.add_argument("--no-cpu", action="store_true",
                    help="skip the oracle cpu_baseline leg")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--only-ttq", action="store_true",
                    help="time only the TTQ step (for profiler runs)")
    return ap.parse_args()


def kernel_src_sha() -> str:
    p = os.path.join(ROOT, "online_activation_aware_ttq_amd", "csrc",
                     "k_fused.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def dev_bf16(bits, torch):
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(
        "cuda").view(torch.bfloat16)


def alg_bytes(d, d_out, T, rank=0):
    return 2 * d_out * d + 2 * T * d + 4 * T * d_out + 2 * rank * (d + d_out)


def alg_flops(d, d_out, T, rank=0):
    return 2 * d_out * d * T + 2 * rank * T * (d + d_out)


def measure(T: int, steps: int, warmup: int, torch, ttq, want_graph: bool,
            want_gemm: bool):
    import numpy as np
    from workloads import configs as wc

    d = d_out = 4096
    prob = wc.make_c2(T=T)
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
              group=prob.group)
    prm = ttq.make_params(d=d, d_out=d_out, T=T, bits=prob.bits,
                          group=prob.group, p=prob.p, lam=prob.lam,
                          alpha=prob.alpha)
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


def cpu_baseline(T: int, seconds: float):
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
    calls = 0
    t0 = time.perf_counter()
    while True:
        X = wc.draw_x(1, 5000 + calls, 1, T, prob.d, "logu10_100", 41)[0]
        oracle.ttq_linear(prob.W, X, bits=prob.bits, group=prob.group,
                          p=prob.p, lam=prob.lam, alpha=prob.alpha)
        calls += 1
        el = time.perf_counter() - t0
        if (el >= seconds and calls >= 3) or el >= 3 * seconds:
            break
    return {"value": calls * T / el, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{calls} full calls of the same workload (T={T}, "
                      f"d=d'=4096), X redrawn per call, {el:.1f} s wall, "
                      f"host cpu_count={os.cpu_count()}"}


def traffic_entry(launch_ms: float):
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except Exception:
        return None
    if rec.get("kernel_src_sha") != kernel_src_sha():
        return None
    return rec.get("bytes_per_launch")


def main():
    a = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the TTQ projection is built and "
              "timed on a single MI355X (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    import online_activation_aware_ttq_amd as ttq

    torch.cuda.init()
    main_m = measure(a.T, a.steps, a.warmup, torch, ttq,
                     want_graph=not a.only_ttq, want_gemm=not a.only_ttq)
    sec = None
    if not a.only_ttq and a.T != 128:
        sec = measure(128, max(100, a.steps // 4), a.warmup, torch, ttq,
                      want_graph=False, want_gemm=True)

    d = d_out = 4096
    T = a.T
    ms = main_m["ms_per_step"]
    value = T / (ms * 1e-3)
    kname = "fused_qdq_mfma" if T <= 128 else "gemm_mfma"
    k_ms = main_m["kernels_ms_avg"].get(kname, float("nan"))
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
    roof["traffic"] = traffic_entry(k_ms)
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
            "workload": f"attention q_proj d=d'=4096 T={T}, 4-bit g128 "
                        "asymmetric, p=2, lambda=1e-3, alpha=0.5, 1% outlier "
                        "channels x10-100 redrawn per call",
            "d": d, "d_out": d_out, "T": T, "bits": 4, "group": 128,
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
        k2 = sec["kernels_ms_avg"].get("fused_qdq_mfma", float("nan"))
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
    if not a.no_cpu and not a.only_ttq:
        line["cpu_baseline"] = cpu_baseline(T, a.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
