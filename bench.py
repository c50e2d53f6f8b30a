#!/usr/bin/env python3
"""Throughput of the TTQ linear projection on one MI355X.

Headline step: one full 7B-class decoder layer of TTQ projections -- q, k, v,
o (4096 -> 4096), gate, up (4096 -> 11008) and down (11008 -> 4096) -- for
R = 8 independent requests of T = 4096 tokens each, every request with its
own activation statistics and its own outlier channels (multitenant), 4-bit
groups of 128, p = 2, lambda = 1e-3, alpha = 0.5, static low rank r = 32 on
all seven projections.  One step = the seven batched calls; ``value`` is the
layer's throughput in tokens/s (R T / step time), inputs resident in HBM.

The JSON line also carries, as keys of their own: the same layer at T = 1,
16 and 256; the 70B-class up projection (8192 -> 28672, T = 512, 2-bit g64,
r = 128) at p = 2 and p = 1; the MLP gate/up and down projections at
T = 2048 (3-bit, r = 64); the 4096 x 4096 projection at T = 1 and T = 128;
for each a plain bf16 GEMM of the same shape (torch -> hipBLASLt) and the
measured overhead ratio against the pages' 1/d' + 3/T.  Then the roofline of
the dominant kernel (event-timed launches on the library's stream; HBM
traffic from committed rocprofv3 counter summaries), two measured ceilings
(a device copy for HBM, a large bf16 GEMM for the matrix cores) and the CPU
oracle on the host cores (cpu_baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("TTQ-linear tokens/s per projection + % HBM/MFMA roofline; "
          "overhead vs bf16 GEMM")
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3
# one vector-ALU lane operation per lane and clock without packed fp32 math:
# 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz (157.3 TFLOP/s counts an FMA as 2
# and a packed pair as 2 more)
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
ROTATE_BYTES = 640 * 2 ** 20
FORMAT_NAMES = {"asym": "asymmetric", "sym": "symmetric",
                "intzp": "integer zero point", "fp8": "FP8 E4M3"}
# timing-kind name -> kernel source (for the counter summaries' freshness)
KERNEL_SOURCES = {"gemv_t1": "k_gemv.hip", "fused_qdq_mfma": "k_fused.hip",
                  "stats_small": "k_stats.hip", "gemm_mfma": "k_gemm_lds.hip",
                  "quant_what": "k_quant.hip", "gemm_quant": "k_gemm_q.hip",
                  "qgemv": "k_qgemv.hip", "stats_z": "k_stats.hip"}
# timing-kind name -> substring of the HIP kernel symbol in rocprofv3 output
KERNEL_SYMBOLS = {"gemv_t1": "k_gemv", "fused_qdq_mfma": "k_fused",
                  "gemm_mfma": "k_gemm_lds", "quant_what": "k_quant",
                  "gemm_quant": "k_gemm_q", "qgemv": "k_qgemv",
                  "stats_small": "k_stats_small", "stats_z": "k_stats_z"}
C5_PROJ = (("q_proj", 4096, 4096), ("k_proj", 4096, 4096),
           ("v_proj", 4096, 4096), ("o_proj", 4096, 4096),
           ("gate_proj", 4096, 11008), ("up_proj", 4096, 11008),
           ("down_proj", 11008, 4096))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10,
                    help="timed steps of the headline layer")
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--leg", default="all",
                    choices=("all", "c5", "c4", "c3", "c2", "decode",
                             "segmented", "pca", "ceilings"),
                    help="run one workload only (profiler runs); 'all' is "
                         "the full line")
    ap.add_argument("--T", type=int, default=0,
                    help="token count of the c5 / c2 leg (default 4096 / 1)")
    ap.add_argument("--p", type=float, default=2.0, help="p of the c4 leg")
    ap.add_argument("--which", default="gate_up", choices=("gate_up", "down"),
                    help="projection of the c3 leg")
    ap.add_argument("--qformat", default="asym",
                    choices=("asym", "sym", "intzp", "fp8"),
                    help="quantizer format of the c2 leg")
    ap.add_argument("--no-cpu", action="store_true",
                    help="skip the oracle cpu_baseline leg")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calib-mb", type=int, default=0,
                    help="after the timed work, run 5 device-to-device copies "
                         "of this many MiB (counter calibration)")
    ap.add_argument("--summarize", nargs=3, metavar=("TRACE", "FETCH", "WRITE"),
                    help="write profiles/ summaries from rocprofv3 output "
                         "directories (kernel trace, FETCH_SIZE, WRITE_SIZE) "
                         "for --kernel on the workload named by --leg")
    ap.add_argument("--kernel", default="",
                    help="timing-kind name of the summarized kernel")
    ap.add_argument("--profile-cmd", default="",
                    help="command lines recorded in the summary (';;' apart)")
    return ap.parse_args()


# ------------------------------------------------------------------ helpers
def dev_bf16(bits, torch):
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(
        "cuda").view(torch.bfloat16)


def draw_x_gpu(torch, seed: int, R: int, T: int, d: int, kind: str,
               n_out: int):
    """Seeded activations [R, T, d] bf16, drawn on the GPU (input generation
    only), a new outlier channel set per request, rounded to bf16 to nearest
    even.  kind ``n``: N(0,1) with ``n_out`` channels multiplied
    log-uniformly by 10-100x; ``x50``: N(0,1) with ``n_out`` channels x50;
    ``t3``: Student-t(3) with ``n_out`` channels x30-100 log-uniform."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    X = torch.empty(R, T, d, dtype=torch.bfloat16, device="cuda")
    for r in range(R):
        if kind == "t3":
            # Student-t(3) = N / sqrt(chi2_3 / 3)
            z = torch.randn(T, d, generator=g, device="cuda")
            c = torch.randn(3, T, d, generator=g, device="cuda").pow_(2).sum(0)
            x = z / torch.sqrt(c / 3.0)
            lo = 1.4771212547196624   # log10 30
        else:
            x = torch.randn(T, d, generator=g, device="cuda")
            lo = 1.0
        ch = torch.randperm(d, generator=g, device="cuda")[:n_out]
        if kind == "x50":
            mult = torch.full((n_out,), 50.0, device="cuda")
        else:
            mult = torch.pow(10.0, lo + (2.0 - lo) * torch.rand(
                n_out, generator=g, device="cuda"))
        x[:, ch] *= mult
        X[r] = x.to(torch.bfloat16)
        del x
    return X


def timed_wall(torch, fn, n: int, w: int) -> float:
    """ms per call: w untimed calls, then n calls bracketed by device
    synchronisations (host wall clock)."""
    for i in range(w):
        fn(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        fn(i)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / n


def kernel_times(torch, ttq, fn, n: int) -> dict:
    """{timing kind: (avg ms per launch, launches per call)} over n calls, from
    the events the runtime stamps around each kernel of the library."""
    ttq.timing_reset()
    ttq.timing_enable(True)
    for i in range(n):
        fn(i)
    torch.cuda.synchronize()
    kt = ttq.timing_query()
    ttq.timing_enable(False)
    ttq.timing_reset()
    return {k: (v[0] / v[1], v[1] / n) for k, v in kt.items() if v[1]}


def gemm_ms(torch, Ws, Xs, n: int, w: int) -> float:
    """Plain bf16 GEMM(s) of the same shapes (torch.nn.functional.linear ->
    hipBLASLt), one per (weight, request) like the TTQ call."""
    import torch.nn.functional as F

    def f(i):
        for W, X in zip(Ws, Xs):
            for r in range(X.shape[0]):
                F.linear(X[r], W)
    return timed_wall(torch, f, n, w)


def alg(d, d_out, T, R=1, rank=0):
    """Algorithmic bytes (W once, X, Y fp32, B and A) and matrix flops of
    one call: R requests of T tokens on one shared W."""
    by = 2 * d_out * d + R * (2 * T * d + 4 * T * d_out) + 2 * rank * (d + d_out)
    fl = R * (2 * d_out * d * T + 2 * rank * T * (d + d_out))
    return by, fl


def kernel_units(kind: str, d, d_out, T, R, rank):
    """Algorithmic (bytes, flops) of one launch of a kernel kind for one
    call of the shape.  The projection GEMMs do the main contraction and the
    low-rank segment Z B^T; the quantize pass reads W once and writes one
    bf16 W_hat per request; the one-pass kernels stream W once."""
    if kind in ("gemm_mfma", "gemm_quant"):
        by = R * (2 * T * d + 4 * T * d_out + 2 * T * rank) + 2 * d_out * rank
        by += 2 * d_out * d * (R if kind == "gemm_mfma" else 1)
        return by, R * 2 * T * d_out * (d + rank)
    if kind == "quant_what":
        return 2 * d_out * d * (1 + R), 0
    if kind in ("gemv_t1", "fused_qdq_mfma"):
        by = 2 * d_out * d + R * (2 * T * d + 4 * T * d_out) + 2 * d_out * rank
        return by, R * 2 * T * d_out * d
    return 0, 0


def alu_ops(kind: str, d, d_out, R) -> float:
    """Vector-ALU operations of the quantization in one launch: per weight
    element and request the scaling u = w D^{1/2}, the group minimum and
    maximum, t = (u - m) / s as a subtraction and a product, the rounding,
    and (one-token kernel only) the product with x' -- 7 and 6 operations."""
    per = {"gemv_t1": 7, "fused_qdq_mfma": 6}.get(kind, 0)
    return float(per) * R * d_out * d


def roofline(kind: str, ms_per_launch: float, bytes_per_launch: float,
             flops_per_launch: float, traffic=None, ops_per_launch: float = 0.0
             ) -> dict:
    t_hbm = bytes_per_launch / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops_per_launch / (BF16_PEAK_TFLOPS * 1e12)
    t_alu = ops_per_launch / (VALU_PEAK_TOPS * 1e12)
    if t_alu > max(t_hbm, t_mfma):
        a = ops_per_launch / (ms_per_launch * 1e-3) / 1e12
        r = {"bound": "alu", "achieved": a, "peak": VALU_PEAK_TOPS,
             "unit": "Tops/s", "frac": a / VALU_PEAK_TOPS}
    elif t_hbm >= t_mfma:
        a = bytes_per_launch / (ms_per_launch * 1e-3) / 1e9
        r = {"bound": "hbm", "achieved": a, "peak": HBM_PEAK_GBS,
             "unit": "GB/s", "frac": a / HBM_PEAK_GBS}
    else:
        a = flops_per_launch / (ms_per_launch * 1e-3) / 1e12
        r = {"bound": "mfma", "achieved": a, "peak": BF16_PEAK_TFLOPS,
             "unit": "TFLOP/s", "frac": a / BF16_PEAK_TFLOPS}
    r["traffic"] = traffic
    r.update(kernel=kind, kernel_ms=ms_per_launch,
             alg_bytes_per_launch=bytes_per_launch,
             alg_flops_per_launch=flops_per_launch)
    if ops_per_launch:
        r["alg_alu_ops_per_launch"] = ops_per_launch
    return r


def _code_only(path: str) -> bytes:
    """Source text without comments and blank space (a comment edit does not
    change what the counters measured)."""
    txt = open(path, encoding="utf-8").read()
    txt = re.sub(r"/\*.*?\*/", " ", txt, flags=re.S)
    txt = re.sub(r"//[^\n]*", " ", txt)
    return " ".join(txt.split()).encode()


def kernel_src_sha(kind: str) -> str:
    cdir = os.path.join(ROOT, "online_activation_aware_ttq_amd", "csrc")
    h = hashlib.sha256(_code_only(os.path.join(
        cdir, KERNEL_SOURCES.get(kind, "k_fused.hip"))))
    # the shared headers change every kernel
    for name in sorted(os.listdir(cdir)):
        if name.endswith(".h"):
            h.update(_code_only(os.path.join(cdir, name)))
    return h.hexdigest()[:16]


def traffic_file(kind: str, leg: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{kind}_{leg}.json")


def traffic_entry(kind: str, leg: str):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel source has changed since it was taken."""
    try:
        rec = json.load(open(traffic_file(kind, leg)))
    except Exception:
        return None
    if rec.get("kernel_src_sha") != kernel_src_sha(kind):
        return None
    return rec.get("bytes_per_launch")


# ------------------------------------------------------------------- legs
def leg_c5(torch, ttq, T: int, steps: int, warmup: int, want_gemm: bool,
           per_projection: bool = True) -> dict:
    """The seven projections of a 7B-class layer for R = 8 requests of T
    tokens each; one step = seven batched calls."""
    from workloads import configs as wc
    R, bits, group, rank = 8, 4, 128, 32
    kw = dict(p=2.0, lam=1e-3, alpha=0.5, bits=bits, group=group)
    projs = []
    for i, (name, d, d_out) in enumerate(C5_PROJ):
        prob = wc.make_c5(T=1, proj=name, R=1)   # W, B, A (seeded per projection)
        projs.append(dict(
            name=name, d=d, d_out=d_out,
            W=dev_bf16(prob.W, torch), B=dev_bf16(prob.B, torch),
            A=dev_bf16(prob.A, torch),
            X=draw_x_gpu(torch, 4000 + 7 * T + i, R, T, d, "n",
                         max(1, round(0.01 * d))),
            Y=torch.empty(R, T, d_out, dtype=torch.float32, device="cuda")))
    ws_bytes = max(ttq.ttq_workspace_bytes(
        ttq.make_params(d=p["d"], d_out=p["d_out"], T=T, rank=rank, bits=bits,
                        group=group, p=2.0, lam=1e-3, alpha=0.5), R)
        for p in projs)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def call(p):
        ttq.ttq_linear_batched(p["W"], p["X"], p["B"], p["A"], Y=p["Y"],
                               workspace=ws, stream=stream, **kw)

    def step(i):
        for p in projs:
            call(p)

    reps = steps if T >= 256 else max(steps, 50)
    ms = timed_wall(torch, step, reps, warmup)
    kt = kernel_times(torch, ttq, step, max(2, min(reps, 20)))
    out = {"workload": f"7B-class layer, 7 projections, R={R} requests x "
                       f"T={T} tokens, 4-bit g128 asymmetric, p=2, "
                       "lambda=1e-3, alpha=0.5, r=32, own outlier set per "
                       "request", "T": T, "R": R, "steps": reps,
           "warmup": warmup, "ms_per_step": ms,
           "tokens_per_s": R * T / (ms * 1e-3),
           "kernels": {k: {"ms_per_launch": v[0], "launches_per_step": v[1]}
                       for k, v in kt.items()},
           "path": ttq.ttq_path(ttq.make_params(
               d=4096, d_out=4096, T=T, rank=rank, bits=bits, group=group,
               p=2.0, lam=1e-3, alpha=0.5), R)}
    by = fl = 0
    for p in projs:
        b_, f_ = alg(p["d"], p["d_out"], T, R, rank)
        by += b_
        fl += f_
    out["alg_bytes_per_step"] = by
    out["alg_flops_per_step"] = fl
    out["hbm_frac_step"] = by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS
    out["mfma_frac_step"] = fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS
    # dominant kernel: the largest share of the step's kernel time
    dom = max(kt, key=lambda k: kt[k][0] * kt[k][1])
    ub = uf = uo = 0
    for p in projs:
        b_, f_ = kernel_units(dom, p["d"], p["d_out"], T, R, rank)
        ub += b_
        uf += f_
        uo += alu_ops(dom, p["d"], p["d_out"], R)
    n_l = kt[dom][1]
    out["roofline"] = roofline(dom, kt[dom][0], ub / n_l, uf / n_l,
                               traffic_entry(dom, f"c5_T{T}"), uo / n_l)
    if per_projection:
        pp = {}
        for p in projs:
            pm = timed_wall(torch, lambda i: call(p), max(3, reps // 2), 1)
            e = {"ms": pm, "tokens_per_s": R * T / (pm * 1e-3)}
            b_, f_ = alg(p["d"], p["d_out"], T, R, rank)
            e["mfma_frac"] = f_ / (pm * 1e-3) / 1e12 / BF16_PEAK_TFLOPS
            e["hbm_frac"] = b_ / (pm * 1e-3) / 1e9 / HBM_PEAK_GBS
            if want_gemm:
                g = gemm_ms(torch, [p["W"]], [p["X"]], max(3, reps // 2), 1)
                e["gemm_bf16_ms"] = g
                e["rho_measured"] = pm / g - 1.0
                e["rho_pages"] = 1.0 / p["d_out"] + 3.0 / T
            pp[p["name"]] = e
        out["per_projection"] = pp
        if want_gemm:
            gl = sum(e["gemm_bf16_ms"] for e in pp.values())
            out["gemm_bf16_layer_ms"] = gl
            out["rho_measured_layer"] = ms / gl - 1.0
    del projs, ws
    torch.cuda.empty_cache()
    return out


def leg_single(torch, ttq, leg: str, name: str, prob_fn, T: int, d: int,
               d_out: int,
               bits: int, group: int, rank: int, p: float, lam: float,
               x_kind: str, n_out: int, steps: int, seed: int,
               want_gemm: bool = True) -> dict:
    """One projection (R = 1) with its weights rotated over enough copies to
    exceed the 256 MB Infinity Cache; a new activation draw per call."""
    prob = prob_fn()
    w_bytes = 2 * d * d_out
    n_w = max(1, -(-ROTATE_BYTES // (w_bytes + 2 * T * d + 4 * T * d_out)))
    W0 = dev_bf16(prob.W, torch)
    Ws = [W0] + [W0.clone() for _ in range(n_w - 1)]
    B = dev_bf16(prob.B, torch) if rank else None
    A = dev_bf16(prob.A, torch) if rank else None
    n_x = max(2, n_w)
    Xs = [draw_x_gpu(torch, seed + c, 1, T, d, x_kind, n_out)[0]
          for c in range(n_x)]
    Ys = [torch.empty(T, d_out, dtype=torch.float32, device="cuda")
          for _ in range(n_x)]
    prm = ttq.make_params(d=d, d_out=d_out, T=T, rank=rank, bits=bits,
                          group=group, p=p, lam=lam, alpha=0.5)
    ws = torch.empty(max(256, ttq.ttq_workspace_bytes(prm)), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    kw = dict(p=p, lam=lam, alpha=0.5, bits=bits, group=group)

    def step(i):
        ttq.ttq_linear(Ws[i % n_w], Xs[i % n_x], B, A, Y=Ys[i % n_x],
                       workspace=ws, stream=stream, **kw)

    ms = timed_wall(torch, step, steps, 2)
    kt = kernel_times(torch, ttq, step, min(steps, 20))
    by, fl = alg(d, d_out, T, 1, rank)
    out = {"workload": name, "d": d, "d_out": d_out, "T": T, "bits": bits,
           "group": group, "rank": rank, "p": p, "lambda": lam,
           "ms": ms, "tokens_per_s": T / (ms * 1e-3),
           "hbm_frac": by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "mfma_frac": fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
           "path": ttq.ttq_path(prm, 1),
           "rotating_w_copies": n_w,
           "kernels": {k: {"ms_per_launch": v[0], "launches_per_call": v[1]}
                       for k, v in kt.items()}}
    dom = max(kt, key=lambda k: kt[k][0] * kt[k][1])
    ub, uf = kernel_units(dom, d, d_out, T, 1, rank)
    out["roofline"] = roofline(dom, kt[dom][0], ub, uf,
                               traffic_entry(dom, leg))
    if want_gemm:
        g = gemm_ms(torch, [Ws[0]], [Xs[0][None]], steps, 2)
        out["gemm_bf16_ms"] = g
        out["rho_measured"] = ms / g - 1.0
        out["rho_pages"] = 1.0 / d_out + 3.0 / T
    del Ws, Xs, Ys, ws
    torch.cuda.empty_cache()
    return out


def leg_c4(torch, ttq, p: float, steps: int) -> dict:
    from workloads import configs as wc
    return leg_single(torch, ttq, f"c4_p{int(p)}", f"c4 up_proj 8192->28672 T=512 2-bit g64 "
                      f"r=128 p={p:g} lambda=1e-2",
                      lambda: wc.make_c4(p=p, T=1), 512, 8192, 28672, 2, 64,
                      128, p, 1e-2, "t3", 41, steps, 7000 + int(p))


def leg_c3(torch, ttq, which: str, steps: int) -> dict:
    from workloads import configs as wc
    d, d_out = (4096, 11008) if which == "gate_up" else (11008, 4096)
    return leg_single(torch, ttq, f"c3_{which}", f"c3 {which} {d}->{d_out} "
                      "T=2048 3-bit g128 r=64, 4 outlier channels x50",
                      lambda: wc.make_c3(which, T=1), 2048, d, d_out, 3, 128,
                      64, 2.0, 1e-3, "x50", 4, steps,
                      8000 + (0 if which == "gate_up" else 50))


def stream_read_ms(torch, ttq, Ws, n: int) -> float:
    """Kernel time of a plain read of the same bytes (ttq_stream_read: the
    one-token kernel's launch shape, rotating W copies so that none is
    cache-resident), averaged over n launches from the library's events."""
    sink = torch.empty(-(-Ws[0].numel() * 2 // (128 * 1024)), dtype=torch.int32,
                       device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def step(i):
        ttq.stream_read(Ws[i % len(Ws)], sink=sink, stream=stream)

    for i in range(5):
        step(i)
    torch.cuda.synchronize()
    return kernel_times(torch, ttq, step, n)["stream_read"][0]


def leg_c2(torch, ttq, T: int, steps: int, warmup: int, qformat: str,
           want_graph: bool, want_gemm: bool) -> dict:
    """The 4096 x 4096 projection at T tokens, W rotated over 20 copies."""
    from workloads import configs as wc
    d = d_out = 4096
    bits = 8 if qformat == "fp8" else 4
    prob = wc.make_c2(T=T)
    n_w = max(2, -(-ROTATE_BYTES // (2 * d * d_out)))
    W0 = dev_bf16(prob.W, torch)
    Ws = [W0] + [W0.clone() for _ in range(n_w - 1)]
    n_x = 64
    Xall = draw_x_gpu(torch, 1000 + T, n_x, T, d, "n", 41)
    Ys = [torch.empty(T, d_out, dtype=torch.float32, device="cuda")
          for _ in range(8)]
    kw = dict(p=2.0, lam=1e-3, alpha=0.5, bits=bits, group=128, qformat=qformat)
    prm = ttq.make_params(d=d, d_out=d_out, T=T, bits=bits, group=128, p=2.0,
                          lam=1e-3, alpha=0.5, qformat=qformat)
    ws = torch.empty(max(256, ttq.ttq_workspace_bytes(prm)), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def step(i):
        ttq.ttq_linear(Ws[i % n_w], Xall[i % n_x], Y=Ys[i % 8], workspace=ws,
                       stream=stream, **kw)

    ms = timed_wall(torch, step, steps, warmup)
    kt = kernel_times(torch, ttq, step, min(steps, 1000))
    by, fl = alg(d, d_out, T)
    out = {"workload": f"q_proj 4096x4096 T={T}, {bits}-bit g128 "
                       f"{FORMAT_NAMES[qformat]}, p=2, lambda=1e-3, alpha=0.5",
           "T": T, "qformat": qformat, "ms": ms,
           "tokens_per_s": T / (ms * 1e-3),
           "hbm_frac": by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "rotating_w_copies": n_w,
           "kernels": {k: {"ms_per_launch": v[0], "launches_per_call": v[1]}
                       for k, v in kt.items()}}
    dom = max(kt, key=lambda k: kt[k][0] * kt[k][1])
    ub, uf = kernel_units(dom, d, d_out, T, 1, 0)
    sfx = "" if qformat == "asym" else f"_{qformat}"
    out["roofline"] = roofline(dom, kt[dom][0], ub, uf,
                               traffic_entry(dom, f"c2_T{T}{sfx}"))
    if want_graph:
        # the ceiling of a one-pass kernel over W: a plain read of the bytes
        # (an auxiliary figure: a failure here is recorded, not fatal)
        wb = 2 * d * d_out
        try:
            sr = stream_read_ms(torch, ttq, Ws, 200)
            out["stream_read"] = {
                "what": "ttq_stream_read over the same W bytes in the one-token "
                        "kernel's launch shape (rotating copies), kernel time",
                "bytes": wb, "ms": sr, "GB_s": wb / (sr * 1e-3) / 1e9,
                "frac_of_peak": wb / (sr * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "dominant_kernel_vs_read": kt[dom][0] / sr}
        except Exception as e:  # noqa: BLE001
            out["stream_read"] = {"error": f"{type(e).__name__}: {e}"}
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(n_w):
                ttq.ttq_linear(Ws[i], Xall[i], Y=Ys[i % 8], workspace=ws,
                               stream=s.cuda_stream, **kw)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            cs = torch.cuda.current_stream().cuda_stream
            for i in range(n_w):
                ttq.ttq_linear(Ws[i], Xall[i], Y=Ys[i % 8], workspace=ws,
                               stream=cs, **kw)
        reps = max(1, steps // n_w)
        out["ms_graph"] = timed_wall(torch, lambda i: g.replay(), reps, 3) / n_w
    if want_gemm:
        gm = gemm_ms(torch, [Ws[0]], [Xall[0][None]], steps, warmup)
        out["gemm_bf16_ms"] = gm
        out["rho_measured"] = ms / gm - 1.0
        out["rho_pages"] = 1.0 / d_out + 3.0 / T
    del Ws, Xall, Ys, ws
    torch.cuda.empty_cache()
    return out


def leg_ceilings(torch) -> dict:
    """Measured ceilings on this machine: HBM from a device-to-device copy of
    2 GiB (read + write bytes over time), matrix cores from a large bf16
    GEMM (torch -> hipBLASLt, 8192^3)."""
    n = 2 * 2 ** 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    ms = timed_wall(torch, lambda i: dst.copy_(src), 20, 3)
    copy = {"bytes_moved": 2 * n, "ms": ms,
            "GB_s": 2 * n / (ms * 1e-3) / 1e9,
            "frac_of_peak": 2 * n / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    del src, dst
    M = 8192
    a = torch.randn(M, M, dtype=torch.bfloat16, device="cuda")
    b = torch.randn(M, M, dtype=torch.bfloat16, device="cuda")
    ms2 = timed_wall(torch, lambda i: torch.matmul(a, b), 20, 3)
    fl = 2.0 * M ** 3
    gemm = {"shape": "8192x8192x8192 bf16", "ms": ms2,
            "TFLOP_s": fl / (ms2 * 1e-3) / 1e12,
            "frac_of_peak": fl / (ms2 * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}
    del a, b
    torch.cuda.empty_cache()
    return {"hbm_copy": copy, "bf16_gemm": gemm}


def leg_decode(torch, ttq, steps: int = 1000) -> dict:
    """One token against codes stored by ttq_quantize (4096 x 4096, 4-bit
    g128): 20 rotating stored copies."""
    from workloads import configs as wc
    d = d_out = 4096
    prob = wc.make_c2(T=16)
    W0 = dev_bf16(prob.W, torch)
    X0 = dev_bf16(prob.X[0], torch)
    kw = dict(bits=4, group=128)
    st = [ttq.ttq_quantize(W0, X0, p=prob.p, lam=prob.lam, alpha=prob.alpha, **kw)
          for _ in range(20)]
    Xs = draw_x_gpu(torch, 3000, 64, 1, d, "n", 41)
    Y = torch.empty(1, d_out, dtype=torch.float32, device="cuda")
    prm = ttq.make_params(d=d, d_out=d_out, T=1, bits=4, group=128, p=1.0,
                          lam=0.0, alpha=0.0)
    ws = torch.empty(max(256, ttq.ttq_qmatmul_workspace_bytes(prm)),
                     dtype=torch.uint8, device="cuda")
    f = lambda i: ttq.ttq_qmatmul(*st[i % 20], Xs[i % 64], Y=Y, workspace=ws, **kw)
    ms = timed_wall(torch, f, steps, 50)
    kt = kernel_times(torch, ttq, f, steps)
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
    gms = timed_wall(torch, lambda i: g.replay(), max(1, steps // 20), 3) / 20
    G = d // 128
    ab = d_out * d // 2 + 8 * d_out * G + 2 * d + 4 * d + 4 * d_out
    k = kt.get("qgemv", (float("nan"), 0))[0]
    # the same stored codes against 16 new tokens (statistics kernel in its
    # stored-D^{-1/2} mode, then the packed-code MFMA kernel)
    X16 = draw_x_gpu(torch, 3100, 16, 16, d, "n", 41)
    Y16 = torch.empty(16, d_out, dtype=torch.float32, device="cuda")
    prm16 = ttq.make_params(d=d, d_out=d_out, T=16, bits=4, group=128, p=1.0,
                            lam=0.0, alpha=0.0)
    ws16 = torch.empty(max(256, ttq.ttq_qmatmul_workspace_bytes(prm16)),
                       dtype=torch.uint8, device="cuda")
    f16 = lambda i: ttq.ttq_qmatmul(*st[i % 20], X16[i % 16], Y=Y16, workspace=ws16, **kw)
    n16 = max(1, steps // 2)
    ms16 = timed_wall(torch, f16, n16, 20)
    kt16 = kernel_times(torch, ttq, f16, n16)
    return {"workload": "4096x4096, 4-bit g128 codes, one token",
            "ms": ms, "tokens_per_s": 1.0 / (ms * 1e-3), "ms_graph": gms,
            "tokens_per_s_graph": 1.0 / (gms * 1e-3), "kernel": "qgemv",
            "kernel_ms": k, "alg_bytes": ab,
            "hbm_frac_kernel": ab / (k * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "traffic": traffic_entry("qgemv", "decode_int4"),
            "T16": {"workload": "the same codes, 16 tokens", "ms": ms16,
                    "tokens_per_s": 16 / (ms16 * 1e-3),
                    "kernels": {kk: {"ms_per_launch": v[0], "launches_per_call": v[1]}
                                for kk, v in kt16.items()}}}


def leg_segmented(torch, ttq, reps: int = 50) -> dict:
    """Continuous batching on the 4096 x 4096 weights (4-bit g128, r = 32):
    22 requests of mixed lengths (16 single tokens, 3, 7, 12, 16, 100, 200;
    354 tokens) in one packed X, each with its own statistics -- one
    ttq_linear_segmented call against one ttq_linear call per request."""
    import numpy as np
    from workloads import configs as wc
    d = d_out = 4096
    prob = wc.make_problem("seg", d=d, d_out=d_out, T=1, bits=4, group=128,
                           rank=32, seed=11)
    lengths = [1] * 16 + [3, 7, 12, 16, 100, 200]
    rng = np.random.default_rng(12)
    lengths = [int(x) for x in rng.permutation(lengths)]
    xs = [draw_x_gpu(torch, 500 + i, 1, t, d, "n", 41)[0]
          for i, t in enumerate(lengths)]
    offs = [0] + [int(x) for x in np.cumsum(lengths)]
    W = dev_bf16(prob.W, torch)
    Bm, A = dev_bf16(prob.B, torch), dev_bf16(prob.A, torch)
    X = torch.cat(xs)
    kw = dict(p=prob.p, lam=prob.lam, alpha=prob.alpha, bits=4, group=128)
    Y = torch.empty(offs[-1], d_out, dtype=torch.float32, device="cuda")

    def seg(i):
        ttq.ttq_linear_segmented(W, X, Bm, A, seg_offsets=offs, Y=Y, **kw)

    def single(i):
        for j, x in enumerate(xs):
            ttq.ttq_linear(W, x, Bm, A, Y=Y[offs[j]:offs[j + 1]], **kw)

    out = {"workload": f"4096x4096 4-bit g128 r=32, {len(lengths)} requests, "
                       f"{offs[-1]} tokens (16 x 1, 3, 7, 12, 16, 100, 200)"}
    for name, f in (("segmented", seg), ("one_call_per_request", single)):
        ms = timed_wall(torch, f, reps, 3)
        out[name] = {"ms": ms, "tokens_per_s": offs[-1] / (ms * 1e-3)}
    return out


def leg_pca(torch, ttq, reps: int = 10) -> dict:
    """Low-rank factors by PCA (4096 x 4096, r = 64, two power iterations,
    static): a per-model initialisation, context for the low-rank row."""
    from workloads.configs import draw_lowrank_w, draw_omega
    d = d_out = 4096
    r, iters = 64, 2
    W = dev_bf16(draw_lowrank_w(1, d_out, d, r), torch)
    Om = torch.from_numpy(draw_omega(2, d, r)).cuda()
    prm = ttq.make_params(d=d, d_out=d_out, T=0, rank=r, bits=4, group=32,
                          p=2.0, lam=0.0, alpha=0.0)
    ws = torch.empty(ttq.ttq_lowrank_pca_workspace_bytes(prm, iters),
                     dtype=torch.uint8, device="cuda")
    f = lambda i: ttq.ttq_lowrank_pca(W, Om, iters=iters, workspace=ws)
    ms = timed_wall(torch, f, reps, 2)
    kt = kernel_times(torch, ttq, f, reps)
    flops_w = (2 + 2 * iters) * 2.0 * d_out * d * r
    sk = kt.get("pca_skinny", (float("nan"), 1))
    sk_ms = sk[0] * sk[1]
    return {"shape": f"{d_out}x{d}, r={r}, {iters} power iterations",
            "ms": ms, "kernels_ms_per_call": {k: v[0] * v[1] for k, v in kt.items()},
            "skinny_tflops_w_products": flops_w / (sk_ms * 1e-3) / 1e12,
            "skinny_frac_fp32_peak": flops_w / (sk_ms * 1e-3) / 1e12 / FP32_PEAK_TFLOPS}


# ------------------------------------------------------------ cpu baseline
def _threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline_c5(T: int, seconds: float) -> dict:
    """The oracle as it stands on the host cores, on a bounded sample of the
    headline workload.  Whole requests (each of the seven projections, all
    output rows, statistics over all T tokens, each request its own X) are
    timed one after another until about `seconds` of oracle time is spent;
    tokens/s = requests timed x T / their time.  On a host where one whole
    request would take far longer than that, each projection is timed on two
    subsets of output rows instead and extrapolated linearly in the row
    count (rows are independent once D is fixed) and times R = 8."""
    import numpy as np
    import oracle
    from workloads import configs as wc
    R = 8
    t_start = time.perf_counter()

    def run(prob, X, rows):
        t0 = time.perf_counter()
        oracle.ttq_linear(prob.W, X, bits=4, group=128, p=2.0, lam=1e-3,
                          alpha=0.5, B_bits=prob.B, A_bits=prob.A, rows=rows)
        return time.perf_counter() - t0

    probs = [wc.make_c5(T=1, proj=name, R=1) for name, _, _ in C5_PROJ]

    def x_of(i, req):
        d = C5_PROJ[i][1]
        return wc.draw_x(4000 + 100 * req + i, 0, 1, T, d, "logu10_100",
                         max(1, round(0.01 * d)))[0]

    # a short timed pass (rows 8 and 24 of q_proj: a fixed part and a cost
    # per row, both taken as proportional to d) estimates one whole request
    X = x_of(0, 0)
    c8, c24 = run(probs[0], X, np.arange(8)), run(probs[0], X, np.arange(24))
    per_row = max((c24 - c8) / 16, 1e-6)
    fixed = max(0.0, c8 - 8 * per_row)
    est_req = sum((fixed + per_row * d_out) * d / 4096
                  for _, d, d_out in C5_PROJ)
    cpu = {"unit": "tokens/s", "cores": _threads(), "kind": "oracle"}
    if est_req <= 2.5 * seconds:
        measured, n = 0.0, 0
        while n < R and (n == 0 or measured < seconds):
            for i in range(len(C5_PROJ)):
                measured += run(probs[i], x_of(i, n), None)
            n += 1
        wall = time.perf_counter() - t_start
        cpu.update(value=n * T / measured,
                   sample=f"{n} whole request(s) of the layer (7 projections, "
                          f"all rows, T={T}), {measured:.1f} s of oracle time "
                          f"({wall:.1f} s wall with input generation); "
                          f"host cpu_count={os.cpu_count()}")
        return {"value": cpu.pop("value"), **cpu}
    n_proj = len(C5_PROJ)
    rows_b = int((seconds / n_proj - 2 * fixed) / (per_row * 4 / 3))
    rows_b = max(24, min(min(d_out for _, _, d_out in C5_PROJ), rows_b))
    rows_a = rows_b // 3
    t_layer = measured = 0.0
    for i, (_, d, d_out) in enumerate(C5_PROJ):
        X = x_of(i, 0)
        ts = [run(probs[i], X, np.arange(rows_a)),
              run(probs[i], X, np.arange(rows_b))]
        measured += sum(ts)
        pr = max(0.0, (ts[1] - ts[0]) / (rows_b - rows_a))
        fx = max(0.0, ts[0] - pr * rows_a)
        t_layer += R * (fx + pr * d_out)
    wall = time.perf_counter() - t_start
    cpu.update(value=R * T / t_layer,
               sample=f"extrapolated x{t_layer / measured:.0f}: one request "
                      f"of each of the 7 projections at T={T}, rows {rows_a} "
                      f"and {rows_b} of d' (statistics over all T tokens), "
                      f"{measured:.1f} s of oracle time ({wall:.1f} s wall "
                      "with input generation), extrapolated linearly in d' "
                      f"and times R=8; host cpu_count={os.cpu_count()}")
    return {"value": cpu.pop("value"), **cpu}


# ---------------------------------------------------------------- profiles
def _read_csv(d, suffix):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)
    rows = []
    for f in files:
        rows += list(csv.DictReader(open(f)))
    return rows


def leg_name(a) -> str:
    if a.leg == "c5":
        return f"c5_T{a.T or 4096}"
    if a.leg == "c4":
        return f"c4_p{int(a.p)}"
    if a.leg == "c3":
        return f"c3_{a.which}"
    if a.leg == "c2":
        sfx = "" if a.qformat == "asym" else f"_{a.qformat}"
        return f"c2_T{a.T or 1}{sfx}"
    if a.leg == "decode":
        return "decode_int4"
    return a.leg


def _stats_table(stats) -> list:
    lines = ["## rocprofv3 --kernel-trace --stats (kernel_stats.csv)", "",
             "| kernel | calls | avg ns | min ns | max ns | share % |",
             "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| {r['Name'][:90]} | {r['Calls']} | "
                     f"{float(r['AverageNs']):.0f} | {r['MinNs']} | {r['MaxNs']} | "
                     f"{float(r.get('Percentage', 0) or 0):.1f} |")
    return lines


def summarize(a):
    """profiles/: kernel-trace summary of one kernel on one workload and its
    HBM traffic per launch from FETCH_SIZE / WRITE_SIZE, each scaled by what
    the same counter reads for a device-to-device copy of known size."""
    trace, fetch, write = a.summarize
    kind = a.kernel or a.leg
    stats = _read_csv(trace, "kernel_stats.csv")
    leg = leg_name(a)
    if fetch == "-" or write == "-":   # kernel trace only (no counters)
        lines = [f"# kernel trace of the {leg} workload", "",
                 "Commands (from the repository root):", "", "```"]
        lines += [c for c in a.profile_cmd.split(";;") if c] + ["```", ""]
        lines += _stats_table(stats)
        open(os.path.join(ROOT, "profiles", f"trace_{leg}.md"), "w").write(
            "\n".join(lines))
        return
    key = KERNEL_SYMBOLS[kind]
    calib_bytes = a.copy_calib_mb * 2 ** 20
    fr = _read_csv(fetch, "counter_collection.csv")
    wr = _read_csv(write, "counter_collection.csv")

    def per_dispatch(rows, counter):
        return [float(r["Counter_Value"]) for r in rows
                if r["Counter_Name"] == counter and key in r["Kernel_Name"]]

    def calls(rows, counter):
        # one timed launch of a kind can be two dispatches (a GEMM's whole
        # rounds of big tiles and its narrow tail): the launches are the
        # dispatches of the most frequent matching kernel
        n = {}
        for r in rows:
            if r["Counter_Name"] == counter and key in r["Kernel_Name"]:
                n[r["Kernel_Name"]] = n.get(r["Kernel_Name"], 0) + 1
        return max(n.values()) if n else 0

    def calib(rows, counter):
        cp = [r for r in rows if r["Counter_Name"] == counter
              and "copyBuffer" in r["Kernel_Name"]]
        cp.sort(key=lambda r: int(r["Dispatch_Id"]))
        vals = [float(r["Counter_Value"]) for r in cp[-5:]]
        return sum(vals) / len(vals) if vals else float("nan")

    k_f, k_w = per_dispatch(fr, "FETCH_SIZE"), per_dispatch(wr, "WRITE_SIZE")
    c_f, c_w = calib(fr, "FETCH_SIZE"), calib(wr, "WRITE_SIZE")
    sf = calib_bytes / (c_f * 1024) if c_f == c_f and c_f > 0 else float("nan")
    sw = calib_bytes / (c_w * 1024) if c_w == c_w and c_w > 0 else float("nan")
    n_f, n_w = calls(fr, "FETCH_SIZE"), calls(wr, "WRITE_SIZE")
    f_kib = sum(k_f) / max(1, n_f)
    w_kib = sum(k_w) / max(1, n_w)
    traffic = f_kib * 1024 * sf + w_kib * 1024 * sw
    rec = {"kernel": kind, "workload": leg, "kernel_src_sha": kernel_src_sha(kind),
           "fetch_kib_per_launch": f_kib, "write_kib_per_launch": w_kib,
           "copy_calib_bytes": calib_bytes, "copy_fetch_kib": c_f,
           "copy_write_kib": c_w, "fetch_scale": sf, "write_scale": sw,
           "bytes_per_launch": traffic, "launches_counted": [n_f, n_w],
           "dispatches_counted": [len(k_f), len(k_w)]}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    json.dump(rec, open(traffic_file(kind, leg), "w"), indent=1)
    lines = [f"# {kind} on {leg}", "", "Commands (from the repository root):",
             "", "```"]
    lines += [c for c in a.profile_cmd.split(";;") if c] + ["```", ""]
    lines += _stats_table(stats)
    lines += ["", "## HBM traffic (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)", "",
              f"- {kind}: FETCH_SIZE {f_kib:.0f} KiB/launch, WRITE_SIZE "
              f"{w_kib:.1f} KiB/launch (summed over {len(k_f)} / {len(k_w)} "
              f"dispatches, {n_f} / {n_w} launches)",
              f"- calibration: device-to-device copy of {calib_bytes} bytes reads "
              f"FETCH_SIZE {c_f:.0f} KiB and WRITE_SIZE {c_w:.0f} KiB; scale "
              f"factors {sf:.4f} (fetch) and {sw:.4f} (write)",
              f"- traffic = {traffic / 1e6:.3f} MB per launch", ""]
    open(os.path.join(ROOT, "profiles", f"{kind}_{leg}.md"), "w").write(
        "\n".join(lines))
    print(json.dumps(rec))


def copy_calibration(mb: int, torch):
    n = mb * 2 ** 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()


# -------------------------------------------------------------------- main
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
    ttq.load_library()

    def emit(obj):
        print(json.dumps(obj), flush=True)

    if a.leg != "all":
        if a.leg == "c5":
            r = leg_c5(torch, ttq, a.T or 4096, a.steps, a.warmup,
                       want_gemm=False, per_projection=False)
        elif a.leg == "c4":
            r = leg_c4(torch, ttq, a.p, a.steps)
        elif a.leg == "c3":
            r = leg_c3(torch, ttq, a.which, a.steps)
        elif a.leg == "c2":
            r = leg_c2(torch, ttq, a.T or 1, a.steps, a.warmup, a.qformat,
                       False, False)
        elif a.leg == "decode":
            r = leg_decode(torch, ttq, a.steps)
        elif a.leg == "segmented":
            r = leg_segmented(torch, ttq, a.steps)
        elif a.leg == "pca":
            r = leg_pca(torch, ttq, a.steps)
        else:
            r = leg_ceilings(torch)
        if a.copy_calib_mb:
            copy_calibration(a.copy_calib_mb, torch)
        emit({a.leg: r})
        return

    T = 4096
    head = leg_c5(torch, ttq, T, a.steps, a.warmup, want_gemm=True)
    print(f"# c5 T={T}: {head['ms_per_step']:.2f} ms/step", file=sys.stderr,
          flush=True)
    legs = {}
    for t in (1, 16, 256):
        legs[f"c5_T{t}"] = leg_c5(torch, ttq, t, 20, 3, want_gemm=True)
        print(f"# c5 T={t} done", file=sys.stderr, flush=True)
    legs["c4_p2"] = leg_c4(torch, ttq, 2.0, 10)
    legs["c4_p1"] = leg_c4(torch, ttq, 1.0, 10)
    legs["c3_gate_up"] = leg_c3(torch, ttq, "gate_up", 10)
    legs["c3_down"] = leg_c3(torch, ttq, "down", 10)
    print("# c4, c3 done", file=sys.stderr, flush=True)
    legs["c2_T1"] = leg_c2(torch, ttq, 1, 2000, 50, "asym", True, True)
    legs["c2_T128"] = leg_c2(torch, ttq, 128, 500, 20, "asym", False, True)
    fmts = {}
    for f in ("sym", "intzp", "fp8"):
        m = leg_c2(torch, ttq, 1, 500, 20, f, False, False)
        fmts[f] = {k: m[k] for k in ("ms", "tokens_per_s", "hbm_frac")}
        fmts[f]["dominant_kernel_ms"] = m["roofline"]["kernel_ms"]
    legs["c2_T1_other_formats"] = fmts
    legs["decode_from_codes"] = leg_decode(torch, ttq)
    legs["continuous_batching"] = leg_segmented(torch, ttq)
    legs["lowrank_pca"] = leg_pca(torch, ttq)
    ceil = leg_ceilings(torch)
    print("# context legs done", file=sys.stderr, flush=True)

    ms = head["ms_per_step"]
    roof = dict(head["roofline"])
    # the same kernel against the measured ceilings (context for frac)
    if roof["bound"] == "mfma":
        roof["frac_of_measured_gemm_ceiling"] = (
            roof["achieved"] / ceil["bf16_gemm"]["TFLOP_s"])
    else:
        roof["frac_of_measured_copy_ceiling"] = (
            roof["achieved"] / ceil["hbm_copy"]["GB_s"])
    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "7B-class decoder layer: q/k/v/o 4096->4096, gate/up "
                        "4096->11008, down 11008->4096; 8 requests x 4096 "
                        "tokens, per-request TTQ statistics and outlier "
                        "channels (1% of channels x10-100 log-uniform); 4-bit "
                        "g128 asymmetric, p=2, lambda=1e-3, alpha=0.5, "
                        "static low rank r=32 on all seven",
            "requests": 8, "T": T, "bits": 4, "group": 128, "rank": 32,
            "global_batch": 8 * T, "parallelism": "single GPU",
        },
        "roofline": roof,
        "step": head,
        "ceilings": ceil,
        **legs,
    }
    if not a.no_cpu:
        line["cpu_baseline"] = cpu_baseline_c5(T, a.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
