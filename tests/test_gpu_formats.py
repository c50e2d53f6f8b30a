"""GPU parity of the quantizer formats (symmetric, integer zero point, FP8
E4M3) against the CPU oracle, through the C ABI.

For every format and every path of ttq_linear (one token; the fused pass at
up to 16 and up to 128 tokens; the in-GEMM quantization at 129..256 tokens;
the quantize pass + GEMM, also forced) the codes, scales and stored offsets
must equal the oracle's float32 decision fed the kernel's own D^{1/2} bit
for bit, mismatches against the oracle's own statistics must lie in the
rounding band (in level units), and Y must meet the bars of ``parity_util``.
Quantize-once and decode (ttq_quantize, ttq_qmatmul on every route) are held
to the oracle the same way, the FP8 codes decoded as E4M3 values.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from parity_util import (BAND_REL, Y_MAX_REL, Y_MEAN_REL, check_problem,
                         run_gpu, to_dev, y_errors)
from workloads import make_problem
from workloads.configs import draw_x

pytestmark = pytest.mark.gpu

FUSED, TWO = 1, 2

FORMATS = [("sym", 4), ("sym", 2), ("intzp", 3), ("intzp", 8), ("fp8", 8)]

# (T, flags): one token; fused up to 16 and up to 128 tokens; in-GEMM
# quantization (T in 129..256, d % 128 == 0); the two-phase path, forced
PATHS = [(1, 0), (16, 0), (100, 0), (200, 0), (40, TWO)]


def _say(name, rep):
    print(f"[parity] {name}: " + " ".join(
        f"{k}={v:.3g}" if isinstance(v, float) else f"{k}={v}"
        for k, v in rep.items()), flush=True)


@pytest.mark.parametrize("fmt,bits", FORMATS, ids=[f"{f}{b}" for f, b in FORMATS])
@pytest.mark.parametrize("T,flags", PATHS, ids=[f"T{t}_f{f}" for t, f in PATHS])
def test_linear_formats(fmt, bits, T, flags):
    group = 64 if bits == 2 else 128
    prob = make_problem(f"{fmt}{bits}", d=1024, d_out=272, T=T, bits=bits,
                        group=group, rank=32 if T > 1 else 0,
                        x_kind="logu10_100", n_outliers=10, seed=60 + bits,
                        qformat=fmt)
    print(f"[case] {fmt} b={bits} g={group} T={T} flags={flags}", flush=True)
    gpu = run_gpu(prob, flags=flags)
    rep = check_problem(prob, gpu)
    _say(f"{fmt}{bits}_T{T}_f{flags}", rep)
    if T > 1 and flags == 0:
        # without exports (other kernel instantiations, and the in-GEMM
        # quantization at T = 200): the same bars
        g2 = run_gpu(prob, flags=flags, exports=False)
        rep2 = check_problem(prob, g2, check_codes=False)
        _say(f"{fmt}{bits}_T{T}_noexport", rep2)


@pytest.mark.parametrize("fmt,bits", [("sym", 4), ("fp8", 8)])
def test_formats_batched_and_group_sizes(fmt, bits):
    for group, T in ((32, 5), (64, 5), (256, 5), (128, 1), (64, 1)):
        prob = make_problem(f"{fmt}_g{group}", d=768, d_out=150, T=T, R=3,
                            bits=bits, group=group, rank=16, seed=70 + group,
                            x_kind="logu10_100", n_outliers=6, qformat=fmt)
        print(f"[case] {fmt} batched g={group} T={T}", flush=True)
        for flags in (0, TWO):
            rep = check_problem(prob, run_gpu(prob, flags=flags))
            _say(f"{fmt}_g{group}_R3_f{flags}", rep)


def test_gemm_quant_formats_match_two_phase():
    """The in-GEMM quantization gives the quantize pass + GEMM's Y bit for
    bit in every format (same decisions, same bf16 operand, same order)."""
    import online_activation_aware_ttq_amd as ttq
    for fmt, bits in (("sym", 4), ("intzp", 3), ("fp8", 8)):
        for group in (32, 64, 128):
            prob = make_problem("gq", d=512, d_out=300, T=170, R=2, bits=bits,
                                group=group, rank=32, seed=80 + group,
                                qformat=fmt)
            prm = ttq.make_params(d=prob.d, d_out=prob.d_out, T=prob.T,
                                  rank=prob.rank, bits=bits, group=group,
                                  p=prob.p, lam=prob.lam, alpha=prob.alpha,
                                  qformat=fmt)
            assert ttq.ttq_path(prm, prob.R) == 3
            print(f"[case] gemm_quant {fmt} g={group}", flush=True)
            g3 = run_gpu(prob, flags=0, exports=False)
            g1 = run_gpu(prob, flags=TWO, exports=False)
            assert not (g3["Y"] != g1["Y"]).any(), (fmt, group)


def test_degenerate_groups_in_every_format():
    # constant rows, an all-zero group (zero activations with lambda = 0 keep
    # D = I there), and a row of zeros
    for fmt, bits in (("sym", 4), ("intzp", 4), ("fp8", 8)):
        prob = make_problem("deg", d=256, d_out=48, T=8, bits=bits, group=64,
                            lam=0.0, seed=41, qformat=fmt)
        prob.W[:5] = prob.W[0, 0]
        prob.W[7] = 0
        prob.X[0][:, :64] = 0
        for flags in (FUSED, TWO):
            gpu = run_gpu(prob, flags=flags)
            rep = check_problem(prob, gpu)
            _say(f"deg_{fmt}_f{flags}", rep)
            assert np.all(gpu["s"][0][7] == 0) and np.all(gpu["m"][0][7] == 0)


# ------------------------------------------------------------ quantize + decode
def _gpu_quantize(prob):
    import torch
    import online_activation_aware_ttq_amd as ttq
    dh = torch.empty(prob.d, dtype=torch.float32, device="cuda")
    codes, s, m, dhi = ttq.ttq_quantize(
        to_dev(prob.W), to_dev(prob.X[0]), dhalf_out=dh, bits=prob.bits,
        group=prob.group, p=prob.p, lam=prob.lam, alpha=prob.alpha,
        qformat=prob.qformat)
    torch.cuda.synchronize()
    return dict(packed=codes.cpu().numpy(), s=s.cpu().numpy(),
                m=m.cpu().numpy(), dhi=dhi.cpu().numpy(), dh=dh.cpu().numpy(),
                dev=(codes, s, m, dhi))


def _gpu_qmatmul(stored, Xs, prob, flags):
    import torch
    import online_activation_aware_ttq_amd as ttq
    codes, s, m, dhi = stored
    Bm = to_dev(prob.B) if prob.rank else None
    A = to_dev(prob.A) if prob.rank else None
    Y = ttq.ttq_qmatmul(codes, s, m, dhi, to_dev(Xs), Bm, A, bits=prob.bits,
                        group=prob.group, flags=flags, qformat=prob.qformat)
    torch.cuda.synchronize()
    return Y.cpu().numpy()


def _upload(*arrs):
    import torch
    return tuple(torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in arrs)


def _check_y(Y, ref, rep, key):
    e, _ = y_errors(Y, ref)
    rep[key] = float(e.max()) if e.size else 0.0
    assert np.all(np.isfinite(Y))
    if e.size:
        assert e.max() <= Y_MAX_REL, (key, e.max())
        assert e.mean() <= Y_MEAN_REL, (key, e.mean())


@pytest.mark.parametrize("fmt,bits,group", [("sym", 4, 128), ("intzp", 2, 64),
                                            ("fp8", 8, 128), ("fp8", 8, 32),
                                            ("sym", 8, 256), ("fp8", 8, 256),
                                            ("intzp", 4, 32)])
def test_quantize_then_decode_formats(fmt, bits, group):
    prob = make_problem(f"q_{fmt}", d=1024, d_out=300, T=40, bits=bits,
                        group=group, rank=32, x_kind="logu10_100",
                        n_outliers=10, seed=90 + bits, qformat=fmt)
    print(f"[case] quantize+decode {fmt} b={bits} g={group}", flush=True)
    rep = {}
    g = _gpu_quantize(prob)
    kw = dict(bits=bits, group=group, p=prob.p, lam=prob.lam, alpha=prob.alpha,
              qformat=fmt)
    qz = oracle.ttq_quantize(prob.W, prob.X[0], **kw)
    # strict: the oracle's decision on the kernel's own D^{1/2}
    qs = oracle.ttq_quantize(prob.W, prob.X[0], dh32_override=g["dh"], **kw)
    np.testing.assert_array_equal(g["packed"], qs["packed"])
    np.testing.assert_array_equal(g["s"].view(np.uint32), qs["s"].view(np.uint32))
    np.testing.assert_array_equal(g["m"].view(np.uint32), qs["m"].view(np.uint32))
    # contract: against the oracle's own statistics, band rule in level units
    ref = oracle.ttq_linear(prob.W, prob.X[0], want_t=True, **kw)
    q_gpu = oracle.unpack_codes(g["packed"], bits, prob.d)
    z_gpu = None
    if fmt == "intzp":
        with np.errstate(divide="ignore", invalid="ignore"):
            z_gpu = np.where(g["s"] > 0, np.rint(g["m"].astype(np.float64) / g["s"]), 0.0)
    lv_g = oracle.format_levels(q_gpu, bits, fmt, z=z_gpu, group=group)
    lv_r = oracle.format_levels(ref["q"], bits, fmt, z=ref.get("z"), group=group)
    nb, ne = oracle.band_excused_levels(lv_g, lv_r, ref["t64"], BAND_REL)
    assert nb == ne, f"{nb - ne} unexcused code mismatches"
    rep.update(code_mismatch=nb)
    stored_or = _upload(qz["packed"], qz["s"], qz["m"], qz["dhi32"])
    for Ts in (1, 7, 100, 200):
        Xs = draw_x(prob.meta["seed"], 1, 1, Ts, prob.d, "logu10_100", 10)[0]
        Y_or = oracle.ttq_qmatmul(qz["packed"], qz["s"], qz["m"], qz["dhi32"], Xs,
                                  bits=bits, group=group, B_bits=prob.B,
                                  A_bits=prob.A, qformat=fmt)
        for flags in (0, TWO):
            _check_y(_gpu_qmatmul(stored_or, Xs, prob, flags), Y_or, rep,
                     f"dec_T{Ts}_f{flags}")
            _check_y(_gpu_qmatmul(g["dev"], Xs, prob, flags), Y_or, rep,
                     f"e2e_T{Ts}_f{flags}")
    _say(f"q_{fmt}{bits}_g{group}", rep)


def test_segmented_with_a_format_equals_single_calls():
    import torch
    import online_activation_aware_ttq_amd as ttq
    lengths = [1, 9, 0, 40, 1, 150]
    base = make_problem("segf", d=512, d_out=272, T=1, bits=8, group=128,
                        rank=16, seed=95, qformat="fp8")
    xs = [draw_x(300 + i, 0, 1, t, 512, "logu10_100", 5)[0]
          for i, t in enumerate(lengths)]
    offs = np.concatenate([[0], np.cumsum(lengths)]).tolist()
    W, Bm, A = to_dev(base.W), to_dev(base.B), to_dev(base.A)
    kw = dict(p=base.p, lam=base.lam, alpha=base.alpha, bits=8, group=128,
              qformat="fp8")
    Y = ttq.ttq_linear_segmented(W, to_dev(np.concatenate(xs)), Bm, A,
                                 seg_offsets=offs, **kw)
    torch.cuda.synchronize()
    Y = Y.cpu().numpy()
    for i, x in enumerate(xs):
        if not x.shape[0]:
            continue
        y1 = ttq.ttq_linear(W, to_dev(x), Bm, A, **kw)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(Y[offs[i]:offs[i + 1]].view(np.uint32),
                                      y1.cpu().numpy().view(np.uint32))
    prob = dataclasses.replace(base, T=40, X=xs[3][None])
    check_problem(prob, {"Y": Y[offs[3]:offs[4]][None]}, check_codes=False)


@pytest.mark.parametrize("fmt,bits", [("sym", 3), ("fp8", 8)])
def test_formats_segmented_with_exports_and_group_256(fmt, bits):
    """Formats through continuous batching with exports (consecutive runs),
    and group 256 on the fused path at 65..128 tokens."""
    import torch
    import online_activation_aware_ttq_amd as ttq
    lengths = [3, 3, 70, 1]
    base = make_problem("segx", d=512, d_out=160, T=1, bits=bits, group=256,
                        rank=0, seed=97, qformat=fmt)
    xs = [draw_x(400 + i, 0, 1, t, 512, "logu10_100", 5)[0]
          for i, t in enumerate(lengths)]
    offs = np.concatenate([[0], np.cumsum(lengths)]).tolist()
    W = to_dev(base.W)
    n = len(xs)
    G = 2
    kw = dict(p=base.p, lam=base.lam, alpha=base.alpha, bits=bits, group=256,
              qformat=fmt)
    ex = dict(codes_out=torch.empty((n, 160, 512), dtype=torch.uint8, device="cuda"),
              scales_out=torch.empty((n, 160, G), dtype=torch.float32, device="cuda"),
              mins_out=torch.empty((n, 160, G), dtype=torch.float32, device="cuda"),
              dhalf_out=torch.empty((n, 512), dtype=torch.float32, device="cuda"))
    Y = ttq.ttq_linear_segmented(W, to_dev(np.concatenate(xs)), seg_offsets=offs,
                                 **kw, **ex)
    torch.cuda.synchronize()
    Yh = Y.cpu().numpy()
    for i, x in enumerate(xs):
        prob = dataclasses.replace(base, T=x.shape[0], X=x[None])
        gpu = {"Y": Yh[offs[i]:offs[i + 1]][None],
               "q": ex["codes_out"][i].cpu().numpy()[None],
               "s": ex["scales_out"][i].cpu().numpy()[None],
               "m": ex["mins_out"][i].cpu().numpy()[None],
               "dh": ex["dhalf_out"][i].cpu().numpy()[None]}
        rep = check_problem(prob, gpu)
        _say(f"seg_{fmt}_g256_req{i}_T{x.shape[0]}", rep)
