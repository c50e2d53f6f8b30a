"""GPU parity of quantize-once / decode-from-codes (ttq_quantize, ttq_qmatmul)
against the CPU oracle, through the C ABI.

Three checks per case:
  * ttq_quantize on the prompt: D^{1/2} and D^{-1/2} within one float32 ulp
    of the oracle's, and the packed codes, scales and minima against the
    oracle's own statistics (bit for bit wherever the group's D^{1/2}
    agrees bit for bit; code mismatches only inside the rounding band of
    ``parity_util``, counted);
  * ttq_qmatmul alone: the oracle's stored values uploaded, the step's Y
    against ``oracle.ttq_qmatmul`` on the same values (Y bars of
    ``parity_util``);
  * end to end: both calls on the GPU against the oracle's quantize +
    decode (Y bars).
Shapes span several row blocks with ragged tails, every container width,
every group size, both statistics routes of ttq_quantize (T <= 128 and
larger) and the three routes of ttq_qmatmul (one token; up to 128 tokens on
the codes; dequantize + GEMM, also forced at small T).
"""
import numpy as np
import pytest

import oracle
from parity_util import BAND_REL, Y_MAX_REL, Y_MEAN_REL, to_dev, y_errors
from workloads import make_c2, make_problem
from workloads.configs import draw_x

pytestmark = pytest.mark.gpu

TWO = 2


def _kw(p):
    return dict(bits=p.bits, group=p.group, p=p.p, lam=p.lam, alpha=p.alpha)


def _step_x(prob, T, call=1):
    return draw_x(prob.meta["seed"], call, 1, T, prob.d, prob.meta["x_kind"],
                  prob.meta["n_outliers"])[0]


def _gpu_quantize(prob):
    import torch
    import online_activation_aware_ttq_amd as ttq
    dh = torch.empty(prob.d, dtype=torch.float32, device="cuda")
    codes, s, m, dhi = ttq.ttq_quantize(to_dev(prob.W), to_dev(prob.X[0]),
                                        dhalf_out=dh, **_kw(prob))
    torch.cuda.synchronize()
    return dict(packed=codes.cpu().numpy(), s=s.cpu().numpy(),
                m=m.cpu().numpy(), dhi=dhi.cpu().numpy(), dh=dh.cpu().numpy(),
                dev=(codes, s, m, dhi))


def _gpu_qmatmul(dev_stored, Xs_bits, prob, flags=0):
    import torch
    import online_activation_aware_ttq_amd as ttq
    codes, s, m, dhi = dev_stored
    Bm = to_dev(prob.B) if prob.rank else None
    A = to_dev(prob.A) if prob.rank else None
    Y = ttq.ttq_qmatmul(codes, s, m, dhi, to_dev(Xs_bits), Bm, A,
                        bits=prob.bits, group=prob.group, flags=flags)
    torch.cuda.synchronize()
    return Y.cpu().numpy()


def _ulps(a, b):
    return np.abs(a.view(np.int32).astype(np.int64)
                  - b.view(np.int32).astype(np.int64))


def check_quantize(prob, g, rep):
    """GPU ttq_quantize outputs against the oracle's own statistics."""
    ref = oracle.ttq_linear(prob.W, prob.X[0], want_t=True, **_kw(prob))
    qz = oracle.ttq_quantize(prob.W, prob.X[0], **_kw(prob))
    assert _ulps(g["dh"], qz["dh32"]).max(initial=0) <= 1
    assert _ulps(g["dhi"], qz["dhi32"]).max(initial=0) <= 1
    rep["dh_mismatch"] = int((g["dh"].view(np.uint32) != qz["dh32"].view(np.uint32)).sum())
    rep["dhi_mismatch"] = int((g["dhi"].view(np.uint32) != qz["dhi32"].view(np.uint32)).sum())
    assert g["packed"].shape == qz["packed"].shape
    q_gpu = oracle.unpack_codes(g["packed"], prob.bits, prob.d)
    # the bytes must be a valid packing (codes < 2^b in every container)
    np.testing.assert_array_equal(oracle.pack_codes(q_gpu, prob.bits), g["packed"])
    nb, ne, nl = oracle.band_excused(q_gpu, ref["q"], ref["t64"], ref["u64"],
                                     ref["m64"], ref["s64"], prob.group,
                                     BAND_REL)
    rep.update(code_mismatch=nb, code_excused=ne, literal_band=nl)
    assert nb == ne, f"{nb - ne} unexcused code mismatches"
    # groups whose D^{1/2} agrees bit for bit decide identically: s, m exact
    G = prob.d // prob.group
    same = (g["dh"].view(np.uint32) == qz["dh32"].view(np.uint32))
    gsame = same.reshape(G, prob.group).all(axis=1)
    np.testing.assert_array_equal(g["s"][:, gsame].view(np.uint32),
                                  qz["s"][:, gsame].view(np.uint32))
    np.testing.assert_array_equal(g["m"][:, gsame].view(np.uint32),
                                  qz["m"][:, gsame].view(np.uint32))
    return qz


def check_y(Y_gpu, Y_ref, rep, key):
    e, nw = y_errors(Y_gpu, Y_ref)
    rep[key + "_max"] = float(e.max()) if e.size else 0.0
    rep[key + "_mean"] = float(e.mean()) if e.size else 0.0
    assert np.all(np.isfinite(Y_gpu))
    if e.size:
        assert e.max() <= Y_MAX_REL, (key, e.max())
        assert e.mean() <= Y_MEAN_REL, (key, e.mean())


CASES = [
    # name, problem kwargs (prompt T), step T values, qmatmul flags
    ("b4_g128_T16", dict(d=1024, d_out=1040, T=16, bits=4, group=128,
                         x_kind="logu10_100", n_outliers=10, seed=41), (1, 5)),
    ("b4_g128_T200", dict(d=1024, d_out=520, T=200, bits=4, group=128, rank=32,
                          x_kind="logu10_100", n_outliers=10, seed=42), (1, 33)),
    ("b3_g32_r64", dict(d=512, d_out=300, T=64, bits=3, group=32, rank=64,
                        seed=43), (1, 130)),
    ("b2_g64", dict(d=1024, d_out=200, T=8, bits=2, group=64, rank=8,
                    p=1.0, lam=1e-2, x_kind="t3_logu30_100", n_outliers=5,
                    seed=44), (1, 4)),
    ("b1_g256", dict(d=1024, d_out=77, T=16, bits=1, group=256, seed=45), (1, 2)),
    ("b8_g64", dict(d=2048, d_out=96, T=1, bits=8, group=64, seed=46), (1, 17)),
    ("b5_g32_T129", dict(d=256, d_out=50, T=129, bits=5, group=32, seed=47),
     (1, 3)),
    ("b4_p_general", dict(d=512, d_out=64, T=4, bits=4, group=128, p=0.5,
                          alpha=0.7, seed=48), (1,)),
    ("b8_d12288", dict(d=12288, d_out=40, T=3, bits=8, group=128, rank=16,
                       seed=49), (1,)),
    ("b4_d30720", dict(d=30720, d_out=24, T=2, bits=4, group=128, seed=50),
     (1,)),
]


@pytest.mark.parametrize("name,kw,steps", CASES, ids=[c[0] for c in CASES])
def test_quantize_then_decode(name, kw, steps):
    prob = make_problem(name, **kw)
    print(f"[case] {name} d={prob.d} d_out={prob.d_out} T={prob.T} "
          f"b={prob.bits} g={prob.group} r={prob.rank} steps={steps}",
          flush=True)
    rep = {}
    g = _gpu_quantize(prob)
    qz = check_quantize(prob, g, rep)
    stored_oracle = tuple(
        t for t in _upload(qz["packed"], qz["s"], qz["m"], qz["dhi32"]))
    for Ts in steps:
        Xs = _step_x(prob, Ts)
        Y_or = oracle.ttq_qmatmul(qz["packed"], qz["s"], qz["m"], qz["dhi32"],
                                  Xs, bits=prob.bits, group=prob.group,
                                  B_bits=prob.B, A_bits=prob.A)
        for flags in (0, TWO):
            # decode kernel alone, on the oracle's stored values
            Y1 = _gpu_qmatmul(stored_oracle, Xs, prob, flags)
            check_y(Y1, Y_or, rep, f"decode_T{Ts}_f{flags}")
            # end to end: the GPU's own stored values
            Y2 = _gpu_qmatmul(g["dev"], Xs, prob, flags)
            check_y(Y2, Y_or, rep, f"e2e_T{Ts}_f{flags}")
    print(f"[parity] {name}: " + " ".join(
        f"{k}={v:.3g}" if isinstance(v, float) else f"{k}={v}"
        for k, v in rep.items()), flush=True)


def _upload(packed, s, m, dhi):
    import torch
    dev = torch.device("cuda")
    return (torch.from_numpy(np.ascontiguousarray(packed)).to(dev),
            torch.from_numpy(np.ascontiguousarray(s)).to(dev),
            torch.from_numpy(np.ascontiguousarray(m)).to(dev),
            torch.from_numpy(np.ascontiguousarray(dhi)).to(dev))


def test_decode_on_the_prompt_matches_one_shot_projection():
    """On the prompt itself, decoding the stored codes gives what ttq_linear
    gives (same codes; D^{-1/2} stored in float32)."""
    import torch
    import online_activation_aware_ttq_amd as ttq
    prob = make_problem("prompt_eq", d=1024, d_out=272, T=1, bits=4,
                        group=128, rank=16, x_kind="logu10_100",
                        n_outliers=10, seed=51)
    g = _gpu_quantize(prob)
    Y_dec = _gpu_qmatmul(g["dev"], prob.X[0], prob)
    Y_lin = ttq.ttq_linear(to_dev(prob.W), to_dev(prob.X[0]), to_dev(prob.B),
                           to_dev(prob.A), **_kw(prob)).cpu().numpy()
    torch.cuda.synchronize()
    e, _ = y_errors(Y_dec, Y_lin.astype(np.float64))
    assert e.max() <= 1e-4, e.max()


def test_empty_and_degenerate():
    import torch
    import online_activation_aware_ttq_amd as ttq
    dev = torch.device("cuda")
    # a step with no tokens: nothing to compute
    prob = make_problem("deg", d=256, d_out=40, T=4, bits=4, group=64, seed=52)
    g = _gpu_quantize(prob)
    codes, s, m, dhi = g["dev"]
    Y = ttq.ttq_qmatmul(codes, s, m, dhi,
                        torch.empty((0, 256), dtype=torch.bfloat16, device=dev),
                        bits=4, group=64)
    assert Y.shape == (0, 40)
    # constant groups (s = 0) decode to the constant; zero channels too.
    # Only some rows get the constant group: a row whose output is one
    # group of equal weights carries the same bf16 rounding of W_hat on the
    # dequantize route in every row, and the mean bar assumes errors that
    # vary from row to row.
    W = prob.W.copy()
    W[0:40:4, :64] = oracle_bits(0.5)
    W[3, :] = oracle_bits(0.0)
    prob2 = make_problem("deg2", d=256, d_out=40, T=4, bits=4, group=64, seed=52)
    prob2.W = W
    X = prob2.X.copy()
    X[:, :, 64:128] = 0
    prob2.X = X
    rep = {}
    g2 = _gpu_quantize(prob2)
    qz = check_quantize(prob2, g2, rep)
    Xs = _step_x(prob2, 3)
    Y_or = oracle.ttq_qmatmul(qz["packed"], qz["s"], qz["m"], qz["dhi32"], Xs,
                              bits=4, group=64)
    for flags in (0, TWO):
        check_y(_gpu_qmatmul(g2["dev"], Xs[:1], prob2, flags), Y_or[:1], rep,
                f"deg_T1_f{flags}")
    check_y(_gpu_qmatmul(g2["dev"], Xs, prob2), Y_or, rep, "deg_T3")


def oracle_bits(v):
    return np.float32(v).view(np.uint32) >> 16


def test_full_size_decode_q_proj():
    """4096 x 4096 attention projection, 4-bit g128: quantize on a 128-token
    prompt, decode one token; sampled rows against the oracle."""
    prob = make_c2(T=128)
    rows = np.unique(np.concatenate([
        np.arange(8), np.arange(prob.d_out - 8, prob.d_out),
        np.random.default_rng(7).choice(prob.d_out, 48, replace=False)]))
    print(f"[case] full-size decode d={prob.d} d_out={prob.d_out} "
          f"prompt T={prob.T}", flush=True)
    g = _gpu_quantize(prob)
    qz = oracle.ttq_quantize(prob.W, prob.X[0], rows=rows, **_kw(prob))
    assert _ulps(g["dh"], qz["dh32"]).max() <= 1
    q_gpu = oracle.unpack_codes(g["packed"][rows], prob.bits, prob.d)
    ref = oracle.ttq_linear(prob.W, prob.X[0], rows=rows, want_t=True,
                            **_kw(prob))
    nb, ne, _ = oracle.band_excused(q_gpu, ref["q"], ref["t64"], ref["u64"],
                                    ref["m64"], ref["s64"], prob.group,
                                    BAND_REL)
    assert nb == ne
    Xs = _step_x(prob, 1)
    Y_or = oracle.ttq_qmatmul(qz["packed"], qz["s"], qz["m"], qz["dhi32"], Xs,
                              bits=prob.bits, group=prob.group)
    Y = _gpu_qmatmul(g["dev"], Xs, prob)[:, rows]
    rep = {"code_mismatch": nb}
    check_y(Y, Y_or, rep, "decode_T1")
    print(f"[parity] full-size decode: {rep}", flush=True)


PREFILL_CASES = [
    # the GEMM that expands the stored codes itself (T > 128): every container
    # width, every group size, ragged token / row tiles, low-rank segments
    ("p_b4_g128_r32", dict(d=1024, d_out=520, T=16, bits=4, group=128, rank=32,
                           x_kind="logu10_100", n_outliers=10, seed=61), (300,)),
    ("p_b3_g32_r64", dict(d=512, d_out=300, T=64, bits=3, group=32, rank=64,
                          seed=62), (130, 257)),
    ("p_b2_g64_r8", dict(d=1024, d_out=200, T=8, bits=2, group=64, rank=8,
                         seed=63), (129,)),
    ("p_b1_g256", dict(d=1024, d_out=77, T=16, bits=1, group=256, seed=64), (200,)),
    ("p_b8_g64", dict(d=2048, d_out=96, T=1, bits=8, group=64, seed=65), (160,)),
    ("p_b5_g32", dict(d=256, d_out=50, T=4, bits=5, group=32, seed=66), (140,)),
]


@pytest.mark.parametrize("name,kw,steps", PREFILL_CASES,
                         ids=[c[0] for c in PREFILL_CASES])
def test_prefill_decode_expands_codes_in_the_gemm(name, kw, steps):
    """Y of the GEMM that expands the codes tile by tile equals the forced
    expand-to-HBM + GEMM route bit for bit (same float32 expansion, same
    rounding, same MFMA order), and meets the oracle's bars."""
    prob = make_problem(name, **kw)
    g = _gpu_quantize(prob)
    rep = {}
    for Ts in steps:
        print(f"[case] {name} prefill decode T={Ts}", flush=True)
        Xs = _step_x(prob, Ts)
        Y3 = _gpu_qmatmul(g["dev"], Xs, prob, 0)
        Y1 = _gpu_qmatmul(g["dev"], Xs, prob, TWO)
        diff = Y3.view(np.uint32) != Y1.view(np.uint32)
        assert not diff.any(), f"T={Ts}: {int(diff.sum())} outputs differ"
        Y_or = oracle.ttq_qmatmul(g["packed"], g["s"], g["m"], g["dhi"], Xs,
                                  bits=prob.bits, group=prob.group,
                                  B_bits=prob.B, A_bits=prob.A)
        check_y(Y3, Y_or, rep, f"T{Ts}")
    print(f"[parity] {name}: " + " ".join(f"{k}={v:.3g}" for k, v in rep.items()),
          flush=True)
