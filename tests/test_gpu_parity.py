"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Reduced shapes span several tiles and ragged tails on both paths (fused
single pass for T <= 128 and the two-phase quantize + GEMM path), every
code path of the kernels (group sizes, bit widths, norm orders, low rank,
batched requests) and the degenerate cases of the method.  The bars are
written in ``parity_util``.
"""
import json
import os

import numpy as np
import pytest

import oracle
from parity_util import check_problem, run_gpu
from workloads import make_c1, make_problem

pytestmark = pytest.mark.gpu

FUSED, TWO = 1, 2


def _say(name, rep):
    print(f"[parity] {name}: " + " ".join(
        f"{k}={v:.3g}" if isinstance(v, float) else f"{k}={v}"
        for k, v in rep.items()), flush=True)
    log = os.environ.get("TTQ_PARITY_LOG")
    if log:
        with open(log, "a") as f:
            f.write(json.dumps(dict(case=name, **rep)) + "\n")


def _run_and_check(prob, flags=0, name=None):
    print(f"[case] {name or prob.name} d={prob.d} d_out={prob.d_out} T={prob.T} "
          f"R={prob.R} b={prob.bits} g={prob.group} r={prob.rank} p={prob.p} "
          f"flags={flags}", flush=True)
    gpu = run_gpu(prob, flags=flags)
    rep = check_problem(prob, gpu)
    _say(name or prob.name, rep)
    return gpu, rep


@pytest.mark.parametrize("flags", [FUSED, TWO])
def test_c1_both_paths(flags):
    _run_and_check(make_c1(), flags)


CASES = [
    # name, kwargs (reduced shapes of the standard workloads + edge shapes)
    ("c2s_T1", dict(d=1024, d_out=1040, T=1, bits=4, group=128,
                    x_kind="logu10_100", n_outliers=10, seed=1)),
    ("c2s_T128", dict(d=1024, d_out=1040, T=128, bits=4, group=128,
                      x_kind="logu10_100", n_outliers=10, seed=1)),
    ("c3s_gateup", dict(d=512, d_out=1376, T=300, bits=3, group=128, rank=64,
                        seed=2)),
    ("c3s_down", dict(d=1376 // 32 * 32, d_out=512, T=200, bits=3, group=32,
                      rank=64, seed=12)),
    ("c4s_p1", dict(d=1024, d_out=896, T=512, bits=2, group=64, rank=128,
                    p=1.0, lam=1e-2, x_kind="t3_logu30_100", n_outliers=5,
                    seed=3)),
    ("c4s_p2", dict(d=1024, d_out=896, T=512, bits=2, group=64, rank=128,
                    p=2.0, lam=1e-2, x_kind="t3_logu30_100", n_outliers=5,
                    seed=3)),
    ("ragged_T17_g256", dict(d=768, d_out=40, T=17, bits=5, group=256, seed=21)),
    ("ragged_T33_g32", dict(d=96, d_out=33, T=33, bits=3, group=32, rank=8,
                            seed=22)),
    ("T65_b8", dict(d=256, d_out=100, T=65, bits=8, group=64, seed=23)),
    ("b1", dict(d=256, d_out=48, T=16, bits=1, group=32, seed=24)),
    ("p_general", dict(d=256, d_out=64, T=16, bits=4, group=128, p=0.5,
                       seed=25)),
    ("p3", dict(d=256, d_out=64, T=129, bits=4, group=64, p=3.0, seed=26)),
    ("alpha0_rtn", dict(d=256, d_out=64, T=16, bits=3, group=128, alpha=0.0,
                        seed=27)),
    ("alpha2_lam0", dict(d=512, d_out=64, T=8, bits=4, group=128, alpha=2.0,
                         lam=0.0, seed=28)),
    # one token: the single-launch kernel, its general-p / general-alpha
    # instantiation and the group sizes
    ("T1_p_general", dict(d=512, d_out=80, T=1, bits=4, group=64, p=0.5,
                          seed=29)),
    ("T1_alpha_general", dict(d=512, d_out=80, T=1, bits=3, group=32,
                              alpha=0.7, seed=30)),
    ("T1_g256_r16", dict(d=1024, d_out=72, T=1, bits=4, group=256, rank=16,
                         seed=32)),
    ("T1_alpha1_p1", dict(d=384, d_out=50, T=1, bits=2, group=128, p=1.0,
                          alpha=1.0, lam=0.0, seed=33)),
    # the small-token low-rank product Z = X A^T: several 32-column rank jobs
    # per 16-token tile (rank 200, padded to 224), a ragged last token tile,
    # channel runs of the 8 waves that end mid-run (d = 800); in the
    # statistics launch (T = 100) and in its own launch (T = 1)
    ("z_r200_T100", dict(d=800, d_out=130, T=100, R=3, bits=4, group=32,
                         rank=200, x_kind="logu10_100", n_outliers=8,
                         seed=34)),
    ("z_r200_T1", dict(d=800, d_out=130, T=1, R=5, bits=4, group=32,
                       rank=200, x_kind="logu10_100", n_outliers=8, seed=35)),
]


@pytest.mark.parametrize("flags", [0, FUSED, TWO])
@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_reduced_cases(name, kw, flags):
    prob = make_problem(name, **kw)
    if flags == FUSED and prob.T > 128:
        pytest.skip("fused path covers T <= 128")
    _run_and_check(prob, flags, name)


@pytest.mark.parametrize("T", [1, 16, 100, 256])
@pytest.mark.parametrize("flags", [0, TWO])
def test_batched_requests(T, flags):
    prob = make_problem("c5s", d=512, d_out=272, T=T, R=8, bits=4, group=128,
                        rank=32, x_kind="logu10_100", n_outliers=5, seed=4)
    gpu, rep = _run_and_check(prob, flags, f"c5s_T{T}")
    # each request has its own statistics: D differs between requests
    assert not np.array_equal(gpu["dh"][0], gpu["dh"][1])


@pytest.mark.parametrize("R", [1, 3])
def test_gemm_more_tiles_than_cus(R):
    """Large-tile GEMM with more output tiles than the chip has CUs (a second,
    partly filled round): R = 1, 9 x 32 tiles of 256 x 128 = 288; R = 3, the
    same tile count over three requests' products, each with its own W_hat;
    the low-rank segment is part of every tile's K range."""
    T = 2304 if R == 1 else 768
    prob = make_problem(f"tail_R{R}", d=1024, d_out=4096, T=T, R=R, bits=4,
                        group=128, rank=32, x_kind="logu10_100", n_outliers=10,
                        seed=60 + R)
    rows = np.unique(np.concatenate([
        np.arange(16), np.arange(3072, 3100), np.arange(4096 - 16, 4096),
        np.random.default_rng(R).choice(4096, 32, replace=False)]))
    print(f"[case] two GEMM rounds R={R} T={T} rows={len(rows)}", flush=True)
    gpu = run_gpu(prob, flags=TWO, rows=rows)
    rep = check_problem(prob, gpu, rows=rows)
    _say(f"tail_R{R}", rep)


def test_persistent_gemm_ragged_tiles():
    """Enough 256 x 256 tiles for the persistent GEMM (more than four rounds
    of the chip's CUs) with every edge at once: ragged token tiles (T = 1000),
    ragged weight-row tiles (d_out = 4000), a channel count that ends in half
    a 64-channel k-tile (d = 544, groups of 32) in the tiled W_hat, a tile
    count whose last round of 32-tile patches is partial (17 requests), and
    a ragged low-rank segment (r = 40)."""
    prob = make_problem("persist", d=544, d_out=4000, T=1000, R=17, bits=4,
                        group=32, rank=40, x_kind="logu10_100", n_outliers=8,
                        seed=71)
    rows = np.unique(np.concatenate([
        np.arange(8), np.arange(3832, 3848), np.arange(4000 - 8, 4000),
        np.random.default_rng(7).choice(4000, 24, replace=False)]))
    print(f"[case] persistent GEMM R=17 T=1000 d=544 d_out=4000 rows={len(rows)}",
          flush=True)
    gpu = run_gpu(prob, rows=rows, exports=False)
    rep = check_problem(prob, gpu, rows=rows, check_codes=False)
    _say("persist", rep)


def test_split_schedule_gemm_ragged_tiles():
    """One partial round of 256 x 256 tiles (one tile per workgroup, the
    split-load schedule) with ragged token and weight-row tiles and a
    channel count ending in half a k-tile of the tiled W_hat."""
    prob = make_problem("split1", d=544, d_out=11000, T=600, bits=4, group=32,
                        rank=24, x_kind="logu10_100", n_outliers=8, seed=72)
    rows = np.unique(np.concatenate([
        np.arange(8), np.arange(10744, 10760), np.arange(11000 - 8, 11000),
        np.random.default_rng(8).choice(11000, 24, replace=False)]))
    print(f"[case] split-schedule GEMM T=600 d=544 d_out=11000 rows={len(rows)}",
          flush=True)
    gpu = run_gpu(prob, rows=rows, exports=False)
    rep = check_problem(prob, gpu, rows=rows, check_codes=False)
    _say("split1", rep)


def test_gemm_whole_rounds_and_narrow_tail():
    """A column count whose last round of 256 x 256 tiles would run partly
    empty: the first 8192 columns as whole rounds of 256 x 256 tiles, the
    ragged rest (356 columns, three 128-wide tiles) in a second launch of
    256 x 128 tiles, both with the ragged low-rank segment (r = 40) and
    the tiled W_hat offset past the split."""
    prob = make_problem("tail_split", d=256, d_out=8548, T=2048, bits=4,
                        group=32, rank=40, x_kind="logu10_100", n_outliers=4,
                        seed=73)
    rows = np.unique(np.concatenate([
        np.arange(8), np.arange(8184, 8200), np.arange(8548 - 12, 8548),
        np.random.default_rng(9).choice(8548, 24, replace=False)]))
    print(f"[case] whole rounds + tail T=2048 d=256 d_out=8548 rows={len(rows)}",
          flush=True)
    gpu = run_gpu(prob, rows=rows, exports=False)
    rep = check_problem(prob, gpu, rows=rows, check_codes=False)
    _say("tail_split", rep)


ROW_PAIR_CASES = [
    # fused path with two 16-row blocks per workgroup (taken for T > 16 when
    # that still leaves at least 256 workgroups): a ragged last pair (odd
    # row-block count), ragged tokens in every token-tile count, group sizes
    # 32 / 64 / 128 with an odd group count, low rank, p = 1, every quantizer
    # format; T = 16 (one row block, hi + lo activations) beside them
    ("rp_T100_g128", dict(d=512, d_out=2064, T=100, R=4, bits=4, group=128,
                          rank=32, x_kind="logu10_100", n_outliers=5,
                          seed=81)),
    ("rp_T40_g64_G9", dict(d=576, d_out=1000, T=40, R=8, bits=3, group=64,
                           rank=8, seed=82)),
    ("rp_T128_g32_p1", dict(d=256, d_out=4080, T=128, R=2, bits=2, group=32,
                            p=1.0, lam=1e-2, x_kind="t3_logu30_100",
                            n_outliers=3, seed=83)),
    ("rp_T16_hilo", dict(d=512, d_out=1040, T=16, R=8, bits=4, group=128,
                         rank=32, x_kind="logu10_100", n_outliers=5, seed=84)),
    ("rp_T17_g64", dict(d=384, d_out=1010, T=17, R=8, bits=4, group=64,
                        seed=85)),
    ("rp_T24_sym4", dict(d=256, d_out=1040, T=24, R=8, bits=4, group=128,
                         qformat="sym", x_kind="logu10_100", n_outliers=3,
                         seed=86)),
    ("rp_T64_intzp3", dict(d=256, d_out=1040, T=64, R=8, bits=3, group=64,
                           qformat="intzp", rank=16, seed=87)),
    ("rp_T128_fp8", dict(d=256, d_out=1040, T=128, R=8, bits=8, group=128,
                         qformat="fp8", x_kind="logu10_100", n_outliers=3,
                         seed=88)),
]


def test_fused_row_pairs_wide_d_without_lds_scales():
    """Two row blocks per workgroup with D^{1/2} read from memory instead of
    LDS (d = 16896 channels: 66 KiB of scales) and exports; sampled rows."""
    prob = make_problem("rp_wide", d=16896, d_out=1040, T=64, R=8, bits=4,
                        group=128, rank=16, x_kind="logu10_100",
                        n_outliers=20, seed=89)
    rows = np.unique(np.concatenate([
        np.arange(8), np.arange(1024, 1040),
        np.random.default_rng(10).choice(1040, 16, replace=False)]))
    print(f"[case] row pairs, d=16896 T=64 R=8 rows={len(rows)}", flush=True)
    gpu = run_gpu(prob, rows=rows)
    rep = check_problem(prob, gpu, rows=rows)
    _say("rp_wide", rep)


@pytest.mark.parametrize("name,kw", ROW_PAIR_CASES,
                         ids=[c[0] for c in ROW_PAIR_CASES])
def test_fused_row_pairs(name, kw):
    prob = make_problem(name, **kw)
    _run_and_check(prob, 0, name)
    # without exports (the other instantiation): the same bars
    rep = check_problem(prob, run_gpu(prob, exports=False), check_codes=False)
    _say(name + "_noexport", rep)


GEMM_Q_CASES = [
    # the GEMM that quantizes its own weight tiles (129 <= T <= 256): every
    # group size, ragged token / row tiles, low-rank segments of one, two and
    # four k-tiles (ragged rank), the shortest channel range (one chunk), an
    # odd number of chunks, batched requests
    ("gq_g128", dict(d=1024, d_out=1040, T=200, bits=4, group=128,
                     x_kind="logu10_100", n_outliers=10, seed=41)),
    ("gq_g64_r128_p1", dict(d=1024, d_out=896, T=256, bits=2, group=64,
                            rank=128, p=1.0, lam=1e-2, x_kind="t3_logu30_100",
                            n_outliers=5, seed=42)),
    ("gq_g32_r72", dict(d=384, d_out=200, T=129, bits=3, group=32, rank=72,
                        seed=43)),
    ("gq_d128_r200", dict(d=128, d_out=130, T=250, bits=5, group=64,
                          rank=200, seed=44)),
    ("gq_b8_r8", dict(d=640, d_out=136, T=200, bits=8, group=128, rank=8,
                      seed=45)),
    ("gq_b1_g32", dict(d=256, d_out=64, T=140, bits=1, group=32, seed=46)),
    ("gq_R3_r32", dict(d=512, d_out=272, T=256, R=3, bits=4, group=128,
                       rank=32, x_kind="logu10_100", n_outliers=5, seed=47)),
]


@pytest.mark.parametrize("name,kw", GEMM_Q_CASES, ids=[c[0] for c in GEMM_Q_CASES])
def test_gemm_quant_path(name, kw):
    """Y of the in-GEMM quantization equals that of the quantize pass + GEMM
    bit for bit (same float32 decisions, same bf16 rounding, same MFMA
    accumulation order) and meets the oracle's bars."""
    import online_activation_aware_ttq_amd as ttq
    prob = make_problem(name, **kw)
    prm = ttq.make_params(d=prob.d, d_out=prob.d_out, T=prob.T, rank=prob.rank,
                          bits=prob.bits, group=prob.group, p=prob.p,
                          lam=prob.lam, alpha=prob.alpha)
    assert ttq.ttq_path(prm, prob.R) == 3
    print(f"[case] {name} gemm_quant vs two-phase", flush=True)
    g3 = run_gpu(prob, flags=0, exports=False)
    g1 = run_gpu(prob, flags=TWO, exports=False)
    diff = g3["Y"] != g1["Y"]
    assert not diff.any(), f"{int(diff.sum())} outputs differ from the two-phase path"
    rep = check_problem(prob, g3, check_codes=False)
    _say(name, rep)


def test_batched_matches_single_calls():
    prob = make_problem("bs", d=512, d_out=160, T=4, R=3, bits=4, group=128,
                        rank=16, seed=31)
    gb = run_gpu(prob)
    for r in range(prob.R):
        single = make_problem("bs", d=512, d_out=160, T=4, R=1, bits=4,
                              group=128, rank=16, seed=31)
        single.X = prob.X[r:r + 1]
        gs = run_gpu(single)
        np.testing.assert_array_equal(gs["q"][0], gb["q"][r])
        np.testing.assert_array_equal(gs["dh"][0], gb["dh"][r])
        np.testing.assert_array_equal(gs["Y"][0], gb["Y"][r])


def test_row_pairs_match_single_calls_bit_for_bit():
    """Eight requests take two row blocks per workgroup (8 x 33 pairs >= 256
    workgroups), one request alone takes one: the same codes and the same Y
    bits (each output's arithmetic does not depend on the row pairing)."""
    kw = dict(d=512, d_out=1040, T=40, bits=4, group=128, rank=32,
              x_kind="logu10_100", n_outliers=5, seed=36)
    prob = make_problem("rpb", R=8, **kw)
    gb = run_gpu(prob)
    for r in (0, 5):
        single = make_problem("rpb", R=1, **kw)
        single.X = prob.X[r:r + 1]
        gs = run_gpu(single)
        np.testing.assert_array_equal(gs["q"][0], gb["q"][r])
        np.testing.assert_array_equal(gs["Y"][0], gb["Y"][r])


def test_degenerate_groups_and_zero_channels():
    # constant weight rows (max == min) and all-zero activation channels with
    # lambda = 0 (n + lambda = 0 -> neutral scale 1)
    prob = make_problem("deg", d=256, d_out=48, T=8, bits=4, group=64, lam=0.0,
                        seed=41)
    prob.W[:5] = prob.W[0, 0]
    prob.X[0][:, :64] = 0
    for flags in (FUSED, TWO):
        gpu, rep = _run_and_check(prob, flags, f"degenerate_f{flags}")
        # group 0: constant weights times the neutral scale -> max == min
        assert np.all(gpu["s"][0][:5, 0] == 0)
        assert np.all(gpu["q"][0][:5, :64] == 0)
        assert np.all(gpu["s"][0][5:, 0] > 0)
        assert np.all(gpu["dh"][0][:64] == 1.0)


def test_empty_shapes():
    import torch
    import online_activation_aware_ttq_amd as ttq
    from parity_util import to_dev
    prob = make_problem("e", d=256, d_out=32, T=0, bits=4, group=128, seed=5)
    gpu, _ = _run_and_check(prob, 0, "T0")
    ref = oracle.ttq_linear(prob.W, prob.X[0], bits=4, group=128, p=2.0,
                            lam=1e-3, alpha=0.5)
    np.testing.assert_array_equal(gpu["q"][0], ref["q"])
    gpu2, _ = _run_and_check(prob, TWO, "T0_two_phase")
    np.testing.assert_array_equal(gpu2["q"][0], ref["q"])
    # d_out = 0: only the statistics are produced
    p2 = make_problem("e2", d=256, d_out=1, T=5, bits=4, group=128, seed=6)
    W = to_dev(p2.W)[:0]
    X = to_dev(p2.X[0])
    dh = torch.empty(256, dtype=torch.float32, device="cuda")
    Y = ttq.ttq_linear(W, X, p=2.0, lam=1e-3, alpha=0.5, bits=4, group=128,
                       dhalf_out=dh)
    torch.cuda.synchronize()
    assert Y.shape == (5, 0)
    # d_out = 0 at T = 1 (the single-launch path): statistics only
    dh1 = torch.empty(256, dtype=torch.float32, device="cuda")
    Y1 = ttq.ttq_linear(W, X[:1], p=2.0, lam=1e-3, alpha=0.5, bits=4,
                        group=128, dhalf_out=dh1)
    torch.cuda.synchronize()
    assert Y1.shape == (1, 0)
    ref1 = oracle.ttq_linear(p2.W, p2.X[0][:1], bits=4, group=128, p=2.0,
                             lam=1e-3, alpha=0.5)
    np.testing.assert_array_equal(dh1.cpu().numpy(), ref1["dh32"])
    ref2 = oracle.ttq_linear(p2.W, p2.X[0], bits=4, group=128, p=2.0,
                             lam=1e-3, alpha=0.5)
    np.testing.assert_array_equal(dh.cpu().numpy(), ref2["dh32"])
    # zero requests
    Xb = to_dev(p2.X)[:0]
    Yb = ttq.ttq_linear_batched(to_dev(p2.W), Xb, p=2.0, lam=1e-3, alpha=0.5,
                                bits=4, group=128)
    assert Yb.shape == (0, 5, 1)


@pytest.mark.parametrize("T", [1, 16, 200])
def test_outputs_without_exports_match(T):
    # the timed path runs a separate kernel instantiation without the
    # optional exports: same Y bit for bit
    prob = make_problem("noexp", d=1024, d_out=272, T=T, bits=4, group=128,
                        rank=32, x_kind="logu10_100", n_outliers=10, seed=61)
    a = run_gpu(prob, exports=True)
    b = run_gpu(prob, exports=False)
    np.testing.assert_array_equal(a["Y"], b["Y"])


def test_deterministic_and_stateless():
    prob = make_problem("det", d=1024, d_out=528, T=16, bits=4, group=128,
                        rank=32, x_kind="logu10_100", n_outliers=10, seed=51)
    for flags in (FUSED, TWO):
        a = run_gpu(prob, flags)
        b = run_gpu(prob, flags)
        for k in ("Y", "q", "s", "m", "dh"):
            np.testing.assert_array_equal(a[k], b[k])
    # a new X (new outlier set) must give new statistics and new codes:
    # nothing is cached between calls
    p2 = make_problem("det", d=1024, d_out=528, T=16, bits=4, group=128,
                      rank=32, x_kind="logu10_100", n_outliers=10, seed=51,
                      call=1)
    c = run_gpu(p2)
    assert not np.array_equal(a["dh"], c["dh"])
    assert not np.array_equal(a["q"], c["q"])
    check_problem(p2, c)


def _with_scaled_channels(prob, big, tiny):
    """The problem with channel sets multiplied by 1e18 and 1e-18 (bf16 has
    float32's exponent range, so such activations are valid inputs)."""
    import dataclasses
    x = oracle.bf16_to_f32(prob.X).astype(np.float64)
    x[..., big] *= 1e18
    x[..., tiny] *= 1e-18
    b = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    return dataclasses.replace(prob, X=b)


@pytest.mark.parametrize("T,alpha", [(1, 0.0), (5, 0.0), (16, 0.5), (3, 1.0)])
def test_fp16_activations_any_magnitude(T, alpha):
    """At T <= 16 the fused kernel takes x' in fp16 scaled by a power of two
    per group and token: activations far beyond fp16's range (and far below)
    must still meet the bars, in groups of their own and mixed with ordinary
    channels of the same group."""
    base = make_problem(f"range_T{T}", d=512, d_out=80, T=T, R=2, bits=4,
                        group=128, alpha=alpha, seed=61 + T)
    big = list(range(0, 8)) + [300]
    tiny = list(range(128, 136)) + [301]
    prob = _with_scaled_channels(base, big, tiny)
    _run_and_check(prob, flags=FUSED, name=f"fp16_range_T{T}_a{alpha}")
