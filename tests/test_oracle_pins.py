"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: values the
pages print, hand-worked examples, library routines, closed forms,
invariants and brute force.  Together they are chosen so that a plausible
slip (a dropped lambda, alpha instead of alpha/2, D^{1/2} and D^{-1/2}
swapped, a transposed X, a wrong rounding rule, a missing low-rank term)
fails at least one of them.
"""
import json
import os

import numpy as np
import pytest

import oracle
from workloads import bf16_round_bits, make_c1, make_problem


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _bits(a):
    return bf16_round_bits(np.asarray(a, dtype=np.float32))


def _run(W, X_tok, **kw):
    return oracle.ttq_linear(_bits(W), _bits(X_tok), **kw)


# ---------------------------------------------------------------- statistics
@pytest.mark.parametrize("p", [1.0, 2.0, 3.0, 0.5])
def test_norms_match_numpy_linalg(p):
    rng = np.random.default_rng(7)
    X = rng.standard_normal((13, 37))
    n = oracle.channel_norms(X, p)
    ref = np.array([np.linalg.norm(X[:, j], ord=p) for j in range(X.shape[1])])
    np.testing.assert_allclose(n, ref, rtol=1e-13)


def test_norm_single_token_is_abs():
    x = np.array([[-3.0, 0.0, 2.5, -1e-3]])
    for p in (1.0, 2.0, 3.0):
        np.testing.assert_allclose(oracle.channel_norms(x, p), np.abs(x[0]),
                                   rtol=1e-15)


def test_norm_is_not_mean_normalised():
    # doubling T by repeating tokens scales the L2 norm by sqrt(2), exactly
    rng = np.random.default_rng(1)
    X = rng.standard_normal((5, 8))
    n1 = oracle.channel_norms(X, 2.0)
    n2 = oracle.channel_norms(np.vstack([X, X]), 2.0)
    np.testing.assert_allclose(n2, np.sqrt(2.0) * n1, rtol=1e-14)


def test_diag_hand_values_pin_lambda_and_half_power():
    # (n + lam)^(alpha/2): n=3, lam=1, alpha=1 -> 2; n=7, lam=9, alpha=0.5 -> 2
    dh, dhi = oracle.diag_scales(np.array([3.0, 7.0, 0.0]), 1.0, 1.0)
    assert dh[0] == 2.0 and dhi[0] == 0.5
    dh, dhi = oracle.diag_scales(np.array([7.0]), 9.0, 0.5)
    assert dh[0] == 2.0 and dhi[0] == 0.5
    # zero channel with lam = 0 is the degenerate case: scale 1
    dh, dhi = oracle.diag_scales(np.array([0.0, 4.0]), 0.0, 1.0)
    assert dh[0] == 1.0 and dhi[0] == 1.0 and dh[1] == 2.0


def test_alpha_zero_gives_identity_and_inverse_invariant():
    n = np.abs(np.random.default_rng(3).standard_normal(50)) * 10
    dh, dhi = oracle.diag_scales(n, 1e-3, 0.0)
    assert np.all(dh == 1.0) and np.all(dhi == 1.0)
    dh, dhi = oracle.diag_scales(n, 1e-3, 0.7)
    np.testing.assert_allclose(dh * dhi, 1.0, rtol=1e-15)


def test_autocorrelation_diagonal_closed_form():
    # p = 2, alpha = 2, lambda = 0  =>  D = diag(X X^T)  (X channel-major)
    rng = np.random.default_rng(11)
    Xcm = rng.standard_normal((9, 6))            # d x T
    n = oracle.channel_norms(Xcm.T, 2.0)
    dh, _ = oracle.diag_scales(n, 0.0, 2.0)
    np.testing.assert_allclose(dh ** 2, np.diag(Xcm @ Xcm.T), rtol=1e-12)


# ---------------------------------------------------------------- quantizer
def test_e1_rtn_tie_handworked(golden_dir):
    g = _load(golden_dir, "e1_rtn_tie.json")
    W = np.array([g["w"]], dtype=np.float32)
    q, s, m = oracle.encode_groups_fp32(W, np.ones(4, np.float32), g["bits"],
                                       g["group"])
    assert q[0].tolist() == g["q"]
    assert float(s[0, 0]) == g["scale"] and float(m[0, 0]) == g["min"]
    u_hat = oracle.dequantize(q, s, m, np.ones(4), g["group"])[0]
    np.testing.assert_array_equal(u_hat, g["u_hat"])
    np.testing.assert_array_equal(np.abs(u_hat - W[0]), g["abs_err"])


def test_e2_ttq_handworked(golden_dir):
    g = _load(golden_dir, "e2_ttq_handworked.json")
    Xtok = np.array(g["X_channel_major"]).T
    W = np.array(g["W"])
    r = _run(W, Xtok, bits=g["bits"], group=g["group"], p=g["p"],
             lam=g["lambda"], alpha=g["alpha"])
    np.testing.assert_array_equal(r["n"], g["n"])
    np.testing.assert_array_equal(r["dh"], g["dh"])
    np.testing.assert_array_equal(r["dhi"], g["dhi"])
    np.testing.assert_array_equal(r["q"], g["q"])
    np.testing.assert_array_equal(r["m"][:, 0], g["min"])
    W_hat = oracle.dequantize(r["q"], r["s"], r["m"], r["dhi"], g["group"])
    np.testing.assert_allclose(W_hat, g["W_hat"], rtol=1e-6)
    np.testing.assert_allclose(r["Y"], g["Y_token_major"], rtol=1e-6)
    # alpha = 0 is plain RTN: different codes and outputs, also hand-worked
    r0 = _run(W, Xtok, bits=g["bits"], group=g["group"], p=g["p"],
              lam=g["lambda"], alpha=0.0)
    np.testing.assert_array_equal(r0["q"], g["rtn_q"])
    np.testing.assert_allclose(r0["Y"], g["rtn_Y_token_major"], rtol=1e-6)
    # a swapped D^{+1/2} / D^{-1/2} would give these codes for row 0
    q_sw, _, _ = oracle.encode_groups_fp32(
        np.float32(W[:1]), np.float32(g["dhi"]), g["bits"], g["group"])
    assert q_sw[0].tolist() == g["swapped_direction_q_row0"]
    assert q_sw[0].tolist() != r["q"][0].tolist()
    # TTQ is closer than RTN to the exact output on the outlier token (t = 0)
    exact = np.array(g["exact_Y_token_major"])
    assert np.abs(r["Y"][0] - exact[0]).sum() < np.abs(r0["Y"][0] - exact[0]).sum()


def _plain_rtn_codes(W, bits, group):
    """Textbook min/max round-to-nearest written with scalar float32 loops."""
    N = np.float32(2 ** bits - 1)
    rows, d = W.shape
    q = np.zeros((rows, d), dtype=np.uint8)
    for i in range(rows):
        for k in range(d // group):
            blk = [np.float32(v) for v in W[i, k * group:(k + 1) * group]]
            lo, hi = min(blk), max(blk)
            step = np.float32(np.float32(hi - lo) / N)
            if step == 0:
                continue
            r = np.float32(np.float32(1.0) / step)
            for j, v in enumerate(blk):
                c = float(np.rint(np.float32(np.float32(v - lo) * r)))
                q[i, k * group + j] = int(min(max(c, 0.0), float(N)))
    return q


def test_alpha_zero_reduces_to_plain_rtn():
    p = make_problem("t", d=64, d_out=12, T=5, bits=3, group=32, seed=5,
                     x_kind="x50", n_outliers=2, alpha=0.0)
    r = oracle.ttq_linear(p.W, p.X[0], bits=3, group=32, p=2.0, lam=1e-3,
                          alpha=0.0)
    ref = _plain_rtn_codes(oracle.bf16_to_f32(p.W), 3, 32)
    np.testing.assert_array_equal(r["q"], ref)


def _c1_small(**kw):
    args = dict(d=256, d_out=48, T=16, bits=4, group=128, seed=0,
                x_kind="x50", n_outliers=3)
    args.update(kw)
    return make_problem("c1s", **args)


@pytest.mark.parametrize("bits,group", [(2, 64), (3, 128), (4, 128), (8, 32)])
def test_code_range_endpoints_and_half_step(bits, group):
    p = _c1_small(bits=bits, group=group)
    r = oracle.ttq_linear(p.W, p.X[0], bits=bits, group=group, p=2.0,
                          lam=1e-3, alpha=0.5)
    N = 2 ** bits - 1
    q = r["q"].reshape(p.d_out, -1, group).astype(np.int64)
    assert q.min() >= 0 and q.max() <= N
    u = (oracle.bf16_to_f32(p.W) * r["dh32"][None, :]).reshape(q.shape)
    s = r["s"].astype(np.float64)
    m = r["m"].astype(np.float64)
    live = s > 0
    # the group min encodes to 0 and the max to N exactly
    am = np.argmin(u, axis=2)
    aM = np.argmax(u, axis=2)
    assert np.all(np.take_along_axis(q, am[:, :, None], 2)[live] == 0)
    assert np.all(np.take_along_axis(q, aM[:, :, None], 2)[live] == N)
    # |u_hat - u| <= s/2 in exact arithmetic; the float32 decision value t
    # carries at most three roundings, |t - t_exact| <= 3 N 2^-24, so the
    # bound becomes s (1/2 + 3 N 2^-24)
    u_hat = m[:, :, None] + s[:, :, None] * q
    err = np.abs(u_hat - u.astype(np.float64))
    bound = s[:, :, None] * (0.5 + 3 * N * 2.0 ** -24)
    assert np.all(err <= bound * (1 + 1e-12))
    # and with no slack at all for every element whose t is not near a tie
    t64 = (u.astype(np.float64) - m[:, :, None]) / np.where(live, s, 1)[:, :, None]
    far = np.abs(t64 - np.floor(t64) - 0.5) > 1e-4
    assert np.all((err <= s[:, :, None] / 2 * (1 + 1e-12))[far & live[:, :, None]])


def test_codes_are_nearest_grid_point_bruteforce():
    rng = np.random.default_rng(2)
    for trial in range(30):
        bits = int(rng.integers(1, 4))
        g = int(rng.choice([2, 4, 8]))
        W = rng.standard_normal((3, 2 * g)).astype(np.float32)
        dh = (np.abs(rng.standard_normal(2 * g)) + 0.1).astype(np.float32)
        q, s, m = oracle.encode_groups_fp32(W, dh, bits, g)
        u = (W * dh).astype(np.float64)
        N = 2 ** bits - 1
        for i in range(3):
            for j in range(2 * g):
                k = j // g
                grid = float(m[i, k]) + float(s[i, k]) * np.arange(N + 1)
                dist = np.abs(grid - u[i, j])
                best = np.flatnonzero(dist <= dist.min() * (1 + 1e-6) + 1e-12)
                assert q[i, j] in best, (trial, i, j)


def test_degenerate_group_has_zero_scale_and_code():
    W = np.full((2, 8), 0.25, dtype=np.float32)
    q, s, m = oracle.encode_groups_fp32(W, np.ones(8, np.float32), 4, 8)
    assert np.all(s == 0) and np.all(q == 0) and np.all(m == 0.25)
    W_hat = oracle.dequantize(q, s, m, np.ones(8), 8)
    assert np.all(W_hat == 0.25)


def test_power_of_two_activation_scaling_is_exact_invariant():
    # lambda = 0, X -> 16 X with alpha = 0.5: D^{1/2} doubles exactly,
    # so the codes and W_hat are unchanged
    p = _c1_small()
    X = oracle.bf16_to_f32(p.X[0])
    kw = dict(bits=4, group=128, p=2.0, lam=0.0, alpha=0.5)
    r1 = oracle.ttq_linear(p.W, _bits(X), **kw)
    r2 = oracle.ttq_linear(p.W, _bits(16.0 * X), **kw)
    np.testing.assert_array_equal(r2["dh"], 2.0 * r1["dh"])
    np.testing.assert_array_equal(r1["q"], r2["q"])
    W1 = oracle.dequantize(r1["q"], r1["s"], r1["m"], r1["dhi"], 128)
    W2 = oracle.dequantize(r2["q"], r2["s"], r2["m"], r2["dhi"], 128)
    np.testing.assert_allclose(W1, W2, rtol=1e-15, atol=0)


def test_token_permutation_invariance():
    p = _c1_small()
    perm = np.random.default_rng(4).permutation(p.T)
    kw = dict(bits=4, group=128, p=2.0, lam=1e-3, alpha=0.5)
    r1 = oracle.ttq_linear(p.W, p.X[0], **kw)
    r2 = oracle.ttq_linear(p.W, p.X[0][perm], **kw)
    np.testing.assert_array_equal(r1["dh32"], r2["dh32"])
    np.testing.assert_array_equal(r1["q"], r2["q"])
    np.testing.assert_allclose(r2["Y"], r1["Y"][perm], rtol=1e-12, atol=1e-12)


def test_uniform_power_of_two_norms_give_rtn_codes():
    # every channel has norm 16 and alpha = 0.5, lambda = 0: D^{1/2} = 2
    d, d_out = 128, 10
    X = np.full((1, d), 16.0)
    W = np.random.default_rng(8).standard_normal((d_out, d)) * 0.02
    kw = dict(bits=3, group=64, p=2.0, lam=0.0)
    r = _run(W, X, alpha=0.5, **kw)
    assert np.all(r["dh"] == 2.0)
    ref = _plain_rtn_codes(oracle.bf16_to_f32(_bits(W)), 3, 64)
    np.testing.assert_array_equal(r["q"], ref)


# ---------------------------------------------------------------- contraction
def test_output_matches_explicit_loops_tiny():
    p = make_problem("tiny", d=64, d_out=5, T=3, bits=2, group=32, rank=2,
                     seed=9, n_outliers=1)
    kw = dict(bits=2, group=32, p=2.0, lam=1e-3, alpha=0.5)
    r = oracle.ttq_linear(p.W, p.X[0], B_bits=p.B, A_bits=p.A, **kw)
    X = oracle.bf16_to_f64(p.X[0])
    A = oracle.bf16_to_f64(p.A)
    B = oracle.bf16_to_f64(p.B)
    W_hat = oracle.dequantize(r["q"], r["s"], r["m"], r["dhi"], 32)
    for t in range(p.T):
        for i in range(p.d_out):
            acc = 0.0
            for j in range(p.d):
                acc += W_hat[i, j] * X[t, j]
            for k in range(p.rank):
                z = 0.0
                for j in range(p.d):
                    z += A[k, j] * X[t, j]
                acc += B[i, k] * z
            assert abs(acc - r["Y"][t, i]) <= 1e-12 * max(1.0, abs(acc))


def test_low_rank_term_equals_dense_product():
    p = make_problem("lr", d=128, d_out=16, T=4, bits=3, group=64, rank=8,
                     seed=10, n_outliers=2)
    kw = dict(bits=3, group=64, p=2.0, lam=1e-3, alpha=0.5)
    r_lr = oracle.ttq_linear(p.W, p.X[0], B_bits=p.B, A_bits=p.A, **kw)
    r_no = oracle.ttq_linear(p.W, p.X[0], **kw)
    X = oracle.bf16_to_f64(p.X[0])
    BA = oracle.bf16_to_f64(p.B) @ oracle.bf16_to_f64(p.A)
    np.testing.assert_allclose(r_lr["Y"] - r_no["Y"], X @ BA.T, rtol=1e-10,
                               atol=1e-13)


def test_row_subset_equals_full():
    p = _c1_small(rank=4)
    kw = dict(bits=4, group=128, p=2.0, lam=1e-3, alpha=0.5, B_bits=p.B,
              A_bits=p.A)
    full = oracle.ttq_linear(p.W, p.X[0], **kw)
    rows = np.array([0, 7, 31, 47])
    sub = oracle.ttq_linear(p.W, p.X[0], rows=rows, **kw)
    np.testing.assert_array_equal(sub["q"], full["q"][rows])
    np.testing.assert_allclose(sub["Y"], full["Y"][:, rows], rtol=1e-13)


# ---------------------------------------------------------------- quality
def _rel_err(p, bits, alpha):
    g = 128 if p.d % 128 == 0 else 32
    r = oracle.ttq_linear(p.W, p.X[0], bits=bits, group=g, p=2.0, lam=1e-3,
                          alpha=alpha)
    X = oracle.bf16_to_f64(p.X[0])
    Y0 = X @ oracle.bf16_to_f64(p.W).T
    return np.linalg.norm(r["Y"] - Y0) / np.linalg.norm(Y0)


def test_error_falls_as_bits_rise():
    p = make_c1()
    errs = [_rel_err(p, b, 0.5) for b in (2, 3, 4, 5, 8)]
    assert all(a > b for a, b in zip(errs, errs[1:])), errs
    assert errs[-1] < 0.01


def test_ttq_beats_rtn_on_outlier_activations():
    p = make_c1()
    for b in (2, 3, 4):
        assert _rel_err(p, b, 0.5) < _rel_err(p, b, 0.0), b


# ---------------------------------------------------------------- pages' example
def test_blog_int4_outlier_example(golden_dir):
    g = _load(golden_dir, "blog_int4_outlier_example.json")
    tol = g["printed_precision"]
    rng = np.random.default_rng(0)
    typical = rng.uniform(-1.0, 1.0, 127)
    typical[0] = 1.0
    grp = np.concatenate([typical, [g["outlier"]]])
    _, s, xh = oracle.symmetric_quantize(grp, g["bits"])
    assert abs(s - g["shared_scale"]) <= tol
    assert abs(s / 2 - g["shared_half_step"]) <= tol
    err = np.abs(xh - grp)
    assert err.max() <= s / 2 + 1e-12
    assert abs(100 * (s / 2) / g["typical"] - g["shared_relative_error_pct"]) <= 1
    _, s2, xh2 = oracle.symmetric_quantize(typical, g["bits"])
    assert abs(s2 - g["segregated_scale"]) <= tol
    assert abs(s2 / 2 - g["segregated_half_step"]) <= tol
    assert np.abs(xh2 - typical).max() <= s2 / 2 + 1e-12
    assert round(100 * (s2 / 2) / g["typical"]) == g["segregated_relative_error_pct"]
    assert round(s / s2) == round(g["outlier"] / g["typical"])


# ---------------------------------------------------------------- band rule
def test_band_rule_classification():
    t = np.array([[2.5 + 1e-9, 2.3, 0.5]])
    u = np.array([[0.1, 0.2, 0.3]])
    m = np.array([[0.0]])
    s = np.array([[0.04]])
    q_ref = np.array([[3, 2, 1]])
    q_gpu = np.array([[2, 3, 1]])
    nb, ne, nl = oracle.band_excused(q_gpu, q_ref, t, u, m, s, 3)
    assert (nb, ne, nl) == (2, 1, 1)


# ------------------------------------------------ float64 pre-rounding value
def test_pre_rounding_fp64_matches_e1_golden_t(golden_dir):
    g = _load(golden_dir, "e1_rtn_tie.json")
    t, u, m, s = oracle.pre_rounding_fp64(np.array([g["w"]]), np.ones(4),
                                          g["bits"], g["group"])
    np.testing.assert_array_equal(t[0], g["t"])
    np.testing.assert_array_equal(u[0], g["w"])
    assert m[0, 0] == g["min"] and s[0, 0] == g["scale"]


def test_pre_rounding_fp64_matches_e2_handworked_t(golden_dir):
    g = _load(golden_dir, "e2_ttq_handworked.json")
    Xtok = np.array(g["X_channel_major"]).T
    r = _run(np.array(g["W"]), Xtok, bits=g["bits"], group=g["group"],
             p=g["p"], lam=g["lambda"], alpha=g["alpha"], want_t=True)
    np.testing.assert_allclose(r["t64"], g["t"], rtol=1e-15, atol=1e-15)
    np.testing.assert_array_equal(r["u64"], g["u"])
    np.testing.assert_array_equal(r["m64"][:, 0], g["min"])
    np.testing.assert_array_equal(r["m64"][:, 0] + r["s64"][:, 0] * 3, g["max"])


def test_pre_rounding_fp64_uses_float64_statistics_closed_form():
    # p = 1, lambda = 0, alpha = 1: channel norms [1, 2, 1, 1] give
    # D^{1/2} = [1, sqrt 2, 1, 1], which float32 cannot hold.  Row [1, 1, 0, 0]
    # has u = [1, sqrt 2, 0, 0], s = sqrt(2)/3, t = [3/sqrt 2, 3, 0, 0]; row
    # [0.5, -1, 1, 0] has u = [0.5, -sqrt 2, 1, 0], s = (1 + sqrt 2)/3,
    # t = [4.5 - 1.5 sqrt 2, 0, 3, 6 - 3 sqrt 2].  A t taken from the float32
    # D^{1/2} or a float32 scale is off by about 1e-8 relative.
    Xtok = np.array([[1.0, 1.0, 0.0, 1.0], [0.0, 1.0, 1.0, 0.0]])
    W = np.array([[1.0, 1.0, 0.0, 0.0], [0.5, -1.0, 1.0, 0.0]])
    r = _run(W, Xtok, bits=2, group=4, p=1.0, lam=0.0, alpha=1.0, want_t=True)
    r2 = np.sqrt(2.0)
    exact = np.array([[3 / r2, 3.0, 0.0, 0.0],
                      [4.5 - 1.5 * r2, 0.0, 3.0, 6 - 3 * r2]])
    np.testing.assert_allclose(r["t64"], exact, rtol=4e-16, atol=1e-15)
    assert np.abs(np.float32(r2) - r2) / r2 > 1e-8   # the slip would show
    np.testing.assert_allclose(r["s64"][:, 0], [r2 / 3, (1 + r2) / 3], rtol=4e-16)
    # the float32 code decision agrees with rint(t) here (no value near a tie)
    assert r["q"].tolist() == [[2, 3, 0, 0], [2, 0, 3, 2]]


def test_pre_rounding_fp64_agrees_with_fp32_codes_outside_the_band():
    rng = np.random.default_rng(7)
    W = _bits(rng.standard_normal((32, 512)) * 0.02)
    X = _bits(rng.standard_normal((8, 512)))
    r = oracle.ttq_linear(W, X, bits=4, group=128, p=2.0, lam=1e-3, alpha=0.5,
                          want_t=True)
    q_ref = np.clip(np.rint(r["t64"]), 0, 15)
    nb, ne, _ = oracle.band_excused(r["q"], q_ref, r["t64"], r["u64"],
                                    r["m64"], r["s64"], 128)
    assert nb == ne   # every disagreement sits on a rounding boundary
