"""GPU parity of the PCA low-rank factors (ttq_lowrank_pca) against the CPU
oracle, through the C ABI.

Bars (float32 panels on the GPU, float64 in the oracle, bf16 outputs):
  * with a spectral gap at r the subspace is well defined: B and A equal the
    oracle's (same Omega, same iterations) to the bf16 rounding of each
    element plus 1e-4 of the largest entry;
  * W_res equals W - B A evaluated in float64 from the GPU's own bf16
    factors to one bf16 ulp plus the float32 summation bound of the r
    products (the residual cancels most of W, so near-zero entries see the
    float32 sum's own rounding);
  * without a gap (Gaussian W), the residual norm is at least the
    Eckart-Young optimum and within 1 % of the oracle's for the same Omega;
  * the factors feed ttq_linear: (W_res, B, A) meet the projection's bars.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from parity_util import check_problem, run_gpu, to_dev
from workloads import make_problem
from workloads.configs import draw_lowrank_w, draw_omega, draw_x

pytestmark = pytest.mark.gpu


def _gpu_pca(Wb, Om, iters, Xb=None, **kw):
    import torch
    import online_activation_aware_ttq_amd as ttq
    X = to_dev(Xb) if Xb is not None else None
    B, A, R = ttq.ttq_lowrank_pca(to_dev(Wb), torch.from_numpy(Om).cuda(),
                                  iters=iters, X=X, **kw)
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    return bits(B), bits(A), bits(R)


def _bf16_ulp(x):
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1e-300)))
    return np.where(a > 0, 2.0 ** (e - 7), 2.0 ** -133)


def _check_factors(Wb, Bg, Ag, Rg, ref, rep):
    B = oracle.bf16_to_f64(Bg)
    A = oracle.bf16_to_f64(Ag)
    tolB = 2.0 ** -8 * np.abs(ref["B"]) + 1e-4 * np.abs(ref["B"]).max()
    tolA = 2.0 ** -8 * np.abs(ref["A"]) + 1e-4 * np.abs(ref["A"]).max()
    rep["B_err"] = float(np.abs(B - ref["B"]).max())
    rep["A_err"] = float(np.abs(A - ref["A"]).max())
    assert np.all(np.abs(B - ref["B"]) <= tolB), rep
    assert np.all(np.abs(A - ref["A"]) <= tolA), rep
    assert np.abs(B.T @ B - np.eye(B.shape[1])).max() < 1e-2
    W = oracle.bf16_to_f64(Wb)
    exact = W - B @ A
    R = oracle.bf16_to_f64(Rg)
    diff = np.abs(R - exact)
    # one bf16 ulp plus the float32 summation bound of the r products
    r = B.shape[1]
    f32 = (r + 2) * 2.0 ** -24 * (np.abs(B) @ np.abs(A) + np.abs(W))
    rep["res_off_half_ulp"] = int((diff > 0.5 * _bf16_ulp(exact) + f32).sum())
    assert np.all(diff <= _bf16_ulp(exact) + f32), rep


@pytest.mark.parametrize("d_out,d,r,iters", [
    (300, 512, 16, 2),
    (520, 1024, 64, 1),
    (72, 200, 8, 3),      # ragged tiles, d not a multiple of 64
    (200, 384, 128, 2),   # the largest rank
    (600, 256, 32, 2),    # more output rows than input channels
])
def test_static_pca_matches_oracle(d_out, d, r, iters):
    Wb = draw_lowrank_w(d_out + d, d_out, d, r)
    Om = draw_omega(r + d, d, r)
    print(f"[case] pca static d_out={d_out} d={d} r={r} iters={iters}", flush=True)
    Bg, Ag, Rg = _gpu_pca(Wb, Om, iters)
    ref = oracle.lowrank_pca(Wb, Om, iters)
    rep = {}
    _check_factors(Wb, Bg, Ag, Rg, ref, rep)
    print(f"[parity] pca {d_out}x{d} r={r}: {rep}", flush=True)


@pytest.mark.parametrize("T", [40, 200])
def test_online_pca_matches_oracle(T):
    d_out, d, r = 256, 512, 16
    Wb = draw_lowrank_w(7, d_out, d, r)
    Xb = draw_x(8, 0, 1, T, d, "logu10_100", 5)[0]
    Om = draw_omega(9, d, r)
    kw = dict(p=2.0, lam=1e-3, alpha=0.5)
    print(f"[case] pca online T={T}", flush=True)
    Bg, Ag, Rg = _gpu_pca(Wb, Om, 2, Xb, **kw)
    ref = oracle.lowrank_pca(Wb, Om, 2, X_bits=Xb, **kw)
    # the activation-aware subspace must have a gap too for the comparison
    s = np.linalg.svd(ref["M"], compute_uv=False)
    assert s[r - 1] / s[r] > 5
    rep = {}
    _check_factors(Wb, Bg, Ag, Rg, ref, rep)
    print(f"[parity] pca online T={T}: {rep}", flush=True)


def test_no_gap_residual_bounds():
    d_out, d, r = 256, 320, 32
    rng = np.random.default_rng(11)
    from workloads.configs import bf16_round_bits
    Wb = bf16_round_bits((rng.standard_normal((d_out, d)) * 0.02).astype(np.float32))
    Om = draw_omega(12, d, r)
    Bg, Ag, Rg = _gpu_pca(Wb, Om, 2)
    W = oracle.bf16_to_f64(Wb)
    res = np.linalg.norm(W - oracle.bf16_to_f64(Bg) @ oracle.bf16_to_f64(Ag))
    s = np.linalg.svd(W, compute_uv=False)
    ref = np.linalg.norm(oracle.lowrank_pca(Wb, Om, 2)["R"])
    print(f"[parity] pca no gap: res={res:.6g} oracle={ref:.6g} "
          f"optimum={np.sqrt(np.sum(s[r:] ** 2)):.6g}", flush=True)
    assert res ** 2 >= np.sum(s[r:] ** 2) * (1 - 1e-6)
    assert abs(res - ref) <= 1e-2 * ref


def test_factors_feed_the_projection():
    d_out, d, r = 300, 512, 32
    Wb = draw_lowrank_w(21, d_out, d, r)
    Om = draw_omega(22, d, r)
    Bg, Ag, Rg = _gpu_pca(Wb, Om, 2)
    base = make_problem("pca_lin", d=d, d_out=d_out, T=24, bits=3, group=64,
                        rank=r, seed=23, x_kind="logu10_100", n_outliers=5)
    prob = dataclasses.replace(base, W=Rg, B=Bg, A=Ag)
    for flags in (0, 2):
        rep = check_problem(prob, run_gpu(prob, flags=flags))
        print(f"[parity] pca -> ttq_linear flags={flags}: y_max={rep['y_max']:.3g}",
              flush=True)
    # and W ~ Q[W_res] + B A approximates W X better than quantizing W alone
    # (the planted part is carried exactly by the factors)
    X = oracle.bf16_to_f64(base.X[0])
    W = oracle.bf16_to_f64(Wb)
    exact = X @ W.T
    kw = dict(bits=3, group=64, p=2.0, lam=1e-3, alpha=0.5)
    with_lr = oracle.ttq_linear(Rg, base.X[0], B_bits=Bg, A_bits=Ag, **kw)["Y"]
    plain = oracle.ttq_linear(Wb, base.X[0], **kw)["Y"]
    assert np.linalg.norm(with_lr - exact) < 0.5 * np.linalg.norm(plain - exact)


def test_pca_is_deterministic():
    Wb = draw_lowrank_w(31, 128, 256, 16)
    Om = draw_omega(32, 256, 16)
    a = _gpu_pca(Wb, Om, 2)
    b = _gpu_pca(Wb, Om, 2)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_degenerate_inputs():
    """Rank-deficient inputs.  With an all-zero W every Gram pivot hits the
    floor; B is then completed to an orthonormal basis (any orthonormal B is
    a valid principal basis of a zero matrix, so B itself is checked for
    orthonormality only), and A = B^T W and the residual are compared with
    the oracle's (both exactly zero).  A W of exact rank 4 with r = 16: the
    rank-4 principal subspace is unique and both B's must contain it; the
    other 12 columns are arbitrary but must stay orthonormal; A and the
    residual (zero up to the bf16 rounding of the factors) match the
    oracle's.  A square W of full rank r = d_out is reproduced by its
    factors."""
    Z = np.zeros((64, 128), dtype=np.uint16)
    Om = draw_omega(41, 128, 16)
    Bg, Ag, Rg = _gpu_pca(Z, Om, 2)
    ref = oracle.lowrank_pca(Z, Om, 2)
    B = oracle.bf16_to_f64(Bg)
    assert np.all(np.isfinite(B))
    np.testing.assert_allclose(B.T @ B, np.eye(16), atol=2e-2)
    np.testing.assert_allclose(ref["B"].T @ ref["B"], np.eye(16), atol=1e-12)
    np.testing.assert_array_equal(oracle.bf16_to_f64(Ag), ref["A"])
    np.testing.assert_array_equal(oracle.bf16_to_f64(Rg), ref["R"])
    # exact rank 4 (small integers: W is exact in bf16)
    rng = np.random.default_rng(7)
    U = rng.integers(-3, 4, (96, 4)).astype(np.float32)
    V = rng.integers(-3, 4, (4, 128)).astype(np.float32)
    from workloads.configs import bf16_round_bits
    W4b = bf16_round_bits(U @ V)
    assert np.array_equal(oracle.bf16_to_f64(W4b), U @ V)
    Om4 = draw_omega(44, 128, 16)
    Bg, Ag, Rg = _gpu_pca(W4b, Om4, 1)
    ref = oracle.lowrank_pca(W4b, Om4, 1)
    W4 = U.astype(np.float64) @ V
    B = oracle.bf16_to_f64(Bg)
    np.testing.assert_allclose(B.T @ B, np.eye(16), atol=2e-2)
    scale = np.linalg.norm(W4)
    for Bx in (B, ref["B"]):   # both contain the unique rank-4 subspace
        assert np.linalg.norm(W4 - Bx @ (Bx.T @ W4)) <= 1e-2 * scale
    # the first 4 columns orthonormalise the same 4 independent columns of
    # M Z (positive R diagonal): unique, equal up to rounding
    np.testing.assert_allclose(B[:, :4], ref["B"][:, :4], atol=2e-2)
    np.testing.assert_allclose(oracle.bf16_to_f64(Ag)[:4], ref["A"][:4],
                               atol=2e-2 * np.abs(ref["A"][:4]).max())
    # residual: zero up to the bf16 rounding of the factors (oracle: exact)
    assert np.linalg.norm(ref["R"]) <= 1e-9 * scale
    assert np.linalg.norm(oracle.bf16_to_f64(Rg) - ref["R"]) <= 1e-2 * scale
    from workloads.configs import bf16_round_bits
    rng = np.random.default_rng(42)
    Wb = bf16_round_bits((rng.standard_normal((32, 96)) * 0.05).astype(np.float32))
    Bg, Ag, Rg = _gpu_pca(Wb, draw_omega(43, 96, 32), 1)
    W = oracle.bf16_to_f64(Wb)
    R = oracle.bf16_to_f64(Rg)
    assert np.linalg.norm(R) <= 1e-2 * np.linalg.norm(W)
