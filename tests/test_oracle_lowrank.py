"""Pins of the oracle's PCA low-rank factors (B orthonormal basis of the
top-r principal subspace of W, or of W D^{1/2} online; A = B^T W) against
things other than the oracle: an independently written Gram-Schmidt, numpy's
SVD (the exact principal subspace, which the iteration must approach at the
rate the spectral gap sets), the Eckart-Young bound, exact identities of an
orthogonal projection, and a hand-built case where the activations decide
which direction is principal.
"""
import numpy as np
import pytest

import oracle
from workloads.configs import bf16_round_bits


def _gs(Y):
    """Classical Gram-Schmidt (twice), written out by loops."""
    Y = np.array(Y, dtype=np.float64)
    Q = np.zeros_like(Y)
    for j in range(Y.shape[1]):
        v = Y[:, j].copy()
        for _ in range(2):
            for i in range(j):
                v -= (Q[:, i] @ v) * Q[:, i]
        Q[:, j] = v / np.linalg.norm(v)
    return Q


def _bits(x):
    return bf16_round_bits(np.asarray(x, dtype=np.float32))


def _planted(dout, d, r, gap, seed, noise=1e-3):
    """W = U S V^T + noise, top r singular values >= gap times the rest."""
    rng = np.random.default_rng(seed)
    U, _ = np.linalg.qr(rng.standard_normal((dout, r)))
    V, _ = np.linalg.qr(rng.standard_normal((d, r)))
    S = np.linspace(2.0, 1.0, r)
    W = (U * S) @ V.T + noise * rng.standard_normal((dout, d)) / np.sqrt(d) * 1.0 / gap
    return _bits(W)


def test_orthonormalize_matches_gram_schmidt():
    rng = np.random.default_rng(0)
    Y = rng.standard_normal((40, 7))
    Q = oracle.orthonormalize(Y)
    np.testing.assert_allclose(Q, _gs(Y), atol=1e-12)
    np.testing.assert_allclose(Q.T @ Q, np.eye(7), atol=1e-13)


def test_iteration_reaches_the_exact_principal_subspace():
    Wb = _planted(96, 80, 6, gap=30.0, seed=1)
    W = oracle.bf16_to_f64(Wb)
    Om = np.random.default_rng(2).standard_normal((80, 6))
    P_exact = (lambda U: U @ U.T)(oracle.pca_exact(W, 6))
    errs = []
    for q in (0, 1, 2):
        B = oracle.lowrank_pca(Wb, Om, q)["B"]
        errs.append(np.linalg.norm(B @ B.T - P_exact, 2))
    assert errs[2] < 1e-9 and errs[1] < 1e-6
    assert errs[0] > errs[1] > errs[2]


def test_eckart_young_bound_and_equality_when_converged():
    rng = np.random.default_rng(3)
    Wb = _bits(rng.standard_normal((60, 50)) * 0.02)
    W = oracle.bf16_to_f64(Wb)
    s = np.linalg.svd(W, compute_uv=False)
    Om = rng.standard_normal((50, 5))
    for q in (0, 2, 30):
        R = oracle.lowrank_pca(Wb, Om, q)["R"]
        assert np.linalg.norm(R) ** 2 >= np.sum(s[5:] ** 2) * (1 - 1e-12)
    # with a spectral gap a few iterations reach the optimum
    Wp = _planted(60, 50, 5, gap=30.0, seed=9)
    sp = np.linalg.svd(oracle.bf16_to_f64(Wp), compute_uv=False)
    R = oracle.lowrank_pca(Wp, Om, 3)["R"]
    assert np.isclose(np.linalg.norm(R) ** 2, np.sum(sp[5:] ** 2), rtol=1e-9)


def test_projection_identities():
    rng = np.random.default_rng(4)
    Wb = _bits(rng.standard_normal((50, 64)))
    out = oracle.lowrank_pca(Wb, rng.standard_normal((64, 8)), 1)
    B, A, R = out["B"], out["A"], out["R"]
    np.testing.assert_allclose(B.T @ B, np.eye(8), atol=1e-12)
    np.testing.assert_allclose(B.T @ R, 0.0, atol=1e-11)     # residual _|_ span B
    np.testing.assert_allclose(B @ A + R, oracle.bf16_to_f64(Wb), atol=1e-12)


def test_exact_for_a_rank_r_matrix():
    rng = np.random.default_rng(5)
    W = _bits(rng.standard_normal((40, 4)) @ rng.standard_normal((4, 32)))
    # bf16 rounding breaks exact rank 4: the residual is at the rounding level
    out = oracle.lowrank_pca(W, rng.standard_normal((32, 4)), 2)
    Wf = oracle.bf16_to_f64(W)
    assert np.linalg.norm(out["R"]) <= 1e-2 * np.linalg.norm(Wf)
    s = np.linalg.svd(Wf, compute_uv=False)
    assert np.isclose(np.linalg.norm(out["R"]) ** 2, np.sum(s[4:] ** 2), rtol=1e-6)


def test_column_operations_on_omega_leave_q_unchanged():
    rng = np.random.default_rng(6)
    Wb = _bits(rng.standard_normal((30, 24)))
    Om = rng.standard_normal((24, 5))
    G = np.triu(rng.uniform(0.5, 2.0, (5, 5)))                 # positive diagonal
    B1 = oracle.lowrank_pca(Wb, Om, 0)["B"]
    B2 = oracle.lowrank_pca(Wb, Om @ G, 0)["B"]
    np.testing.assert_allclose(B1, B2, atol=1e-10)


def test_online_alpha_zero_is_static():
    rng = np.random.default_rng(7)
    Wb = _bits(rng.standard_normal((32, 64)))
    Xb = _bits(rng.standard_normal((5, 64)))
    Om = rng.standard_normal((64, 4))
    st = oracle.lowrank_pca(Wb, Om, 2)
    on = oracle.lowrank_pca(Wb, Om, 2, X_bits=Xb, p=2.0, lam=1e-3, alpha=0.0)
    np.testing.assert_allclose(on["B"], st["B"], atol=1e-12)


def test_online_follows_the_activations():
    # two rank-one parts on disjoint channel sets: statically the first is
    # principal (1.5 > 1); activations 100x larger on the second part's
    # channels make it principal in W D^{1/2} (alpha = 1: D^{1/2} = n^{1/2})
    d, dout = 64, 16
    u1 = np.zeros(dout); u1[:8] = 1 / np.sqrt(8)
    u2 = np.zeros(dout); u2[8:] = 1 / np.sqrt(8)
    v1 = np.zeros(d); v1[:32] = 1 / np.sqrt(32)
    v2 = np.zeros(d); v2[32:] = 1 / np.sqrt(32)
    W = 1.5 * np.outer(u1, v1) + 1.0 * np.outer(u2, v2)
    Wb = _bits(W)
    X = np.ones((4, d)); X[:, 32:] *= 100.0
    Om = np.random.default_rng(8).standard_normal((d, 1))
    st = oracle.lowrank_pca(Wb, Om, 3)["B"][:, 0]
    on = oracle.lowrank_pca(Wb, Om, 3, X_bits=_bits(X), p=2.0, lam=0.0,
                            alpha=1.0)["B"][:, 0]
    assert abs(st @ u1) > 0.999 and abs(on @ u2) > 0.999
