"""Numerical arguments the kernels rely on, checked on the CPU (no GPU).

The one-token kernel evaluates D^{1/2} = (|x| + lambda)^{1/4} (alpha = 1/2)
in [1e-30, 1e30] as a float32 seed (two square roots) refined by one float64
Newton step, z + z e / 4 with e = (base - z^4) / z^4, where the oracle takes
the float64 value and rounds it once to float32.  The claim is that the
rounded float32 results are equal; here it is checked for every finite bf16
input at several lambdas, with the seed and the reciprocal perturbed by a
few float32 ulps (the hardware square root and reciprocal are not correctly
rounded).
"""
import numpy as np
import pytest


def _bf16_values():
    u = np.arange(65536, dtype=np.uint32) << 16
    x = u.view(np.float32)
    return np.abs(x[np.isfinite(x)]).astype(np.float64)


def _seeded_fourth_root(base, rng, seed_ulps, rcp_ulps):
    z32 = np.sqrt(np.sqrt(base.astype(np.float32)))
    if seed_ulps:
        z32 = (z32.view(np.int32) + rng.integers(-seed_ulps, seed_ulps + 1,
                                                 z32.size).astype(np.int32)).view(np.float32)
    z = z32.astype(np.float64)
    z4 = (z * z) * (z * z)
    r = np.float32(1) / z4.astype(np.float32)
    if rcp_ulps:
        r = (r.view(np.int32) + rng.integers(-rcp_ulps, rcp_ulps + 1,
                                             r.size).astype(np.int32)).view(np.float32)
    e = ((base - z4).astype(np.float32) * r).astype(np.float64)
    return z + z * (e * 0.25)


@pytest.mark.parametrize("lam", [0.0, 1e-3, 1e-2, 0.37, 3.0])
@pytest.mark.parametrize("ulps", [0, 3])
def test_seeded_fourth_root_rounds_like_float64(lam, ulps):
    rng = np.random.default_rng(int(lam * 1000) + ulps)
    base = _bf16_values() + lam
    base = base[(base >= 1e-30) & (base <= 1e30)]
    ref = np.sqrt(np.sqrt(base)).astype(np.float32)
    got = _seeded_fourth_root(base, rng, ulps, 1 if ulps else 0).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_seeded_fourth_root_error_bound():
    rng = np.random.default_rng(7)
    base = 10.0 ** rng.uniform(-30, 30, 200_000)
    exact = np.sqrt(np.sqrt(base))
    got = _seeded_fourth_root(base, rng, 3, 1)
    # the neglected terms are about 3 e^2 / 32 with e up to a few 2^-21
    assert np.max(np.abs(got - exact) / exact) < 2.0 ** -40
