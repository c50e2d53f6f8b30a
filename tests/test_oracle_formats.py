"""Pins of the oracle's format variants of Q (symmetric, integer zero point,
FP8 E4M3) against things other than the oracle itself: the blog's worked
INT4 example, hand-worked groups, library quantizers that implement the
same definitions (torch's float8_e4m3fn cast and its per-tensor affine fake
quantizer), brute-force nearest-level searches and invariants.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import ttq_oracle as O

torch = pytest.importorskip("torch")


def _ones(d):
    return np.ones(d, dtype=np.float32)


# ---------------------------------------------------------------- E4M3 codec
def test_e4m3_decode_matches_torch_float8_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok].astype(np.float64))


def test_e4m3_hand_values():
    # largest finite, smallest subnormal, smallest normal, one
    assert oracle.e4m3_decode(np.array([0x7e]))[0] == 448.0
    assert oracle.e4m3_decode(np.array([0x01]))[0] == 2.0 ** -9
    assert oracle.e4m3_decode(np.array([0x08]))[0] == 2.0 ** -6
    assert oracle.e4m3_decode(np.array([0x38]))[0] == 1.0
    assert oracle.e4m3_decode(np.array([0xb8]))[0] == -1.0
    # ties go to the even mantissa
    r = oracle.e4m3_round(np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10,
                                    432.0, 440.0, -1.0625, 0.0]))
    np.testing.assert_array_equal(r, [1.0, 1.25, 0.0, 2.0 ** -8, 448.0, 448.0,
                                      -1.0, 0.0])
    with pytest.raises(ValueError):
        oracle.e4m3_round(np.array([449.0]))


def test_e4m3_round_matches_torch_cast_including_every_tie():
    rng = np.random.default_rng(3)
    vals = oracle.e4m3_decode(np.arange(0x7f))
    mids = (vals[1:] + vals[:-1]) / 2           # exact in float32
    t = np.concatenate([rng.uniform(-448, 448, 50000),
                        rng.standard_normal(50000) * 0.01,
                        mids, -mids, vals, -vals]).astype(np.float32)
    ours = oracle.e4m3_round(t.astype(np.float64))
    ref = torch.from_numpy(t).to(torch.float8_e4m3fn).float().numpy()
    np.testing.assert_array_equal(ours, ref.astype(np.float64))


def test_e4m3_encode_round_trip():
    codes = np.array([c for c in range(256) if (c & 0x7f) != 0x7f and c != 0x80],
                     dtype=np.uint8)
    np.testing.assert_array_equal(oracle.e4m3_encode(oracle.e4m3_decode(codes)),
                                  codes)
    # the sign is kept, also for a zero: as torch's float8_e4m3fn cast does
    t = np.array([-0.0, 0.0, -1e-5, 1e-5, -2.0 ** -11], dtype=np.float32)
    ours = oracle.e4m3_encode(oracle.e4m3_round(t.astype(np.float64)))
    ref = torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(ours, [0x80, 0x00, 0x80, 0x00, 0x80])


# ---------------------------------------------------------------- symmetric
def test_sym_reproduces_the_blog_int4_example(golden_dir):
    with open(os.path.join(golden_dir, "blog_int4_outlier_example.json")) as f:
        g = json.load(f)
    tol = g["printed_precision"]
    rng = np.random.default_rng(0)
    typical = rng.uniform(-1.0, 1.0, 127).astype(np.float32)
    typical[0] = 1.0
    grp = np.concatenate([typical, [np.float32(g["outlier"])]])[None, :]
    k, s = oracle.encode_sym_fp32(grp, _ones(128), g["bits"], 128)
    assert abs(float(s[0, 0]) - g["shared_scale"]) <= tol
    assert int(np.abs(k).max()) == g["levels"]
    err = np.abs(float(s[0, 0]) * k[0] - grp[0].astype(np.float64))
    assert err.max() <= float(s[0, 0]) / 2 * (1 + 1e-6)
    # every value of magnitude <= 1 is below half a step: all collapse to 0
    assert float(s[0, 0]) / 2 > g["typical"] and not k[0, :127].any()
    k2, s2 = oracle.encode_sym_fp32(np.concatenate([typical, typical[:1]])[None, :],
                                    _ones(128), g["bits"], 128)
    assert abs(float(s2[0, 0]) - g["segregated_scale"]) <= tol
    err2 = np.abs(float(s2[0, 0]) * k2[0, :127] - typical.astype(np.float64))
    assert err2.max() <= g["segregated_half_step"] + tol


def test_sym_hand_worked_group():
    # u = [0.25, 1.0, -0.25, 2.0]: b = 3 (Z = 3): s = fl(2/3), inv = 1.5,
    # t = [0.375, 1.5, -0.375, 3] -> levels [0, 2, 0, 3] (1.5 ties to 2);
    # b = 2 (Z = 1): s = 2, inv = 0.5, t = [0.125, 0.5, -0.125, 1] -> [0, 0, 0, 1]
    u = np.array([[0.25, 1.0, -0.25, 2.0]], dtype=np.float32)
    k, s = oracle.encode_sym_fp32(u, _ones(4), 3, 4)
    assert s[0, 0] == np.float32(2.0) / np.float32(3.0)
    np.testing.assert_array_equal(k[0], [0, 2, 0, 3])
    f = oracle.quantize_format(u, _ones(4), 3, 4, "sym")
    np.testing.assert_array_equal(f["codes"][0], [3, 5, 3, 6])
    k, s = oracle.encode_sym_fp32(u, _ones(4), 2, 4)
    assert s[0, 0] == 2.0
    np.testing.assert_array_equal(k[0], [0, 0, 0, 1])


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_sym_matches_torch_fake_quantize(bits):
    rng = np.random.default_rng(bits)
    W = rng.standard_normal((5, 256)).astype(np.float32)
    dh = rng.uniform(0.5, 4.0, 256).astype(np.float32)
    k, s = oracle.encode_sym_fp32(W, dh, bits, 64)
    Z = 2 ** (bits - 1) - 1
    u = W * dh
    for i in range(5):
        for g in range(4):
            x = torch.from_numpy(u[i, g * 64:(g + 1) * 64].copy())
            ref = torch.fake_quantize_per_tensor_affine(x, float(s[i, g]), 0, -Z, Z)
            ours = (np.float64(s[i, g]) * k[i, g * 64:(g + 1) * 64]).astype(np.float32)
            np.testing.assert_array_equal(ours, ref.numpy())


def test_sym_is_odd_and_nearest_level():
    rng = np.random.default_rng(5)
    W = rng.standard_normal((7, 128)).astype(np.float32)
    k, s = oracle.encode_sym_fp32(W, _ones(128), 4, 32)
    kn, sn = oracle.encode_sym_fp32(-W, _ones(128), 4, 32)
    np.testing.assert_array_equal(sn, s)
    np.testing.assert_array_equal(kn, -k)
    # brute force: every value sits at a nearest level of s * {-7..7}
    levels = np.arange(-7, 8, dtype=np.float64)
    for i in range(7):
        for g in range(4):
            x = W[i, g * 32:(g + 1) * 32].astype(np.float64)
            grid = float(s[i, g]) * levels
            d = np.abs(x[:, None] - grid[None, :])
            mine = np.abs(x - float(s[i, g]) * k[i, g * 32:(g + 1) * 32])
            assert np.all(mine <= d.min(axis=1) * (1 + 1e-6) + 1e-12)


def test_sym_rejects_one_bit():
    with pytest.raises(ValueError):
        oracle.encode_sym_fp32(np.ones((1, 32), np.float32), _ones(32), 1, 32)


# ---------------------------------------------------------------- integer zero point
@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_intzp_matches_torch_fake_quantize(bits):
    rng = np.random.default_rng(10 + bits)
    W = rng.standard_normal((5, 256)).astype(np.float32)
    W[0, :64] = np.abs(W[0, :64])        # a group with min > 0
    W[1, 64:128] = -np.abs(W[1, 64:128])  # a group with max < 0
    dh = rng.uniform(0.5, 4.0, 256).astype(np.float32)
    q, s, z = oracle.encode_intzp_fp32(W, dh, bits, 64)
    N = 2 ** bits - 1
    u = W * dh
    for i in range(5):
        for g in range(4):
            x = torch.from_numpy(u[i, g * 64:(g + 1) * 64].copy())
            ref = torch.fake_quantize_per_tensor_affine(
                x, float(s[i, g]), int(-z[i, g]), 0, N)
            ours = (np.float64(s[i, g]) * (q[i, g * 64:(g + 1) * 64].astype(np.float64)
                                           + z[i, g])).astype(np.float32)
            np.testing.assert_array_equal(ours, ref.numpy())


def test_intzp_zero_is_exact_and_range_holds():
    rng = np.random.default_rng(21)
    W = rng.standard_normal((9, 256)).astype(np.float32)
    W[:, ::7] = 0.0
    q, s, z = oracle.encode_intzp_fp32(W, _ones(256), 4, 64)
    assert q.max() <= 15 and np.all((z <= 0) & (z >= -15))
    uh = oracle.reconstruct_format(q, s, 4, 64, "intzp", z=z)
    assert np.all(uh[:, ::7] == 0.0)
    # half-step bound away from the clipped top end
    err = np.abs(uh - W.astype(np.float64))
    ss = np.repeat(s.astype(np.float64), 64, axis=1)
    assert np.all(err <= ss * (1.0 + 1e-5))


def test_intzp_hand_worked_group():
    # u = [-0.5, 0.125, 0.75, 1.0], b = 2: lo = -0.5, hi = 1, s = 0.5,
    # inv = 2, z = rint(-1) = -1, rint(u*2) = [-1, 0 (0.25), 2 (1.5 tie), 2]
    # q = [0, 1, 3, 3], u_hat = 0.5 * (q - 1) = [-0.5, 0, 1, 1]
    u = np.array([[-0.5, 0.125, 0.75, 1.0]], dtype=np.float32)
    q, s, z = oracle.encode_intzp_fp32(u, _ones(4), 2, 4)
    assert s[0, 0] == 0.5 and z[0, 0] == -1
    np.testing.assert_array_equal(q[0], [0, 1, 3, 3])
    np.testing.assert_array_equal(
        oracle.reconstruct_format(q, s, 2, 4, "intzp", z=z)[0], [-0.5, 0.0, 1.0, 1.0])
    # an all-zero group: s = 0, every code 0, exact zeros
    q0, s0, z0 = oracle.encode_intzp_fp32(np.zeros((1, 4), np.float32), _ones(4), 2, 4)
    assert s0[0, 0] == 0 and z0[0, 0] == 0 and not q0.any()


# ---------------------------------------------------------------- FP8 codes
def test_fp8_group_matches_torch_cast_of_scaled_values():
    rng = np.random.default_rng(31)
    W = rng.standard_normal((6, 256)).astype(np.float32)
    dh = rng.uniform(0.5, 4.0, 256).astype(np.float32)
    v, s = oracle.encode_fp8_fp32(W, dh, 128)
    u = (W * dh).reshape(6, 2, 128)
    inv = (np.float32(1.0) / s)[:, :, None]
    ref = torch.from_numpy((u * inv).astype(np.float32)).to(torch.float8_e4m3fn)
    np.testing.assert_array_equal(v.reshape(6, 2, 128), ref.float().numpy())
    # the group maximum lands on +-448 exactly
    assert np.all(np.abs(v).reshape(6, 2, 128).max(axis=2) == 448.0)
    f = oracle.quantize_format(W, dh, 8, 128, "fp8")
    np.testing.assert_array_equal(f["codes"], ref.view(torch.uint8).numpy().reshape(6, 256))
    with pytest.raises(ValueError):
        oracle.quantize_format(W, dh, 4, 128, "fp8")


def test_fp8_relative_error_bound():
    # normal E4M3 values carry 3 mantissa bits: relative error <= 2^-4
    rng = np.random.default_rng(32)
    W = rng.standard_normal((4, 512)).astype(np.float32)
    f = oracle.quantize_format(W, _ones(512), 8, 64, "fp8")
    uh = oracle.reconstruct_format(f["codes"], f["s"], 8, 64, "fp8")
    w = W.astype(np.float64)
    ss = np.repeat(f["s"].astype(np.float64), 64, axis=1)
    normal = np.abs(w) >= ss * 2.0 ** -6
    rel = np.abs(uh - w)[normal] / np.abs(w)[normal]
    assert rel.max() <= 2.0 ** -4 * (1 + 1e-5)
    assert np.all(np.abs(uh - w)[~normal] <= ss[~normal] * 2.0 ** -10 * (1 + 1e-5))


# ---------------------------------------------------------------- shared helpers
def test_format_offsets_reconstruct_integer_formats():
    rng = np.random.default_rng(41)
    W = rng.standard_normal((8, 256)).astype(np.float32)
    dh = rng.uniform(0.5, 2.0, 256).astype(np.float32)
    for fmt, bits in (("asym", 4), ("sym", 4), ("intzp", 3)):
        f = oracle.quantize_format(W, dh, bits, 64, fmt)
        off = oracle.format_offsets(f["s"], bits, fmt, m=f.get("m"), z=f.get("z"))
        exact = oracle.reconstruct_format(f["codes"], f["s"], bits, 64, fmt,
                                          m=f.get("m"), z=f.get("z"))
        folded = (np.repeat(off.astype(np.float64), 64, axis=1)
                  + np.repeat(f["s"].astype(np.float64), 64, axis=1) * f["codes"])
        scale = np.repeat(np.abs(off).astype(np.float64), 64, axis=1)
        assert np.all(np.abs(folded - exact) <= scale * 2.0 ** -24 + 1e-30)


def test_pre_rounding_agrees_with_fp32_levels_outside_the_band():
    rng = np.random.default_rng(42)
    W = rng.standard_normal((16, 256)).astype(np.float32)
    dh = rng.uniform(0.5, 2.0, 256)
    for fmt, bits in (("sym", 4), ("intzp", 4), ("fp8", 8)):
        f = oracle.quantize_format(W, dh.astype(np.float32), bits, 64, fmt)
        lv = oracle.format_levels(f["codes"], bits, fmt, z=f.get("z"), group=64)
        t = oracle.pre_rounding_format_fp64(W.astype(np.float64),
                                            dh.astype(np.float32).astype(np.float64),
                                            bits, 64, fmt)
        if fmt == "fp8":
            r = oracle.e4m3_round(np.clip(t, -448, 448))
        elif fmt == "sym":
            r = np.clip(np.rint(t), -(2 ** (bits - 1) - 1), 2 ** (bits - 1) - 1)
        else:
            z = np.repeat(f["z"].astype(np.float64), 64, axis=1)
            r = np.clip(np.rint(t), z, z + 2 ** bits - 1)
        nb, ne = oracle.band_excused_levels(lv, r, t, 1e-6)
        assert nb == ne, (fmt, nb, ne)


def test_band_rule_in_level_units():
    t = np.array([2.5 + 1e-9, 2.3, 1.0625 + 1e-8, 1.0625 + 0.01])
    a = np.array([3.0, 3.0, 1.125, 1.125])
    b = np.array([2.0, 2.0, 1.0, 1.0])
    nb, ne = oracle.band_excused_levels(a, b, t, 1e-6)
    assert (nb, ne) == (4, 2)
    # not neighbours on the grid
    nb, ne = oracle.band_excused_levels(np.array([4.0]), np.array([2.0]),
                                        np.array([3.0]), 1e-6)
    assert (nb, ne) == (1, 0)


@pytest.mark.parametrize("fmt,bits", [("sym", 4), ("intzp", 4), ("fp8", 8)])
def test_linear_with_format_equals_dense_product_of_reconstruction(fmt, bits):
    from workloads import make_problem
    prob = make_problem("fmt", d=256, d_out=24, T=5, bits=bits, group=64,
                        rank=8, seed=3)
    out = oracle.ttq_linear(prob.W, prob.X[0], bits=bits, group=64, p=2.0,
                            lam=1e-3, alpha=0.5, B_bits=prob.B, A_bits=prob.A,
                            qformat=fmt)
    W32 = oracle.bf16_to_f32(prob.W)
    f = oracle.quantize_format(W32, out["dh32"], bits, 64, fmt)
    np.testing.assert_array_equal(f["codes"], out["q"])
    uh = oracle.reconstruct_format(f["codes"], f["s"], bits, 64, fmt, z=f.get("z"))
    X = oracle.bf16_to_f64(prob.X[0])
    Y = X @ (uh * out["dhi"][None, :]).T + (X @ oracle.bf16_to_f64(prob.A).T) @ \
        oracle.bf16_to_f64(prob.B).T
    np.testing.assert_allclose(out["Y"], Y, rtol=1e-12, atol=1e-12)
    # quantize-once + decode of the same prompt gives the same Y
    qz = oracle.ttq_quantize(prob.W, prob.X[0], bits=bits, group=64, p=2.0,
                             lam=1e-3, alpha=0.5, qformat=fmt)
    Yq = oracle.ttq_qmatmul(qz["packed"], qz["s"], qz["m"], qz["dhi32"], prob.X[0],
                            bits=bits, group=64, B_bits=prob.B, A_bits=prob.A,
                            qformat=fmt)
    rel = np.abs(Yq - out["Y"]).max() / np.abs(out["Y"]).max()
    assert rel < 1e-6
