"""Pins of the oracle's quantize-once / decode-from-codes functions (CPU).

What fixes them, besides the oracle itself:
  * the code storage format (a design choice, stated in the oracle): hand
    packed bytes for every container width;
  * round trip of pack / unpack over every bit width;
  * on the prompt that produced the codes, decoding from stored codes gives
    the projection of the pinned one-shot path (``ttq_linear``);
  * on a later step, the statistics are those of the prompt, not the step's;
  * linearity in the activations, exact power-of-two scaling, token
    permutation, and the low-rank identity B(AX) = (BA)X;
  * alpha = 0 makes the stored weights independent of the prompt (plain RTN).
"""
import numpy as np
import pytest

import oracle
from workloads import bf16_round_bits, make_problem


def _bf16(x):
    return bf16_round_bits(np.asarray(x, dtype=np.float32))


@pytest.mark.parametrize("bits,cb", [(1, 1), (2, 2), (3, 4), (4, 4), (5, 8),
                                     (6, 8), (7, 8), (8, 8)])
def test_container_bits(bits, cb):
    assert oracle.code_container_bits(bits) == cb


def test_pack_hand_examples():
    # 4-bit: two codes per byte, first channel in the low nibble
    q = np.array([[1, 2, 3, 4, 15, 0]], dtype=np.uint8)
    assert oracle.pack_codes(q, 4).tolist() == [[0x21, 0x43, 0x0F]]
    # 3-bit codes use the 4-bit container
    assert oracle.pack_codes(np.array([[7, 5]], np.uint8), 3).tolist() == [[0x57]]
    # 2-bit: four per byte, 1 | 2<<2 | 3<<4 | 0<<6 = 0x39
    q = np.array([[1, 2, 3, 0, 3, 3, 3, 3]], dtype=np.uint8)
    assert oracle.pack_codes(q, 2).tolist() == [[0x39, 0xFF]]
    # 1-bit: eight per byte, bit j = channel j
    q = np.array([[1, 0, 1, 1, 0, 0, 0, 1]], dtype=np.uint8)
    assert oracle.pack_codes(q, 1).tolist() == [[0x8D]]
    # 8-bit: the codes themselves
    q = np.array([[0, 200, 255, 17]], dtype=np.uint8)
    assert oracle.pack_codes(q, 8).tolist() == [[0, 200, 255, 17]]


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 8])
def test_pack_round_trip(bits):
    rng = np.random.default_rng(bits)
    q = rng.integers(0, 1 << bits, size=(7, 64), dtype=np.uint8)
    packed = oracle.pack_codes(q, bits)
    assert packed.shape == (7, 64 * oracle.code_container_bits(bits) // 8)
    np.testing.assert_array_equal(oracle.unpack_codes(packed, bits, 64), q)
    if bits < 8:
        with pytest.raises(ValueError):
            bad = q.copy()
            bad[0, 0] = 1 << bits
            oracle.pack_codes(bad, bits)


def _prob(seed=3, T=8, rank=0, alpha=0.5):
    return make_problem("qm", d=256, d_out=48, T=T, bits=4, group=64,
                        rank=rank, alpha=alpha, seed=seed,
                        x_kind="logu10_100", n_outliers=5)


def _kw(p):
    return dict(bits=p.bits, group=p.group, p=p.p, lam=p.lam, alpha=p.alpha)


def test_same_prompt_matches_one_shot_projection():
    p = _prob(rank=16)
    qz = oracle.ttq_quantize(p.W, p.X[0], **_kw(p))
    Y = oracle.ttq_qmatmul(qz["packed"], qz["s"], qz["m"], qz["dhi32"], p.X[0],
                           bits=p.bits, group=p.group, B_bits=p.B, A_bits=p.A)
    ref = oracle.ttq_linear(p.W, p.X[0], B_bits=p.B, A_bits=p.A, **_kw(p))
    np.testing.assert_array_equal(qz["q"], ref["q"])
    # only difference: D^{-1/2} stored in float32 (relative 2^-24 per term)
    rms = np.sqrt(np.mean(ref["Y"] ** 2))
    np.testing.assert_allclose(Y, ref["Y"], rtol=0, atol=1e-6 * rms)


def test_later_step_uses_the_prompt_statistics():
    p1, p2 = _prob(seed=3), _prob(seed=4)
    qz = oracle.ttq_quantize(p1.W, p1.X[0], **_kw(p1))
    Y = oracle.ttq_qmatmul(qz["packed"], qz["s"], qz["m"], qz["dhi32"], p2.X[0],
                           bits=p1.bits, group=p1.group)
    # the weights that the prompt's one-shot projection applies ...
    ref1 = oracle.ttq_linear(p1.W, p1.X[0], **_kw(p1))
    W_hat1 = oracle.dequantize(ref1["q"], ref1["s"], ref1["m"], ref1["dhi"], p1.group)
    X2 = oracle.bf16_to_f64(p2.X[0])
    ref = X2 @ W_hat1.T
    rms = np.sqrt(np.mean(ref ** 2))
    np.testing.assert_allclose(Y, ref, rtol=0, atol=1e-6 * rms)
    # ... differ from re-deriving the statistics from the step itself
    ref2 = oracle.ttq_linear(p1.W, p2.X[0], **_kw(p1))
    assert not np.allclose(Y, ref2["Y"], rtol=1e-3)


def test_linearity_scaling_and_permutation():
    p = _prob(T=6)
    qz = oracle.ttq_quantize(p.W, p.X[0], **_kw(p))
    args = (qz["packed"], qz["s"], qz["m"], qz["dhi32"])
    kw = dict(bits=p.bits, group=p.group)
    X = oracle.bf16_to_f32(p.X[0])
    Y = oracle.ttq_qmatmul(*args, p.X[0], **kw)
    # exact power-of-two scaling of the activations
    Y4 = oracle.ttq_qmatmul(*args, _bf16(4.0 * X), **kw)
    np.testing.assert_array_equal(Y4, 4.0 * Y)
    # token permutation permutes the rows of Y
    perm = np.array([3, 0, 5, 1, 4, 2])
    Yp = oracle.ttq_qmatmul(*args, p.X[0][perm], **kw)
    np.testing.assert_array_equal(Yp, Y[perm])
    # additivity over a split of the tokens' values (exact halves)
    Xa = _bf16(X * 0.5)
    Y2 = oracle.ttq_qmatmul(*args, Xa, **kw) * 2.0
    np.testing.assert_allclose(Y2, Y, rtol=1e-12, atol=1e-12)


def test_low_rank_identity():
    p = _prob(rank=16)
    qz = oracle.ttq_quantize(p.W, p.X[0], **_kw(p))
    args = (qz["packed"], qz["s"], qz["m"], qz["dhi32"], p.X[0])
    kw = dict(bits=p.bits, group=p.group)
    Y0 = oracle.ttq_qmatmul(*args, **kw)
    Y1 = oracle.ttq_qmatmul(*args, B_bits=p.B, A_bits=p.A, **kw)
    BA = oracle.bf16_to_f64(p.B) @ oracle.bf16_to_f64(p.A)
    np.testing.assert_allclose(Y1 - Y0, oracle.bf16_to_f64(p.X[0]) @ BA.T,
                               rtol=1e-9, atol=1e-12)


def test_alpha0_stored_weights_do_not_depend_on_the_prompt():
    pa, pb = _prob(seed=3, alpha=0.0), _prob(seed=9, alpha=0.0)
    qa = oracle.ttq_quantize(pa.W, pa.X[0], **_kw(pa))
    qb = oracle.ttq_quantize(pa.W, pb.X[0], **_kw(pa))
    np.testing.assert_array_equal(qa["packed"], qb["packed"])
    np.testing.assert_array_equal(qa["s"], qb["s"])
    np.testing.assert_array_equal(qa["dhi32"], np.ones_like(qa["dhi32"]))
