"""Seeded synthetic workloads for the TTQ linear projection.

The pages evaluate TTQ on language-model perplexity with trained OPT, Qwen3
and Gemma3 weights and on VLM/VLA suites; none of that is reproduced here.
These generators stand in for those workloads with the structure the pages
describe: activation outlier channels of 10-100x the typical magnitude
(blog TL;DR and mechanism sections), whose positions depend on the input and
therefore are redrawn per call and per request (multitenant traffic).

Every array is drawn in float32 from ``numpy.random.Generator(PCG64)`` fed
by ``SeedSequence(seed).spawn`` sub-streams, scaled, and rounded to bfloat16
with round-to-nearest-even.  Arrays are returned as raw bfloat16 bit
patterns (``uint16``) so that the oracle and the GPU see identical bytes.

Shapes and distributions of the five standard workloads:

* ``c1``: d = d' = 512, T = 16, seed 0.  X ~ N(0,1) with 4 channels x50;
  W ~ N(0, 0.02^2); 4-bit, g = 128, p = 2, lambda = 1e-3, alpha = 0.5.
* ``c2``: d = d' = 4096 (a 7B-class attention projection), T in {1, 128}.
  X ~ N(0,1) with 1 % of channels (41) scaled by 10**U(1,2); 4-bit, g = 128.
* ``c3``: 7B-class MLP gate/up (4096 -> 11008) and down (11008 -> 4096),
  T = 2048; X as c1 (4 channels x50, redrawn per call); 3-bit, g = 128;
  low rank r = 64 with B, A ~ N(0, 0.01^2).
* ``c4``: 70B-class MLP up projection 8192 -> 28672, T = 512; X Student-t
  (nu = 3) with 0.5 % of channels (41) scaled log-uniformly 30-100x; 2-bit,
  g = 64, lambda = 1e-2, p in {1, 2}; r = 128.
* ``c5``: the seven projections of a 7B-class decoder layer, R = 8
  requests each with its own outlier set, T in {1, 16, 256, 4096}; 4-bit,
  g = 128, p = 2, lambda = 1e-3, r = 32.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "Problem",
    "bf16_round_bits",
    "make_problem",
    "make_c1",
    "make_c2",
    "make_c3",
    "make_c4",
    "make_c5",
    "C5_PROJECTIONS",
    "draw_x",
    "draw_omega",
    "draw_lowrank_w",
]

# (name, d_in, d_out) of the seven projections of a 7B-class decoder layer.
C5_PROJECTIONS = (
    ("q_proj", 4096, 4096),
    ("k_proj", 4096, 4096),
    ("v_proj", 4096, 4096),
    ("o_proj", 4096, 4096),
    ("gate_proj", 4096, 11008),
    ("up_proj", 4096, 11008),
    ("down_proj", 11008, 4096),
)


@dataclasses.dataclass
class Problem:
    """One TTQ linear call: bf16 bit patterns plus the method's scalars."""

    name: str
    d: int
    d_out: int
    T: int
    R: int
    bits: int
    group: int
    rank: int
    p: float
    lam: float
    alpha: float
    W: np.ndarray  # uint16 [d_out, d]
    X: np.ndarray  # uint16 [R, T, d]
    B: Optional[np.ndarray] = None  # uint16 [d_out, rank]
    A: Optional[np.ndarray] = None  # uint16 [rank, d]
    meta: dict = dataclasses.field(default_factory=dict)
    qformat: str = "asym"  # quantizer format: asym, sym, intzp, fp8

    @property
    def params(self) -> dict:
        return dict(d=self.d, d_out=self.d_out, T=self.T, rank=self.rank,
                    bits=self.bits, group=self.group, p=self.p,
                    lam=self.lam, alpha=self.alpha)


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite input)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    # chunked to keep temporaries bounded on very large arrays
    out = np.empty(b.shape, dtype=np.uint16)
    flat_b = b.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 24
    for i in range(0, flat_b.size, step):
        v = flat_b[i:i + step]
        lsb = (v >> np.uint32(16)) & np.uint32(1)
        r = (v + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
        flat_o[i:i + step] = r.astype(np.uint16)
    return out


def _rng(seed: int, *path: int) -> np.random.Generator:
    ss = np.random.SeedSequence(seed)
    for k in path:
        ss = ss.spawn(k + 1)[k]
    return np.random.Generator(np.random.PCG64(ss))


def _normal_bits(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    step = 1 << 24
    for i in range(0, n, step):
        m = min(step, n - i)
        v = rng.standard_normal(m, dtype=np.float32)
        v *= np.float32(sigma)
        out[i:i + m] = bf16_round_bits(v)
    return out.reshape(shape)


# Stream indices under each problem seed.
_S_W, _S_B, _S_A, _S_X, _S_OMEGA, _S_LR = 0, 1, 2, 3, 4, 5


def draw_x(seed: int, call: int, R: int, T: int, d: int, kind: str,
           n_outliers: int) -> np.ndarray:
    """Activations [R, T, d] as bf16 bits; one outlier set per request.

    kind:
      ``"x50"``        N(0,1), outlier channels multiplied by 50;
      ``"logu10_100"`` N(0,1), outlier channels multiplied by 10**U(1,2);
      ``"t3_logu30_100"`` Student-t(3), outliers multiplied by 10**U(log10 30, 2).
    """
    out = np.empty((R, T, d), dtype=np.uint16)
    for r in range(R):
        rng = _rng(seed, _S_X, call, r)
        if kind.startswith("t3"):
            x = rng.standard_t(3.0, size=(T, d)).astype(np.float32)
        else:
            x = rng.standard_normal((T, d), dtype=np.float32)
        k = min(n_outliers, d)
        ch = rng.choice(d, size=k, replace=False)
        if kind == "x50":
            mult = np.full(k, 50.0, dtype=np.float32)
        elif kind == "logu10_100":
            mult = (10.0 ** rng.uniform(1.0, 2.0, size=k)).astype(np.float32)
        elif kind == "t3_logu30_100":
            mult = (10.0 ** rng.uniform(np.log10(30.0), 2.0, size=k)).astype(np.float32)
        else:
            raise ValueError(f"unknown activation kind {kind!r}")
        x[:, ch] *= mult[None, :]
        out[r] = bf16_round_bits(x)
    return out


def make_problem(name: str, *, d: int, d_out: int, T: int, R: int = 1,
                 bits: int, group: int, rank: int = 0, p: float = 2.0,
                 lam: float = 1e-3, alpha: float = 0.5, seed: int = 0,
                 x_kind: str = "x50", n_outliers: int = 4,
                 w_sigma: float = 0.02, lr_sigma: float = 0.01,
                 call: int = 0, qformat: str = "asym") -> Problem:
    """Generic seeded problem; the standard workloads call this."""
    W = _normal_bits(_rng(seed, _S_W), (d_out, d), w_sigma)
    B = A = None
    if rank > 0:
        B = _normal_bits(_rng(seed, _S_B), (d_out, rank), lr_sigma)
        A = _normal_bits(_rng(seed, _S_A), (rank, d), lr_sigma)
    X = draw_x(seed, call, R, T, d, x_kind, n_outliers)
    return Problem(name=name, d=d, d_out=d_out, T=T, R=R, bits=bits,
                   group=group, rank=rank, p=p, lam=lam, alpha=alpha,
                   W=W, X=X, B=B, A=A,
                   meta=dict(seed=seed, x_kind=x_kind, n_outliers=n_outliers,
                             w_sigma=w_sigma, lr_sigma=lr_sigma, call=call),
                   qformat=qformat)


def make_c1(**kw) -> Problem:
    """512x512 single linear, T = 16, 4-bit g128, no low rank."""
    args = dict(d=512, d_out=512, T=16, bits=4, group=128, rank=0, p=2.0,
                lam=1e-3, alpha=0.5, seed=0, x_kind="x50", n_outliers=4)
    args.update(kw)
    return make_problem("c1", **args)


def make_c2(T: int = 1, **kw) -> Problem:
    """4096x4096 attention projection at decode (T=1) or T=128."""
    args = dict(d=4096, d_out=4096, T=T, bits=4, group=128, rank=0, p=2.0,
                lam=1e-3, alpha=0.5, seed=1, x_kind="logu10_100",
                n_outliers=41)
    args.update(kw)
    return make_problem(f"c2_T{T}", **args)


def make_c3(which: str = "gate_up", **kw) -> Problem:
    """MLP gate/up (4096->11008) or down (11008->4096), T = 2048, 3-bit, r=64."""
    d, d_out = (4096, 11008) if which == "gate_up" else (11008, 4096)
    args = dict(d=d, d_out=d_out, T=2048, bits=3, group=128, rank=64, p=2.0,
                lam=1e-3, alpha=0.5, seed=2 if which == "gate_up" else 12,
                x_kind="x50", n_outliers=4)
    args.update(kw)
    return make_problem(f"c3_{which}", **args)


def make_c4(p: float = 2.0, **kw) -> Problem:
    """8192 -> 28672 up projection, T = 512, 2-bit g64, r = 128."""
    args = dict(d=8192, d_out=28672, T=512, bits=2, group=64, rank=128, p=p,
                lam=1e-2, alpha=0.5, seed=3, x_kind="t3_logu30_100",
                n_outliers=41)
    args.update(kw)
    return make_problem(f"c4_p{int(p)}", **args)


def make_c5(T: int, proj: str = "q_proj", R: int = 8, **kw) -> Problem:
    """One projection of a 7B-class layer, R requests with own outlier sets."""
    names = [n for n, _, _ in C5_PROJECTIONS]
    i = names.index(proj)
    _, d, d_out = C5_PROJECTIONS[i]
    args = dict(d=d, d_out=d_out, T=T, R=R, bits=4, group=128, rank=32,
                p=2.0, lam=1e-3, alpha=0.5, seed=4 + 100 * (i + 1),
                x_kind="logu10_100", n_outliers=max(1, round(0.01 * d)))
    args.update(kw)
    return make_problem(f"c5_{proj}_T{T}", **args)


def draw_omega(seed: int, d: int, r: int) -> np.ndarray:
    """Gaussian test matrix [d, r] (float32) for the PCA range finder."""
    return _rng(seed, _S_OMEGA).standard_normal((d, r)).astype(np.float32)


def draw_lowrank_w(seed: int, d_out: int, d: int, r: int, gap: float = 30.0,
                   sigma: float = 0.02) -> np.ndarray:
    """bf16 weights with a planted rank-r part: W = U S V^T + E with the
    planted singular values (2 .. 1) x sigma sqrt(d) and a Gaussian E whose
    singular values sit about ``gap`` times lower (a clear spectral gap at r,
    as the PCA tests need).  U, V are Gaussian (not orthonormalised: the
    planted part is then only approximately of singular values S)."""
    rng = _rng(seed, _S_LR)
    U = rng.standard_normal((d_out, r)) / np.sqrt(d_out)
    V = rng.standard_normal((d, r)) / np.sqrt(d)
    S = np.linspace(2.0, 1.0, r) * sigma * np.sqrt(d)
    E = rng.standard_normal((d_out, d)) * (sigma / gap) / np.sqrt(max(d_out, d)) \
        * np.sqrt(d) / 2.0
    return bf16_round_bits(((U * S) @ V.T + E).astype(np.float32))
