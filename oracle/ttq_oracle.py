"""CPU oracle for the TTQ (activation-aware test-time quantization) linear
projection.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check in ``__graft_entry__``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP implementation; the only thing both sides consume is the seeded
bfloat16 input bytes from the ``workloads`` package.

Sources (pages as titled; sections as headed on each page):

* [ZH]  "TTQ: Activation-Aware Test-Time Quantization to Accelerate LLM
  Inference On The Fly", gist.science zh summary of arXiv:2603.19296.
  Sec. 2.1 (online activation-aware quantization): the diagonal
  D_ii = (||X_{i,:}||_p + lambda)^alpha and W_hat = Q[W D^{1/2}] D^{-1/2};
  Sec. 2.2 (low-rank integration): W ~ W_q + BA with static B, A;
  Sec. 2.3 (complexity): overhead O[dT + 3d'd] against O[d'dT].
* [NL], [IT]  the nl and it summaries of the same paper, Sec. 2
  (methodology), which restate the same formulas.
* [BLOG-EN] "Test-time quantization: quantising on the fly with no
  calibration dataset", section "The maths that matter": the affine
  quantizer (integer code, scale s, zero point) with |x - x_hat| <= s/2, the
  symmetric scale M / (2^{b-1} - 1), and the INT4 outlier example.

Notation: X has d input channels and T tokens.  Arrays here store it
token-major, ``X[t, j]`` = channel j of token t, as a linear layer receives
it.  W is ``[d_out, d]``; Y = W_hat X is stored ``[T, d_out]``.

Readings taken where the pages leave a step open:

1. Quantizer Q: asymmetric b-bit, groups of ``group`` consecutive input
   channels of one output row, min-anchored with a real zero point:
   s = (max - min) / (2^b - 1), q = clamp(round((u - min) / s), 0, 2^b - 1),
   u_hat = min + s q.  A group with max == min gets s = 0 and q = 0.
2. round = round half to even.
3. ||X_{i,:}||_p is the plain (unnormalised) L_p norm over the T tokens.
4. lambda is added to the norm before the power: (n + lambda)^alpha.
5. D^{1/2}, D^{-1/2} are the elementwise powers +-alpha/2 of the diagonal;
   D^{-1/2} is evaluated as 1 / D^{1/2}.  A channel with n + lambda = 0 gets
   D^{1/2} = D^{-1/2} = 1 (it multiplies zero activations only).
6. Low rank: the W passed in is already the residual W_q; Y = Q_D[W] X +
   B (A X), with B, A unquantized and untouched by D.
7. Decision precision: the pages fix none, so the integer codes are decided
   in IEEE float32 by this fixed sequence (no fused multiply-add):
     dh32 = float32(D^{1/2});  u = fl(w * dh32);  m, M = min, max of u;
     s = fl(fl(M - m) / N);    inv = fl(1 / s) (0 if s == 0);
     t = fl(fl(u - m) * inv);  q = clamp(rint(t), 0, N).
   Statistics (norms, powers) and the dequantized contraction are float64.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

__all__ = [
    "bf16_to_f64",
    "bf16_to_f32",
    "channel_norms",
    "diag_scales",
    "encode_groups_fp32",
    "pre_rounding_fp64",
    "dequantize",
    "ttq_linear",
    "ttq_linear_batched",
    "band_excused",
    "symmetric_quantize",
    "code_container_bits",
    "pack_codes",
    "unpack_codes",
    "ttq_quantize",
    "ttq_qmatmul",
    "QFORMATS",
    "e4m3_decode",
    "e4m3_round",
    "e4m3_encode",
    "encode_sym_fp32",
    "encode_intzp_fp32",
    "encode_fp8_fp32",
    "quantize_format",
    "reconstruct_format",
    "format_offsets",
    "format_levels",
    "pre_rounding_format_fp64",
    "band_excused_levels",
    "orthonormalize",
    "subspace_iteration",
    "lowrank_pca",
    "pca_exact",
]


# --------------------------------------------------------------------------
# input decoding (the oracle's own; bfloat16 is the top half of a float32)
# --------------------------------------------------------------------------
def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_to_f32(bits).astype(np.float64)


# --------------------------------------------------------------------------
# statistics: [ZH] Sec. 2.1, [NL]/[IT] Sec. 2
# --------------------------------------------------------------------------
def channel_norms(X: np.ndarray, p: float) -> np.ndarray:
    """n_j = ||X_{j,:}||_p, the L_p norm of channel j over all T tokens.

    ``X`` is ``[T, d]`` float64.  Reading 3: no 1/T normalisation.
    """
    X = np.asarray(X, dtype=np.float64)
    if X.shape[0] == 0:
        return np.zeros(X.shape[1], dtype=np.float64)
    if p == 2.0:
        return np.sqrt(np.sum(X * X, axis=0))
    if p == 1.0:
        return np.sum(np.abs(X), axis=0)
    return np.sum(np.abs(X) ** p, axis=0) ** (1.0 / p)


def diag_scales(n: np.ndarray, lam: float, alpha: float):
    """D^{1/2} and D^{-1/2} for D_ii = (n_i + lambda)^alpha ([ZH] Sec. 2.1).

    Returns float64 ``(dh, dhi)``; readings 4 and 5.
    """
    base = np.asarray(n, dtype=np.float64) + float(lam)
    dh = np.ones_like(base)
    ok = base > 0.0
    dh[ok] = base[ok] ** (0.5 * float(alpha))
    dhi = 1.0 / dh
    return dh, dhi


# --------------------------------------------------------------------------
# quantizer Q[W D^{1/2}]: [ZH] Sec. 2.1; affine form from [BLOG-EN] maths
# --------------------------------------------------------------------------
def encode_groups_fp32(W32: np.ndarray, dh32: np.ndarray, bits: int,
                       group: int):
    """Integer codes of W D^{1/2}, decided in float32 (reading 7).

    ``W32`` is ``[rows, d]`` float32 (exact bf16 values), ``dh32`` is ``[d]``
    float32.  Returns ``(q uint8 [rows, d], s f32 [rows, G], m f32 [rows, G])``
    with G = d / group.
    """
    W32 = np.asarray(W32, dtype=np.float32)
    dh32 = np.asarray(dh32, dtype=np.float32)
    rows, d = W32.shape
    G = d // group
    N = np.float32(2 ** bits - 1)
    u = (W32 * dh32[None, :]).reshape(rows, G, group)       # fl(w * dh)
    m = u.min(axis=2)
    M = u.max(axis=2)
    s = (M - m) / N                                          # fl(fl(M-m)/N)
    pos = s > np.float32(0)
    inv = np.zeros_like(s)
    inv[pos] = np.float32(1.0) / s[pos]                      # fl(1/s)
    t = (u - m[:, :, None]) * inv[:, :, None]                # fl(fl(u-m)*inv)
    q = np.clip(np.rint(t), np.float32(0), N)
    q = np.where(pos[:, :, None], q, np.float32(0))
    return q.astype(np.uint8).reshape(rows, d), s, m


def pre_rounding_fp64(W64: np.ndarray, dh64: np.ndarray, bits: int,
                      group: int):
    """The real-valued pre-rounding code t* = (u - min) / s in float64.

    Used only to decide whether a code mismatch sits on a rounding boundary.
    Returns ``(t, u, m, s)`` with t, u ``[rows, d]`` and m, s ``[rows, G]``.
    """
    W64 = np.asarray(W64, dtype=np.float64)
    rows, d = W64.shape
    G = d // group
    N = float(2 ** bits - 1)
    u = (W64 * dh64[None, :]).reshape(rows, G, group)
    m = u.min(axis=2)
    s = (u.max(axis=2) - m) / N
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(s[:, :, None] > 0, (u - m[:, :, None]) / s[:, :, None], 0.0)
    return t.reshape(rows, d), u.reshape(rows, d), m, s


def dequantize(q: np.ndarray, s: np.ndarray, m: np.ndarray, dhi: np.ndarray,
               group: int) -> np.ndarray:
    """W_hat = (min + s q) D^{-1/2}, float64 ([ZH] Sec. 2.1)."""
    rows, d = q.shape
    G = d // group
    u_hat = (m.astype(np.float64)[:, :, None]
             + s.astype(np.float64)[:, :, None]
             * q.reshape(rows, G, group).astype(np.float64))
    return u_hat.reshape(rows, d) * np.asarray(dhi, dtype=np.float64)[None, :]


# --------------------------------------------------------------------------
# the whole projection
# --------------------------------------------------------------------------
def ttq_linear(W_bits: np.ndarray, X_bits: np.ndarray, *, bits: int,
               group: int, p: float, lam: float, alpha: float,
               B_bits: Optional[np.ndarray] = None,
               A_bits: Optional[np.ndarray] = None,
               rows: Optional[np.ndarray] = None,
               dh32_override: Optional[np.ndarray] = None,
               want_t: bool = False, qformat: str = "asym") -> dict:
    """One TTQ linear call for one request.

    ``W_bits`` uint16 ``[d_out, d]``, ``X_bits`` uint16 ``[T, d]``, optional
    ``B_bits`` ``[d_out, r]`` and ``A_bits`` ``[r, d]``.  ``rows`` restricts
    the quantization and the output to a subset of output channels (rows of
    W are independent once D is fixed; D always uses the full X).
    ``dh32_override`` replaces the float32 D^{1/2} fed to the code decision
    (used to check a kernel's codes against its own exported statistics).

    ``qformat`` picks the quantizer (``QFORMATS``; default the asymmetric
    one of reading 1).

    Returns a dict with ``n, dh, dhi`` (float64 [d]), ``dh32`` (float32
    [d]), ``q`` (uint8 [rows, d], the stored codes), ``s, m`` (float32
    [rows, G]; for formats other than asym ``m`` is ``format_offsets``),
    ``Y`` (float64 [T, rows]) and, if ``want_t``, the float64 pre-rounding
    values (``t64`` in level units for formats other than asym).
    """
    X = bf16_to_f64(X_bits)
    T, d = X.shape
    d_out = W_bits.shape[0]
    if d % group != 0:
        raise ValueError("group must divide d")
    sel = np.arange(d_out) if rows is None else np.asarray(rows)
    Wsel = np.asarray(W_bits)[sel]

    n = channel_norms(X, p)
    dh, dhi = diag_scales(n, lam, alpha)
    dh32 = dh.astype(np.float32) if dh32_override is None else \
        np.asarray(dh32_override, dtype=np.float32)

    if qformat == "asym":
        q, s, m = encode_groups_fp32(bf16_to_f32(Wsel), dh32, bits, group)
        W_hat = dequantize(q, s, m, dhi, group)
        extra = {}
    else:
        f = quantize_format(bf16_to_f32(Wsel), dh32, bits, group, qformat)
        q, s = f["codes"], f["s"]
        m = format_offsets(s, bits, qformat, z=f.get("z"))
        W_hat = reconstruct_format(q, s, bits, group, qformat, z=f.get("z")) \
            * dhi[None, :]
        extra = {"z": f["z"]} if "z" in f else {}
    Y = X @ W_hat.T
    if B_bits is not None and A_bits is not None and np.asarray(A_bits).size:
        A = bf16_to_f64(A_bits)
        Bm = bf16_to_f64(np.asarray(B_bits)[sel])
        Z = X @ A.T                       # (A X) stored token-major [T, r]
        Y = Y + Z @ Bm.T                  # + B (A X)   ([ZH] Sec. 2.2)
    out = dict(n=n, dh=dh, dhi=dhi, dh32=dh32, q=q, s=s, m=m, Y=Y, rows=sel,
               qformat=qformat, **extra)
    if want_t:
        if qformat == "asym":
            t, u, mm, ss = pre_rounding_fp64(bf16_to_f64(Wsel), dh, bits, group)
            out.update(t64=t, u64=u, m64=mm, s64=ss)
        else:
            out.update(t64=pre_rounding_format_fp64(bf16_to_f64(Wsel), dh, bits,
                                                    group, qformat))
    return out


def ttq_linear_batched(W_bits, X_bits, **kw) -> list:
    """R independent requests on a shared W (and B, A): one D per request."""
    return [ttq_linear(W_bits, X_bits[r], **kw) for r in range(X_bits.shape[0])]


# --------------------------------------------------------------------------
# quantize once per prompt, then contract later tokens with stored codes
# --------------------------------------------------------------------------
# The statistics are computed per input prompt ([NL] Sec. 2, methodology),
# and the speed-up of the deployed model comes from integer-matmul kernels
# over stored low-bit weights ([NL] Sec. 3, efficiency; [ZH] Sec. 3) because
# moving the weights is the bottleneck at scale ([ZH] Sec. 4).  Reading:
# the deployed form keeps the codes, the per-group (s, min) and D^{-1/2} of
# the prompt, and every later step computes
# Y = ((min + s q) D^{-1/2}) X + B (A X) with those stored values.
#
# Storage of the codes: each code takes the smallest of 1, 2, 4, 8 bits that
# holds b bits ("container"), channel j of a row at bit (j * cb) % 8 of byte
# (j * cb) // 8 (least significant bits first).

def code_container_bits(bits: int) -> int:
    """Storage width in bits of one b-bit code."""
    if not 1 <= bits <= 8:
        raise ValueError("bits must be in 1..8")
    for cb in (1, 2, 4, 8):
        if bits <= cb:
            return cb
    raise AssertionError


def pack_codes(q: np.ndarray, bits: int) -> np.ndarray:
    """uint8 codes [rows, d] -> packed bytes [rows, d * cb / 8]."""
    cb = code_container_bits(bits)
    q = np.asarray(q, dtype=np.uint8)
    rows, d = q.shape
    if (d * cb) % 8:
        raise ValueError("d * container bits must be a whole number of bytes")
    if q.size and int(q.max()) >= (1 << bits):
        raise ValueError("code out of range")
    per = 8 // cb                         # codes per byte
    qq = q.reshape(rows, d // per, per).astype(np.uint16)
    out = np.zeros((rows, d // per), dtype=np.uint16)
    for k in range(per):
        out |= qq[:, :, k] << (k * cb)
    return out.astype(np.uint8)


def unpack_codes(packed: np.ndarray, bits: int, d: int) -> np.ndarray:
    """Inverse of ``pack_codes``."""
    cb = code_container_bits(bits)
    per = 8 // cb
    packed = np.asarray(packed, dtype=np.uint8)
    rows = packed.shape[0]
    mask = (1 << cb) - 1
    parts = [(packed >> (k * cb)) & mask for k in range(per)]
    return np.stack(parts, axis=-1).reshape(rows, d).astype(np.uint8)


def ttq_quantize(W_bits: np.ndarray, X_bits: np.ndarray, *, bits: int,
                 group: int, p: float, lam: float, alpha: float,
                 rows: Optional[np.ndarray] = None,
                 dh32_override: Optional[np.ndarray] = None,
                 qformat: str = "asym") -> dict:
    """Statistics of one prompt X and the quantized weights to keep.

    Same steps as ``ttq_linear`` up to the codes; returns ``q`` (uint8),
    ``packed`` (``pack_codes``), ``s, m`` (float32 [rows, G]), ``dh32`` and
    ``dhi32`` = float32(1 / D^{1/2}) (the stored D^{-1/2}), and the float64
    ``dh, dhi``.
    """
    X = bf16_to_f64(X_bits)
    d_out = W_bits.shape[0]
    sel = np.arange(d_out) if rows is None else np.asarray(rows)
    Wsel = np.asarray(W_bits)[sel]
    n = channel_norms(X, p)
    dh, dhi = diag_scales(n, lam, alpha)
    dh32 = dh.astype(np.float32) if dh32_override is None else \
        np.asarray(dh32_override, dtype=np.float32)
    f = quantize_format(bf16_to_f32(Wsel), dh32, bits, group, qformat)
    q, s = f["codes"], f["s"]
    m = f["m"] if qformat == "asym" else format_offsets(s, bits, qformat,
                                                        z=f.get("z"))
    return dict(q=q, packed=pack_codes(q, bits), s=s, m=m, dh=dh, dhi=dhi,
                dh32=dh32, dhi32=dhi.astype(np.float32), rows=sel,
                qformat=qformat)


def ttq_qmatmul(packed: np.ndarray, s: np.ndarray, m: np.ndarray,
                dhi32: np.ndarray, X_bits: np.ndarray, *, bits: int,
                group: int, B_bits: Optional[np.ndarray] = None,
                A_bits: Optional[np.ndarray] = None,
                qformat: str = "asym") -> np.ndarray:
    """Y [T, rows] = X ((min + s q) D^{-1/2})^T + (X A^T) B^T, float64, from
    the stored codes, (s, min) and D^{-1/2} of an earlier prompt.

    For the other formats the group term ``m`` is the stored offset of
    ``format_offsets``; the reconstruction follows the format's definition
    (the intzp zero point is z = rint(m / s), exact for |z| <= 255)."""
    X = bf16_to_f64(X_bits)
    d = X.shape[1]
    q = unpack_codes(packed, bits, d)
    dhi64 = np.asarray(dhi32, dtype=np.float64)
    if qformat == "asym":
        W_hat = dequantize(q, s, m, dhi64, group)
    else:
        z = None
        if qformat == "intzp":
            s32 = np.asarray(s, dtype=np.float64)
            with np.errstate(divide="ignore", invalid="ignore"):
                z = np.where(s32 > 0, np.rint(np.asarray(m, dtype=np.float64) / s32), 0.0)
        W_hat = reconstruct_format(q, s, bits, group, qformat, z=z) * dhi64[None, :]
    Y = X @ W_hat.T
    if B_bits is not None and A_bits is not None and np.asarray(A_bits).size:
        Y = Y + (X @ bf16_to_f64(A_bits).T) @ bf16_to_f64(B_bits).T
    return Y


# --------------------------------------------------------------------------
# code-parity band
# --------------------------------------------------------------------------
def band_excused(q_gpu: np.ndarray, q_ref: np.ndarray, t64: np.ndarray,
                 u64: np.ndarray, m64: np.ndarray, s64: np.ndarray,
                 group: int, rel: float = 1e-6):
    """Classify code mismatches.

    A mismatch is excused iff the two codes are adjacent (k, k+1) and the
    float64 pre-rounding value t* lies within ``rel`` of the boundary k + 1/2,
    relative to max(|t*|, (|u| + |min|)/s), the size of the operands that
    enter the subtraction.  Returns ``(n_mismatch, n_excused, n_literal)``,
    where ``n_literal`` counts mismatches inside the literal band
    ``rel * (k + 1/2)``.
    """
    q_gpu = np.asarray(q_gpu).astype(np.int64)
    q_ref = np.asarray(q_ref).astype(np.int64)
    bad = q_gpu != q_ref
    nb = int(bad.sum())
    if nb == 0:
        return 0, 0, 0
    rows, d = q_ref.shape
    G = d // group
    mm = np.repeat(m64, group, axis=1)
    ss = np.repeat(s64, group, axis=1)
    k = np.minimum(q_gpu, q_ref)
    adjacent = np.abs(q_gpu - q_ref) == 1
    dist = np.abs(t64 - (k + 0.5))
    with np.errstate(divide="ignore", invalid="ignore"):
        scale = np.maximum(np.abs(t64), (np.abs(u64) + np.abs(mm)) / ss)
    exc = bad & adjacent & (dist <= rel * scale)
    lit = bad & adjacent & (dist <= rel * (k + 0.5))
    return nb, int(exc.sum()), int(lit.sum())


# --------------------------------------------------------------------------
# [BLOG-EN] maths: the symmetric b-bit quantizer of the worked example
# --------------------------------------------------------------------------
def symmetric_quantize(x: np.ndarray, bits: int):
    """Symmetric round-to-nearest with s = max|x| / (2^{b-1} - 1).

    Returns ``(q, s, x_hat)``; q in [-(2^{b-1}-1), 2^{b-1}-1], x_hat = s q.
    """
    x = np.asarray(x, dtype=np.float64)
    L = 2 ** (bits - 1) - 1
    s = float(np.max(np.abs(x))) / L
    if s == 0.0:
        return np.zeros_like(x, dtype=np.int64), 0.0, np.zeros_like(x)
    q = np.clip(np.rint(x / s), -L, L).astype(np.int64)
    return q, s, s * q


# --------------------------------------------------------------------------
# format variants of Q: the pages call TTQ orthogonal to the code format
# ([BLOG-EN] section "What TTQ is NOT": the scale source is what defines the
# method, so the same D-scaled groups can feed an INT4 or an FP8 quantizer;
# its table names E4M3 and E5M2 as the FP8 formats).
# Each variant below decides its codes in float32 by a fixed sequence, like
# reading 7, and reconstructs by its own definition in float64.
#
#   "asym"   min-anchored real zero point (reading 1; encode_groups_fp32)
#   "sym"    symmetric b-bit ([BLOG-EN] maths): s = max|u| / Z, Z = 2^{b-1}-1,
#            level k = clamp(round(u / s), -Z, Z), u_hat = s k;
#            stored code k + Z in [0, 2Z]
#   "intzp"  the affine form of [BLOG-EN] maths with an integer zero point z:
#            code q = round(u / s) - z in [0, N], u_hat = s (q + z).  Reading:
#            the range is widened to contain 0 (zero is then exactly
#            representable, the usual convention for integer zero points),
#            s = (hi - lo) / N with lo = min(min u, 0), hi = max(max u, 0),
#            z = round(lo / s)
#   "fp8"    FP8 E4M3 codes (OCP 8-bit float: 1 sign, 4 exponent bits with
#            bias 7, 3 mantissa bits, largest finite 448, no infinities) with
#            one float32 scale per group from the D-scaled weights
#            (TTQ over FP8, [BLOG-EN] "What TTQ is NOT"): s = max|u| / 448,
#            value v = E4M3 rounding (nearest, ties to even mantissa) of u / s,
#            u_hat = s v; stored code = the E4M3 bit pattern of v, whose sign
#            bit is the sign of u / s (a conversion to a floating-point format
#            keeps the sign, also of a result that rounds to zero)
# --------------------------------------------------------------------------
QFORMATS = ("asym", "sym", "intzp", "fp8")
E4M3_MAX = 448.0


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    """float64 value of E4M3 bit patterns (codes 0x7f / 0xff are NaN)."""
    c = np.asarray(code).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    mnt = (c & 7).astype(np.float64)
    val = np.where(e == 0, mnt * 2.0 ** -9,
                   (1.0 + mnt / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = np.where((c & 0x7f) == 0x7f, np.nan, val)
    return sign * val


def _e4m3_nonneg_grid():
    """All finite non-negative E4M3 values, ascending, with their codes."""
    codes = np.arange(0x7f)                       # 0x00 .. 0x7e
    return e4m3_decode(codes), codes


def e4m3_round(t: np.ndarray) -> np.ndarray:
    """Round each finite |t| <= 448 to the nearest E4M3 value; a tie goes to
    the neighbour with the even mantissa (its code is even); the sign of t
    is kept (also for a zero result).  float64 out."""
    t = np.asarray(t, dtype=np.float64)
    if np.any(np.abs(t) > E4M3_MAX):
        raise ValueError("outside the E4M3 range")
    vals, codes = _e4m3_nonneg_grid()
    a = np.abs(t)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    dlo = a - vals[lo]
    dhi = vals[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (codes[hi] % 2 == 0))
    r = np.where(pick_hi, vals[hi], vals[lo])
    return np.where(np.signbit(t), -r, r)


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Bit pattern of exact E4M3 values; the sign bit is the sign bit of v
    (a negative zero is 0x80)."""
    v = np.asarray(v, dtype=np.float64)
    vals, codes = _e4m3_nonneg_grid()
    a = np.abs(v)
    idx = np.searchsorted(vals, a)
    if np.any(idx >= len(vals)) or np.any(vals[np.minimum(idx, len(vals) - 1)] != a):
        raise ValueError("not an E4M3 value")
    return (codes[idx] | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def _grouped_u32(W32, dh32, group):
    W32 = np.asarray(W32, dtype=np.float32)
    dh32 = np.asarray(dh32, dtype=np.float32)
    rows, d = W32.shape
    return (W32 * dh32[None, :]).reshape(rows, d // group, group), rows, d


def _inv32(s):
    inv = np.zeros_like(s)
    pos = s > np.float32(0)
    inv[pos] = np.float32(1.0) / s[pos]                      # fl(1/s)
    return inv


def encode_sym_fp32(W32, dh32, bits: int, group: int):
    """Symmetric codes: A = max|u|; s = fl(A / Z); inv = fl(1/s) (0 if s = 0);
    k = clamp(rint(fl(u * inv)), -Z, Z).  Returns (k int16 [rows, d], s)."""
    if bits < 2:
        raise ValueError("the symmetric quantizer needs bits >= 2")
    u, rows, d = _grouped_u32(W32, dh32, group)
    Z = np.float32(2 ** (bits - 1) - 1)
    s = np.abs(u).max(axis=2) / Z
    inv = _inv32(s)
    k = np.clip(np.rint(u * inv[:, :, None]), -Z, Z)
    return k.astype(np.int16).reshape(rows, d), s


def encode_intzp_fp32(W32, dh32, bits: int, group: int):
    """Integer zero point: lo = min(min u, 0), hi = max(max u, 0);
    s = fl(fl(hi - lo) / N); inv = fl(1/s) (0 if s = 0); z = rint(fl(lo * inv));
    q = clamp(rint(fl(u * inv)) - z, 0, N).  Returns (q uint8, s, z int16)."""
    u, rows, d = _grouped_u32(W32, dh32, group)
    N = np.float32(2 ** bits - 1)
    lo = np.minimum(u.min(axis=2), np.float32(0))
    hi = np.maximum(u.max(axis=2), np.float32(0))
    s = (hi - lo) / N
    inv = _inv32(s)
    z = np.rint(lo * inv)
    q = np.clip(np.rint(u * inv[:, :, None]) - z[:, :, None], np.float32(0), N)
    return q.astype(np.uint8).reshape(rows, d), s, z.astype(np.int16)


def encode_fp8_fp32(W32, dh32, group: int):
    """FP8 E4M3 codes: A = max|u|; s = fl(A / 448); inv = fl(1/s) (0 if s = 0);
    t = fl(u * inv) clamped to [-448, 448]; v = E4M3 rounding of t.
    Returns (v float64 E4M3 values [rows, d], s)."""
    u, rows, d = _grouped_u32(W32, dh32, group)
    s = np.abs(u).max(axis=2) / np.float32(E4M3_MAX)
    inv = _inv32(s)
    t = np.clip(u * inv[:, :, None], np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3_round(t.astype(np.float64)).reshape(rows, d), s


def quantize_format(W32, dh32, bits: int, group: int, fmt: str) -> dict:
    """Codes of W D^{1/2} in format ``fmt``.  Returns ``codes`` (uint8, the
    stored code), ``s`` (float32 [rows, G]) and the format's own group term:
    ``m`` (asym minimum), ``z`` (intzp zero point), else nothing."""
    if fmt == "asym":
        q, s, m = encode_groups_fp32(W32, dh32, bits, group)
        return dict(codes=q, s=s, m=m)
    if fmt == "sym":
        k, s = encode_sym_fp32(W32, dh32, bits, group)
        return dict(codes=(k + (2 ** (bits - 1) - 1)).astype(np.uint8), s=s)
    if fmt == "intzp":
        q, s, z = encode_intzp_fp32(W32, dh32, bits, group)
        return dict(codes=q, s=s, z=z)
    if fmt == "fp8":
        if bits != 8:
            raise ValueError("fp8 codes are 8 bits wide")
        v, s = encode_fp8_fp32(W32, dh32, group)
        return dict(codes=e4m3_encode(v), s=s)
    raise ValueError(f"unknown format {fmt!r}")


def reconstruct_format(codes, s, bits: int, group: int, fmt: str, m=None,
                       z=None) -> np.ndarray:
    """u_hat (before D^{-1/2}) from stored codes, float64, by each format's
    definition."""
    codes = np.asarray(codes)
    rows, d = codes.shape
    G = d // group
    s64 = np.asarray(s, dtype=np.float64)[:, :, None]
    c = codes.reshape(rows, G, group)
    if fmt == "asym":
        v = np.asarray(m, dtype=np.float64)[:, :, None] + s64 * c.astype(np.float64)
    elif fmt == "sym":
        v = s64 * (c.astype(np.float64) - (2 ** (bits - 1) - 1))
    elif fmt == "intzp":
        v = s64 * (c.astype(np.float64) + np.asarray(z, dtype=np.float64)[:, :, None])
    elif fmt == "fp8":
        v = s64 * e4m3_decode(c)
    else:
        raise ValueError(f"unknown format {fmt!r}")
    return v.reshape(rows, d)


def format_offsets(s, bits: int, fmt: str, m=None, z=None) -> np.ndarray:
    """The float32 per-group offset o with u_hat = o + s code for the integer
    formats (asym: the minimum; sym: -fl(Z s); intzp: fl(z s)); 0 for fp8.
    This is the group term the library exports and stores beside the scales."""
    s = np.asarray(s, dtype=np.float32)
    if fmt == "asym":
        return np.asarray(m, dtype=np.float32)
    if fmt == "sym":
        return -(np.float32(2 ** (bits - 1) - 1) * s)
    if fmt == "intzp":
        return np.asarray(z).astype(np.float32) * s
    if fmt == "fp8":
        return np.zeros_like(s)
    raise ValueError(f"unknown format {fmt!r}")


def format_levels(codes, bits: int, fmt: str, z=None, group: int = 1):
    """Signed levels in units of s (the value the rounding decided):
    asym code; sym code - Z; intzp code + z; fp8 the E4M3 value."""
    c = np.asarray(codes)
    if fmt == "asym":
        return c.astype(np.float64)
    if fmt == "sym":
        return c.astype(np.float64) - (2 ** (bits - 1) - 1)
    if fmt == "intzp":
        zz = np.repeat(np.asarray(z, dtype=np.float64), group, axis=1)
        return c.astype(np.float64) + zz
    return e4m3_decode(c)


def pre_rounding_format_fp64(W64, dh64, bits: int, group: int, fmt: str):
    """float64 pre-rounding value in level units for each format (u/s for the
    formats without a real minimum, (u - min)/s for asym).  Returns t [rows, d]."""
    if fmt == "asym":
        return pre_rounding_fp64(W64, dh64, bits, group)[0]
    W64 = np.asarray(W64, dtype=np.float64)
    rows, d = W64.shape
    G = d // group
    u = (W64 * np.asarray(dh64)[None, :]).reshape(rows, G, group)
    if fmt == "sym":
        s = np.abs(u).max(axis=2) / (2 ** (bits - 1) - 1)
    elif fmt == "intzp":
        lo = np.minimum(u.min(axis=2), 0.0)
        hi = np.maximum(u.max(axis=2), 0.0)
        s = (hi - lo) / (2 ** bits - 1)
    elif fmt == "fp8":
        s = np.abs(u).max(axis=2) / E4M3_MAX
    else:
        raise ValueError(f"unknown format {fmt!r}")
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(s[:, :, None] > 0, u / s[:, :, None], 0.0)
    return t.reshape(rows, d)


def band_excused_levels(lv_gpu, lv_ref, t64, rel: float = 1e-6):
    """Band rule in level units for any format: a mismatch is excused iff the
    two levels are neighbours on the format's grid (no level between them:
    distance 1 for the integer formats, adjacent E4M3 values for fp8) and
    the float64 pre-rounding value lies within ``rel * max(|t*|, 1)`` of
    their midpoint.  Returns ``(n_mismatch, n_excused)``."""
    a = np.asarray(lv_gpu, dtype=np.float64)
    b = np.asarray(lv_ref, dtype=np.float64)
    bad = a != b
    nb = int(bad.sum())
    if nb == 0:
        return 0, 0
    lo = np.minimum(a, b)
    hi = np.maximum(a, b)
    vals, _ = _e4m3_nonneg_grid()
    grid = np.concatenate([-vals[:0:-1], vals])
    ilo = np.searchsorted(grid, lo)
    ihi = np.searchsorted(grid, hi)
    on_grid = (np.take(grid, np.minimum(ilo, len(grid) - 1)) == lo) & \
        (np.take(grid, np.minimum(ihi, len(grid) - 1)) == hi)
    integer = (lo == np.rint(lo)) & (hi == np.rint(hi))
    neighbours = (integer & (hi - lo == 1)) | (on_grid & (ihi - ilo == 1))
    mid = 0.5 * (lo + hi)
    t = np.asarray(t64, dtype=np.float64)
    near = np.abs(t - mid) <= rel * np.maximum(np.abs(t), 1.0)
    return nb, int((bad & neighbours & near).sum())


# --------------------------------------------------------------------------
# low-rank factors by PCA: [NL] Sec. 2 (static factors initialised by PCA,
# dynamic adaptation supported), [IT] Sec. 2 (B, A static or adapted online by
# PCA), [ZH] Sec. 2.2 (B, A statically initialised, e.g. by PCA).  The pages
# give no algorithm.  Readings:
#   * the principal subspace is that of the output rows: B (d' x r) is an
#     orthonormal basis of the top-r left singular subspace of M, and
#     A = B^T W, so B A = B B^T W is the rank-r PCA projection of W;
#   * M = W for the static initialisation; online, M = W D^{1/2} with D from
#     the current activations (the activation-aware principal directions);
#   * the residual W - B A is what the quantizer sees (reading 6);
#   * the subspace is found by randomized subspace iteration (Halko,
#     Martinsson and Tropp, "Finding structure with randomness", 2011: range
#     finder with q power iterations), the Gaussian test matrix Omega (d x r)
#     given by the caller; every orthonormalisation is a QR factorisation with
#     a positive diagonal of R (so Q is unique for full-rank input).
# --------------------------------------------------------------------------
def orthonormalize(Y: np.ndarray) -> np.ndarray:
    """Q of the QR factorisation Y = Q R with diag(R) > 0, float64."""
    Q, R = np.linalg.qr(np.asarray(Y, dtype=np.float64))
    sgn = np.sign(np.diag(R))
    sgn[sgn == 0] = 1.0
    return Q * sgn[None, :]


def subspace_iteration(M: np.ndarray, Omega: np.ndarray, iters: int) -> np.ndarray:
    """Orthonormal basis (d' x r) of the range of M after ``iters`` power
    iterations from Y = M Omega: Q = orth(M Omega); then ``iters`` times
    Z = orth(M^T Q), Q = orth(M Z)."""
    M = np.asarray(M, dtype=np.float64)
    Q = orthonormalize(M @ np.asarray(Omega, dtype=np.float64))
    for _ in range(iters):
        Z = orthonormalize(M.T @ Q)
        Q = orthonormalize(M @ Z)
    return Q


def lowrank_pca(W_bits: np.ndarray, Omega: np.ndarray, iters: int, *,
                X_bits: Optional[np.ndarray] = None, p: float = 2.0,
                lam: float = 0.0, alpha: float = 0.0) -> dict:
    """Low-rank factors of W by PCA.  Returns ``B`` (d' x r), ``A`` (r x d),
    ``R`` = W - B A (all float64) and ``M`` (the matrix whose principal
    subspace was taken).  With ``X_bits`` ([T, d] bf16) the online variant:
    M = W D^{1/2}, D from X with (p, lam, alpha) as in ``ttq_linear``."""
    W = bf16_to_f64(W_bits)
    M = W
    if X_bits is not None:
        n = channel_norms(bf16_to_f64(X_bits), p)
        dh, _ = diag_scales(n, lam, alpha)
        M = W * dh[None, :]
    B = subspace_iteration(M, Omega, iters)
    A = B.T @ W
    return dict(B=B, A=A, R=W - B @ A, M=M)


def pca_exact(M: np.ndarray, r: int) -> np.ndarray:
    """Exact top-r left singular vectors of M (numpy SVD), float64."""
    U, _, _ = np.linalg.svd(np.asarray(M, dtype=np.float64), full_matrices=False)
    return U[:, :r]


def overhead_ratio(d_out: int, T: int) -> float:
    """The pages' relative overhead of the online statistics, 1/d' + 3/T
    ([ZH] Sec. 2.3)."""
    return 1.0 / d_out + 3.0 / T if T > 0 else math.inf
