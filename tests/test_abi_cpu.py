"""Host-side tests of the C ABI (no GPU needed, no kernel is launched).

The library is loaded, every entry point include/ttq.h declares must be
exported, and every validation error is forced from the host: all of these
calls return before the library makes any HIP call.
"""
import ctypes
import os
import re

import pytest

import online_activation_aware_ttq_amd as ttq
from online_activation_aware_ttq_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ttq.h")

FAKE = 0x7f0000000000  # 256-byte aligned, never dereferenced by validation


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ttq_[a-z_]+)\s*\(", src)))


def lib():
    return ttq.load_library()


def prm(**kw):
    base = dict(d=256, d_out=64, T=16, rank=0, bits=4, group=128, p=2.0,
                lam=1e-3, alpha=0.5, flags=0)
    base.update(kw)
    return ttq.make_params(**base)


def call_linear(p, W=FAKE, X=FAKE, Bm=None, A=None, Y=FAKE, codes=None,
                scales=None, mins=None, dh=None, ws=FAKE, ws_bytes=1 << 40,
                R=None):
    L = lib()
    args = [W, X, Bm, A, Y, codes, scales, mins, dh, ws, ws_bytes, None]
    if R is None:
        return L.ttq_linear(ctypes.byref(p) if p is not None else None, *args)
    return L.ttq_linear_batched(ctypes.byref(p) if p is not None else None, R,
                                *args)


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 12
    L = lib()
    for n in names:
        assert hasattr(L, n), n
        assert n in B.EXPORTS, f"binding lacks a signature for {n}"
    assert set(B.EXPORTS) == set(names)


def test_params_struct_matches_header_layout():
    assert ctypes.sizeof(ttq.ttq_params) == 8 * 4 + 4 * 2 + 8 * 3 + 4 * 2
    assert ttq.ttq_params.p.offset == 40 and ttq.ttq_params.flags.offset == 64


def test_status_strings_and_version():
    for st in (0, -1, -2, -3, -4, -5, -100, 12345):
        s = ttq.ttq_status_string(st)
        assert isinstance(s, str) and s
    assert ttq.ttq_status_string(-4).startswith("workspace")
    assert "gfx950" in ttq.ttq_version()


@pytest.mark.parametrize("kw,status", [
    (dict(bits=0), ttq.TTQ_EINVAL),
    (dict(bits=9), ttq.TTQ_EINVAL),
    (dict(d=0), ttq.TTQ_EINVAL),
    (dict(d=-1), ttq.TTQ_EINVAL),
    (dict(d_out=-1), ttq.TTQ_EINVAL),
    (dict(T=-1), ttq.TTQ_EINVAL),
    (dict(rank=-1), ttq.TTQ_EINVAL),
    (dict(group=0), ttq.TTQ_EINVAL),
    (dict(d=256, group=96), ttq.TTQ_EINVAL),        # does not divide d
    (dict(d=256, group=16), ttq.TTQ_EUNSUPPORTED),  # divides, not supported
    (dict(p=0.0), ttq.TTQ_EINVAL),
    (dict(p=-2.0), ttq.TTQ_EINVAL),
    (dict(p=float("nan")), ttq.TTQ_EINVAL),
    (dict(p=float("inf")), ttq.TTQ_EINVAL),
    (dict(lam=-1e-3), ttq.TTQ_EINVAL),
    (dict(lam=float("inf")), ttq.TTQ_EINVAL),
    (dict(alpha=-0.5), ttq.TTQ_EINVAL),
    (dict(alpha=float("nan")), ttq.TTQ_EINVAL),
    (dict(rank=12), ttq.TTQ_EUNSUPPORTED),
    (dict(rank=2048), ttq.TTQ_EUNSUPPORTED),
    (dict(flags=3), ttq.TTQ_EINVAL),
    (dict(flags=4), ttq.TTQ_EINVAL),
    (dict(T=129, flags=1), ttq.TTQ_EUNSUPPORTED),
    (dict(qformat=4), ttq.TTQ_EINVAL),
    (dict(qformat=1, bits=1), ttq.TTQ_EINVAL),  # symmetric needs b >= 2
    (dict(qformat=3, bits=4), ttq.TTQ_EINVAL),  # E4M3 codes are 8 bits
])
def test_invalid_params_rejected_everywhere(kw, status):
    p = prm(**kw)
    out = ctypes.c_size_t(7)
    assert lib().ttq_workspace_bytes(ctypes.byref(p), 1, ctypes.byref(out)) == status
    assert out.value == 7
    assert lib().ttq_path(ctypes.byref(p), 1) == status
    assert call_linear(p) == status
    assert call_linear(p, R=2) == status


def test_valid_edge_params_accepted():
    for kw in (dict(bits=1), dict(bits=8), dict(group=32, d=32), dict(d_out=0),
               dict(T=0), dict(rank=8), dict(rank=1024), dict(alpha=0.0),
               dict(lam=0.0), dict(p=0.37), dict(group=256, d=512),
               dict(T=128, flags=1), dict(T=1, flags=2), dict(qformat=1, bits=2),
               dict(qformat=2, bits=1), dict(qformat=3, bits=8)):
        assert ttq.ttq_workspace_bytes(prm(**kw)) >= 0, kw


def test_format_names_map_to_the_header_values():
    assert ttq.QFORMATS == {"asym": 0, "sym": 1, "intzp": 2, "fp8": 3}
    assert ttq.make_params(d=128, d_out=1, T=1, bits=8, group=128, p=2.0,
                           lam=0.0, alpha=0.5, qformat="fp8").qformat == 3
    with pytest.raises(ValueError):
        ttq.qformat_code("int3")


def test_null_pointers():
    p = prm()
    assert lib().ttq_workspace_bytes(None, 1, ctypes.byref(ctypes.c_size_t())) == ttq.TTQ_ENULL
    assert lib().ttq_workspace_bytes(ctypes.byref(p), 1, None) == ttq.TTQ_ENULL
    assert call_linear(None) == ttq.TTQ_ENULL
    assert call_linear(p, W=None) == ttq.TTQ_ENULL
    assert call_linear(p, X=None) == ttq.TTQ_ENULL
    assert call_linear(p, Y=None) == ttq.TTQ_ENULL
    assert call_linear(p, ws=None) == ttq.TTQ_ENULL
    pr = prm(rank=8)
    assert call_linear(pr, Bm=FAKE, A=None) == ttq.TTQ_ENULL
    assert call_linear(pr, Bm=None, A=FAKE) == ttq.TTQ_ENULL
    # scales without mins (or the reverse) is a usage error
    assert call_linear(p, scales=FAKE) == ttq.TTQ_EINVAL
    assert call_linear(p, mins=FAKE) == ttq.TTQ_EINVAL


def test_alignment_rules():
    p = prm()
    assert call_linear(p, W=FAKE + 8) == ttq.TTQ_EALIGN
    assert call_linear(p, X=FAKE + 2) == ttq.TTQ_EALIGN
    assert call_linear(p, Y=FAKE + 2) == ttq.TTQ_EALIGN
    assert call_linear(p, codes=FAKE + 4) == ttq.TTQ_EALIGN
    assert call_linear(p, dh=FAKE + 1) == ttq.TTQ_EALIGN
    assert call_linear(p, ws=FAKE + 128) == ttq.TTQ_EALIGN
    pr = prm(rank=8)
    assert call_linear(pr, Bm=FAKE + 8, A=FAKE) == ttq.TTQ_EALIGN


def test_workspace_too_small():
    p = prm()
    need = ttq.ttq_workspace_bytes(p)
    assert need > 0
    assert call_linear(p, ws_bytes=need - 1) == ttq.TTQ_EWORKSPACE
    assert call_linear(p, ws_bytes=0) == ttq.TTQ_EWORKSPACE
    need2 = ttq.ttq_workspace_bytes(p, 3)
    assert need2 > need
    assert call_linear(p, ws_bytes=need2 - 1, R=3) == ttq.TTQ_EWORKSPACE


def test_zero_requests_is_a_no_op():
    p = prm()
    assert ttq.ttq_workspace_bytes(p, 0) == 0
    assert call_linear(p, W=None, X=None, Y=None, ws=None, ws_bytes=0, R=0) == ttq.TTQ_OK
    assert call_linear(p, R=-1) == ttq.TTQ_EINVAL


def test_injected_hip_error_is_reported(monkeypatch):
    monkeypatch.setenv("TTQ_INJECT_HIP_ERROR", "1")
    p = prm()
    assert call_linear(p) == ttq.TTQ_EHIP
    assert lib().ttq_last_hip_error() != 0
    with pytest.raises(ttq.TTQError) as ei:
        raise ttq.TTQError(ttq.TTQ_EHIP, "x")
    assert "hipError" in str(ei.value)


def test_path_selection():
    assert ttq.ttq_path(prm(T=1)) == 2
    assert ttq.ttq_path(prm(T=1, d=12288 + 128)) == 0
    assert ttq.ttq_path(prm(T=1, flags=ttq.TTQ_FLAG_FORCE_FUSED)) == 0
    assert ttq.ttq_path(prm(T=2)) == 0
    assert ttq.ttq_path(prm(T=128)) == 0
    assert ttq.ttq_path(prm(T=129)) == 3
    assert ttq.ttq_path(prm(T=256)) == 3
    assert ttq.ttq_path(prm(T=257)) == 1
    assert ttq.ttq_path(prm(T=129, group=256)) == 1
    assert ttq.ttq_path(prm(T=129, d=192, group=64)) == 1
    assert ttq.ttq_path(prm(T=129, flags=ttq.TTQ_FLAG_FORCE_TWO_PHASE)) == 1
    assert ttq.ttq_path(prm(T=2048)) == 1
    assert ttq.ttq_path(prm(T=2048, flags=ttq.TTQ_FLAG_FORCE_FUSED & 0)) == 1
    assert ttq.ttq_path(prm(T=64, flags=ttq.TTQ_FLAG_FORCE_TWO_PHASE)) == 1
    assert ttq.ttq_path(prm(T=100, flags=ttq.TTQ_FLAG_FORCE_FUSED)) == 0


def test_workspace_grows_with_shape():
    small = ttq.ttq_workspace_bytes(prm(T=1))
    big = ttq.ttq_workspace_bytes(prm(T=2048, d_out=11008, rank=64))
    assert big > small
    # the two-phase path holds the dequantized bf16 weights
    assert big >= 11008 * 256 * 2


def test_gemm_quantizing_path_reserves_no_dequantized_weights():
    # 8 requests of 256 tokens on an 8192 -> 28672 projection: the path that
    # quantizes inside the GEMM needs statistics, Z and partial sums only,
    # far less than one request's bf16 W_hat (470 MB)
    p3 = prm(d=8192, d_out=28672, T=256, rank=128, group=64, bits=2)
    assert ttq.ttq_path(p3, 8) == 3
    ws = ttq.ttq_workspace_bytes(p3, 8)
    assert ws < 28672 * 8192 * 2 // 8
    # forcing the quantize pass brings W_hat back
    p1 = prm(d=8192, d_out=28672, T=256, rank=128, group=64, bits=2,
             flags=ttq.TTQ_FLAG_FORCE_TWO_PHASE)
    assert ttq.ttq_workspace_bytes(p1, 8) >= ws + 28672 * 8192 * 2


def test_noalloc_checks_size_before_touching_the_device():
    L = lib()
    # validation as for the batched call
    assert L.ttq_linear_noalloc(None, 1, *([None] * 9), None) == ttq.TTQ_ENULL
    assert L.ttq_linear_noalloc(ctypes.byref(prm(bits=9)), 1, *([None] * 9),
                                None) == ttq.TTQ_EINVAL
    assert L.ttq_linear_noalloc(ctypes.byref(prm()), 0, *([None] * 9),
                                None) == ttq.TTQ_OK
    # a plan beyond the static scratch is refused on the host
    big = prm(d=4096, d_out=11008, T=4096, rank=32)
    assert ttq.ttq_workspace_bytes(big, 8) > ttq.TTQ_NOALLOC_SCRATCH_BYTES
    assert L.ttq_linear_noalloc(ctypes.byref(big), 8, *([FAKE] * 5),
                                None, None, None, None, None) == ttq.TTQ_EWORKSPACE


def test_timing_api_without_launches():
    L = lib()
    n = L.ttq_kernel_count()
    assert n >= 5
    names = [L.ttq_kernel_name(k).decode() for k in range(n)]
    assert "fused_qdq_mfma" in names and "gemm_mfma" in names
    assert L.ttq_kernel_name(n) is None
    ttq.timing_reset()
    q = ttq.timing_query()
    assert all(v == (0.0, 0) for v in q.values())
    ms = ctypes.c_double()
    cnt = ctypes.c_int64()
    assert L.ttq_timing_query(-1, ctypes.byref(ms), ctypes.byref(cnt)) == ttq.TTQ_EINVAL


# ---------------------------------------------- quantize once / decode calls
def call_quantize(p, W=FAKE, X=FAKE, codes=FAKE, scales=FAKE, mins=FAKE,
                  dhi=FAKE, dh=None, ws=FAKE, ws_bytes=1 << 40):
    return lib().ttq_quantize(ctypes.byref(p) if p is not None else None, W, X,
                              codes, scales, mins, dhi, dh, ws, ws_bytes, None)


def call_qmatmul(p, codes=FAKE, scales=FAKE, mins=FAKE, dhi=FAKE, X=FAKE,
                 Bm=None, A=None, Y=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return lib().ttq_qmatmul(ctypes.byref(p) if p is not None else None,
                             codes, scales, mins, dhi, X, Bm, A, Y, ws,
                             ws_bytes, None)


@pytest.mark.parametrize("bits,d,row_bytes", [
    (4, 256, 128), (3, 256, 128), (8, 256, 256), (5, 4096, 4096),
    (2, 256, 64), (1, 256, 32), (4, 4096, 2048), (2, 4096, 1024),
])
def test_packed_row_bytes(bits, d, row_bytes):
    assert B.container_bits(bits) * d // 8 == row_bytes
    assert ttq.ttq_packed_row_bytes(prm(bits=bits, d=d)) == row_bytes


def test_packed_rows_must_fill_16_bytes():
    # 1-bit codes of 64 channels are 8 bytes a row: not supported
    p = prm(bits=1, d=64, group=32)
    out = ctypes.c_int64(-7)
    assert lib().ttq_packed_row_bytes(ctypes.byref(p), ctypes.byref(out)) == ttq.TTQ_EUNSUPPORTED
    assert out.value == -7
    assert call_quantize(p) == ttq.TTQ_EUNSUPPORTED
    assert call_qmatmul(p) == ttq.TTQ_EUNSUPPORTED
    # 2-bit codes of 64 channels are 16 bytes: fine
    assert ttq.ttq_packed_row_bytes(prm(bits=2, d=64, group=32)) == 16


@pytest.mark.parametrize("kw,status", [
    (dict(bits=0), ttq.TTQ_EINVAL),
    (dict(bits=9), ttq.TTQ_EINVAL),
    (dict(d=0), ttq.TTQ_EINVAL),
    (dict(d_out=-1), ttq.TTQ_EINVAL),
    (dict(T=-1), ttq.TTQ_EINVAL),
    (dict(d=256, group=96), ttq.TTQ_EINVAL),
    (dict(d=256, group=16), ttq.TTQ_EUNSUPPORTED),
])
def test_packed_calls_validate_shapes(kw, status):
    p = prm(**kw)
    out = ctypes.c_size_t(7)
    assert lib().ttq_quantize_workspace_bytes(ctypes.byref(p), ctypes.byref(out)) == status
    assert lib().ttq_qmatmul_workspace_bytes(ctypes.byref(p), ctypes.byref(out)) == status
    assert out.value == 7
    assert call_quantize(p) == status
    assert call_qmatmul(p) == status


def test_quantize_checks_statistics_constants_only():
    # statistics constants are validated by ttq_quantize ...
    assert call_quantize(prm(p=0.0)) == ttq.TTQ_EINVAL
    assert call_quantize(prm(alpha=-1.0)) == ttq.TTQ_EINVAL
    # ... but rank and the path flags are not read (unknown flags still are)
    assert ttq.ttq_quantize_workspace_bytes(prm(rank=12, flags=3)) > 0
    assert call_quantize(prm(flags=4)) == ttq.TTQ_EINVAL
    # ttq_qmatmul does not read the statistics constants or FORCE_FUSED
    assert ttq.ttq_qmatmul_workspace_bytes(prm(p=0.0, alpha=-1.0, flags=1)) >= 0
    assert call_qmatmul(prm(rank=12)) == ttq.TTQ_EUNSUPPORTED
    assert call_qmatmul(prm(flags=4)) == ttq.TTQ_EINVAL


def test_packed_calls_null_and_alignment():
    p = prm()
    assert call_quantize(None) == ttq.TTQ_ENULL
    for k in ("W", "X", "codes", "scales", "mins", "dhi", "ws"):
        assert call_quantize(p, **{k: None}) == ttq.TTQ_ENULL, k
    for k, off in (("W", 8), ("X", 2), ("codes", 8), ("scales", 2),
                   ("mins", 2), ("dhi", 4), ("dh", 2), ("ws", 128)):
        assert call_quantize(p, **{k: FAKE + off}) == ttq.TTQ_EALIGN, k
    assert call_qmatmul(None) == ttq.TTQ_ENULL
    for k in ("codes", "scales", "mins", "dhi", "X", "Y"):
        assert call_qmatmul(p, **{k: None}) == ttq.TTQ_ENULL, k
    for k, off in (("codes", 8), ("scales", 2), ("mins", 2), ("dhi", 4),
                   ("X", 2), ("Y", 2), ("ws", 128)):
        assert call_qmatmul(p, **{k: FAKE + off}) == ttq.TTQ_EALIGN, k
    pr = prm(rank=8)
    assert call_qmatmul(pr) == ttq.TTQ_ENULL
    assert call_qmatmul(pr, Bm=FAKE, A=None) == ttq.TTQ_ENULL
    assert call_qmatmul(pr, Bm=FAKE + 8, A=FAKE) == ttq.TTQ_EALIGN


def test_packed_calls_workspace():
    p = prm(T=1, rank=8)
    need = ttq.ttq_qmatmul_workspace_bytes(p)
    assert need > 0
    assert call_qmatmul(p, Bm=FAKE, A=FAKE, ws_bytes=need - 1) == ttq.TTQ_EWORKSPACE
    # T <= 128: x' of the step (one bf16 plane of 64 tokens here)
    assert ttq.ttq_qmatmul_workspace_bytes(prm(T=64)) >= 64 * 256 * 2
    # larger T expands the codes inside the GEMM (no workspace without the
    # low-rank term); the forced route holds the expanded bf16 weights
    assert ttq.ttq_qmatmul_workspace_bytes(prm(T=200)) == 0
    assert ttq.ttq_qmatmul_workspace_bytes(
        prm(T=200, flags=ttq.TTQ_FLAG_FORCE_TWO_PHASE)) >= 64 * 256 * 2
    assert ttq.ttq_qmatmul_workspace_bytes(prm(T=8, flags=2)) >= 64 * 256 * 2
    assert ttq.ttq_qmatmul_workspace_bytes(prm(T=1)) == 0
    q = prm(T=2048)
    qneed = ttq.ttq_quantize_workspace_bytes(q)
    assert qneed >= 256 * 4
    assert call_quantize(q, ws_bytes=qneed - 1) == ttq.TTQ_EWORKSPACE


def test_packed_calls_report_injected_hip_error(monkeypatch):
    monkeypatch.setenv("TTQ_INJECT_HIP_ERROR", "1")
    assert call_quantize(prm()) == ttq.TTQ_EHIP
    assert call_qmatmul(prm()) == ttq.TTQ_EHIP


# ---------------------------------------------- requests of different lengths
def _offs(*v):
    arr = (ctypes.c_int64 * len(v))(*v)
    return ctypes.cast(arr, ctypes.c_void_p), arr


def seg_ws(p, offsets):
    ptr, _keep = _offs(*offsets)
    out = ctypes.c_size_t(0)
    st = lib().ttq_segmented_workspace_bytes(ctypes.byref(p), len(offsets) - 1,
                                             ptr, ctypes.byref(out))
    return st, out.value


def call_segmented(p, offsets, ws_bytes=1 << 40, n=None, Y=FAKE, ws=FAKE):
    ptr, _keep = _offs(*offsets) if offsets is not None else (None, None)
    n = len(offsets) - 1 if n is None else n
    return lib().ttq_linear_segmented(ctypes.byref(p), n, ptr, FAKE, FAKE,
                                      None, None, Y, None, None, None, None,
                                      ws, ws_bytes, None)


def test_segmented_offsets_validated():
    p = prm(T=7)
    assert seg_ws(p, [0, 3, 7])[0] == ttq.TTQ_OK
    assert seg_ws(p, [1, 3, 7])[0] == ttq.TTQ_EINVAL       # does not start at 0
    assert seg_ws(p, [0, 3, 6])[0] == ttq.TTQ_EINVAL       # does not end at T
    assert seg_ws(p, [0, 5, 3, 7])[0] == ttq.TTQ_EINVAL    # decreasing
    assert call_segmented(p, None, n=2) == ttq.TTQ_ENULL
    assert call_segmented(p, [0, 5, 3, 7]) == ttq.TTQ_EINVAL
    assert call_segmented(prm(T=7, bits=0), [0, 3, 7]) == ttq.TTQ_EINVAL


def test_segmented_no_requests_is_a_no_op():
    p = prm(T=0)
    assert seg_ws(p, [0]) == (ttq.TTQ_OK, 0)
    assert call_segmented(p, [0], ws=None, ws_bytes=0) == ttq.TTQ_OK


def test_segmented_workspace_plan():
    # equal lengths, consecutive: one batched call, no copies
    p = prm(T=3)
    st, need = seg_ws(p, [0, 1, 2, 3])
    assert st == ttq.TTQ_OK and need == ttq.ttq_workspace_bytes(prm(T=1), 3)
    # 1 token, then 5 and 16 tokens (one run, padded to 16 through copies)
    p = prm(T=22)
    st, need = seg_ws(p, [0, 1, 6, 22])
    batch = ttq.ttq_workspace_bytes(prm(T=16), 2)
    assert st == ttq.TTQ_OK and need > batch
    # a path flag: every request alone at its own length
    p = prm(T=22, flags=ttq.TTQ_FLAG_FORCE_TWO_PHASE)
    st, need = seg_ws(p, [0, 1, 6, 22])
    alone = max(ttq.ttq_workspace_bytes(prm(T=t, flags=ttq.TTQ_FLAG_FORCE_TWO_PHASE), 1)
                for t in (1, 5, 16))
    assert st == ttq.TTQ_OK and need == alone
    # the call checks the workspace against the plan before any launch
    st, need = seg_ws(prm(T=22), [0, 1, 6, 22])
    assert call_segmented(prm(T=22), [0, 1, 6, 22], ws_bytes=need - 1) == ttq.TTQ_EWORKSPACE
    assert call_segmented(prm(T=22), [0, 1, 6, 22], Y=None) == ttq.TTQ_ENULL


# ---------------------------------------------------------------- PCA factors
def _pca_prm(**kw):
    base = dict(d=256, d_out=128, T=0, rank=16, bits=4, group=32, p=2.0,
                lam=1e-3, alpha=0.5)
    base.update(kw)
    return ttq.make_params(**base)


@pytest.mark.parametrize("kw,iters,status", [
    (dict(rank=12), 2, ttq.TTQ_EUNSUPPORTED),
    (dict(rank=256, d=512, d_out=512), 2, ttq.TTQ_EUNSUPPORTED),
    (dict(rank=0), 2, ttq.TTQ_EINVAL),
    (dict(rank=16, d_out=8), 2, ttq.TTQ_EINVAL),       # rank > d_out
    (dict(rank=16), -1, ttq.TTQ_EINVAL),
    (dict(rank=16), 17, ttq.TTQ_EINVAL),
    (dict(d_out=0), 2, ttq.TTQ_EINVAL),
    (dict(T=-1), 2, ttq.TTQ_EINVAL),
    (dict(T=4, d=260), 2, ttq.TTQ_EUNSUPPORTED),       # token rows of 16 bytes
    (dict(T=4, p=0.0), 2, ttq.TTQ_EINVAL),
    (dict(T=4, alpha=-1.0), 2, ttq.TTQ_EINVAL),
])
def test_pca_validation(kw, iters, status):
    p = _pca_prm(**kw)
    out = ctypes.c_size_t(5)
    assert lib().ttq_lowrank_pca_workspace_bytes(ctypes.byref(p), iters,
                                                 ctypes.byref(out)) == status
    assert out.value == 5
    assert lib().ttq_lowrank_pca(ctypes.byref(p), iters, FAKE, FAKE, FAKE, FAKE,
                                 FAKE, None, FAKE, 1 << 40, None) == status


def test_pca_pointers_and_workspace():
    p = _pca_prm()
    need = ttq.ttq_lowrank_pca_workspace_bytes(p, 2)
    assert need > 0
    # bits / group / flags / qformat are not read; T = 0 needs no X
    assert ttq.ttq_lowrank_pca_workspace_bytes(_pca_prm(bits=1, group=7), 2) == need
    call = lambda **k: lib().ttq_lowrank_pca(
        ctypes.byref(k.get("p", p)), 2, k.get("W", FAKE), k.get("X", None),
        k.get("Om", FAKE), k.get("B", FAKE), k.get("A", FAKE), None,
        k.get("ws", FAKE), k.get("wsb", need), None)
    assert call(W=None) == ttq.TTQ_ENULL
    assert call(Om=None) == ttq.TTQ_ENULL
    assert call(B=None) == ttq.TTQ_ENULL
    assert call(A=None) == ttq.TTQ_ENULL
    assert call(ws=None) == ttq.TTQ_ENULL
    assert call(p=_pca_prm(T=4)) == ttq.TTQ_ENULL       # T > 0 needs X
    assert call(wsb=need - 1) == ttq.TTQ_EWORKSPACE
    assert call(W=FAKE + 8) == ttq.TTQ_EALIGN
    # online statistics need their own workspace
    assert ttq.ttq_lowrank_pca_workspace_bytes(_pca_prm(T=300), 2) > need


def test_stream_read_validation():
    # the measurement read validates on the host before anything is enqueued
    L = lib()
    sink = FAKE + 1024
    assert L.ttq_stream_read(FAKE, 0, None, None) == ttq.TTQ_OK       # nothing to read
    assert L.ttq_stream_read(FAKE, -16, sink, None) == ttq.TTQ_EINVAL
    assert L.ttq_stream_read(FAKE, 24, sink, None) == ttq.TTQ_EINVAL  # not a multiple of 16
    assert L.ttq_stream_read(None, 4096, sink, None) == ttq.TTQ_ENULL
    assert L.ttq_stream_read(FAKE, 4096, None, None) == ttq.TTQ_ENULL
    assert L.ttq_stream_read(FAKE + 8, 4096, sink, None) == ttq.TTQ_EALIGN
    assert L.ttq_stream_read(FAKE, 4096, sink + 2, None) == ttq.TTQ_EALIGN
