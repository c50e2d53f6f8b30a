"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding, run the oracle on the same bytes, compare.

Bars (written here, used by every parity test):
  * D^{1/2}: the kernel's float32 values against float32(oracle's float64).
  * codes, strict: the oracle's float32 decision fed the kernel's own D^{1/2}
    must reproduce every code, scale and minimum bit for bit.
  * codes, contract: against the oracle's own statistics, a mismatch is
    allowed only when the float64 pre-rounding value lies within 1e-6
    (relative to the operands of the subtraction) of the rounding boundary;
    such mismatches are counted and reported.
  * Y: e = |Y_gpu - Y_ref| / max(|Y_ref|, rms_t), rms_t the RMS of the
    reference token row over the checked outputs; max e <= 2e-2 and
    mean e <= 2e-3 against the float64-accumulated oracle.
"""
from __future__ import annotations

import numpy as np

import oracle

Y_MAX_REL = 2e-2
Y_MEAN_REL = 2e-3
BAND_REL = 1e-6


def to_dev(bits: np.ndarray, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def run_gpu(prob, flags: int = 0, exports: bool = True, rows=None):
    """Run one problem (R == 1 -> ttq_linear, else ttq_linear_batched)."""
    import torch
    import online_activation_aware_ttq_amd as ttq
    dev = torch.device("cuda")
    W = to_dev(prob.W)
    Bm = to_dev(prob.B) if prob.rank else None
    A = to_dev(prob.A) if prob.rank else None
    batched = prob.R != 1
    X = to_dev(prob.X if batched else prob.X[0])
    lead = (prob.R,) if batched else ()
    G = prob.d // prob.group
    out = {}
    kw = dict(p=prob.p, lam=prob.lam, alpha=prob.alpha, bits=prob.bits,
              group=prob.group, flags=flags)
    if prob.qformat != "asym":
        kw["qformat"] = prob.qformat
    if exports:
        kw.update(
            codes_out=torch.empty(lead + (prob.d_out, prob.d), dtype=torch.uint8, device=dev),
            scales_out=torch.empty(lead + (prob.d_out, G), dtype=torch.float32, device=dev),
            mins_out=torch.empty(lead + (prob.d_out, G), dtype=torch.float32, device=dev),
            dhalf_out=torch.empty(lead + (prob.d,), dtype=torch.float32, device=dev))
    fn = ttq.ttq_linear_batched if batched else ttq.ttq_linear
    Y = fn(W, X, Bm, A, **kw)
    torch.cuda.synchronize()
    sel = slice(None) if rows is None else torch.as_tensor(rows, device=dev)

    def host(t, row_axis):
        if t is None:
            return None
        if rows is not None:
            t = t.index_select(row_axis, sel)
        return t.cpu().numpy()

    ax = 1 if batched else 0
    out["Y"] = host(Y, Y.dim() - 1)
    if exports:
        out["q"] = host(kw["codes_out"], ax)
        out["s"] = host(kw["scales_out"], ax)
        out["m"] = host(kw["mins_out"], ax)
        out["dh"] = kw["dhalf_out"].cpu().numpy()
    if not batched:
        out = {k: (v[None] if v is not None else None) for k, v in out.items()}
    return out


def y_errors(Y_gpu: np.ndarray, Y_ref: np.ndarray):
    """Per-element relative error with the token-row RMS floor."""
    Y_gpu = np.asarray(Y_gpu, dtype=np.float64)
    if Y_ref.size == 0:
        return np.zeros(0), 0.0
    rms = np.sqrt(np.mean(Y_ref * Y_ref, axis=-1, keepdims=True))
    den = np.maximum(np.abs(Y_ref), rms)
    den = np.where(den > 0, den, 1.0)
    e = np.abs(Y_gpu - Y_ref) / den
    nw = np.linalg.norm(Y_gpu - Y_ref) / max(np.linalg.norm(Y_ref), 1e-300)
    return e, nw


def check_problem(prob, gpu: dict, rows=None, report: dict = None,
                  check_codes: bool = True):
    """Compare a GPU result with the oracle; assert every bar; fill report."""
    rep = report if report is not None else {}
    rep.update(dh_mismatch=0, strict_mismatch=0, contract_mismatch=0,
               contract_excused=0, literal_band=0, y_max=0.0, y_mean=0.0,
               y_normwise=0.0)
    sel = np.arange(prob.d_out) if rows is None else np.asarray(rows)
    W32 = oracle.bf16_to_f32(np.asarray(prob.W)[sel])
    for r in range(prob.R):
        fmt = prob.qformat
        ref = oracle.ttq_linear(
            prob.W, prob.X[r], bits=prob.bits, group=prob.group, p=prob.p,
            lam=prob.lam, alpha=prob.alpha, B_bits=prob.B, A_bits=prob.A,
            rows=sel, want_t=check_codes, qformat=fmt)
        if check_codes and "dh" in gpu:
            dh_gpu = gpu["dh"][r]
            mis = dh_gpu.view(np.uint32) != ref["dh32"].view(np.uint32)
            rep["dh_mismatch"] += int(mis.sum())
            if mis.any():  # never more than one float32 ulp apart
                ulps = np.abs(dh_gpu.view(np.int32).astype(np.int64)
                              - ref["dh32"].view(np.int32).astype(np.int64))
                assert ulps.max() <= 1, ulps.max()
            # strict: the oracle's float32 decision with the kernel's D^{1/2}
            if fmt == "asym":
                q_s, s_s, m_s = oracle.encode_groups_fp32(W32, dh_gpu, prob.bits,
                                                         prob.group)
            else:
                f = oracle.quantize_format(W32, dh_gpu, prob.bits, prob.group, fmt)
                q_s, s_s = f["codes"], f["s"]
                m_s = oracle.format_offsets(s_s, prob.bits, fmt, z=f.get("z"))
            n_strict = int((q_s != gpu["q"][r]).sum())
            rep["strict_mismatch"] += n_strict
            assert n_strict == 0, f"request {r}: {n_strict} code mismatches (strict)"
            np.testing.assert_array_equal(s_s.view(np.uint32), gpu["s"][r].view(np.uint32))
            np.testing.assert_array_equal(m_s.view(np.uint32), gpu["m"][r].view(np.uint32))
            # contract: against the oracle's own statistics, band rule
            if fmt == "asym":
                nb, ne, nl = oracle.band_excused(
                    gpu["q"][r], ref["q"], ref["t64"], ref["u64"], ref["m64"],
                    ref["s64"], prob.group, BAND_REL)
            else:
                z_gpu = None
                if fmt == "intzp":
                    with np.errstate(divide="ignore", invalid="ignore"):
                        z_gpu = np.where(s_s > 0, np.rint(gpu["m"][r].astype(np.float64)
                                                          / s_s), 0.0)
                lv_gpu = oracle.format_levels(gpu["q"][r], prob.bits, fmt, z=z_gpu,
                                              group=prob.group)
                lv_ref = oracle.format_levels(ref["q"], prob.bits, fmt,
                                              z=ref.get("z"), group=prob.group)
                nb, ne = oracle.band_excused_levels(lv_gpu, lv_ref, ref["t64"], BAND_REL)
                nl = 0
            rep["contract_mismatch"] += nb
            rep["contract_excused"] += ne
            rep["literal_band"] += nl
            assert nb == ne, f"request {r}: {nb - ne} unexcused code mismatches"
        if prob.T > 0 and len(sel) > 0:
            e, nw = y_errors(gpu["Y"][r], ref["Y"])
            rep["y_max"] = max(rep["y_max"], float(e.max()))
            rep["y_mean"] = max(rep["y_mean"], float(e.mean()))
            rep["y_normwise"] = max(rep["y_normwise"], float(nw))
            assert np.all(np.isfinite(gpu["Y"][r]))
            assert e.max() <= Y_MAX_REL, (r, e.max())
            assert e.mean() <= Y_MEAN_REL, (r, e.mean())
    return rep
