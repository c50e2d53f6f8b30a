"""Continuous batching on the GPU: requests of different lengths packed in one
X, each with its own statistics (``ttq_linear_segmented``).

Every request's Y rows, codes, scales, minima and D^{1/2} must equal, bit for
bit, those of ``ttq_linear`` on that request alone (itself held to the oracle
by the other parity tests), and two requests are also checked against the
oracle directly.  The lengths cover every length class (one token, 2..16,
17..32 / 33..64 / 65..128 padded runs, longer requests alone), empty
requests, runs of equal lengths (no copies) and of mixed lengths (padded
through workspace copies).
"""
import dataclasses

import numpy as np
import pytest

from parity_util import check_problem, to_dev
from workloads import make_problem
from workloads.configs import draw_x

pytestmark = pytest.mark.gpu

LENGTHS = [1, 5, 1, 16, 0, 33, 130, 1, 1, 7, 64, 20, 300, 2]


def _problem(d_out, group, rank, seed):
    base = make_problem("seg", d=512, d_out=d_out, T=1, bits=4, group=group,
                        rank=rank, seed=seed)
    xs = [draw_x(seed + 100 + i, 0, 1, t, 512, "logu10_100", 5)[0]
          for i, t in enumerate(LENGTHS)]
    return base, xs


def _run_single(base, X, flags=0, exports=True):
    import torch
    import online_activation_aware_ttq_amd as ttq
    W = to_dev(base.W)
    Bm = to_dev(base.B) if base.rank else None
    A = to_dev(base.A) if base.rank else None
    dev = W.device
    T = X.shape[0]
    G = base.d // base.group
    Xd = to_dev(X) if T > 0 else torch.empty((0, base.d), dtype=torch.bfloat16, device=dev)
    kw = {}
    if exports:
        kw = dict(codes_out=torch.empty((base.d_out, base.d), dtype=torch.uint8, device=dev),
                  scales_out=torch.empty((base.d_out, G), dtype=torch.float32, device=dev),
                  mins_out=torch.empty((base.d_out, G), dtype=torch.float32, device=dev),
                  dhalf_out=torch.empty((base.d,), dtype=torch.float32, device=dev))
    Y = ttq.ttq_linear(W, Xd, Bm, A, p=base.p, lam=base.lam, alpha=base.alpha,
                       bits=base.bits, group=base.group, flags=flags, **kw)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in dict(Y=Y, **kw).items()}


def _run_segmented(base, xs, exports, flags=0):
    import torch
    import online_activation_aware_ttq_amd as ttq
    W = to_dev(base.W)
    Bm = to_dev(base.B) if base.rank else None
    A = to_dev(base.A) if base.rank else None
    dev = W.device
    offs = np.concatenate([[0], np.cumsum([x.shape[0] for x in xs])]).tolist()
    X = to_dev(np.concatenate(xs, axis=0))
    n = len(xs)
    G = base.d // base.group
    kw = {}
    if exports:
        kw = dict(codes_out=torch.empty((n, base.d_out, base.d), dtype=torch.uint8, device=dev),
                  scales_out=torch.empty((n, base.d_out, G), dtype=torch.float32, device=dev),
                  mins_out=torch.empty((n, base.d_out, G), dtype=torch.float32, device=dev),
                  dhalf_out=torch.empty((n, base.d), dtype=torch.float32, device=dev))
    Y = ttq.ttq_linear_segmented(W, X, Bm, A, seg_offsets=offs, p=base.p,
                                 lam=base.lam, alpha=base.alpha, bits=base.bits,
                                 group=base.group, flags=flags, **kw)
    torch.cuda.synchronize()
    return offs, {k: v.cpu().numpy() for k, v in dict(Y=Y, **kw).items()}


@pytest.mark.parametrize("d_out,group,rank,exports", [
    (272, 128, 32, True),     # 16-byte output rows, low rank, exports
    (270, 64, 0, False),      # 4-byte output rows, the no-export kernels
    (272, 32, 16, False),
])
def test_segments_equal_single_requests(d_out, group, rank, exports):
    base, xs = _problem(d_out, group, rank, seed=70 + group)
    print(f"[case] segmented d_out={d_out} g={group} r={rank} exports={exports} "
          f"lengths={LENGTHS}", flush=True)
    offs, seg = _run_segmented(base, xs, exports)
    for i, x in enumerate(xs):
        # (the kernels that also write codes are other instantiations: Y is
        # compared with the single call of the same kind)
        one = _run_single(base, x, exports=exports)
        a, b = offs[i], offs[i + 1]
        np.testing.assert_array_equal(seg["Y"][a:b].view(np.uint32),
                                      one["Y"].view(np.uint32), err_msg=f"request {i}")
        if exports:
            np.testing.assert_array_equal(seg["codes_out"][i], one["codes_out"])
            for k in ("scales_out", "mins_out", "dhalf_out"):
                np.testing.assert_array_equal(seg[k][i].view(np.uint32),
                                              one[k].view(np.uint32),
                                              err_msg=f"request {i} {k}")
    # two requests against the oracle directly (a padded short one, a long one)
    for i in (1, 12):
        prob = dataclasses.replace(base, T=xs[i].shape[0], X=xs[i][None])
        gpu = {"Y": seg["Y"][offs[i]:offs[i + 1]][None]}
        rep = check_problem(prob, gpu, check_codes=False)
        print(f"[parity] segment {i} T={xs[i].shape[0]}: y_max={rep['y_max']:.3g} "
              f"y_mean={rep['y_mean']:.3g}", flush=True)


def test_segments_with_a_path_flag_run_alone():
    base, xs = _problem(272, 128, 32, seed=91)
    flags = 2  # TTQ_FLAG_FORCE_TWO_PHASE
    offs, seg = _run_segmented(base, xs, exports=False, flags=flags)
    for i in (0, 1, 6, 12):
        one = _run_single(base, xs[i], flags=flags, exports=False)
        np.testing.assert_array_equal(seg["Y"][offs[i]:offs[i + 1]].view(np.uint32),
                                      one["Y"].view(np.uint32), err_msg=f"request {i}")


def test_all_requests_empty_or_one_token():
    """Only empty requests and single tokens: one batched one-token launch per
    run of consecutive single tokens, nothing for the empty ones."""
    import online_activation_aware_ttq_amd as ttq
    base, _ = _problem(272, 128, 0, seed=93)
    lengths = [0, 1, 1, 1, 0, 0, 1]
    xs = [draw_x(200 + i, 0, 1, t, 512, "logu10_100", 5)[0] for i, t in enumerate(lengths)]
    offs, seg = _run_segmented(base, xs, exports=False)
    assert seg["Y"].shape == (4, 272)
    for i, x in enumerate(xs):
        if x.shape[0]:
            one = _run_single(base, x, exports=False)
            np.testing.assert_array_equal(seg["Y"][offs[i]:offs[i + 1]].view(np.uint32),
                                          one["Y"].view(np.uint32))
    # the workspace covers both plans: with exports, runs of consecutive
    # requests (the three single tokens, each empty request alone, the last
    # token alone; an empty request still needs its statistics workspace in
    # case codes are asked for); without, requests grouped by length (the
    # four single tokens in one batch, gathered into padded X and Y copies)
    def ws(T, R):
        return ttq.ttq_workspace_bytes(
            ttq.make_params(d=512, d_out=272, T=T, bits=4, group=128, p=2.0,
                            lam=1e-3, alpha=0.5), R)

    def up(n):
        return -(-n // 256) * 256
    prm = ttq.make_params(d=512, d_out=272, T=4, bits=4, group=128, p=2.0,
                          lam=1e-3, alpha=0.5)
    gathered = up(ws(1, 4)) + up(4 * 1 * 512 * 2) + up(4 * 1 * 272 * 4)
    assert ttq.ttq_segmented_workspace_bytes(prm, offs) == max(ws(1, 3), ws(0, 1),
                                                               ws(1, 1), gathered)
