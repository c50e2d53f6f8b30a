"""The allocation-free entry point ttq_linear_noalloc, called through the C
ABI, against the workspace-taking entry point ttq_linear_batched on the same
inputs: several calls in a row on the library's static scratch, each later
call smaller than the one before, over the statistics-split path with
quantization inside the GEMM (with and without exports), the fused path and
the one-token path.  Both entry points run the same kernels with the same
plan, so the outputs must agree bit for bit."""
import ctypes

import numpy as np
import pytest

import online_activation_aware_ttq_amd as ttq
from workloads import make_problem

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

# (d, d_out, T, R, rank, bits, group, exports), largest first
CASES = [
    (4096, 1024, 200, 2, 32, 4, 128, False),
    (2048, 768, 160, 2, 16, 3, 64, True),
    (1024, 512, 48, 2, 16, 4, 128, True),
    (512, 256, 1, 1, 0, 4, 128, False),
]


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(
        torch.bfloat16)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


@pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
def test_noalloc_equals_workspace_entry_point_on_consecutive_calls():
    lib = ttq.load_library()
    stream = torch.cuda.current_stream().cuda_stream
    for i, (d, d_out, T, R, rank, bits, group, exports) in enumerate(CASES):
        print(f"noalloc case {i}: d={d} d_out={d_out} T={T} R={R} r={rank}",
              flush=True)
        prob = make_problem(f"na{i}", d=d, d_out=d_out, T=T, R=R, bits=bits,
                            group=group, rank=rank, seed=900 + i,
                            x_kind="logu10_100", n_outliers=max(1, d // 100))
        W, X = _dev(prob.W), _dev(prob.X)
        B = _dev(prob.B) if rank else None
        A = _dev(prob.A) if rank else None
        G = d // group
        kw = dict(p=prob.p, lam=prob.lam, alpha=prob.alpha, bits=bits,
                  group=group)

        def outs():
            if not exports:
                return None, None, None, None
            return (torch.empty(R, d_out, d, dtype=torch.uint8, device="cuda"),
                    torch.empty(R, d_out, G, dtype=torch.float32, device="cuda"),
                    torch.empty(R, d_out, G, dtype=torch.float32, device="cuda"),
                    torch.empty(R, d, dtype=torch.float32, device="cuda"))

        rc, rs, rm, rd = outs()
        Yref = ttq.ttq_linear_batched(W, X, B, A, codes_out=rc, scales_out=rs,
                                      mins_out=rm, dhalf_out=rd, **kw)
        prm = ttq.make_params(d=d, d_out=d_out, T=T, rank=rank, bits=bits,
                              group=group, p=prob.p, lam=prob.lam,
                              alpha=prob.alpha)
        Y = torch.full((R, T, d_out), float("nan"), dtype=torch.float32,
                       device="cuda")
        c, s, m, dh = outs()
        st = lib.ttq_linear_noalloc(ctypes.byref(prm), R, _ptr(W), _ptr(X),
                                    _ptr(B), _ptr(A), _ptr(Y), _ptr(c), _ptr(s),
                                    _ptr(m), _ptr(dh), ctypes.c_void_p(stream))
        assert st == ttq.TTQ_OK, ttq.ttq_status_string(st)
        torch.cuda.synchronize()
        assert torch.equal(Y, Yref), f"case {i}: Y differs"
        if exports:
            assert torch.equal(c, rc) and torch.equal(s, rs)
            assert torch.equal(m, rm) and torch.equal(dh, rd)


@pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
def test_noalloc_rejects_calls_beyond_the_scratch_size():
    lib = ttq.load_library()
    # the quantize pass + GEMM path keeps one bf16 W_hat per request: 8 of
    # 4096 x 11008 need far more than the scratch holds
    prm = ttq.make_params(d=4096, d_out=11008, T=4096, rank=32, bits=4,
                          group=128, p=2.0, lam=1e-3, alpha=0.5)
    assert ttq.ttq_workspace_bytes(prm, 8) > ttq.TTQ_NOALLOC_SCRATCH_BYTES
    st = lib.ttq_linear_noalloc(ctypes.byref(prm), 8, *([ctypes.c_void_p(16)] * 5),
                                None, None, None, None, None)
    assert st == ttq.TTQ_EWORKSPACE
