"""Parity at the full sizes of the standard workloads, on sampled outputs.

Every workload is run at its real shape on the GPU, twice:
  * without exports: the launch configuration the benchmark times (for one
    token, the single-launch kernel instantiation without export stores);
    Y is checked on the sampled output channels, all tokens;
  * with codes / scales / minimums / D^{1/2} exported: the same bars as the
    reduced-shape tests (D^{1/2} within one float32 ulp, codes strict against
    the kernel's own D^{1/2}, contract band rule against the oracle's own
    statistics, Y bars) on the sampled channels.
The oracle computes the statistics from the full activations and quantizes
only the sampled weight rows (rows are independent once D is fixed).
"""
import numpy as np
import pytest

from workloads import configs as wc
from parity_util import run_gpu, check_problem

pytestmark = pytest.mark.gpu

N_ROWS = 48


def sample_rows(d_out, seed):
    rng = np.random.default_rng(seed)
    rows = rng.choice(d_out, size=min(N_ROWS, d_out), replace=False)
    return np.unique(np.concatenate([rows, [0, d_out - 1]]))


def _say(tag, rep):
    print(f"[fullsize] {tag}: " + " ".join(f"{k}={v:.3g}" if isinstance(v, float)
                                          else f"{k}={v}" for k, v in rep.items()),
          flush=True)


def _check(prob):
    print(f"[case] {prob.name} d={prob.d} d_out={prob.d_out} T={prob.T} "
          f"R={prob.R} b={prob.bits} g={prob.group} r={prob.rank} p={prob.p}",
          flush=True)
    rows = sample_rows(prob.d_out, 1234 + prob.d_out + prob.T)
    plain = run_gpu(prob, exports=False, rows=rows)
    rep = check_problem(prob, plain, rows=rows, check_codes=False)
    _say(prob.name + " (no exports)", rep)
    full = run_gpu(prob, exports=True, rows=rows)
    rep = check_problem(prob, full, rows=rows)
    _say(prob.name + " (exports)", rep)
    # the two launches compute the same Y up to the fp32 summation order (the
    # one-token kernel's export instantiation splits the contraction over 8
    # instead of 16 waves): error per element relative to max(|Y|, RMS of the
    # token's row), the scale of the Y bars
    yp, yf = np.asarray(plain["Y"], np.float64), np.asarray(full["Y"], np.float64)
    rms = np.sqrt(np.mean(yf * yf, axis=-1, keepdims=True))
    e = np.abs(yp - yf) / np.maximum(np.maximum(np.abs(yf), rms), 1e-30)
    assert e.max() <= 1e-4, e.max()


@pytest.mark.parametrize("T", [1, 128])
def test_c2_q_proj(T):
    _check(wc.make_c2(T))


@pytest.mark.parametrize("which", ["gate_up", "down"])
def test_c3_mlp_prefill(which):
    _check(wc.make_c3(which))


@pytest.mark.parametrize("p", [1.0, 2.0])
def test_c4_up_proj(p):
    _check(wc.make_c4(p))


# all three projection shapes (square, 4096 -> 11008, 11008 -> 4096) at
# every token count of the layer
@pytest.mark.parametrize("T,proj", [(1, "q_proj"), (1, "gate_proj"),
                                    (1, "down_proj"),
                                    (16, "gate_proj"), (16, "k_proj"),
                                    (16, "down_proj"),
                                    (256, "down_proj"), (256, "up_proj"),
                                    (256, "v_proj"), (4096, "o_proj"),
                                    (4096, "gate_proj"), (4096, "down_proj")])
def test_c5_layer_requests(T, proj):
    _check(wc.make_c5(T, proj))
