"""Why the intermediates between the stages stay fp32 (the fp16/bf16
intermediates option is rejected by this error analysis).

"Round 30 Track C Audit: gdn_pre, gdn_post, and gdn_scanr_4", section 1
(gdn_pre): the pre stage hands q, k, v and the gates to the scan as float4
vectors, i.e. fp32.  Storing them (and the scan's o) as fp16 would halve the
bytes between the stages; this module measures, with the oracle alone, what
that rounding does to the results the parity bars judge:

* the final state: per value head, relative Frobenius error against the
  unrounded run, bar 1e-4;
* y: absolute error, bar 2e-3 (fp32 output).

The same run with the intermediates rounded to fp32 (what the path stores)
stays far inside both bars, so the margin the fp32 intermediates leave is
measured too.  Inputs: the production-width T=512 workload (value heads 0, 17
and 40 only, to keep the CPU time short), its own seed and distributions.
"""
import numpy as np
import pytest

from gated_deltanet_linear_pre_amd import synth
from oracle import gdn_oracle as orc

HEADS = [0, 17, 40]
STATE_BAR = 1e-4
Y_BAR = 2e-3


def _run(dims, cu, pr, inp, cast):
    """Scan and post from the pre intermediates rounded through `cast`."""
    r = {k: cast(pr[k]) for k in ("qn", "kn", "vc", "g", "beta")}
    o, S = orc.scan(dims, cu, r["qn"], r["kn"], r["vc"], r["g"], r["beta"], inp["S0"],
                    heads=HEADS)
    o = cast(o)
    T = o.shape[0]
    z = np.asarray(inp["z"], np.float64).reshape(T, dims.hv, dims.dv)
    y = orc.post(o[:, HEADS, :], z[:, HEADS, :], inp["gamma"], 1e-6)
    return S[:, HEADS], y


def _state_err(S, S_ref):
    num = np.sqrt(((S - S_ref) ** 2).sum(axis=(-1, -2)))
    den = np.sqrt((S_ref ** 2).sum(axis=(-1, -2)))
    return float((num / den).max())


@pytest.fixture(scope="module")
def runs():
    w = synth.WORKLOADS["prod_t512_fp16"]
    inp = synth.layer_inputs(w)
    dims = orc.Dims(w.hk, w.hv)
    cu = w.cu_seqlens()
    pr = orc.pre(dims, cu, inp["qkv"], inp["conv_w"], inp["a"], inp["b"], inp["A_log"],
                 inp["dt_bias"], inp["hist"], 1e-6)
    exact = _run(dims, cu, pr, inp, lambda x: np.asarray(x, np.float64))
    f32 = _run(dims, cu, pr, inp, lambda x: np.asarray(x, np.float32).astype(np.float64))
    f16 = _run(dims, cu, pr, inp, lambda x: np.asarray(x, np.float16).astype(np.float64))
    return exact, f32, f16


def test_fp32_intermediates_stay_inside_the_bars(runs):
    (S, y), (S32, y32), _ = runs
    assert _state_err(S32, S) < STATE_BAR / 20
    assert np.abs(y32 - y).max() < Y_BAR / 20


def test_fp16_intermediates_break_the_state_bar(runs):
    (S, y), _, (S16, y16) = runs
    err = _state_err(S16, S)
    # fp16 keeps 11 significant bits: rounding q, k and v alone puts the
    # state error well above the 1e-4 bar
    assert err > STATE_BAR, err
    # and y moves by more than the fp32-output bar somewhere
    assert np.abs(y16 - y).max() > Y_BAR
