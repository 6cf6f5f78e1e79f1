"""Stage-level parity of the HIP kernels against the fp64 oracle.

Each stage gets identical inputs on both sides (stage isolation, as in "round
10 track b: gdn vectorization and scan", "correctness": every stage is fed the
same inputs even if an earlier one is wrong).  Inputs come from the seeded
generator, or from the oracle's own earlier stage rounded to the fp32 storage of
the intermediates, never from the GPU.  Every output buffer is wrapped in
canary bands that must survive the call.
"""
import math

import numpy as np
import pytest
import torch

from gated_deltanet_linear_pre_amd import binding as B
from gated_deltanet_linear_pre_amd import synth
from gated_deltanet_linear_pre_amd import buffers
from gated_deltanet_linear_pre_amd.buffers import upload
from oracle import gdn_oracle as orc

from . import parity
from .gpu_util import Guarded, banner, np_

pytestmark = pytest.mark.gpu

F32 = torch.float32


def scratch(s):
    return buffers.scratch(B.gdn_scan_workspace_bytes(s), "cuda")


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


PRE_CASES = [
    # name, hk, hv, seqlens, io, hist_std
    ("tiny_t37_fp32", 2, 6, (37,), "f32", 0.0),
    ("tiny_varlen_fp32_hist", 2, 6, (1, 2, 3, 9, 0, 20), "f32", 1.0),
    ("prod_t512_fp16", 16, 48, (512,), "f16", 0.0),
    ("prod_varlen_fp16_hist", 16, 48, (1, 3, 37, 300, 17, 2), "f16", 1.0),
]


@pytest.mark.parametrize("case", PRE_CASES, ids=[c[0] for c in PRE_CASES])
def test_pre_matches_oracle(gpu, case):
    name, hk, hv, lens, io, hist_std = case
    w = synth.Workload(name, hk=hk, hv=hv, seqlens=lens, io=io, seed=(3,), hist_std=hist_std)
    inp = synth.layer_inputs(w)
    cu = _cu(lens)
    T, n = int(cu[-1]), len(lens)
    ref = orc.pre(orc.Dims(hk, hv), cu, inp["qkv"], inp["conv_w"], inp["a"], inp["b"],
                  inp["A_log"], inp["dt_bias"], inp["hist"], 1e-6)
    dev = "cuda"
    hist = Guarded(inp["hist"].shape, torch.float16 if io == "f16" else F32, init=torch.from_numpy(inp["hist"]))
    outs = {k: Guarded(s, F32) for k, s in
            dict(qn=(T, hk, 128), kn=(T, hk, 128), vc=(T, hv, 128), g=(T, hv), beta=(T, hv)).items()}
    s = B.make_shape(hk, hv, n, T, max(lens), io=io, out="f32")
    banner("gdn_pre", name, f"T={T}", f"lens={lens}")
    B.gdn_pre(s, upload(cu, dev), upload(inp["qkv"], dev), upload(inp["conv_w"], dev),
              upload(inp["a"], dev), upload(inp["b"], dev), upload(inp["A_log"], dev),
              upload(inp["dt_bias"], dev), hist.t, outs["qn"].t, outs["kn"].t, outs["vc"].t,
              outs["g"].t, outs["beta"].t)
    torch.cuda.synchronize()
    for k, gbuf in outs.items():
        assert gbuf.intact(), f"{k}: canary overwritten"
    assert hist.intact()
    parity.check_close("qn", np_(outs["qn"].t), ref["qn"])
    parity.check_close("kn", np_(outs["kn"].t), ref["kn"])
    parity.check_close("vc", np_(outs["vc"].t), ref["vc"])
    parity.check_close("g", np_(outs["g"].t), ref["g"], rtol=1e-5, atol=1e-7)
    parity.check_close("beta", np_(outs["beta"].t), ref["beta"])
    parity.check_exact("hist", np_(hist.t).astype(np.float64), ref["hist"])


SCAN_CASES = [
    # name, hk, hv, seqlens, s0_std
    ("tiny_t37_zero_state", 2, 6, (37,), 0.0),
    ("tiny_varlen", 2, 6, (1, 16, 17, 0, 33), 0.05),
    ("prod_t300", 16, 48, (300,), 0.05),
    ("prod_varlen_ragged", 16, 48, (5, 129, 64, 1), 0.05),
    ("g1_heads", 4, 4, (50, 3), 0.05),
]


@pytest.mark.parametrize("case", SCAN_CASES, ids=[c[0] for c in SCAN_CASES])
def test_scan_matches_oracle(gpu, case):
    name, hk, hv, lens, s0_std = case
    d = synth.scan_inputs(hk, hv, lens, seed=(4,), s0_std=s0_std)
    cu = _cu(lens)
    T, n = int(cu[-1]), len(lens)
    o_ref, S_ref = orc.scan(orc.Dims(hk, hv), cu, d["qn"], d["kn"], d["vc"], d["g"], d["beta"], d["S0"])
    dev = "cuda"
    state = Guarded(d["S0"].shape, F32, init=torch.from_numpy(d["S0"]))
    o = Guarded((T, hv, 128), F32)
    s = B.make_shape(hk, hv, n, T, max(lens), io="f32", out="f32")
    ws = Guarded((B.gdn_scan_workspace_bytes(s) // 4,), F32)
    banner("gdn_scan", name, f"T={T}", f"lens={lens}")
    B.gdn_scan(s, upload(cu, dev), upload(d["qn"], dev), upload(d["kn"], dev),
               upload(d["vc"], dev), upload(d["g"], dev), upload(d["beta"], dev), state.t, o.t,
               ws.t)
    torch.cuda.synchronize()
    assert state.intact() and o.intact() and ws.intact()
    parity.check_o(np_(o.t), o_ref)
    parity.check_state(np_(state.t), S_ref)
    # sequences of length 0 keep their state bit for bit
    for k, L in enumerate(lens):
        if L == 0:
            assert np.array_equal(np_(state.t)[k], d["S0"][k])


def test_scan_on_layer_intermediates(gpu):
    # the scan fed with what the oracle's pre stage makes of a production-width
    # layer (T = 1365, non-zero state, decays and gates from the layer's own
    # parameters), rounded to the fp32 storage of the intermediates
    w = synth.WORKLOADS["prod_continuation_fp16"]
    inp = synth.layer_inputs(w)
    cu = w.cu_seqlens()
    pr = orc.pre(orc.Dims(w.hk, w.hv), cu, inp["qkv"], inp["conv_w"], inp["a"], inp["b"],
                 inp["A_log"], inp["dt_bias"], inp["hist"], 1e-6)
    f32 = {k: pr[k].astype(np.float32) for k in ("qn", "kn", "vc", "g", "beta")}
    S0 = inp["S0"].astype(np.float32)
    o_ref, S_ref = orc.scan(orc.Dims(w.hk, w.hv), cu, f32["qn"], f32["kn"], f32["vc"], f32["g"],
                            f32["beta"], S0)
    T, dev = int(cu[-1]), "cuda"
    state = Guarded(S0.shape, F32, init=torch.from_numpy(S0))
    o = Guarded((T, w.hv, 128), F32)
    s = B.make_shape(w.hk, w.hv, 1, T, T, io="f32", out="f32")
    ws = Guarded((B.gdn_scan_workspace_bytes(s) // 4,), F32)
    banner("gdn_scan", w.name, f"T={T}")
    B.gdn_scan(s, upload(cu, dev), *(upload(f32[k], dev) for k in ("qn", "kn", "vc", "g", "beta")),
               state.t, o.t, ws.t)
    torch.cuda.synchronize()
    assert state.intact() and o.intact() and ws.intact()
    parity.check_o(np_(o.t), o_ref)
    parity.check_state(np_(state.t), S_ref)


def test_scan_invariant_beta0_g0_keeps_state_bitwise(gpu):
    hk, hv, T = 16, 48, 40
    d = synth.scan_inputs(hk, hv, (T,), seed=(8,), s0_std=0.05)
    d["g"][:] = 0.0
    d["beta"][:] = 0.0
    dev = "cuda"
    state = upload(d["S0"], dev)
    o = torch.empty((T, hv, 128), dtype=F32, device=dev)
    s = B.make_shape(hk, hv, 1, T, T, io="f32", out="f32")
    banner("gdn_scan", "beta=0,g=0")
    B.gdn_scan(s, upload(_cu([T]), dev),
               upload(d["qn"], dev), upload(d["kn"], dev), upload(d["vc"], dev),
               upload(d["g"], dev), upload(d["beta"], dev), state, o, scratch(s))
    torch.cuda.synchronize()
    assert np.array_equal(np_(state), d["S0"])
    # o_t = S0 q_t / sqrt(dk): compare with the oracle's scan of the same inputs
    o_or, _ = orc.scan(orc.Dims(hk, hv), _cu([T]), d["qn"], d["kn"], d["vc"], d["g"], d["beta"],
                       d["S0"])
    parity.check_o(np_(o), o_or)


def test_scan_invariant_unit_key_writes_value(gpu):
    # k = e_j (a basis vector, fed straight to the scan), beta = 1, alpha = 1:
    # after each token the state column j equals v_t (up to fp32 rounding).
    hk, hv, T = 2, 6, 24
    rs = np.random.default_rng(9)
    d = synth.scan_inputs(hk, hv, (T,), seed=(9,), s0_std=0.05)
    js = rs.integers(0, 128, T)
    d["kn"][:] = 0.0
    for t in range(T):
        d["kn"][t, :, js[t]] = 1.0
    d["g"][:] = 0.0
    d["beta"][:] = 1.0
    dev = "cuda"
    for t_end in (1, 7, 24):
        state = upload(d["S0"], dev)
        o = torch.empty((t_end, hv, 128), dtype=F32, device=dev)
        s = B.make_shape(hk, hv, 1, t_end, t_end, io="f32", out="f32")
        banner("gdn_scan", "unit-key", f"T={t_end}")
        B.gdn_scan(s, upload(_cu([t_end]), dev), upload(d["qn"][:t_end], dev),
                   upload(d["kn"][:t_end], dev), upload(d["vc"][:t_end], dev),
                   upload(d["g"][:t_end], dev), upload(d["beta"][:t_end], dev), state, o,
                   scratch(s))
        torch.cuda.synchronize()
        S = np_(state)[0]
        col = S[:, :, js[t_end - 1]]
        np.testing.assert_allclose(col, d["vc"][t_end - 1], rtol=0, atol=4e-6)


POST_CASES = [("f16", "f16"), ("f16", "f32"), ("f32", "f32"), ("f32", "f16")]


@pytest.mark.parametrize("io,out", POST_CASES, ids=[f"{a}in_{b}out" for a, b in POST_CASES])
@pytest.mark.parametrize("o_std", [8e-4, 1.0], ids=["eps_regime", "unit_scale"])
def test_post_matches_oracle(gpu, io, out, o_std):
    T, hv = 333, 48
    d = synth.post_inputs(T, hv, seed=(6,), o_std=o_std, io=io)
    y_ref = orc.post(d["o"], d["z"].reshape(T, hv, 128), d["gamma"], 1e-6)
    dev = "cuda"
    y = Guarded((T, hv * 128), torch.float16 if out == "f16" else F32)
    banner("gdn_post", io, out, o_std)
    B.gdn_post(B.make_shape(16, hv, 1, T, T, io=io, out=out), upload(d["o"], dev),
               upload(d["z"], dev), upload(d["gamma"], dev), y.t)
    torch.cuda.synchronize()
    assert y.intact()
    parity.check_y(np_(y.t), y_ref, out)


def test_post_checker_catches_one_corrupted_fp16_element(gpu):
    # negative control ("round 10 track b", "correctness": a deliberately
    # corrupted fp16 output must fail the check)
    T, hv = 64, 48
    d = synth.post_inputs(T, hv, seed=(7,), io="f16")
    y_ref = orc.post(d["o"], d["z"].reshape(T, hv, 128), d["gamma"], 1e-6)
    dev = "cuda"
    y = torch.empty((T, hv * 128), dtype=torch.float16, device=dev)
    B.gdn_post(B.make_shape(16, hv, 1, T, T, io="f16", out="f16"), upload(d["o"], dev),
               upload(d["z"], dev), upload(d["gamma"], dev), y)
    yh = np_(y).copy()
    parity.check_y(yh, y_ref, "f16")
    bad = yh.copy()
    i = np.argmax(np.abs(y_ref.reshape(-1)) < 1)
    bad.reshape(-1)[i] = np.float16(bad.reshape(-1)[i] + np.float16(0.01))
    with pytest.raises(parity.ParityError):
        parity.check_y(bad, y_ref, "f16")
