"""gdn_step (one decode token per sequence through the whole layer) against
the fp64 oracle, and against the prefill path.

"Round 30 Track C Audit: gdn_pre, gdn_post, and gdn_scanr_4", section 1: the
single-token step is what every scan variant is checked against; section 2:
T steps must agree with one T-token pass.  The oracle runs the same layer with
one token per sequence (cu_seqlens = 0, 1, 2, ...), so no oracle code is
specific to the step.
"""
import numpy as np
import pytest
import torch

from gated_deltanet_linear_pre_amd import binding as B
from gated_deltanet_linear_pre_amd import synth
from gated_deltanet_linear_pre_amd.buffers import LayerBuffers
from oracle import gdn_oracle as orc

from . import parity
from .gpu_util import Guarded, banner, np_

pytestmark = pytest.mark.gpu


def _step(buf, y=None, state=None, hist=None):
    B.gdn_step(buf.shape, buf.qkv, buf.conv_w, buf.a, buf.b, buf.A_log, buf.dt_bias, buf.z,
               buf.gamma, buf.hist if hist is None else hist,
               buf.state if state is None else state, buf.y if y is None else y)


CASES = [
    # name, hk, hv, n_seq, io, out
    ("prod_batch5_fp16", 16, 48, 5, "f16", "f16"),
    ("prod_batch3_fp16in_fp32out", 16, 48, 3, "f16", "f32"),
    ("tiny_batch4_fp32", 2, 6, 4, "f32", "f32"),
    ("tiny_batch1_fp32in_fp16out", 2, 6, 1, "f32", "f16"),
    # one value head per key head (one 256-thread group per block), and five
    # (value heads handled three at a time: two rounds)
    ("g1_batch3_fp16", 4, 4, 3, "f16", "f16"),
    ("g5_batch2_fp16in_fp32out", 2, 10, 2, "f16", "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_step_matches_oracle(gpu, case):
    name, hk, hv, n, io, out = case
    w = synth.Workload(name, hk=hk, hv=hv, seqlens=(1,) * n, io=io, out=out, seed=(31, n),
                       s0_std=0.05, hist_std=1.0)
    inp = synth.layer_inputs(w)
    buf = LayerBuffers.create(w, inp)
    y = Guarded(tuple(buf.y.shape), buf.y.dtype)
    state = Guarded(tuple(buf.state.shape), torch.float32, init=buf.state)
    hist = Guarded(tuple(buf.hist.shape), buf.hist.dtype, init=buf.hist)
    banner("gdn_step", name, f"n_seq={n}")
    _step(buf, y=y.t, state=state.t, hist=hist.t)
    torch.cuda.synchronize()
    assert y.intact() and state.intact() and hist.intact()
    ref = orc.layer(orc.Dims(hk, hv), w.cu_seqlens(), inp)
    parity.check_y(np_(y.t).reshape(n, hv, 128), ref["y"], out)
    parity.check_state(np_(state.t), ref["S"])
    parity.check_exact("hist", np_(hist.t).astype(np.float64), ref["hist"])


def test_steps_match_prefill_and_oracle(gpu):
    # 37 decode steps of one sequence vs one 37-token prefill call: both
    # against the oracle, and against each other within the same bars
    T = 37
    w = synth.Workload("steps_vs_prefill", hk=16, hv=48, seqlens=(T,), seed=(32,), s0_std=0.05,
                       hist_std=1.0)
    inp = synth.layer_inputs(w)
    ref = orc.layer(orc.Dims(w.hk, w.hv), w.cu_seqlens(), inp)
    banner("gdn_prefill_layer", w.name, f"T={T}")
    pre = LayerBuffers.create(w, inp)
    ws = pre.workspace()
    pre.run_layer(ws)
    torch.cuda.synchronize()
    one = synth.Workload("steps_vs_prefill_1", hk=16, hv=48, seqlens=(1,), seed=(32,))
    hist, state = inp["hist"], inp["S0"]
    ys = []
    for t in range(T):
        part = dict(inp, hist=hist, S0=state)
        for k in ("qkv", "a", "b", "z"):
            part[k] = inp[k][t:t + 1]
        banner("gdn_step", w.name, f"token {t}")
        buf = LayerBuffers.create(one, part)
        _step(buf)
        torch.cuda.synchronize()
        ys.append(np_(buf.y))
        hist, state = np_(buf.hist), np_(buf.state)
    y = np.concatenate(ys).reshape(T, w.hv, 128)
    parity.check_y(y, ref["y"], "f16", what="y (steps)")
    parity.check_state(state, ref["S"])
    parity.check_exact("hist (steps)", hist.astype(np.float64), ref["hist"])
    parity.check_y(np_(pre.y).reshape(T, w.hv, 128), ref["y"], "f16", what="y (prefill)")
    parity.check_state(state, np_(pre.state).astype(np.float64))
    assert np.array_equal(hist.view(np.uint16), np_(pre.hist).view(np.uint16))


def test_step_is_bitwise_deterministic(gpu):
    w = synth.Workload("step_det", hk=16, hv=48, seqlens=(1,) * 8, seed=(33,), s0_std=0.05,
                       hist_std=1.0)
    inp = synth.layer_inputs(w)
    outs = []
    for _ in range(2):
        buf = LayerBuffers.create(w, inp)
        banner("gdn_step", w.name)
        _step(buf)
        torch.cuda.synchronize()
        outs.append((np_(buf.y).view(np.uint16), np_(buf.state).view(np.uint32)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


def test_step_graph_replay_matches_eager(gpu):
    # A decode step over 4 layers (each with its own weights, state and
    # history) captured once in a HIP graph and replayed three times from the
    # same initial state and history, with eager copies and a synchronisation
    # between the replays: every replay equals the eager run bit for bit.
    L = 4
    w = synth.Workload("step_graph", hk=16, hv=48, seqlens=(1,) * 8, seed=(34,), s0_std=0.05,
                       hist_std=1.0)
    bufs = [LayerBuffers.create(w, synth.layer_inputs(w, l)) for l in range(L)]
    init = [(b.state.clone(), b.hist.clone()) for b in bufs]

    def run_all():
        for b in bufs:
            _step(b)

    def restore():
        for b, (s, h) in zip(bufs, init):
            b.state.copy_(s)
            b.hist.copy_(h)

    banner("gdn_step", w.name, "eager")
    run_all()
    torch.cuda.synchronize()
    ref = [(np_(b.y).copy(), np_(b.state).copy(), np_(b.hist).copy()) for b in bufs]
    restore()
    torch.cuda.synchronize()
    banner("gdn_step", w.name, "capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_all()
    torch.cuda.synchronize()
    for rep in range(3):
        restore()
        banner("gdn_step", w.name, f"replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for b, (y, s, h) in zip(bufs, ref):
            assert np.array_equal(np_(b.y).view(np.uint16), y.view(np.uint16)), f"y, replay {rep}"
            assert np.array_equal(np_(b.state).view(np.uint32), s.view(np.uint32)), f"state, replay {rep}"
            assert np.array_equal(np_(b.hist).view(np.uint16), h.view(np.uint16)), f"hist, replay {rep}"



def _step_out(buf, hist_in, hist_out, y=None, state=None, qkv=None):
    B.gdn_step(buf.shape, buf.qkv if qkv is None else qkv, buf.conv_w, buf.a, buf.b, buf.A_log,
               buf.dt_bias, buf.z, buf.gamma, hist_in, buf.state if state is None else state,
               buf.y if y is None else y, hist_out=hist_out)


@pytest.mark.parametrize("case", [CASES[0], CASES[2], CASES[4], CASES[5]], ids=lambda c: c[0])
def test_step_hist_out_matches_in_place(gpu, case):
    # the new history written to a buffer of its own (one launch) gives the
    # in-place call's y, state and history bit for bit, and leaves the input
    # history untouched
    name, hk, hv, n, io, out = case
    w = synth.Workload(name, hk=hk, hv=hv, seqlens=(1,) * n, io=io, out=out, seed=(35, n),
                       s0_std=0.05, hist_std=1.0)
    inp = synth.layer_inputs(w)
    a = LayerBuffers.create(w, inp)
    b = LayerBuffers.create(w, inp)
    banner("gdn_step", name, "in place")
    _step(a)
    hist0 = b.hist.clone()
    y = Guarded(tuple(b.y.shape), b.y.dtype)
    state = Guarded(tuple(b.state.shape), torch.float32, init=b.state)
    hist_out = Guarded(tuple(b.hist.shape), b.hist.dtype)
    banner("gdn_step", name, "hist_out")
    _step_out(b, b.hist, hist_out.t, y=y.t, state=state.t)
    torch.cuda.synchronize()
    assert y.intact() and state.intact() and hist_out.intact()
    bits = np.uint16 if io == "f16" else np.uint32
    ybits = np.uint16 if out == "f16" else np.uint32
    assert np.array_equal(np_(y.t).view(ybits), np_(a.y).view(ybits))
    assert np.array_equal(np_(state.t).view(np.uint32), np_(a.state).view(np.uint32))
    assert np.array_equal(np_(hist_out.t).view(bits), np_(a.hist).view(bits))
    assert np.array_equal(np_(b.hist).view(bits), np_(hist0).view(bits))


def test_steps_alternating_history_match_in_place(gpu):
    # 9 decode steps over 3 layers with each layer's history alternating
    # between two buffers (one launch per step and layer) equal the in-place
    # steps bit for bit, run eagerly and replayed from a HIP graph of two
    # steps (the graph reads the token rows from fixed staging buffers that
    # are refilled between replays)
    L, T, n = 3, 9, 4
    w = synth.Workload("step_alternating", hk=16, hv=48, seqlens=(1,) * n, seed=(36,),
                       s0_std=0.05, hist_std=1.0)
    inps = [synth.layer_inputs(w, l) for l in range(L)]
    rng = np.random.default_rng(36)
    toks = [[torch.from_numpy(rng.standard_normal(inps[l]["qkv"].shape).astype(np.float16)).cuda()
             for l in range(L)] for _ in range(T)]
    ref = [LayerBuffers.create(w, inp) for inp in inps]
    banner("gdn_step", w.name, "in place")
    for t in range(T):
        for l, b in enumerate(ref):
            _step_out(b, b.hist, None, qkv=toks[t][l])
    torch.cuda.synchronize()

    def check(bufs, hs, mode):
        for l, b in enumerate(bufs):
            assert np.array_equal(np_(b.y).view(np.uint16), np_(ref[l].y).view(np.uint16)), mode
            assert np.array_equal(np_(b.state).view(np.uint32), np_(ref[l].state).view(np.uint32)), mode
            assert np.array_equal(np_(hs[l][T % 2]).view(np.uint16), np_(ref[l].hist).view(np.uint16)), mode

    def fresh():
        bufs = [LayerBuffers.create(w, inp) for inp in inps]
        return bufs, [[b.hist, torch.empty_like(b.hist)] for b in bufs]

    banner("gdn_step", w.name, "alternating, eager")
    bufs, hs = fresh()
    for t in range(T):
        for l, b in enumerate(bufs):
            _step_out(b, hs[l][t % 2], hs[l][1 - t % 2], qkv=toks[t][l])
    torch.cuda.synchronize()
    check(bufs, hs, "eager")

    banner("gdn_step", w.name, "alternating, graph of two steps")
    bufs, hs = fresh()
    stage = [[torch.empty_like(toks[0][l]) for l in range(L)] for _ in range(2)]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s in range(2):
            for l, b in enumerate(bufs):
                _step_out(b, hs[l][s], hs[l][1 - s], qkv=stage[s][l])
    torch.cuda.synchronize()
    for t in range(0, T - 1, 2):
        for s in range(2):
            for l in range(L):
                stage[s][l].copy_(toks[t + s][l])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
    for l, b in enumerate(bufs):  # the odd last step, eagerly
        _step_out(b, hs[l][(T - 1) % 2], hs[l][T % 2], qkv=toks[T - 1][l])
    torch.cuda.synchronize()
    check(bufs, hs, "graph")
