"""Whole-layer parity (gdn_prefill_layer) against the fp64 oracle, on every
workload: the tiny fp32 layer, the production-width T=512 layer and the
continuation sweep (the 36-layer stack and the long varlen batch, at full
size, are in test_gpu_stack.py).

Also: bitwise determinism, a long sequence alone equal to the same sequence
packed with another, graph replays of the layer equal to the eager call, key
heads shared by 8 and 10 value heads, and split invariance of the path ("Round 30
Track C Audit: gdn_pre, gdn_post, and gdn_scanr_4", section 2: the
token-blocked scan must equal the single pass) -- bitwise for splits on the
32-token chunk grid, within tolerance for any other split.
"""
import numpy as np
import pytest
import torch

from gated_deltanet_linear_pre_amd import binding as B
from gated_deltanet_linear_pre_amd import synth
from gated_deltanet_linear_pre_amd.buffers import LayerBuffers
from oracle import gdn_oracle as orc

from . import parity
from .gpu_util import banner, np_

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _run_layer(w, inp, out=None, cu=None):
    buf = LayerBuffers.create(w, inp, out=out, cu=cu)
    ws = buf.workspace()
    buf.run_layer(ws)
    torch.cuda.synchronize()
    return buf


def _check_layer(w, buf, ref, out, heads=None):
    T = buf.shape.total_T
    y = np_(buf.y).reshape(T, w.hv, 128)
    y_ref = ref["y"]
    if heads is not None:
        y, y_ref = y[:, heads], y_ref[:, heads]
    rep = parity.check_y(y, y_ref, out)
    worst = parity.check_state(np_(buf.state), ref["S"], heads=heads)
    parity.check_exact("hist", np_(buf.hist).astype(np.float64), ref["hist"])
    return rep, worst


@pytest.mark.parametrize("name", ["tiny_h2x6_t37_fp32", "prod_t512_fp16"])
def test_layer_full_oracle(gpu, name):
    w = W[name]
    inp = synth.layer_inputs(w)
    banner("gdn_prefill_layer", name)
    buf = _run_layer(w, inp)
    ref = orc.layer(orc.Dims(w.hk, w.hv), w.cu_seqlens(), inp)
    _check_layer(w, buf, ref, w.out)


def _run_segments(w, inp, segments):
    """Run the layer over consecutive segments, carrying state and history."""
    hist, state = inp["hist"], inp["S0"]
    ys, s = [], 0
    for L in segments:
        part = dict(inp, hist=hist, S0=state)
        for k in ("qkv", "a", "b", "z"):
            part[k] = inp[k][s:s + L]
        banner("gdn_prefill_layer", w.name, f"segment [{s}, {s + L})")
        buf = _run_layer(w, part, cu=[0, L])
        ys.append(np_(buf.y))
        hist, state = np_(buf.hist), np_(buf.state)
        s += L
    return np.concatenate(ys), state, hist


def test_continuation_split_matches_whole_and_oracle(gpu):
    # segments 1, 3, 37, 300, 1024 carrying state and history vs one call:
    # both within tolerance of the oracle, the history bit-exact, and the two
    # GPU results within rounding of each other (the chunk grid moves with the
    # split, so they need not be bit-identical)
    w = W["prod_continuation_fp16"]
    inp = synth.layer_inputs(w)
    banner("gdn_prefill_layer", w.name, "whole")
    whole = _run_layer(w, inp)
    ref = orc.layer(orc.Dims(w.hk, w.hv), w.cu_seqlens(), inp)
    _check_layer(w, whole, ref, w.out)
    y, state, hist = _run_segments(w, inp, w.segments)
    T = w.total_T
    parity.check_y(y.reshape(T, w.hv, 128), ref["y"], w.out, what="y (split)")
    parity.check_state(state, ref["S"])
    parity.check_exact("hist (split)", hist.astype(np.float64), ref["hist"])
    # split and whole GPU runs agree to the same bars they each meet against
    # the oracle
    parity.check_state(state, np_(whole.state).astype(np.float64))
    d = np.abs(y.astype(np.float32) - np_(whole.y).astype(np.float32))
    assert d.max() <= 2 * parity.Y_ABS


def test_split_on_chunk_boundaries_is_bitwise(gpu):
    # splits at multiples of 32 tokens keep the chunk grid: bit-identical
    w = W["prod_continuation_fp16"]
    inp = synth.layer_inputs(w)
    banner("gdn_prefill_layer", w.name, "whole")
    whole = _run_layer(w, inp)
    y, state, hist = _run_segments(w, inp, (32, 64, 256, 992, 21))
    assert np.array_equal(y.view(np.uint16), np_(whole.y).view(np.uint16))
    assert np.array_equal(state.view(np.uint32), np_(whole.state).view(np.uint32))
    assert np.array_equal(hist.view(np.uint16), np_(whole.hist).view(np.uint16))


def test_varlen_packing_equals_separate_calls(gpu):
    # several sequences packed in one call == one call per sequence (bitwise),
    # including empty sequences and ones shorter than the 3-token history
    lens = (0, 1, 2, 3, 19, 0, 70)
    w = synth.Workload("pack", hk=16, hv=48, seqlens=lens, seed=(12,), s0_std=0.05, hist_std=1.0)
    inp = synth.layer_inputs(w)
    banner("gdn_prefill_layer", "varlen packed", f"lens={lens}")
    packed = _run_layer(w, inp)
    cu = w.cu_seqlens()
    for n, L in enumerate(lens):
        if L == 0:
            assert np.array_equal(np_(packed.state)[n], inp["S0"][n])
            assert np.array_equal(np_(packed.hist)[n], inp["hist"][n])
            continue
        part = dict(inp, hist=inp["hist"][n:n + 1], S0=inp["S0"][n:n + 1])
        for k in ("qkv", "a", "b", "z"):
            part[k] = inp[k][cu[n]:cu[n + 1]]
        banner("gdn_prefill_layer", "varlen single", f"seq={n}", f"T={L}")
        one = _run_layer(w, part, cu=[0, L])
        assert np.array_equal(np_(one.y), np_(packed.y)[cu[n]:cu[n + 1]])
        assert np.array_equal(np_(one.state)[0], np_(packed.state)[n])
        assert np.array_equal(np_(one.hist)[0], np_(packed.hist)[n])
    ref = orc.layer(orc.Dims(w.hk, w.hv), cu, inp)
    _check_layer(w, packed, ref, w.out)


def test_layer_is_bitwise_deterministic(gpu):
    w = W["prod_t512_fp16"]
    inp = synth.layer_inputs(w)
    banner("gdn_prefill_layer", "determinism")
    a = _run_layer(w, inp)
    b = _run_layer(w, inp)
    assert np.array_equal(np_(a.y).view(np.uint16), np_(b.y).view(np.uint16))
    assert np.array_equal(np_(a.state).view(np.uint32), np_(b.state).view(np.uint32))
    assert np.array_equal(np_(a.hist).view(np.uint16), np_(b.hist).view(np.uint16))


def test_stages_equal_layer_entry_point(gpu):
    # gdn_pre + gdn_scan + gdn_post called one by one == gdn_prefill_layer (bitwise)
    w = W["prod_t512_fp16"]
    inp = synth.layer_inputs(w)
    banner("gdn_pre/gdn_scan/gdn_post vs gdn_prefill_layer")
    st = LayerBuffers.create(w, inp)
    st.run_pre()
    st.run_scan()
    st.run_post()
    torch.cuda.synchronize()
    ly = _run_layer(w, inp)
    assert np.array_equal(np_(st.y).view(np.uint16), np_(ly.y).view(np.uint16))
    assert np.array_equal(np_(st.state), np_(ly.state))
    assert np.array_equal(np_(st.hist), np_(ly.hist))


def _single_vs_packed(w1, w2):
    # one long sequence alone == the same sequence packed first with a short
    # second one, bitwise: y of its rows, its state and its history
    inp2 = synth.layer_inputs(w2)
    T1 = w1.seqlens[0]
    inp1 = dict(inp2, hist=inp2["hist"][:1], S0=inp2["S0"][:1])
    for k in ("qkv", "a", "b", "z"):
        inp1[k] = inp2[k][:T1]
    banner("gdn_prefill_layer", "single", w1.name, f"T={T1}", w1.io)
    one = _run_layer(w1, inp1)
    banner("gdn_prefill_layer", "packed", w2.name, f"lens={w2.seqlens}", w2.io)
    packed = _run_layer(w2, inp2)
    assert np.array_equal(np_(one.y).view(np.uint8), np_(packed.y)[:T1].view(np.uint8))
    assert np.array_equal(np_(one.state)[0].view(np.uint32), np_(packed.state)[0].view(np.uint32))
    assert np.array_equal(np_(one.hist)[0].view(np.uint8), np_(packed.hist)[0].view(np.uint8))
    return inp1, one


@pytest.mark.parametrize("io", ["f16", "f32"])
def test_long_sequence_alone_equals_packed(gpu, io):
    hk, hv = (16, 48) if io == "f16" else (2, 6)
    kw = dict(hk=hk, hv=hv, io=io, out=io, seed=(31,), s0_std=0.05, hist_std=1.0)
    w1 = synth.Workload(f"long_{io}", seqlens=(1500,), **kw)
    w2 = synth.Workload(f"long_plus_short_{io}", seqlens=(1500, 5), **kw)
    inp1, one = _single_vs_packed(w1, w2)
    if io == "f32":
        ref = orc.layer(orc.Dims(hk, hv), w1.cu_seqlens(), inp1)
        _check_layer(w1, one, ref, io)


def test_layer_graph_replay_matches_eager(gpu):
    # gdn_prefill_layer captured in a graph: every replay, with eager work and
    # synchronisation between replays, equals the eager call bitwise
    w = synth.Workload("long_graph", hk=16, hv=48, seqlens=(1200,), seed=(33,), s0_std=0.05,
                       hist_std=1.0)
    inp = synth.layer_inputs(w)
    banner("gdn_prefill_layer", "graph replay", w.name)
    eager = _run_layer(w, inp)
    buf = LayerBuffers.create(w, inp)
    ws = buf.workspace()
    hist0, state0 = buf.hist.clone(), buf.state.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        buf.run_layer(ws)  # warm-up outside the capture
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        buf.run_layer(ws)
    for r in range(3):
        buf.hist.copy_(hist0)
        buf.state.copy_(state0)
        buf.y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(np_(buf.y).view(np.uint16), np_(eager.y).view(np.uint16)), r
        assert np.array_equal(np_(buf.state).view(np.uint32), np_(eager.state).view(np.uint32)), r
        assert np.array_equal(np_(buf.hist).view(np.uint16), np_(eager.hist).view(np.uint16)), r


GROUP_CASES = [
    # (hk, hv, io): value heads per key head G = hv / hk.  The fused fp32-io
    # prep splits its tasks by G (G = 1: 5 token parts per unit; G = 4 and 8:
    # 2 parts, and at G = 8 twenty tasks take two rounds of the block's 16
    # rows); the fused fp16 prep is fixed-shape; G = 10 runs the three stages.
    (2, 2, "f32"), (2, 8, "f32"), (1, 8, "f32"), (2, 2, "f16"), (1, 8, "f16"), (1, 10, "f16"),
]


@pytest.mark.parametrize("hk,hv,io", GROUP_CASES,
                         ids=[f"G{hv // hk}_{io}" + ("_staged" if hv // hk > 8 else "_fused")
                              for hk, hv, io in GROUP_CASES])
def test_layer_group_sizes_match_oracle_and_stages(gpu, hk, hv, io):
    # key heads shared by G value heads: against the oracle, and bit for bit
    # against gdn_pre + gdn_scan + gdn_post, ragged with an empty sequence
    lens = (70, 0, 33)
    w = synth.Workload(f"group{hv}_{hk}_{io}", hk=hk, hv=hv, seqlens=lens, seed=(35,), io=io, out=io,
                       s0_std=0.05, hist_std=1.0)
    inp = synth.layer_inputs(w)
    banner("gdn_prefill_layer", w.name, f"lens={lens}")
    ly = _run_layer(w, inp)
    ref = orc.layer(orc.Dims(w.hk, w.hv), w.cu_seqlens(), inp)
    _check_layer(w, ly, ref, w.out)
    st = LayerBuffers.create(w, inp)
    st.run_pre()
    st.run_scan()
    st.run_post()
    torch.cuda.synchronize()
    assert np.array_equal(np_(st.y).view(np.uint8), np_(ly.y).view(np.uint8))
    assert np.array_equal(np_(st.state).view(np.uint32), np_(ly.state).view(np.uint32))
    assert np.array_equal(np_(st.hist).view(np.uint8), np_(ly.hist).view(np.uint8))


@pytest.mark.parametrize("hk,hv,T,out", [(16, 48, 2048, "f16"), (16, 48, 517, "f32"), (8, 16, 40, "f16"),
                                         (2, 6, 1, "f16")])
def test_post_in_chunk_launch_equals_separate_post(gpu, hk, hv, T, out, monkeypatch):
    # post run by the chunk kernel's launch (its idle CUs; each (chunk, value
    # head) once its eight output waves have counted it) gives the separate
    # post kernel's y bit for bit, on workspaces first filled with 0xFF bytes
    # and with random bytes; the status word shows that no wait gave up.
    # (16 and 8 key heads: value heads of XCD x on XCD x; 6 value heads: in
    # plain chunk order)
    w = synth.Workload("post_fused", hk=hk, hv=hv, seqlens=(T,), seed=(43,), io="f16", out=out,
                       s0_std=0.05, hist_std=1.0)
    inp = synth.layer_inputs(w)
    banner("gdn_prefill_layer", "post in the chunk launch vs separate", f"hk={hk} hv={hv} T={T} out={out}")
    monkeypatch.setenv("GDN_LAYER_POST_FUSED", "0")
    sep = _run_layer(w, inp)
    monkeypatch.delenv("GDN_LAYER_POST_FUSED")
    nbytes = B.gdn_prefill_workspace_bytes(sep.shape)
    n_count = (T + 31) // 32 * hv
    sync_at = nbytes - (n_count + 1) * 256   # the last region: a 256-byte line per counter
    status_at = sync_at + n_count * 256
    g = torch.Generator(device="cpu").manual_seed(7)
    for fill in ("ff", "random"):
        if fill == "ff":
            src = torch.full((nbytes,), 255, dtype=torch.uint8)
        else:
            src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g)
        buf = LayerBuffers.create(w, inp)
        ws = buf.workspace()
        ws.copy_(src.cuda())
        buf.run_layer(ws)
        torch.cuda.synchronize()
        assert np.array_equal(np_(buf.y).view(np.uint8), np_(sep.y).view(np.uint8)), fill
        assert np.array_equal(np_(buf.state).view(np.uint32), np_(sep.state).view(np.uint32)), fill
        assert np.array_equal(np_(buf.hist).view(np.uint16), np_(sep.hist).view(np.uint16)), fill
        status = ws[status_at:status_at + 4].cpu().numpy().view(np.uint32)[0]
        assert status == 0, f"a wait for o gave up ({fill})"


def test_post_in_chunk_launch_wait_bound(gpu, monkeypatch):
    # the post waves' wait for o is bounded: with the bound forced to zero
    # polls from the host, they give up at once, the call still completes and
    # the status word says so; the next call with the normal bound is exact
    w = synth.Workload("post_bound", hk=16, hv=48, seqlens=(300,), seed=(44,), s0_std=0.05,
                       hist_std=1.0)
    inp = synth.layer_inputs(w)
    banner("gdn_prefill_layer", "post wait bound forced to 0")
    monkeypatch.setenv("GDN_LAYER_POST_FUSED", "0")
    sep = _run_layer(w, inp)
    monkeypatch.delenv("GDN_LAYER_POST_FUSED")
    nbytes = B.gdn_prefill_workspace_bytes(sep.shape)
    n_count = (300 + 31) // 32 * 48
    status_at = nbytes - 256
    assert status_at == nbytes - (n_count + 1) * 256 + n_count * 256
    buf = LayerBuffers.create(w, inp)
    ws = buf.workspace()
    monkeypatch.setenv("GDN_POST_WAIT_POLLS", "0")
    buf.run_layer(ws)
    torch.cuda.synchronize()
    assert ws[status_at:status_at + 4].cpu().numpy().view(np.uint32)[0] & 1 == 1
    # the state and history do not depend on post
    assert np.array_equal(np_(buf.state).view(np.uint32), np_(sep.state).view(np.uint32))
    monkeypatch.delenv("GDN_POST_WAIT_POLLS")
    again = LayerBuffers.create(w, inp)
    again.run_layer(ws)
    torch.cuda.synchronize()
    assert ws[status_at:status_at + 4].cpu().numpy().view(np.uint32)[0] == 0
    assert np.array_equal(np_(again.y).view(np.uint16), np_(sep.y).view(np.uint16))
