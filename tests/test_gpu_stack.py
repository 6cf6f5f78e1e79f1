"""The two full-size workloads through the launch the benchmark times
(gdn_prefill_layer), against the fp64 oracle on every value head:

- the 36-layer T=2048 stack: every layer, with fp16 and with fp32 output;
- the long varlen batch (T = 16384, 8192, 2048, 511 packed, fp32 output):
  layers 0, 17 and 35.

("round 10 track b: gdn vectorization and scan", "correctness": every buffer
checked for every T and output-precision combination; "Round 30 Track C
Audit: gdn_pre, gdn_post, and gdn_scanr_4", section 2: the ten buffers
compared per stage.)
"""
import numpy as np
import pytest
import torch

from gated_deltanet_linear_pre_amd import synth
from gated_deltanet_linear_pre_amd.buffers import LayerBuffers
from oracle import gdn_oracle as orc

from . import parity
from .gpu_util import banner, np_

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _gpu_layer(w, inp, out):
    buf = LayerBuffers.create(w, inp, out=out)
    buf.run_layer(buf.workspace())
    torch.cuda.synchronize()
    T = w.total_T
    res = dict(y=np_(buf.y).reshape(T, w.hv, 128), S=np_(buf.state), hist=np_(buf.hist))
    del buf
    return res


def _check(w, g, ref, out):
    rep = parity.check_y(g["y"], ref["y"], out)
    st = parity.check_state(g["S"], ref["S"], report=True)
    parity.check_exact("hist", g["hist"].astype(np.float64), ref["hist"])
    return rep, st


@pytest.mark.parametrize("layer", range(36))
def test_stack36_every_layer_and_head(gpu, layer):
    w16 = W["prod36_t2048_fp16out"]
    inp = synth.layer_inputs(w16, layer)
    banner("gdn_prefill_layer", w16.name, f"layer={layer}", "out=f16 and f32")
    g16 = _gpu_layer(w16, inp, "f16")
    g32 = _gpu_layer(w16, inp, "f32")
    ref = orc.layer(orc.Dims(w16.hk, w16.hv), w16.cu_seqlens(), inp)
    r16, st = _check(w16, g16, ref, "f16")
    r32, _ = _check(w16, g32, ref, "f32")
    # the output precision does not touch the state or the history
    assert np.array_equal(g16["S"].view(np.uint32), g32["S"].view(np.uint32))
    banner(f"  y16 max|dy| {r16['max_abs_small']:.2e}, y32 max|dy| {r32['max_abs']:.2e}, state "
           f"fro {st['fro']:.2e} elem {st['elem_rms']:.2e}")


@pytest.mark.parametrize("layer", [0, 17, 35])
def test_varlen_long_batch_every_head(gpu, layer):
    w = W["prod36_varlen4_fp32out"]
    inp = synth.layer_inputs(w, layer)
    banner("gdn_prefill_layer", w.name, f"layer={layer}", f"lens={w.seqlens}")
    g = _gpu_layer(w, inp, "f32")
    banner("  oracle")
    ref = orc.layer(orc.Dims(w.hk, w.hv), w.cu_seqlens(), inp)
    r, st = _check(w, g, ref, "f32")
    banner(f"  y max|dy| {r['max_abs']:.2e}, state fro {st['fro']:.2e} elem {st['elem_rms']:.2e}")
