"""Pins for the oracle's post stage and the whole layer.

Post ("Round 30 Track C Audit: gdn_pre, gdn_post, and gdn_scanr_4", section 1;
"opus_r25_gdn -- round 25 track A", "shipped"): one sum of squares per
(token, value head) row, gamma, and a sigmoid gate.  It is the library
RMSNorm with weight gamma times the library SiLU of z.
"""
import numpy as np
import torch
import torch.nn.functional as F

from gated_deltanet_linear_pre_amd import synth
from oracle import gdn_oracle as orc


def test_post_matches_library_rmsnorm_times_silu():
    rs = np.random.default_rng(30)
    for o_std in (1e-4, 8e-4, 1.0):
        o = o_std * rs.standard_normal((33, 5, 128))
        z = rs.standard_normal((33, 5, 128))
        gamma = 1 + 0.1 * rs.standard_normal(128)
        y = orc.post(o, z, gamma, 1e-6)
        ref = (F.rms_norm(torch.from_numpy(o), [128], torch.from_numpy(gamma), 1e-6)
               * F.silu(torch.from_numpy(z))).numpy()
        np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-15)


def test_post_zero_cases_and_scale_invariance():
    rs = np.random.default_rng(31)
    o = rs.standard_normal((4, 3, 16))
    z = rs.standard_normal((4, 3, 16))
    gamma = 1 + 0.1 * rs.standard_normal(16)
    assert np.array_equal(orc.post(np.zeros_like(o), z, gamma, 1e-6), np.zeros_like(o))
    assert not np.any(orc.post(o, np.zeros_like(z), gamma, 1e-6))
    # relative effect of eps is about eps / (2 ms); here ms >= 0.1
    np.testing.assert_allclose(orc.post(37.0 * o, z, gamma, 1e-6), orc.post(o, z, gamma, 1e-6),
                               rtol=1e-5)
    # in the eps-dominated regime the norm is no longer scale-free
    small = 1e-5 * o
    assert not np.allclose(orc.post(small, z, gamma, 1e-6), orc.post(o, z, gamma, 1e-6), rtol=1e-2)


def test_layer_continuation_is_bitwise():
    # one call over the concatenation == segment calls carrying state and
    # history (pages: single-pass vs token-blocked scan, prompt chunks).
    w = synth.Workload("t", hk=2, hv=4, seqlens=(45,), io="f32", out="f32",
                       s0_std=0.05, hist_std=1.0, dk=16, dv=8)
    inp = synth.layer_inputs(w)
    dims = orc.Dims(2, 4, 16, 8)
    whole = orc.layer(dims, [0, 45], inp)
    S, hist, s = inp["S0"], inp["hist"], 0
    ys, os_ = [], []
    for L in (1, 3, 2, 20, 19):
        part = dict(inp, S0=S, hist=hist)
        for k in ("qkv", "a", "b", "z"):
            part[k] = inp[k][s:s + L]
        r = orc.layer(dims, [0, L], part)
        ys.append(r["y"])
        os_.append(r["o"])
        S, hist, s = r["S"], r["hist"], s + L
    assert np.array_equal(np.concatenate(os_), whole["o"])
    assert np.array_equal(np.concatenate(ys), whole["y"])
    assert np.array_equal(S, whole["S"]) and np.array_equal(hist, whole["hist"])


def test_layer_head_subset_matches_full():
    w = synth.Workload("t", hk=2, hv=6, seqlens=(9, 4), io="f32", out="f32", dk=8, dv=8)
    inp = synth.layer_inputs(w)
    dims = orc.Dims(2, 6, 8, 8)
    cu = w.cu_seqlens()
    full = orc.layer(dims, cu, inp)
    sub = orc.layer(dims, cu, inp, heads=[5, 0])
    for k in ("y", "o"):
        assert np.array_equal(sub[k][:, [0, 5]], full[k][:, [0, 5]])
    assert np.array_equal(sub["S"][:, [0, 5]], full["S"][:, [0, 5]])
