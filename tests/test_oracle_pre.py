"""Pins for the oracle's pre stage (conv, history, SiLU, L2 norm, gates).

Each check ties the oracle to something other than itself: a library routine
that computes the same definition by another route, a closed form, an
impulse response, or an exact invariant.  See "Round 30 Track C Audit: gdn_pre,
gdn_post, and gdn_scanr_4", section 1, for the stage structure these follow.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

from oracle import gdn_oracle as orc


def _rand(rs, *shape):
    return rs.standard_normal(shape)


# ------------------------------------------------------------------ conv

def test_conv_impulse_response_fixes_tap_orientation():
    # zero history, unit impulse at (t0, c): output at t0 + r is w[c, 3 - r]
    # (tap 3 multiplies the current token); nothing leaks to other channels
    # or earlier tokens, and there is no bias.
    rs = np.random.default_rng(0)
    T, C, t0, c = 12, 3, 5, 1
    x = np.zeros((T, C))
    x[t0, c] = 1.0
    w = _rand(rs, C, 4)
    out = orc.conv(x, w, np.zeros((1, 3, C)), [0, T])
    expect = np.zeros((T, C))
    for r in range(4):
        expect[t0 + r, c] = w[c, 3 - r]
    assert np.array_equal(out, expect)


def test_conv_history_impulse():
    # an impulse in history row r (of 3, oldest first) reaches tokens 0..r
    # through taps r, r-1, ..., 0... i.e. token tau sees it through tap r - tau
    rs = np.random.default_rng(1)
    T, C = 6, 2
    w = _rand(rs, C, 4)
    for r in range(3):
        hist = np.zeros((1, 3, C))
        hist[0, r, 0] = 1.0
        out = orc.conv(np.zeros((T, C)), w, hist, [0, T])
        expect = np.zeros((T, C))
        for tau in range(T):
            m = r - tau
            if 0 <= m <= 3:
                expect[tau, 0] = w[0, m]
        assert np.array_equal(out, expect), r


def test_conv_matches_torch_depthwise_conv1d():
    # library route: torch depthwise conv1d (a cross-correlation) over the
    # history-extended input, no padding, one group per channel.
    rs = np.random.default_rng(2)
    T, C = 29, 40
    x, w, h = _rand(rs, T, C), _rand(rs, C, 4), _rand(rs, 1, 3, C)
    out = orc.conv(x, w, h, [0, T])
    xbar = torch.from_numpy(np.concatenate([h[0], x], 0).T[None].copy())
    ref = F.conv1d(xbar, torch.from_numpy(w[:, None, :].copy()), groups=C)[0].T.numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-13)


def test_conv_matches_banded_matrix_product():
    # another route: each channel's conv is a (T x (T+3)) banded matrix times
    # the extended column.
    rs = np.random.default_rng(3)
    T, C = 17, 5
    x, w, h = _rand(rs, T, C), _rand(rs, C, 4), _rand(rs, 1, 3, C)
    out = orc.conv(x, w, h, [0, T])
    xbar = np.concatenate([h[0], x], 0)
    for c in range(C):
        M = np.zeros((T, T + 3))
        for tau in range(T):
            M[tau, tau:tau + 4] = w[c]
        np.testing.assert_allclose(out[:, c], M @ xbar[:, c], rtol=1e-13, atol=1e-13)


def test_conv_varlen_uses_own_history():
    rs = np.random.default_rng(4)
    lens = [5, 1, 2, 9]
    C = 7
    cu = np.concatenate([[0], np.cumsum(lens)])
    x, w, h = _rand(rs, cu[-1], C), _rand(rs, C, 4), _rand(rs, len(lens), 3, C)
    out = orc.conv(x, w, h, cu)
    for n, L in enumerate(lens):
        part = orc.conv(x[cu[n]:cu[n + 1]], w, h[n:n + 1], [0, L])
        assert np.array_equal(out[cu[n]:cu[n + 1]], part)


# --------------------------------------------------------------- history

@pytest.mark.parametrize("T", [0, 1, 2, 3, 4, 11])
def test_history_is_last_three_rows_of_extended_input(T):
    rs = np.random.default_rng(5 + T)
    C = 6
    x, h = _rand(rs, T, C), _rand(rs, 1, 3, C)
    out = orc.history(x, h, [0, T])
    xbar = np.concatenate([h[0], x], 0)
    assert np.array_equal(out[0], xbar[-3:])
    if T == 0:
        assert np.array_equal(out, h)


def test_conv_and_history_split_invariance():
    # processing a sequence in pieces, carrying the history, is bit-identical
    # to one call (pages: single-pass vs token-blocked scan; prompt chunks).
    rs = np.random.default_rng(7)
    C, pieces = 9, [1, 3, 2, 7, 4]
    T = sum(pieces)
    x, w, h = _rand(rs, T, C), _rand(rs, C, 4), _rand(rs, 1, 3, C)
    whole = orc.conv(x, w, h, [0, T])
    hw = orc.history(x, h, [0, T])
    hc, s, parts = h, 0, []
    for L in pieces:
        parts.append(orc.conv(x[s:s + L], w, hc, [0, L]))
        hc = orc.history(x[s:s + L], hc, [0, L])
        s += L
    assert np.array_equal(np.concatenate(parts), whole)
    assert np.array_equal(hc, hw)


# ------------------------------------------------------------------ silu

def test_silu_against_library_and_special_values():
    x = np.concatenate([np.linspace(-40, 40, 2001), [0.0, -800.0, 800.0]])
    y = orc.silu(x)
    np.testing.assert_allclose(y, x * scipy.special.expit(x), rtol=1e-15, atol=1e-300)
    assert orc.silu([0.0])[0] == 0.0
    assert orc.silu([800.0])[0] == 800.0
    assert abs(orc.silu([-800.0])[0]) == 0.0
    # SiLU(x) - SiLU(-x) = x
    xs = np.linspace(-10, 10, 101)
    np.testing.assert_allclose(orc.silu(xs) - orc.silu(-xs), xs, atol=1e-14)


# ---------------------------------------------------------------- l2norm

def test_l2norm_closed_form_and_direction():
    rs = np.random.default_rng(8)
    eps = 1e-6
    x = _rand(rs, 50, 128) * np.logspace(-4, 1, 50)[:, None]
    y = orc.l2norm(x, eps)
    s = (x * x).sum(-1)
    np.testing.assert_allclose((y * y).sum(-1), s / (s + eps), rtol=1e-13)
    # same direction: y = c x with c > 0 per row
    c = y / x
    np.testing.assert_allclose(c, c[:, :1].repeat(128, 1), rtol=1e-13)
    assert (c > 0).all()
    assert np.array_equal(orc.l2norm(np.zeros((2, 4)), eps), np.zeros((2, 4)))


def test_l2norm_scale_invariance_when_eps_negligible():
    rs = np.random.default_rng(9)
    x = _rand(rs, 10, 128)
    np.testing.assert_allclose(orc.l2norm(1000 * x, 1e-6), orc.l2norm(x, 1e-6), rtol=1e-8)


# ----------------------------------------------------------------- gates

def test_gates_special_values_and_asymptotes():
    A_log = np.array([0.0, math.log(4.0), 1.3])
    dt = np.array([0.0, 0.5, -0.25])
    hv = 3
    # a + dt_bias = 0: g = -exp(A_log) ln 2 ; b = 0: beta = 1/2
    a = -dt[None, :].copy()
    b = np.zeros((1, hv))
    g, beta = orc.gates(a, b, A_log, dt)
    np.testing.assert_allclose(g[0], -np.exp(A_log) * math.log(2.0), rtol=1e-15)
    assert np.array_equal(beta[0], np.full(hv, 0.5))
    # large argument: softplus(x) -> x ; very negative: softplus(x) -> e^x
    a = np.array([[60.0, 60.0, 60.0], [-60.0, -60.0, -60.0]]) - dt
    g, _ = orc.gates(a, np.zeros((2, hv)), A_log, dt)
    np.testing.assert_allclose(g[0], -np.exp(A_log) * 60.0, rtol=1e-15)
    np.testing.assert_allclose(g[1], -np.exp(A_log) * math.exp(-60.0), rtol=1e-13)


def test_gates_against_library_softplus_and_sigmoid():
    rs = np.random.default_rng(10)
    T, hv = 64, 5
    a, b = 4 * _rand(rs, T, hv), 4 * _rand(rs, T, hv)
    A_log, dt = rs.uniform(0, math.log(16), hv), 0.5 * _rand(rs, hv)
    g, beta = orc.gates(a, b, A_log, dt)
    sp = np.logaddexp(0.0, a + dt)  # library softplus
    np.testing.assert_allclose(-g / np.exp(A_log), sp, rtol=1e-14)
    np.testing.assert_allclose(beta, scipy.special.expit(b), rtol=1e-15)
    np.testing.assert_allclose(beta + orc.gates(a, -b, A_log, dt)[1], 1.0, atol=1e-15)
    assert (g < 0).all() and ((beta > 0) & (beta < 1)).all()


# -------------------------------------------------------- whole pre stage

def test_pre_block_split_head_order_and_norm_via_library():
    # identity conv (tap 3 = 1), zero history: the pre outputs are the
    # library SiLU of each channel block, q and k normalised per key head.
    rs = np.random.default_rng(11)
    dims = orc.Dims(hk=2, hv=6, dk=8, dv=4)
    T, C = 7, dims.C
    x = _rand(rs, T, C)
    w = np.zeros((C, 4))
    w[:, 3] = 1.0
    a, b = _rand(rs, T, 6), _rand(rs, T, 6)
    A_log, dt = rs.uniform(0, 2, 6), _rand(rs, 6)
    out = orc.pre(dims, [0, T], x, w, a, b, A_log, dt, np.zeros((1, 3, C)), 1e-6)
    s = F.silu(torch.from_numpy(x)).numpy()
    q = s[:, :16].reshape(T, 2, 8)
    k = s[:, 16:32].reshape(T, 2, 8)
    v = s[:, 32:].reshape(T, 6, 4)
    nq = F.normalize(torch.from_numpy(q), dim=-1).numpy()
    nk = F.normalize(torch.from_numpy(k), dim=-1).numpy()
    # F.normalize divides by the norm; the oracle by sqrt(norm^2 + 1e-6)
    np.testing.assert_allclose(out["qn"], nq, rtol=1e-5)
    np.testing.assert_allclose(out["kn"], nk, rtol=1e-5)
    rq = out["qn"] / nq
    assert np.all(rq < 1.0)  # the epsilon only ever shrinks the norm
    np.testing.assert_allclose(out["vc"], v, rtol=1e-15)
    g, beta = orc.gates(a, b, A_log, dt)
    assert np.array_equal(out["g"], g) and np.array_equal(out["beta"], beta)
    assert np.array_equal(out["hist"][0], x[-3:])
