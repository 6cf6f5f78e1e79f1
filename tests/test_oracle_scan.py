"""Pins for the oracle's gated delta-rule scan.

The recurrence per value head h (key head j = h // (hv // hk)), with a dv x dk
state S, alpha_t = exp(g_t):
    S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T,
    o_t = S_t q_t / sqrt(dk).
"Round 30 Track C Audit: gdn_pre, gdn_post, and gdn_scanr_4", section 1,
describes the kernel that runs it (one state per value head, updated in the
loop that forms the dot products against the old state); section 2 lists the
checks the pages run on it (token-blocked vs single pass, and against a
one-token step kernel).

The brute force below runs in exact rational arithmetic through a different
algebraic route, the transition-matrix form
    S_t = S_{t-1} (alpha_t (I - beta_t k_t k_t^T)) + beta_t v_t k_t^T,
with explicit dk x dk matrices.
"""
import math
from fractions import Fraction as Fr

import numpy as np
import pytest

from oracle import gdn_oracle as orc


def _mat(r, c, val=0):
    return [[Fr(val) for _ in range(c)] for _ in range(r)]


def _matmul(A, B):
    return [[sum((A[i][k] * B[k][j] for k in range(len(B))), Fr(0))
             for j in range(len(B[0]))] for i in range(len(A))]


def brute_force_scan(hk, hv, dk, dv, cu, qn, kn, vc, alpha, beta, S0, sqrt_dk):
    """Exact rational scan through the transition-matrix route."""
    G = hv // hk
    T = cu[-1]
    o = [[[None] * dv for _ in range(hv)] for _ in range(T)]
    S_out = []
    for n in range(len(cu) - 1):
        S_seq = []
        for h in range(hv):
            j = h // G
            S = [row[:] for row in S0[n][h]]
            for t in range(cu[n], cu[n + 1]):
                k, q, v = kn[t][j], qn[t][j], vc[t][h]
                a, b = alpha[t][h], beta[t][h]
                M = _mat(dk, dk)
                for r in range(dk):
                    for c in range(dk):
                        M[r][c] = a * ((1 if r == c else 0) - b * k[r] * k[c])
                S = _matmul(S, M)
                for i in range(dv):
                    for c in range(dk):
                        S[i][c] += b * v[i] * k[c]
                for i in range(dv):
                    o[t][h][i] = sum((S[i][c] * q[c] for c in range(dk)), Fr(0)) / sqrt_dk
            S_seq.append(S)
        S_out.append(S_seq)
    return o, S_out


def _rat(rs, shape, den=8, span=8):
    return rs.integers(-span, span + 1, size=shape).astype(object) * Fr(1, den)


def test_scan_matches_exact_rational_brute_force():
    rs = np.random.default_rng(12)
    hk, hv, dk, dv = 2, 4, 4, 3          # G = 2: heads 0,1 -> key 0; heads 2,3 -> key 1
    cu = [0, 5, 6, 9]                    # three sequences, ragged
    T = cu[-1]
    qn = _rat(rs, (T, hk, dk))
    kn = _rat(rs, (T, hk, dk))
    vc = _rat(rs, (T, hv, dv))
    alpha = rs.choice([Fr(1), Fr(1, 2), Fr(3, 4), Fr(1, 8), Fr(7, 8)], size=(T, hv))
    beta = rs.choice([Fr(0), Fr(1, 4), Fr(1, 2), Fr(1)], size=(T, hv))
    S0 = _rat(rs, (3, hv, dv, dk), den=4, span=4)
    o_ex, S_ex = brute_force_scan(hk, hv, dk, dv, cu, qn.tolist(), kn.tolist(), vc.tolist(),
                                  alpha.tolist(), beta.tolist(), S0.tolist(), Fr(2))
    f = np.vectorize(float)
    g = np.log(f(alpha))
    o, S = orc.scan(orc.Dims(hk, hv, dk, dv), cu, f(qn), f(kn), f(vc), g, f(beta), f(S0))
    o_ex, S_ex = f(np.array(o_ex, dtype=object)), f(np.array(S_ex, dtype=object))
    np.testing.assert_allclose(o, o_ex, rtol=1e-12, atol=1e-12 * np.abs(o_ex).max())
    np.testing.assert_allclose(S, S_ex, rtol=1e-12, atol=1e-12 * np.abs(S_ex).max())


def test_scan_worked_example_by_hand():
    # dk = dv = 2, one head, S0 = 0.  Derived by hand:
    # t=0: k=(1,0) q=(1,0) v=(2,4) beta=1/2 alpha=1:
    #      u=(1,2), S=[[1,0],[2,0]], o=S q/sqrt2=(1,2)/sqrt2
    # t=1: k=(.6,.8) q=(0,1) v=(1,0) beta=1 alpha=1/2:
    #      A=[[.5,0],[1,0]], p=A k=(.3,.6), u=(.7,-.6),
    #      S=A+u k^T=[[.92,.56],[.64,-.48]], o=(.56,-.48)/sqrt2
    kn = np.array([[[1.0, 0.0]], [[0.6, 0.8]]])
    qn = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    vc = np.array([[[2.0, 4.0]], [[1.0, 0.0]]])
    g = np.log(np.array([[1.0], [0.5]]))
    beta = np.array([[0.5], [1.0]])
    o, S = orc.scan(orc.Dims(1, 1, 2, 2), [0, 2], qn, kn, vc, g, beta, np.zeros((1, 1, 2, 2)))
    r2 = math.sqrt(2.0)
    np.testing.assert_allclose(o[0, 0], [1 / r2, 2 / r2], rtol=1e-15)
    np.testing.assert_allclose(o[1, 0], [0.56 / r2, -0.48 / r2], rtol=1e-14)
    np.testing.assert_allclose(S[0, 0], [[0.92, 0.56], [0.64, -0.48]], rtol=1e-14)


def _rand_inputs(rs, hk, hv, dk, dv, T, n_seq=1):
    return dict(qn=rs.standard_normal((T, hk, dk)) / math.sqrt(dk),
                kn=rs.standard_normal((T, hk, dk)) / math.sqrt(dk),
                vc=rs.standard_normal((T, hv, dv)),
                g=-rs.exponential(1.0, (T, hv)),
                beta=rs.uniform(0, 1, (T, hv)),
                S0=0.1 * rs.standard_normal((n_seq, hv, dv, dk)))


def test_invariant_beta0_g0_leaves_state_unchanged():
    rs = np.random.default_rng(13)
    d = _rand_inputs(rs, 2, 4, 16, 8, 10)
    d["g"][:] = 0.0
    d["beta"][:] = 0.0
    o, S = orc.scan(orc.Dims(2, 4, 16, 8), [0, 10], **d)
    assert np.array_equal(S, d["S0"])
    for h in range(4):
        ref = d["qn"][:, h // 2, :] @ d["S0"][0, h].T / 4.0
        np.testing.assert_allclose(o[:, h, :], ref, rtol=1e-13, atol=1e-15)


def test_invariant_unit_key_beta1_alpha1_writes_value():
    # k a basis vector e_j, beta = 1, alpha = 1: after the step S e_j = v
    rs = np.random.default_rng(14)
    dk, dv, T = 8, 6, 9
    d = _rand_inputs(rs, 1, 1, dk, dv, T)
    d["kn"][:] = 0.0
    js = rs.integers(0, dk, T)
    d["kn"][np.arange(T), 0, js] = 1.0
    d["g"][:] = 0.0
    d["beta"][:] = 1.0
    for t in range(1, T + 1):
        _, S = orc.scan(orc.Dims(1, 1, dk, dv), [0, t],
                        **{k: (v[:t] if k != "S0" else v) for k, v in d.items()})
        col = S[0, 0][:, js[t - 1]]
        np.testing.assert_allclose(col, d["vc"][t - 1, 0], rtol=0, atol=4e-16 * 8)


def test_closed_form_first_step_from_zero_state():
    rs = np.random.default_rng(15)
    hk, hv, dk, dv = 2, 6, 16, 8
    d = _rand_inputs(rs, hk, hv, dk, dv, 1)
    d["S0"][:] = 0.0
    o, S = orc.scan(orc.Dims(hk, hv, dk, dv), [0, 1], **d)
    for h in range(hv):
        j = h // 3
        kq = float(d["kn"][0, j] @ d["qn"][0, j])
        ref = d["beta"][0, h] * d["vc"][0, h] * kq / 4.0
        np.testing.assert_allclose(o[0, h], ref, rtol=1e-13, atol=1e-16)
        np.testing.assert_allclose(S[0, h], d["beta"][0, h] * np.outer(d["vc"][0, h], d["kn"][0, j]),
                                   rtol=1e-14, atol=1e-17)


def test_closed_form_beta0_pure_decay():
    rs = np.random.default_rng(16)
    d = _rand_inputs(rs, 1, 2, 8, 8, 12)
    d["beta"][:] = 0.0
    _, S = orc.scan(orc.Dims(1, 2, 8, 8), [0, 12], **d)
    for h in range(2):
        decay = math.exp(d["g"][:, h].sum())
        np.testing.assert_allclose(S[0, h], decay * d["S0"][0, h], rtol=1e-12)


def test_closed_form_ema_along_fixed_unit_key():
    # fixed unit key k: S_t k = alpha_t (1 - beta_t) S_{t-1} k + beta_t v_t, while
    # the components orthogonal to k only decay.
    rs = np.random.default_rng(17)
    dk, dv, T = 8, 5, 15
    d = _rand_inputs(rs, 1, 1, dk, dv, T)
    k = rs.standard_normal(dk)
    k /= np.linalg.norm(k)
    d["kn"][:, 0, :] = k
    _, S = orc.scan(orc.Dims(1, 1, dk, dv), [0, T], **d)
    a = np.exp(d["g"][:, 0])
    b = d["beta"][:, 0]
    m = d["S0"][0, 0] @ k
    P = np.eye(dk) - np.outer(k, k)
    perp = d["S0"][0, 0] @ P
    for t in range(T):
        m = a[t] * (1 - b[t]) * m + b[t] * d["vc"][t, 0]
        perp = a[t] * perp
    np.testing.assert_allclose(S[0, 0] @ k, m, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S[0, 0] @ P, perp, rtol=1e-10, atol=1e-14)


def test_closed_form_orthonormal_keys_associative_lookup():
    # alpha = beta = 1 with orthonormal keys: S_T e_j is the last value
    # written at key e_j (untouched keys keep S0's column)
    rs = np.random.default_rng(18)
    dk, dv, T = 6, 4, 20
    Q, _ = np.linalg.qr(rs.standard_normal((dk, dk)))
    d = _rand_inputs(rs, 1, 1, dk, dv, T)
    idx = rs.integers(0, dk - 1, T)        # key dk-1 is never written
    d["kn"][:, 0, :] = Q[:, idx].T
    d["g"][:] = 0.0
    d["beta"][:] = 1.0
    _, S = orc.scan(orc.Dims(1, 1, dk, dv), [0, T], **d)
    for j in range(dk):
        hits = np.nonzero(idx == j)[0]
        want = d["vc"][hits[-1], 0] if len(hits) else d["S0"][0, 0] @ Q[:, j]
        np.testing.assert_allclose(S[0, 0] @ Q[:, j], want, rtol=1e-12, atol=1e-13)


def test_split_invariance_is_bitwise():
    rs = np.random.default_rng(19)
    hk, hv, dk, dv = 2, 4, 16, 16
    T = 40
    d = _rand_inputs(rs, hk, hv, dk, dv, T)
    dims = orc.Dims(hk, hv, dk, dv)
    o_whole, S_whole = orc.scan(dims, [0, T], **d)
    S = d["S0"]
    outs = []
    s = 0
    for L in [1, 3, 7, 16, 13]:
        part = {k: v[s:s + L] for k, v in d.items() if k != "S0"}
        o, S = orc.scan(dims, [0, L], S0=S, **part)
        outs.append(o)
        s += L
    assert np.array_equal(np.concatenate(outs), o_whole)
    assert np.array_equal(S, S_whole)


def test_varlen_and_head_subset_agree_with_single_runs():
    rs = np.random.default_rng(20)
    hk, hv, dk, dv = 2, 6, 8, 8
    lens = [4, 0, 9, 1]
    cu = np.concatenate([[0], np.cumsum(lens)])
    d = _rand_inputs(rs, hk, hv, dk, dv, cu[-1], n_seq=4)
    dims = orc.Dims(hk, hv, dk, dv)
    o, S = orc.scan(dims, cu, **d)
    for n, L in enumerate(lens):
        part = {k: v[cu[n]:cu[n + 1]] for k, v in d.items() if k != "S0"}
        on, Sn = orc.scan(dims, [0, L], S0=d["S0"][n:n + 1], **part)
        assert np.array_equal(o[cu[n]:cu[n + 1]], on)
        assert np.array_equal(S[n:n + 1], Sn)
    # T = 0 leaves the state unchanged
    assert np.array_equal(S[1], d["S0"][1])
    os_, Ss = orc.scan(dims, cu, heads=[4, 1], **d)
    assert np.array_equal(os_[:, [1, 4]], o[:, [1, 4]])
    assert np.isnan(os_[:, 0]).all() and np.array_equal(Ss[:, [1, 4]], S[:, [1, 4]])


@pytest.mark.parametrize("G", [1, 3])
def test_key_head_grouping_is_contiguous(G):
    # value head h must read key head h // G: giving each key head its own
    # distinct key and checking the first-step closed form per head pins it.
    rs = np.random.default_rng(21)
    hk, dk, dv = 2, 8, 4
    hv = hk * G
    d = _rand_inputs(rs, hk, hv, dk, dv, 1)
    d["S0"][:] = 0.0
    _, S = orc.scan(orc.Dims(hk, hv, dk, dv), [0, 1], **d)
    for h in range(hv):
        for j in range(hk):
            ref = d["beta"][0, h] * np.outer(d["vc"][0, h], d["kn"][0, j])
            assert np.allclose(S[0, h], ref, rtol=1e-14) == (j == h // G)
