"""NumPy-facing wrapper around the fp64 C oracle (``gdn_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg use this module; the GPU library never does, and this module
imports nothing from it.

Every function takes arrays of any float dtype, widens them to float64 (exact
for fp16 and fp32 storage), calls the C routine and returns float64 arrays.
The layouts are those documented at the top of ``gdn_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
# A test may point this at a deliberately broken build of the oracle to show
# that the pins catch it (tests/test_oracle_mutants.py).
_LIB_OVERRIDE = os.environ.get("GDN_ORACLE_LIB")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
             "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"],
            check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            path = _LIB_OVERRIDE
        else:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            path = _LIB
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L = ctypes.c_int64
        D = ctypes.c_double
        lib.gdn_oracle_set_threads.argtypes = [I]
        lib.gdn_oracle_max_threads.restype = I
        lib.gdn_oracle_conv.argtypes = [I, I, P, P, P, P, P]
        lib.gdn_oracle_history.argtypes = [I, I, P, P, P, P]
        lib.gdn_oracle_silu.argtypes = [L, P, P]
        lib.gdn_oracle_l2norm.argtypes = [L, I, P, D, P]
        lib.gdn_oracle_gates.argtypes = [L, I, P, P, P, P, P, P]
        lib.gdn_oracle_pre.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, P, D,
                                       P, P, P, P, P, P, P]
        lib.gdn_oracle_scan.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, I]
        lib.gdn_oracle_post.argtypes = [L, I, P, P, P, D, P]
        for f in ("gdn_oracle_conv", "gdn_oracle_history", "gdn_oracle_silu",
                  "gdn_oracle_l2norm", "gdn_oracle_gates", "gdn_oracle_pre",
                  "gdn_oracle_scan", "gdn_oracle_post", "gdn_oracle_set_threads"):
            getattr(lib, f).restype = None
        _lib = lib
    return _lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x), dtype=np.float64)


def _cu(cu) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(cu), dtype=np.int64)


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def set_threads(n: int) -> None:
    _load().gdn_oracle_set_threads(int(n))


def max_threads() -> int:
    return int(_load().gdn_oracle_max_threads())


@dataclass
class Dims:
    hk: int
    hv: int
    dk: int = 128
    dv: int = 128

    @property
    def C(self) -> int:
        return 2 * self.hk * self.dk + self.hv * self.dv


# ---------------------------------------------------------------- steps

def conv(qkv, conv_w, hist, cu) -> np.ndarray:
    qkv, conv_w, hist, cu = _f64(qkv), _f64(conv_w), _f64(hist), _cu(cu)
    T, C = qkv.shape
    n_seq = len(cu) - 1
    assert conv_w.shape == (C, 4) and hist.shape == (n_seq, 3, C) and cu[-1] == T
    out = np.empty((T, C))
    _load().gdn_oracle_conv(C, n_seq, _p(cu), _p(qkv), _p(conv_w), _p(hist), _p(out))
    return out


def history(qkv, hist, cu) -> np.ndarray:
    qkv, hist, cu = _f64(qkv), _f64(hist), _cu(cu)
    T, C = qkv.shape
    n_seq = len(cu) - 1
    out = np.empty_like(hist)
    _load().gdn_oracle_history(C, n_seq, _p(cu), _p(qkv), _p(hist), _p(out))
    return out


def silu(x) -> np.ndarray:
    x = _f64(x)
    y = np.empty_like(x)
    _load().gdn_oracle_silu(x.size, _p(x), _p(y))
    return y


def l2norm(x, eps: float) -> np.ndarray:
    x = _f64(x)
    d = x.shape[-1]
    y = np.empty_like(x)
    _load().gdn_oracle_l2norm(x.size // d, d, _p(x), float(eps), _p(y))
    return y


def gates(a, b, A_log, dt_bias):
    a, b, A_log, dt_bias = _f64(a), _f64(b), _f64(A_log), _f64(dt_bias)
    T, hv = a.shape
    g = np.empty_like(a)
    beta = np.empty_like(a)
    _load().gdn_oracle_gates(T, hv, _p(a), _p(b), _p(A_log), _p(dt_bias), _p(g), _p(beta))
    return g, beta


def pre(dims: Dims, cu, qkv, conv_w, a, b, A_log, dt_bias, hist, eps_l2: float):
    """Returns dict qn [T,hk,dk], kn [T,hk,dk], vc [T,hv,dv], g, beta [T,hv],
    hist [n_seq,3,C] (the carried history after the call)."""
    cu = _cu(cu)
    qkv, conv_w, a, b = _f64(qkv), _f64(conv_w), _f64(a), _f64(b)
    A_log, dt_bias, hist = _f64(A_log), _f64(dt_bias), _f64(hist)
    T = int(cu[-1])
    n_seq = len(cu) - 1
    hk, hv, dk, dv = dims.hk, dims.hv, dims.dk, dims.dv
    assert qkv.shape == (T, dims.C) and a.shape == (T, hv) and b.shape == (T, hv)
    assert hist.shape == (n_seq, 3, dims.C)
    qn = np.empty((T, hk, dk))
    kn = np.empty((T, hk, dk))
    vc = np.empty((T, hv, dv))
    g = np.empty((T, hv))
    beta = np.empty((T, hv))
    hist_out = np.empty_like(hist)
    work = np.empty(2 * T * dims.C)
    _load().gdn_oracle_pre(hk, hv, dk, dv, n_seq, _p(cu), _p(qkv), _p(conv_w), _p(a), _p(b),
                           _p(A_log), _p(dt_bias), _p(hist), float(eps_l2), _p(qn), _p(kn),
                           _p(vc), _p(g), _p(beta), _p(hist_out), _p(work))
    return dict(qn=qn, kn=kn, vc=vc, g=g, beta=beta, hist=hist_out)


def scan(dims: Dims, cu, qn, kn, vc, g, beta, S0, heads=None):
    """Returns (o [T,hv,dv], S [n_seq,hv,dv,dk]).  With `heads`, only those value
    heads are run; o and S of the other heads are NaN."""
    cu = _cu(cu)
    qn, kn, vc, g, beta, S0 = _f64(qn), _f64(kn), _f64(vc), _f64(g), _f64(beta), _f64(S0)
    T = int(cu[-1])
    n_seq = len(cu) - 1
    hk, hv, dk, dv = dims.hk, dims.hv, dims.dk, dims.dv
    assert qn.shape == (T, hk, dk) and kn.shape == (T, hk, dk) and vc.shape == (T, hv, dv)
    assert g.shape == (T, hv) and beta.shape == (T, hv) and S0.shape == (n_seq, hv, dv, dk)
    o = np.full((T, hv, dv), np.nan)
    S = np.full_like(S0, np.nan)
    if heads is None:
        hp, nh = None, 0
    else:
        harr = np.ascontiguousarray(np.asarray(heads), dtype=np.int32)
        assert harr.min() >= 0 and harr.max() < hv
        hp, nh = _p(harr), int(harr.size)
    _load().gdn_oracle_scan(hk, hv, dk, dv, n_seq, _p(cu), _p(qn), _p(kn), _p(vc), _p(g),
                            _p(beta), _p(S0), _p(S), _p(o), hp, nh)
    return o, S


def post(o, z, gamma, eps_rms: float) -> np.ndarray:
    """y (unrounded), same shape as o ([..., dv])."""
    o, z, gamma = _f64(o), _f64(z), _f64(gamma)
    dv = o.shape[-1]
    assert z.shape == o.shape and gamma.shape == (dv,)
    y = np.empty_like(o)
    _load().gdn_oracle_post(o.size // dv, dv, _p(o), _p(z), _p(gamma), float(eps_rms), _p(y))
    return y


def layer(dims: Dims, cu, inp: dict, eps_l2: float = 1e-6, eps_rms: float = 1e-6, heads=None):
    """The whole path, pre -> scan -> post, on one layer's inputs.

    `inp` holds qkv, conv_w, a, b, A_log, dt_bias, z, gamma, hist, S0 (any float
    dtype).  Returns the pre intermediates plus o, y (unrounded), the new hist
    and the final state S.  With `heads`, the scan and post run on those value
    heads only (y and o of the other heads are NaN)."""
    pr = pre(dims, cu, inp["qkv"], inp["conv_w"], inp["a"], inp["b"], inp["A_log"],
             inp["dt_bias"], inp["hist"], eps_l2)
    o, S = scan(dims, cu, pr["qn"], pr["kn"], pr["vc"], pr["g"], pr["beta"], inp["S0"],
                heads=heads)
    T = o.shape[0]
    z = _f64(inp["z"]).reshape(T, dims.hv, dims.dv)
    if heads is None:
        y = post(o, z, inp["gamma"], eps_rms)
    else:
        y = np.full_like(o, np.nan)
        hs = np.asarray(heads)
        y[:, hs, :] = post(o[:, hs, :], z[:, hs, :], inp["gamma"], eps_rms)
    out = dict(pr)
    out.update(o=o, y=y, S=S)
    return out
