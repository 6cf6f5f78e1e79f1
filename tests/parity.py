"""Comparison rules between the GPU path and the fp64 oracle.

Bars (each written here once and used by every GPU test):
- y stored as fp16: compared with the UNROUNDED fp64 oracle.  Where the fp16
  half-spacing at y_ref is below 2e-3 (|y_ref| < 8) the error must be
  <= 2e-3.  Above that no fp16 value can meet 2e-3, so the GPU value must be
  one of the two fp16 neighbours of y_ref.
- y stored as fp32: max |dy| <= 2e-3.
- state: per (sequence, value head) ||S_gpu - S_ref||_F / ||S_ref||_F <= 1e-4,
  and elementwise max|dS| <= 2e-4 x RMS(S_ref) of the head (the Frobenius
  ratio averages one bad element of a 128 x 128 head away: a lost low half of
  a split operand moves it by ~4e-6, but that element by ~2^-11 of its size).
  max|dS| / max|S_ref| is reported beside it.
- o (fp32 scan output): the same 1e-4 relative Frobenius bar per value head,
  and elementwise max|do| <= 2e-4 x RMS(o_ref) of the head.  The second bar
  catches isolated bad elements that a Frobenius norm averages away: an
  fp32-accurate product chain stays near 1e-5 x RMS per element, while one
  product that loses the low half of a split operand (error ~2^-11 of a term)
  lands near 2e-3 x RMS.
- history: bit-exact (a copy of stored input rows).
- pre intermediates (fp32, one short fp32 chain per element): qn, kn, vc and
  beta within 1e-5 relative + 1e-6 absolute; g (|g| up to ~80) 1e-5 relative.
"""
from __future__ import annotations

import numpy as np

Y_ABS = 2e-3
STATE_REL = 1e-4
STATE_MAX_REL = 2e-4
O_REL = 1e-4
O_MAX_REL = 2e-4
PRE_RTOL, PRE_ATOL = 1e-5, 1e-6


class ParityError(AssertionError):
    pass


def _fail(msg):
    raise ParityError(msg)


def fp16_neighbours(ref: np.ndarray):
    r16 = ref.astype(np.float16)
    up = np.nextafter(r16, np.float16(np.inf))
    dn = np.nextafter(r16, np.float16(-np.inf))
    lo = np.where(r16.astype(np.float64) <= ref, r16, dn)
    hi = np.where(r16.astype(np.float64) >= ref, r16, up)
    return lo, hi


def check_y(y_gpu: np.ndarray, y_ref: np.ndarray, out: str, what="y") -> dict:
    """Returns a small report; raises ParityError on failure.  NaN in y_ref marks
    elements the oracle did not compute (sampled checks)."""
    ref = np.asarray(y_ref, np.float64).reshape(-1)
    g = np.asarray(y_gpu).reshape(-1)
    m = ~np.isnan(ref)
    ref, g = ref[m], g[m]
    if not np.isfinite(g.astype(np.float64)).all():
        _fail(f"{what}: non-finite GPU values")
    gd = g.astype(np.float64)
    if out == "f32":
        err = np.abs(gd - ref).max(initial=0.0)
        if err > Y_ABS:
            _fail(f"{what} fp32: max|dy| = {err:.3e} > {Y_ABS}")
        return dict(n=int(ref.size), max_abs=float(err))
    small = np.abs(ref) < 8.0
    err_s = np.abs(gd[small] - ref[small]).max(initial=0.0)
    if err_s > Y_ABS:
        _fail(f"{what} fp16: max|dy| = {err_s:.3e} > {Y_ABS} where |y_ref| < 8")
    big = ~small
    n_big_bad = 0
    if big.any():
        lo, hi = fp16_neighbours(ref[big])
        gb = g[big].astype(np.float16)
        ok = (gb == lo) | (gb == hi)
        n_big_bad = int((~ok).sum())
        if n_big_bad:
            _fail(f"{what} fp16: {n_big_bad} values with |y_ref| >= 8 are not an fp16 "
                  f"neighbour of y_ref")
    return dict(n=int(ref.size), max_abs_small=float(err_s), n_big=int(big.sum()))


def rel_fro_per_head(x_gpu, x_ref, axes) -> np.ndarray:
    d = np.asarray(x_gpu, np.float64) - x_ref
    num = np.sqrt((d * d).sum(axis=axes))
    den = np.sqrt((np.asarray(x_ref) ** 2).sum(axis=axes))
    return num / np.maximum(den, 1e-300)


def check_state(S_gpu, S_ref, heads=None, report=False):
    """S: [n_seq, hv, dv, dk].  Returns the worst per-head relative Frobenius
    error, or with report=True a dict of it, the worst elementwise error in
    units of the head's RMS and max|dS| / max|S_ref| over the checked heads."""
    S_gpu, S_ref = np.asarray(S_gpu), np.asarray(S_ref, np.float64)
    if heads is not None:
        S_gpu, S_ref = S_gpu[:, heads], S_ref[:, heads]
    if not np.isfinite(np.asarray(S_gpu, np.float64)).all():
        _fail("state: non-finite GPU values")
    r = rel_fro_per_head(S_gpu, S_ref, axes=(2, 3))
    zero = np.sqrt((S_ref ** 2).sum(axis=(2, 3))) == 0
    r = np.where(zero, np.abs(np.asarray(S_gpu, np.float64)).max(axis=(2, 3)), r)
    worst = float(r.max(initial=0.0))
    if not np.isfinite(worst) or worst > STATE_REL:
        _fail(f"state: worst per-head relative Frobenius error {worst:.3e} > {STATE_REL}")
    d = np.abs(np.asarray(S_gpu, np.float64) - S_ref)
    dmax = d.max(axis=(2, 3))
    rms = np.sqrt((S_ref ** 2).mean(axis=(2, 3)))
    e = np.where(zero, dmax, dmax / np.maximum(rms, 1e-300))
    elem = float(e.max(initial=0.0))
    if elem > STATE_MAX_REL:
        n, h = np.unravel_index(int(np.argmax(e)), e.shape)
        _fail(f"state: sequence {n} head {h} max|dS| = {dmax[n, h]:.3e} is {elem:.2e} x "
              f"RMS(S_ref) > {STATE_MAX_REL}")
    if not report:
        return worst
    smax = float(np.abs(S_ref).max(initial=0.0))
    return dict(fro=worst, elem_rms=elem,
                max_over_max=float(d.max(initial=0.0)) / smax if smax > 0 else float(d.max(initial=0.0)))


def check_o(o_gpu, o_ref, heads=None) -> float:
    """o: [T, hv, dv]; per value head over all tokens."""
    o_gpu, o_ref = np.asarray(o_gpu), np.asarray(o_ref)
    if heads is not None:
        o_gpu, o_ref = o_gpu[:, heads], o_ref[:, heads]
    r = rel_fro_per_head(o_gpu, o_ref, axes=(0, 2))
    worst = float(r.max(initial=0.0))
    if not np.isfinite(worst) or worst > O_REL:
        _fail(f"o: worst per-head relative Frobenius error {worst:.3e} > {O_REL}")
    d = np.abs(np.asarray(o_gpu, np.float64) - o_ref).max(axis=(0, 2))
    rms = np.sqrt((np.asarray(o_ref, np.float64) ** 2).mean(axis=(0, 2)))
    e = d / np.maximum(rms, 1e-300)
    h = int(np.argmax(e)) if e.size else 0
    if e.size and e[h] > O_MAX_REL:
        _fail(f"o: head {h} max|do| = {d[h]:.3e} is {e[h]:.2e} x RMS(o_ref) > {O_MAX_REL}")
    return worst


def check_close(name, gpu, ref, rtol=PRE_RTOL, atol=PRE_ATOL) -> float:
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(gpu - ref)
    bad = err > atol + rtol * np.abs(ref)
    if not np.isfinite(gpu).all() or bad.any():
        i = np.argmax(err - rtol * np.abs(ref))
        _fail(f"{name}: {int(bad.sum())} elements outside rtol={rtol} atol={atol}; worst "
              f"gpu={gpu.reshape(-1)[i]!r} ref={ref.reshape(-1)[i]!r}")
    return float(err.max(initial=0.0))


def check_exact(name, gpu, ref):
    if not np.array_equal(np.asarray(gpu), np.asarray(ref)):
        _fail(f"{name}: not bit-exact")
