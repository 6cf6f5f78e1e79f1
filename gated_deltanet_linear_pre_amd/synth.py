"""Seeded synthetic inputs for the GDN prefill path.

This module only draws random numbers and rounds them to a storage dtype; it
holds none of the path's arithmetic.  The GPU tests, the benchmark and the
oracle-side checks all take their inputs from here, so both sides read the
same bytes.

Recipe (every tensor gets its own PCG64 stream, so any one layer or tensor
can be drawn alone):
    rng(seed_words, tensor) = numpy.random.default_rng([*seed_words, TENSOR_ID])
    normal draws are float32 standard normals times the stated standard
    deviation (plus mean), then rounded (RNE) to the storage dtype.

    qkv      [T, C]          N(0, 1)
    conv_w   [C, 4]          N(0, 0.25)
    a, b     [T, hv]         N(0, 1)
    A_log    [hv]            U[0, ln 16)
    dt_bias  [hv]            N(0, 0.5)
    z        [T, hv*dv]      N(0, 1)
    gamma    [dv]            1 + N(0, 0.1)
    S0       [n_seq, hv, dv, dk]  fp32, zero or N(0, s0_std)
    hist     [n_seq, 3, C]   zero or N(0, hist_std)

The production widths (hk=16, hv=48, head dim 128, 10240 channels) are those
of "round 10 track b: gdn vectorization and scan", "source and execution".
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Sequence

import numpy as np

TENSOR_ID = {"qkv": 1, "conv_w": 2, "a": 3, "b": 4, "A_log": 5, "dt_bias": 6,
             "z": 7, "gamma": 8, "S0": 9, "hist": 10,
             # stage-isolated draws
             "s_qn": 21, "s_kn": 22, "s_vc": 23, "s_g": 24, "s_beta": 25,
             "p_o": 31}

NP_DTYPE = {"f32": np.float32, "f16": np.float16}


def rng(seed_words: Sequence[int], tensor: str) -> np.random.Generator:
    return np.random.default_rng([*map(int, seed_words), TENSOR_ID[tensor]])


def normal(seed_words, tensor, shape, std, mean=0.0, dtype="f32") -> np.ndarray:
    x = rng(seed_words, tensor).standard_normal(shape, dtype=np.float32)
    x *= np.float32(std)
    if mean:
        x += np.float32(mean)
    return x.astype(NP_DTYPE[dtype])


def uniform(seed_words, tensor, shape, lo, hi, dtype="f32") -> np.ndarray:
    return rng(seed_words, tensor).uniform(lo, hi, shape).astype(NP_DTYPE[dtype])


@dataclass(frozen=True)
class Workload:
    """One named workload: head counts, sequence lengths, dtypes, layers, seeds."""
    name: str
    hk: int
    hv: int
    seqlens: tuple
    io: str = "f16"            # storage of qkv, conv_w, a, b, A_log, dt_bias, z, gamma, hist
    out: str = "f16"           # storage of y
    layers: int = 1
    seed: tuple = (21,)        # seed words of layer 0
    per_layer_seed: str = "offset"   # "offset": (seed[0] + l,), "append": (*seed, l)
    s0_std: float = 0.0
    hist_std: float = 0.0
    dk: int = 128
    dv: int = 128
    segments: tuple = field(default=())   # continuation split of the single sequence

    @property
    def C(self) -> int:
        return 2 * self.hk * self.dk + self.hv * self.dv

    @property
    def total_T(self) -> int:
        return int(sum(self.seqlens))

    @property
    def max_T(self) -> int:
        return int(max(self.seqlens)) if self.seqlens else 0

    @property
    def n_seq(self) -> int:
        return len(self.seqlens)

    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seqlens)]).astype(np.int32)

    def layer_seed(self, layer: int) -> tuple:
        if self.per_layer_seed == "offset":
            return (self.seed[0] + layer,)
        return (*self.seed, layer)


# The five workloads.  Names say what they are; sizes are per layer.
WORKLOADS = {
    w.name: w for w in (
        Workload("tiny_h2x6_t37_fp32", hk=2, hv=6, seqlens=(37,), io="f32", out="f32",
                 seed=(21,)),
        Workload("prod_t512_fp16", hk=16, hv=48, seqlens=(512,), seed=(1,)),
        Workload("prod36_t2048_fp16out", hk=16, hv=48, seqlens=(2048,), layers=36,
                 seed=(100,)),
        Workload("prod36_t2048_fp32out", hk=16, hv=48, seqlens=(2048,), layers=36,
                 out="f32", seed=(100,)),
        Workload("prod_continuation_fp16", hk=16, hv=48, seqlens=(1365,), seed=(21,),
                 s0_std=0.05, hist_std=1.0, segments=(1, 3, 37, 300, 1024)),
        Workload("prod36_varlen4_fp32out", hk=16, hv=48, seqlens=(16384, 8192, 2048, 511),
                 layers=36, out="f32", seed=(7,), per_layer_seed="append"),
    )
}


def layer_inputs(w: Workload, layer: int = 0) -> dict:
    """All inputs of one layer as numpy arrays in their storage dtypes."""
    s = w.layer_seed(layer)
    T, C, hv, dv, dk, io = w.total_T, w.C, w.hv, w.dv, w.dk, w.io
    d = dict(
        qkv=normal(s, "qkv", (T, C), 1.0, dtype=io),
        conv_w=normal(s, "conv_w", (C, 4), 0.25, dtype=io),
        a=normal(s, "a", (T, hv), 1.0, dtype=io),
        b=normal(s, "b", (T, hv), 1.0, dtype=io),
        A_log=uniform(s, "A_log", (hv,), 0.0, math.log(16.0), dtype=io),
        dt_bias=normal(s, "dt_bias", (hv,), 0.5, dtype=io),
        z=normal(s, "z", (T, hv * dv), 1.0, dtype=io),
        gamma=normal(s, "gamma", (dv,), 0.1, mean=1.0, dtype=io),
    )
    n = w.n_seq
    if w.s0_std:
        d["S0"] = normal(s, "S0", (n, hv, dv, dk), w.s0_std, dtype="f32")
    else:
        d["S0"] = np.zeros((n, hv, dv, dk), np.float32)
    if w.hist_std:
        d["hist"] = normal(s, "hist", (n, 3, C), w.hist_std, dtype=io)
    else:
        d["hist"] = np.zeros((n, 3, C), NP_DTYPE[io])
    return d


def scan_inputs(hk: int, hv: int, seqlens, seed=(5,), dk=128, dv=128,
                s0_std=0.05, g_scale=1.5) -> dict:
    """Stage-isolated fp32 scan inputs with the scales the pre stage produces:
    q and k entries N(0, 1/sqrt(dk)) (so |q|, |k| are near 1), v N(0, 1),
    log decay g = -Exp(g_scale), beta U(0, 1), S0 N(0, s0_std)."""
    T = int(sum(seqlens))
    n = len(seqlens)
    sd = 1.0 / math.sqrt(dk)
    g = -rng(seed, "s_g").exponential(g_scale, (T, hv)).astype(np.float32)
    return dict(
        qn=normal(seed, "s_qn", (T, hk, dk), sd),
        kn=normal(seed, "s_kn", (T, hk, dk), sd),
        vc=normal(seed, "s_vc", (T, hv, dv), 1.0),
        g=g,
        beta=uniform(seed, "s_beta", (T, hv), 0.0, 1.0),
        S0=normal(seed, "S0", (n, hv, dv, dk), s0_std) if s0_std else
        np.zeros((n, hv, dv, dk), np.float32),
    )


def post_inputs(n_tok: int, hv: int, dv=128, seed=(6,), o_std=8e-4, io="f16") -> dict:
    """Stage-isolated post inputs: o N(0, o_std) fp32 (the scan's output scale,
    where the RMS epsilon matters), z N(0, 1), gamma 1 + N(0, 0.1)."""
    return dict(
        o=normal(seed, "p_o", (n_tok, hv, dv), o_std),
        z=normal(seed, "z", (n_tok, hv * dv), 1.0, dtype=io),
        gamma=normal(seed, "gamma", (dv,), 0.1, mean=1.0, dtype=io),
    )


def layer_inputs_device(w: Workload, layer: int, device) -> dict:
    """One layer's inputs drawn on the device with torch's generator (Philox),
    with the same shapes, dtypes and distributions as layer_inputs but not the
    same values: for throughput runs whose inputs are too large to draw on the
    host in time (the long varlen batch).  Parity checks use layer_inputs."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.default_rng([*map(int, w.layer_seed(layer)), 99]).integers(2**62)))
    dt = {"f32": torch.float32, "f16": torch.float16}[w.io]
    T, C, hv, dv, dk, n = w.total_T, w.C, w.hv, w.dv, w.dk, w.n_seq

    def nrm(shape, std, mean=0.0, dtype=dt):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std
        return (x + mean).to(dtype)

    A_log = (torch.rand((hv,), generator=g, device=device) * math.log(16.0)).to(dt)
    return dict(
        qkv=nrm((T, C), 1.0), conv_w=nrm((C, 4), 0.25), a=nrm((T, hv), 1.0), b=nrm((T, hv), 1.0),
        A_log=A_log, dt_bias=nrm((hv,), 0.5), z=nrm((T, hv * dv), 1.0), gamma=nrm((dv,), 0.1, 1.0),
        S0=nrm((n, hv, dv, dk), w.s0_std, dtype=torch.float32) if w.s0_std else
        torch.zeros((n, hv, dv, dk), device=device, dtype=torch.float32),
        hist=nrm((n, 3, C), w.hist_std) if w.hist_std else torch.zeros((n, 3, C), device=device, dtype=dt),
    )
