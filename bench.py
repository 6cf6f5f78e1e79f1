#!/usr/bin/env python3
"""GDN prefill benchmark: 36 layers of pre -> scan -> post at T=2048.

One step = one pass of the whole path for each of the 36 layers, launched in
order on one stream, over one 2048-token batch at production width (16 key
heads, 48 value heads, head dim 128, fp16 activations and weights, fp32
state).  The timed step calls gdn_prefill_layer per layer (the layer entry
point: the pre stage fused into the scan's prep step, the chunk kernel, the
post stage).  Every layer has its own inputs, state, history and output
buffers, all resident in HBM before timing starts; the intermediates live in
one workspace reused layer after layer, as in a real prefill.

Prints ONE JSON line: tokens/s of the layer path with fp16 output (the
headline) and fp32 output; the staged path (gdn_pre, gdn_scan, gdn_post) with
per-stage times from HIP events recorded on the launch stream inside the
timed region; the scan's roofline fraction (gdn_scan of the staged path);
gdn_step decode timings; the long varlen batch (36 layers of four packed
sequences, T = 16384, 8192, 2048 and 511, fp32 output) through
gdn_prefill_layer; and the fp64 oracle timed on the host cores on a bounded
sample of both workloads.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN prefill tokens/sec (pre+scan+post, 36 layers, T=2048); % of roofline"
# MI355X published peaks
HBM_PEAK_GBS = 8000.0
FP16_MFMA_PEAK_TFLOPS = 2500.0       # dense fp16 matrix: the scan's contractions run on it
FP32_MFMA_PEAK_TFLOPS = 157.3        # dense fp32 matrix, for comparison
COUNTERS_FILE = os.path.join(ROOT, "profiles", "scan_counters.json")


def scan_flops(T, hv, dv=128, dk=128):
    # S k: 2, decay + rank-1 write: 3, S q: 2 flop per state element per token
    return 7.0 * T * hv * dv * dk


def pre_bytes(T, hk, hv, io_bytes=2, n_seq=1):
    C = 2 * hk * 128 + hv * 128
    per_tok = C * io_bytes + 2 * hv * io_bytes + (2 * hk * 128 + hv * 128) * 4 + 2 * hv * 4
    fixed = C * 4 * io_bytes + 2 * hv * io_bytes + n_seq * 2 * 3 * C * io_bytes
    return T * per_tok + fixed


def scan_bytes(T, hk, hv, n_seq=1):
    per_tok = (2 * hk * 128 + hv * 128) * 4 + 2 * hv * 4 + hv * 128 * 4
    return T * per_tok + n_seq * 2 * hv * 128 * 128 * 4


def post_bytes(T, hv, io_bytes=2, out_bytes=2):
    return T * hv * 128 * (4 + io_bytes + out_bytes) + 128 * io_bytes


def kernel_source_hash(name):
    p = os.path.join(ROOT, "gated_deltanet_linear_pre_amd", "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def load_counters():
    """rocprofv3 counter figures of the scan (HBM bytes per launch, MFMA and
    VALU utilisation), if they were taken on the scan kernel as it is now
    (source hash match); else {}."""
    try:
        d = json.load(open(COUNTERS_FILE))
    except (OSError, ValueError):
        return {}
    if d.get("kernel_source_sha256_16") != kernel_source_hash("gdn_scan.hip"):
        return {}
    return d


def cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(budget_s=12.0, layers_total=36):
    """The fp64 oracle, as it stands, on whole layers of the same workload
    (T=2048, all 48 value heads, pre+scan+post), one layer after another until
    ~budget_s of oracle time; tokens/s is scaled to the 36-layer pass the
    metric counts (T / (mean seconds per layer x 36)).  Also one layer on one
    thread."""
    import numpy as np
    from gated_deltanet_linear_pre_amd import synth
    from oracle import gdn_oracle as orc

    w = synth.WORKLOADS["prod36_t2048_fp16out"]
    dims = orc.Dims(w.hk, w.hv)
    times = []
    while len(times) < layers_total and sum(times) < budget_s:
        inp = synth.layer_inputs(w, len(times))
        t0 = time.perf_counter()
        orc.layer(dims, w.cu_seqlens(), inp)
        times.append(time.perf_counter() - t0)
    per_layer = float(np.mean(times))
    cores = orc.max_threads()
    inp = synth.layer_inputs(w, 0)
    orc.set_threads(1)
    try:
        t0 = time.perf_counter()
        orc.layer(dims, w.cu_seqlens(), inp)
        one = time.perf_counter() - t0
    finally:
        orc.set_threads(cores)
    return dict(value=round(w.total_T / (per_layer * layers_total), 2), unit="tokens/s",
                cores=cores, kind="oracle",
                sample=f"{len(times)} of the 36 layers (layers 0..{len(times) - 1}), each full "
                       f"T=2048, all 48 value heads, pre+scan+post in fp64; "
                       f"{per_layer:.2f} s per layer, scaled to 36 layers",
                cpu_model=cpu_model(),
                one_core={"s_per_layer": round(one, 3), "tokens_per_s": round(w.total_T / (one * 36), 2),
                          "sample": "layer 0, T=2048, all 48 value heads, 1 thread, scaled to 36 layers"})


def chunk_step_schedule(seqlens, hv, n_cu, chunk=32, blocks_per_head=4):
    """Chunk steps on the longest sequence's chain, and the makespan of the
    chunk kernel's blocks dealt longest sequence first to n_cu CUs, one block
    per CU at a time (its LDS use), each block running ceil(len / chunk) steps."""
    import heapq
    lens = sorted(seqlens, reverse=True)
    free = [0] * n_cu
    for L_ in lens:
        for _ in range(hv * blocks_per_head):
            t = heapq.heappop(free)
            heapq.heappush(free, t + (L_ + chunk - 1) // chunk)
    crit = (lens[0] + chunk - 1) // chunk
    work = sum(hv * blocks_per_head * ((L_ + chunk - 1) // chunk) for L_ in lens)
    return {"critical_path": crit, "list_schedule_makespan": max(free),
            "work_over_cus": round(work / n_cu, 1)}


def cpu_baseline_varlen(layers_total=36):
    """The fp64 oracle on one whole layer of the long varlen batch (layer 0:
    all four sequences, all 48 value heads), extrapolated to 36 layers."""
    from gated_deltanet_linear_pre_amd import synth
    from oracle import gdn_oracle as orc

    w = synth.WORKLOADS["prod36_varlen4_fp32out"]
    inp = synth.layer_inputs(w, 0)
    t0 = time.perf_counter()
    orc.layer(orc.Dims(w.hk, w.hv), w.cu_seqlens(), inp)
    sec = time.perf_counter() - t0
    return dict(value=round(w.total_T / (sec * layers_total), 2), unit="tokens/s",
                cores=orc.max_threads(), kind="oracle",
                sample=f"layer 0 of 36 ({w.total_T} tokens, all 48 value heads, pre+scan+post "
                       f"in fp64), {sec:.2f} s; tokens/s extrapolated to 36 layers as "
                       f"T / (36 x that time)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=36)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--legs", default="prefill,staged,varlen,decode",
                    help="comma-separated subset of prefill (the layer path, the headline), staged "
                         "(gdn_pre, gdn_scan, gdn_post; the roofline), varlen (the long varlen "
                         "batch) and decode; a profiler run can take one workload at a time")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (for scaling the HBM "
                         "byte counters of a profiler run)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path would shard by value heads, with no exchange inside it)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": src.numel() * 4,
                          "copy_calibration_bytes_written": dst.numel() * 4, "launches": 5}))
        return
    from gated_deltanet_linear_pre_amd import binding as B
    from gated_deltanet_linear_pre_amd import synth
    from gated_deltanet_linear_pre_amd.buffers import TORCH_DTYPE, upload

    def log(*a):
        if not args.quiet:
            print("[bench]", *a, file=sys.stderr, flush=True)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    B.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w16 = synth.WORKLOADS["prod36_t2048_fp16out"]
    L = args.layers
    T, hk, hv = w16.total_T, w16.hk, w16.hv

    # ---- inputs for all layers, resident in HBM --------------------------
    t0 = time.perf_counter()
    layers = []
    for l in range(L):
        inp = synth.layer_inputs(w16, l)
        layers.append({k: upload(v, dev) for k, v in inp.items()})
        if l % 6 == 5:
            log(f"generated layer {l + 1}/{L} ({time.perf_counter() - t0:.1f}s)")
    cu = upload(w16.cu_seqlens(), dev)
    f32 = dict(dtype=torch.float32, device=dev)
    qn = torch.empty((T, hk, 128), **f32)
    kn = torch.empty((T, hk, 128), **f32)
    vc = torch.empty((T, hv, 128), **f32)
    g = torch.empty((T, hv), **f32)
    beta = torch.empty((T, hv), **f32)
    o = torch.empty((T, hv, 128), **f32)
    from gated_deltanet_linear_pre_amd.buffers import scratch
    stream = torch.cuda.current_stream()

    def run_layer(out, steps, warmup):
        # the whole path per layer: gdn_prefill_layer (pre fused into the scan's
        # prep step, then the chunk kernel and post), 36 layers in order
        ys = [torch.empty((T, hv * 128), dtype=TORCH_DTYPE[out], device=dev) for _ in range(L)]
        shape = B.make_shape(hk, hv, 1, T, T, io="f16", out=out)
        ws = scratch(B.gdn_prefill_workspace_bytes(shape), dev)

        def step():
            for l, d in enumerate(layers):
                B.gdn_prefill_layer(shape, cu, d["qkv"], d["conv_w"], d["a"], d["b"], d["A_log"],
                                    d["dt_bias"], d["z"], d["gamma"], d["hist"], d["S0"], ys[l], ws,
                                    stream=stream)
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps

        # the same 36-layer step captured once in a HIP graph and replayed (no
        # host launches per layer); the calls go to the current stream, which
        # is the capture stream while the graph is captured
        def step_cur():
            for l, d in enumerate(layers):
                B.gdn_prefill_layer(shape, cu, d["qkv"], d["conv_w"], d["a"], d["b"], d["A_log"],
                                    d["dt_bias"], d["z"], d["gamma"], d["hist"], d["S0"], ys[l], ws)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step_cur()
        graph.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return dict(ms_per_step=ms, ms_per_step_graph=e0.elapsed_time(e1) / steps)

    def run(out, steps, warmup):
        # the staged path (gdn_pre, gdn_scan, gdn_post per layer): the whole pass
        # timed as one, then each stage alone over the 36 layers back to back
        # (one event pair per stage loop: the per-launch average of that
        # kernel, without events between launches), for the per-stage times
        # and the scan's roofline
        ys = [torch.empty((T, hv * 128), dtype=TORCH_DTYPE[out], device=dev) for _ in range(L)]
        shape = B.make_shape(hk, hv, 1, T, T, io="f16", out=out)
        sws = scratch(B.gdn_scan_workspace_bytes(shape), dev)

        def pre(d):
            B.gdn_pre(shape, cu, d["qkv"], d["conv_w"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                      d["hist"], qn, kn, vc, g, beta, stream=stream)

        def scan(d):
            B.gdn_scan(shape, cu, qn, kn, vc, g, beta, d["S0"], o, sws, stream=stream)

        def post(d, l):
            B.gdn_post(shape, o, d["z"], d["gamma"], ys[l], stream=stream)

        def step():
            for l, d in enumerate(layers):
                pre(d)
                scan(d)
                post(d, l)

        def timed(fn, n):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(n):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        total_ms = timed(step, steps)
        per = {}
        for name, fn in (("pre", lambda: [pre(d) for d in layers]),
                         ("scan", lambda: [scan(d) for d in layers]),
                         ("post", lambda: [post(d, l) for l, d in enumerate(layers)])):
            fn()
            torch.cuda.synchronize()
            per[name] = timed(fn, steps) / L
        return dict(ms_per_step=total_ms, pre_ms=per["pre"], scan_ms=per["scan"], post_ms=per["post"])

    legs = set(args.legs.split(","))
    if "prefill" in legs:
        log("timing the layer path, fp16 output")
        l16 = run_layer("f16", args.steps, args.warmup)
        log("timing the layer path, fp32 output")
        l32 = run_layer("f32", args.steps, args.warmup)
    else:
        l16 = l32 = {"ms_per_step": float("nan")}
    if "staged" in legs:
        log("timing the staged path (per-stage events), fp16 output")
        r16 = run("f16", args.steps, args.warmup)
        log("timing the staged path, fp32 output")
        r32 = run("f32", args.steps, args.warmup)
    else:
        nan = float("nan")
        r16 = r32 = dict(ms_per_step=nan, pre_ms=nan, scan_ms=nan, post_ms=nan)

    scan_s = r16["scan_ms"] / 1e3
    achieved_tf = scan_flops(T, hv) / scan_s / 1e12
    ctr = load_counters()
    traffic = ctr.get("bytes_per_launch")
    # achieved = the recurrence's fp32 flops (7 per state element and token) per call / the
    # call's event-timed duration; the contractions execute as three fp16 MFMA products per
    # fp32 product, so the peak is the dense fp16 MFMA figure
    roof = {"bound": "mfma", "achieved": round(achieved_tf, 3), "peak": FP16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved_tf / FP16_MFMA_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "kernel": "gdn_scan (scan_prep_kernel + scan_chunk_kernel), per layer launch",
            "flops_per_launch": scan_flops(T, hv),
            "frac_of_fp32_mfma_peak": round(achieved_tf / FP32_MFMA_PEAK_TFLOPS, 4),
            "frac_of_split_fp16_peak": round(achieved_tf / (FP16_MFMA_PEAK_TFLOPS / 3), 4),
            # chunk kernel, from the counters: MFMA busy cycles over all SIMD cycles (%), VALU
            # issue (%), and the fp16 MFMA flops the two kernels execute per launch
            "mfma_util_pct": ctr.get("mfma_util_pct"), "valu_busy_pct": ctr.get("valu_busy_pct"),
            "mfma_flops_executed_per_launch": ctr.get("mfma_flops_executed_per_launch")}

    def stage_report(r, out_bytes):
        return {
            "pre_us": round(r["pre_ms"] * 1e3, 2),
            "scan_us": round(r["scan_ms"] * 1e3, 2),
            "post_us": round(r["post_ms"] * 1e3, 2),
            "pre_hbm_frac": round(pre_bytes(T, hk, hv) / (r["pre_ms"] / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "post_hbm_frac": round(post_bytes(T, hv, out_bytes=out_bytes) / (r["post_ms"] / 1e3)
                                   / 1e9 / HBM_PEAK_GBS, 4),
            "scan_tflops": round(scan_flops(T, hv) / (r["scan_ms"] / 1e3) / 1e12, 3),
        }

    def decode(batch, layers=36, steps=20):
        # gdn_step over `layers` layers, each with its own weights, state and
        # history (distinct buffers), one token per sequence per step
        wd = synth.Workload(f"decode_b{batch}", hk=hk, hv=hv, seqlens=(1,) * batch, seed=(41,),
                            s0_std=0.05, hist_std=1.0)
        shape = B.make_shape(hk, hv, batch, batch, 1, io="f16", out="f16")
        ls = []
        for l in range(layers):
            inp = synth.layer_inputs(wd, l)
            ls.append({k: upload(v, dev) for k, v in inp.items()})
        y = torch.empty((batch, hv * 128), dtype=torch.float16, device=dev)

        def one():
            # on the current stream: the capture stream while a graph is captured
            for d in ls:
                B.gdn_step(shape, d["qkv"], d["conv_w"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                           d["z"], d["gamma"], d["hist"], d["S0"], y)

        # the history alternating between two buffers per layer: one launch
        # per layer and step (two steps per call, back to the first buffer)
        hists = [[d["hist"], torch.empty_like(d["hist"])] for d in ls]

        def two_alt():
            for s_ in range(2):
                for d, hs in zip(ls, hists):
                    B.gdn_step(shape, d["qkv"], d["conv_w"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                               d["z"], d["gamma"], hs[s_], d["S0"], y, hist_out=hs[1 - s_])
        def timed(fn):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(steps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / (steps * layers)

        for _ in range(3):
            one()
        us = timed(one)
        # the same 36-layer step captured once in a HIP graph (no host
        # launches per layer), replayed
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            one()
        graph.replay()
        us_g = timed(graph.replay)
        for _ in range(2):
            two_alt()
        us_a = timed(two_alt) / 2
        graph_a = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph_a):
            two_alt()
        graph_a.replay()
        us_ag = timed(graph_a.replay) / 2
        C = 2 * hk * 128 + hv * 128
        byts = batch * (2 * hv * 128 * 128 * 4 + C * 2 + 4 * 3 * C * 2 + 2 * hv * 2 + 2 * hv * 128 * 2)
        return {"batch": batch, "us_per_layer": round(us, 2),
                "tokens_per_s": round(batch / (us * 1e-6 * layers), 1),
                "us_per_layer_graph": round(us_g, 2),
                "tokens_per_s_graph": round(batch / (us_g * 1e-6 * layers), 1),
                "bytes_per_layer": byts, "hbm_frac": round(byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "hbm_frac_graph": round(byts / (us_g * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "us_per_layer_alternating": round(us_a, 2),
                "us_per_layer_alternating_graph": round(us_ag, 2),
                "tokens_per_s_alternating_graph": round(batch / (us_ag * 1e-6 * layers), 1)}

    def varlen(steps, warmup):
        # the long varlen batch through gdn_prefill_layer, 36 layers in order,
        # each with its own inputs (drawn on the device), state, history and
        # output; then gdn_scan alone over 36 per-layer states (the roofline
        # kernel), reading one layer's intermediates
        wv = synth.WORKLOADS["prod36_varlen4_fp32out"]
        Tv = wv.total_T
        lv = [synth.layer_inputs_device(wv, l, dev) for l in range(L)]
        cuv = upload(wv.cu_seqlens(), dev)
        shape = B.make_shape(hk, hv, wv.n_seq, Tv, wv.max_T, io="f16", out="f32")
        ys = [torch.empty((Tv, hv * 128), dtype=torch.float32, device=dev) for _ in range(L)]
        ws = scratch(B.gdn_prefill_workspace_bytes(shape), dev)

        def step():
            for l, d in enumerate(lv):
                B.gdn_prefill_layer(shape, cuv, d["qkv"], d["conv_w"], d["a"], d["b"], d["A_log"],
                                    d["dt_bias"], d["z"], d["gamma"], d["hist"], d["S0"], ys[l], ws,
                                    stream=stream)
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        del ys, ws
        # gdn_scan alone: one layer's intermediates from gdn_pre, 36 states
        f = dict(dtype=torch.float32, device=dev)
        iq, ik = torch.empty((Tv, hk, 128), **f), torch.empty((Tv, hk, 128), **f)
        iv, io_ = torch.empty((Tv, hv, 128), **f), torch.empty((Tv, hv, 128), **f)
        ig, ib = torch.empty((Tv, hv), **f), torch.empty((Tv, hv), **f)
        d0 = lv[0]
        B.gdn_pre(shape, cuv, d0["qkv"], d0["conv_w"], d0["a"], d0["b"], d0["A_log"], d0["dt_bias"],
                  d0["hist"].clone(), iq, ik, iv, ig, ib, stream=stream)
        sws = scratch(B.gdn_scan_workspace_bytes(shape), dev)
        states = [d["S0"] for d in lv]

        def scans():
            for S in states:
                B.gdn_scan(shape, cuv, iq, ik, iv, ig, ib, S, io_, sws, stream=stream)
        scans()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            scans()
        e1.record(stream)
        torch.cuda.synchronize()
        scan_us = e0.elapsed_time(e1) * 1e3 / (steps * L)
        del lv, iq, ik, iv, io_, ig, ib, sws
        torch.cuda.empty_cache()
        tf = scan_flops(Tv, hv) / (scan_us * 1e-6) / 1e12
        return {"workload": wv.name, "layers": L, "seqlens": list(wv.seqlens), "T_total": Tv,
                "io": "fp16", "state": "fp32", "out": "fp32",
                "value": round(Tv / (ms / 1e3), 1), "unit": "tokens/s", "ms_per_step": round(ms, 3),
                "inputs": "drawn on the device (torch Philox), same shapes and distributions as the "
                          "parity tests' host-drawn inputs",
                "roofline": {"bound": "mfma", "kernel": "gdn_scan (scan_prep_kernel + scan_chunk_kernel)",
                             "achieved": round(tf, 3), "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(tf / FP16_MFMA_PEAK_TFLOPS, 4), "us_per_call": round(scan_us, 1),
                             "flops_per_launch": scan_flops(Tv, hv)},
                "chunk_steps": chunk_step_schedule(wv.seqlens, hv,
                                                   torch.cuda.get_device_properties(dev).multi_processor_count),
                "cpu_baseline": None}

    var = None
    if "varlen" in legs:
        log("timing the long varlen batch (36 layers, T = 16384 + 8192 + 2048 + 511)")
        var = varlen(max(3, args.steps // 4), 1)

    dec = None
    if "decode" in legs:
        log("timing gdn_step decode")
        dec = [decode(b) for b in (1, 8, 64)]

    res = {
        "metric": METRIC,
        "value": round(T / (l16["ms_per_step"] / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(l16["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 (state, elementwise); contractions as split fp16 x3 on MFMA",
        "data": "synthetic",
        "config": {"workload": w16.name, "layers": L, "T": T, "batch": 1, "hk": hk, "hv": hv,
                   "head_dim": 128, "io": "fp16", "state": "fp32", "out": "fp16",
                   "parallelism": "single-gpu"},
        "roofline": roof,
        "graph_replay": {"value": round(T / (l16.get("ms_per_step_graph", float("nan")) / 1e3), 1),
                         "unit": "tokens/s",
                         "ms_per_step": round(l16.get("ms_per_step_graph", float("nan")), 4)},
        "fp32_out": {"value": round(T / (l32["ms_per_step"] / 1e3), 1), "unit": "tokens/s",
                     "ms_per_step": round(l32["ms_per_step"], 4),
                     "graph_replay_ms_per_step": round(l32.get("ms_per_step_graph", float("nan")), 4)},
        "staged_fp16_out": {"value": round(T / (r16["ms_per_step"] / 1e3), 1),
                            "ms_per_step": round(r16["ms_per_step"], 4), **stage_report(r16, 2)},
        "staged_fp32_out": {"value": round(T / (r32["ms_per_step"] / 1e3), 1),
                            "ms_per_step": round(r32["ms_per_step"], 4), **stage_report(r32, 4)},
        "varlen4": var,
        "decode_gdn_step": dec,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on the host cores")
        res["cpu_baseline"] = cpu_baseline()
        if var is not None:
            log("timing the fp64 oracle on one layer of the long varlen batch")
            res["varlen4"]["cpu_baseline"] = cpu_baseline_varlen()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
