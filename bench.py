#!/usr/bin/env python3
"""E2-TTT chunk-update throughput on one MI355X.

One step = one e2ttt_chunk_forward call over the whole workload (scalar
kernels, fast-weight forward/backward at the chunk-start weights, both
gradient aggregations, state transition and chunk outputs for every chunk of
every (batch, head)), inputs resident in HBM.  Prints one JSON line.

Timing protocol: W warm-up calls, then K timed calls.  Before each timed call
a 512 MiB buffer is overwritten on the same stream (outside the call's
events), so that neither the L2 caches nor the 256 MB last-level cache still
hold the previous call's inputs or state.  Each call is timed by HIP events
recorded inside it, on its own stream; ``ms_per_step`` and ``value`` use the
median call time, and p10 / p90 / mean / min are reported beside it.
``--no-flush`` times back-to-back calls instead.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--backward]

With --backward one step is one e2ttt_chunk_backward call instead (forward
recompute, reverse chunk loop, scalar-kernel backward): the gradients of a
training step for the same workload.  With --train one step is a training
step: e2ttt_chunk_forward with E2TTT_FLAG_SAVE_STATES, then
e2ttt_chunk_backward on the same workspace (no recompute).  With --peaks it
measures the chip's own bf16 MFMA and HBM ceilings instead; --graph times
replays of the forward call captured in a HIP graph.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "E2-TTT chunk-update tokens/sec at 1 GPU + % of MFMA/HBM roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 (MFMA / packed VALU)
PEAK_HBM_GBS = 8000.0
LOOP_SRC = os.path.join(ROOT, "chunk_weight_rnn_amd", "csrc", "swiglu_loop.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_swiglu_loop_1p3b.json")


def flops_per_token_head(cfg: synth.Config) -> dict:
    """Algorithmic MFMA-able flops per token per head, split by stage."""
    D, Hd = cfg.D, cfg.Hd
    sets = 2 if cfg.momentum else 1  # weighted aggregations: G^M and G^W, or G^W alone
    if cfg.kind == "swiglu":
        return {"grad": 6 * D * Hd, "aggregate": 6 * sets * D * Hd, "apply": 6 * D * Hd}
    if cfg.kind == "mlp":
        fwd = 4 * D * Hd if cfg.loss == "mse" else 2 * D * Hd
        return {"grad": fwd + 2 * D * Hd, "aggregate": 4 * sets * D * Hd, "apply": 4 * D * Hd}
    return {"grad": 2 * D * D, "aggregate": 2 * sets * D * D, "apply": 2 * D * D}


def bwd_flops_per_token_head(cfg: synth.Config) -> dict:
    """MFMA-able flops per token per head of the backward (SwiGLU path), by kernel:
    recompute = the forward chunk loop; token = projections of k, v at W_c and
    the cotangents, dk and dv, and the output path's projections and dq;
    weight = the chunk's dW contraction over its tokens."""
    D, Hd = cfg.D, cfg.Hd
    mom = cfg.momentum
    token = (9 if mom else 6) * 2 * D * Hd + (6 if mom else 4) * 2 * D * Hd + (3 if mom else 2) * 2 * D * Hd \
        + 3 * 2 * D * Hd + 2 * 2 * D * Hd
    return {"recompute": 6 * D * Hd + 6 * (2 if mom else 1) * D * Hd, "token": token, "weight": 12 * D * Hd}


def alg_bytes(cfg: synth.Config) -> int:
    es = 2 if cfg.io_dtype == "bf16" else 4
    BH = cfg.B * cfg.H
    states = 4 if cfg.momentum else 2  # W0, M0 read + W_end, M_end written (no momentum: W only)
    gates = 3 if cfg.momentum else 2
    return BH * cfg.T * cfg.D * es * 4 + BH * cfg.T * 4 * gates + BH * cfg.P * 4 * states


class HipEvents:
    """hipEvent_t handles through the HIP runtime (timing on the library's stream)."""

    def __init__(self, n: int):
        self.rt = ctypes.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            assert self.rt.hipEventCreate(ctypes.byref(h)) == 0
            self.ev.append(h)

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        assert self.rt.hipEventSynchronize(b) == 0
        assert self.rt.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return float(ms.value)


FLUSH_BYTES = 512 << 20


class Flusher:
    """Overwrites a 512 MiB device buffer on the current stream between timed
    calls (a fill kernel: every cache line it writes evicts older data)."""

    def __init__(self, torch, enabled: bool):
        self.buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda") if enabled else None
        self.n = 0

    def __call__(self):
        if self.buf is not None:
            self.n += 1
            self.buf.fill_(self.n & 255)


def stats(ms: list) -> dict:
    """median, p10, p90, mean, min of per-call times (ms)."""
    v = sorted(ms)
    q = lambda f: v[min(len(v) - 1, max(0, int(round(f * (len(v) - 1)))))]
    return {"median": q(0.5), "p10": q(0.1), "p90": q(0.9), "mean": sum(v) / len(v), "min": v[0], "n": len(v)}


def timing_record(call: dict, wall_ms: float, args) -> dict:
    """How the step time was taken, for the JSON line."""
    return {"per_call_ms": call, "wall_ms_per_step": wall_ms,
            "flush": None if args.no_flush else f"{FLUSH_BYTES >> 20} MiB overwritten before each timed call",
            "ms_per_step_is": "median of the per-call HIP-event times (the wall time per step includes the "
                              "flush and host launch gaps)"}


def code_fingerprint(path: str) -> str:
    """sha256 of a C++/HIP source with its comments and whitespace removed, so
    that a comment edit does not count as a kernel change."""
    src = open(path).read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return hashlib.sha256(" ".join(src.split()).encode()).hexdigest()


def measured_traffic(loop_launch_bytes_alg: float):
    """HBM traffic per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel code (comments aside); else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        if t.get("code_sha256") != code_fingerprint(LOOP_SRC):
            return None
        return float(t["bytes_per_launch"])
    except (OSError, ValueError, KeyError):
        return None


def cpu_baseline_backward(cfg: synth.Config, budget_s: float) -> dict:
    """The fp64 backward oracle (autograd of the closed form) on a bounded
    sample: single (b, h) heads, cycling over the workload's heads, until
    about budget_s seconds of host work have been timed."""
    import torch
    import oracle
    cores = torch.get_num_threads()
    x = synth.make_inputs(cfg, seed=0)
    c = synth.make_cotangents(cfg, seed=1)
    f = lambda t: t.double().numpy()
    n, wall = 0, 0.0
    while wall < budget_s:
        b, h = (n // cfg.H) % cfg.B, n % cfg.H
        xs = synth.head_slice(x, [(b, h)])
        cs = synth.head_slice(c, [(b, h)])
        t0 = time.perf_counter()
        oracle.chunk_backward(cfg.kind, cfg.loss, f(xs["q"]), f(xs["k"]), f(xs["v"]), f(xs["eta"]),
                              f(xs["alpha"]), f(xs["beta"]), f(xs["W0"]), f(xs["M0"]), f(cs["dout"]),
                              f(cs["dW_end"]), f(cs["dM_end"]), cfg.chunk, cfg.Hd, momentum=cfg.momentum,
                              chunk_avg=cfg.chunk_avg)
        wall += time.perf_counter() - t0
        n += 1
    # tokens/s of the whole workload: each sampled head is 1/H of a sequence's work
    return {"value": n * cfg.T / cfg.H / wall, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n} single (b, h) heads x {cfg.T} tokens (one head = 1/{cfg.H} of a sequence), fp64 "
                      f"torch autograd of the closed form, {wall:.1f} s"}


def run_backward(args, cfg, lib, e2, torch) -> dict:
    """Time e2ttt_chunk_backward on the workload; returns the JSON record."""
    xin = synth.make_inputs(cfg, seed=0)
    if cfg.kind == "mlp":  # the MLP/MSE state leaves fp32 range with the default gates (as in the tests)
        gen = torch.Generator().manual_seed(1234)
        xin["alpha"] = torch.sigmoid(8.0 + torch.randn(xin["alpha"].shape, generator=gen))
        xin["eta"] = xin["eta"] / cfg.D
    x = {n: t.cuda() for n, t in xin.items()}
    c = {n: t.cuda() for n, t in synth.make_cotangents(cfg, seed=1).items()}
    g = {n: torch.empty_like(x[n]) for n in ("q", "k", "v", "eta", "alpha", "beta", "W0", "M0")}
    desc = e2._lib.make_desc(cfg.kind, cfg.loss, cfg.io_dtype, cfg.B, cfg.H, cfg.T, cfg.D, cfg.Hd, cfg.chunk,
                             cfg.flags)
    ws_bytes = int(lib.e2ttt_backward_workspace_size(ctypes.byref(desc)))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    hs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    hev = HipEvents(4 * max(args.steps, 1))

    def step(i=None):
        evs = None if i is None else (ctypes.c_void_p * 4)(*hev.ev[4 * i:4 * i + 4])
        st = lib.e2ttt_chunk_backward_events(
            ctypes.byref(desc), p(x["q"]), p(x["k"]), p(x["v"]), p(x["eta"]), p(x["alpha"]), p(x["beta"]),
            p(x["W0"]), p(x["M0"]), p(c["dout"]), p(c["dW_end"]), p(c["dM_end"]), p(g["q"]), p(g["k"]),
            p(g["v"]), p(g["eta"]), p(g["alpha"]), p(g["beta"]), p(g["W0"]), p(g["M0"]), p(ws),
            ctypes.c_size_t(ws_bytes), hs, evs)
        if st != 0:
            raise e2.E2TTTError("e2ttt_chunk_backward_events", st)

    flush = Flusher(torch, not args.no_flush)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        flush()
        step(i)
    torch.cuda.synchronize()
    wall_ms = 1e3 * (time.perf_counter() - t0) / args.steps
    st = {"recompute": [], "reverse_loop": [], "scalar": []}
    calls = []
    for i in range(args.steps):
        e = hev.ev[4 * i:4 * i + 4]
        st["recompute"].append(hev.elapsed_ms(e[0], e[1]))
        st["reverse_loop"].append(hev.elapsed_ms(e[1], e[2]))
        st["scalar"].append(hev.elapsed_ms(e[2], e[3]))
        calls.append(hev.elapsed_ms(e[0], e[3]))
    st_ms = {k: sum(v) / len(v) for k, v in st.items()}
    call = stats(calls)
    ms_step = call["median"]
    th = cfg.B * cfg.H * cfg.T
    mfma_path = bool(lib.e2ttt_path(ctypes.byref(desc)) == 1)
    if mfma_path:
        fpt = bwd_flops_per_token_head(cfg)
        loop_flops = (fpt["token"] + fpt["weight"]) * th
        loop_tflops = loop_flops / (st_ms["reverse_loop"] * 1e-3) / 1e12
        call_tflops = sum(fpt.values()) * th / (ms_step * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": "bwd_tok_kernel + bwd_wt_kernel (reverse chunk loop)",
                "achieved": loop_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": loop_tflops / PEAK_BF16_TFLOPS, "traffic": None,
                "per_launch": f"{fpt['token'] + fpt['weight']} flop/token/head x {th} token-heads = "
                              f"{loop_flops:.4g} flop over the reverse loop"}
        whole = {"tflops": call_tflops, "frac_of_peak": call_tflops / PEAK_BF16_TFLOPS}
    else:  # the portable fp32 path: one workgroup per head, no roofline model
        roof = None
        whole = None
    res = {
        "metric": "E2-TTT chunk-update backward (VJP) tokens/sec at 1 GPU + % of MFMA roofline",
        "value": cfg.B * cfg.T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if cfg.io_dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.notes}, backward", "kind": cfg.kind, "loss": cfg.loss,
                   "B": cfg.B, "H": cfg.H, "T": cfg.T, "D": cfg.D, "Hd": cfg.Hd, "chunk": cfg.chunk,
                   "io": cfg.io_dtype, "state": "f32", "momentum": cfg.momentum, "chunk_avg": cfg.chunk_avg},
        "roofline": roof,
        "whole_call": whole,
        "stages_ms": st_ms,
        "timing": timing_record(call, wall_ms, args),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_backward(cfg, args.cpu_budget)
    return res


def run_train(args, cfg, lib, e2, torch) -> dict:
    """Time forward (saving states) + backward (from them) on the workload."""
    x = {n: t.cuda() for n, t in synth.make_inputs(cfg, seed=0).items()}
    c = {n: t.cuda() for n, t in synth.make_cotangents(cfg, seed=1).items()}
    g = {n: torch.empty_like(x[n]) for n in ("q", "k", "v", "eta", "alpha", "beta", "W0", "M0")}
    out, W, M = torch.empty_like(x["q"]), torch.empty_like(x["W0"]), torch.empty_like(x["M0"])
    desc = e2._lib.make_desc(cfg.kind, cfg.loss, cfg.io_dtype, cfg.B, cfg.H, cfg.T, cfg.D, cfg.Hd, cfg.chunk,
                             cfg.flags | e2._lib.FLAG_SAVE_STATES)
    ws_bytes = int(lib.e2ttt_backward_workspace_size(ctypes.byref(desc)))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    hs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    hev = HipEvents(8 * max(args.steps, 1))
    ins = [p(x[n]) for n in ("q", "k", "v", "eta", "alpha", "beta", "W0", "M0")]

    def step(i=None):
        ef = eb = None
        if i is not None:
            ef = (ctypes.c_void_p * 4)(*hev.ev[8 * i:8 * i + 4])
            eb = (ctypes.c_void_p * 4)(*hev.ev[8 * i + 4:8 * i + 8])
        st = lib.e2ttt_chunk_forward_events(ctypes.byref(desc), *ins, p(out), p(W), p(M), p(ws),
                                            ctypes.c_size_t(ws_bytes), hs, ef)
        if st != 0:
            raise e2.E2TTTError("e2ttt_chunk_forward_events", st)
        st = lib.e2ttt_chunk_backward_events(
            ctypes.byref(desc), *ins, p(c["dout"]), p(c["dW_end"]), p(c["dM_end"]),
            *[p(g[n]) for n in ("q", "k", "v", "eta", "alpha", "beta", "W0", "M0")], p(ws),
            ctypes.c_size_t(ws_bytes), hs, eb)
        if st != 0:
            raise e2.E2TTTError("e2ttt_chunk_backward_events", st)

    flush = Flusher(torch, not args.no_flush)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        flush()
        step(i)
    torch.cuda.synchronize()
    wall_ms = 1e3 * (time.perf_counter() - t0) / args.steps
    fw = [hev.elapsed_ms(hev.ev[8 * i], hev.ev[8 * i + 3]) for i in range(args.steps)]
    bw = [hev.elapsed_ms(hev.ev[8 * i + 4], hev.ev[8 * i + 7]) for i in range(args.steps)]
    call = stats([hev.elapsed_ms(hev.ev[8 * i], hev.ev[8 * i + 7]) for i in range(args.steps)])
    ms_step = call["median"]
    th = cfg.B * cfg.H * cfg.T
    f_fwd = sum(flops_per_token_head(cfg).values())
    fb = bwd_flops_per_token_head(cfg)
    f_bwd = fb["token"] + fb["weight"]
    tflops = (f_fwd + f_bwd) * th / (ms_step * 1e-3) / 1e12
    return {
        "metric": "E2-TTT chunk-update training step (forward + backward) tokens/sec at 1 GPU",
        "value": cfg.B * cfg.T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if cfg.io_dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.notes}, forward + backward", "kind": cfg.kind, "loss": cfg.loss,
                   "B": cfg.B, "H": cfg.H, "T": cfg.T, "D": cfg.D, "Hd": cfg.Hd, "chunk": cfg.chunk,
                   "io": cfg.io_dtype, "state": "f32", "momentum": cfg.momentum, "chunk_avg": cfg.chunk_avg},
        "whole_step": {"tflops": tflops, "frac_of_peak": tflops / PEAK_BF16_TFLOPS,
                       "flop_model": f"forward {f_fwd} + backward (token and weight kernels) {f_bwd} flop per "
                                     f"token and head"},
        "stages_ms": {"forward": sum(fw) / len(fw), "backward": sum(bw) / len(bw)},
        "timing": timing_record(call, wall_ms, args),
    }


def cpu_baseline(cfg: synth.Config, budget_s: float) -> dict:
    """The fp64 oracle on a bounded sample of the same workload: whole batch
    rows (every head of one sequence), cycling over the batch until about
    budget_s seconds of host work have been timed."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    x = synth.make_inputs(cfg, seed=0)
    f = lambda t: t.double().numpy()
    rows, wall = 0, 0.0
    while wall < budget_s:
        b = rows % cfg.B
        sl = {n: f(t[b:b + 1]) for n, t in x.items()}
        t0 = time.perf_counter()
        oracle.chunk_forward(cfg.kind, cfg.loss, sl["q"], sl["k"], sl["v"], sl["eta"], sl["alpha"], sl["beta"],
                             sl["W0"], sl["M0"], cfg.chunk, cfg.Hd, momentum=cfg.momentum, chunk_avg=cfg.chunk_avg)
        wall += time.perf_counter() - t0
        rows += 1
    tokens = rows * cfg.T
    return {"value": tokens / wall, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{rows} batch rows of {cfg.H} heads x {cfg.T} tokens (cycling over the {cfg.B} rows of "
                      f"the workload), fp64 numpy closed form, {wall:.1f} s"}


def run_peaks(torch) -> dict:
    """The chip's own ceilings, next to the vendor peaks the roofline uses: bf16
    MFMA throughput of the shapes the kernels issue (independent
    accumulations, 8 wavefronts per SIMD), the overlap of MFMA and VALU work
    on one SIMD, LDS bandwidth per compute unit, HBM read bandwidth
    (grid-stride 16-byte loads) and a plain torch copy (read + write)."""
    probe = ctypes.CDLL(os.path.join(ROOT, "chunk_weight_rnn_amd", "libe2ttt_probe.so"))
    probe.e2ttt_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    probe.e2ttt_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def timed(fn, reps=5):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            best = min(best, a.elapsed_time(b) * 1e-3)
        return best

    res = {"probe": "peaks", "vendor": {"bf16_mfma_TFLOPs": PEAK_BF16_TFLOPS, "hbm_GBs": PEAK_HBM_GBS}}
    grid, iters = ncu * 8, 2000
    out = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    for shape, name, flop_wave_iter in [(0, "mfma_16x16x32_bf16", 8 * 16 * 16 * 32 * 2),
                                        (2, "mfma_16x16x32_bf16_16acc", 16 * 16 * 16 * 32 * 2),
                                        (3, "mfma_16x16x16_bf16", 8 * 16 * 16 * 16 * 2),
                                        (1, "mfma_32x32x16_bf16", 4 * 32 * 32 * 16 * 2)]:
        def launch(shape=shape):
            assert probe.e2ttt_probe_mfma(shape, iters, ctypes.c_void_p(out.data_ptr()), grid, sp) == 0
        t = timed(launch)
        res[name + "_TFLOPs"] = grid * 4 * iters * flop_wave_iter / t / 1e12
    # MFMA and VALU of two wavefronts on one SIMD: 16 MFMAs per round against
    # 16 V FMAs per round, alone and together
    probe.e2ttt_probe_overlap.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                          ctypes.c_void_p]
    ogrid = ncu
    oout = torch.empty(ogrid * 512, dtype=torch.float32, device="cuda")
    ov = {}
    for mode, v, name in [(1, 2, "mfma_alone"), (2, 2, "valu2_alone"), (3, 2, "mfma_with_valu2"),
                          (2, 4, "valu4_alone"), (3, 4, "mfma_with_valu4")]:
        def launch(mode=mode, v=v):
            assert probe.e2ttt_probe_overlap(mode, v, iters, ctypes.c_void_p(oout.data_ptr()), ogrid, sp) == 0
        ov[name + "_us"] = timed(launch) * 1e6
    ov["note"] = ("per SIMD: one wavefront with 16 x iters independent 16x16x32 bf16 MFMAs, another with 16 V x iters "
                  "fp32 FMAs; together vs alone shows the overlap")
    res["mfma_valu_overlap"] = ov
    # LDS bytes per ns per compute unit, 12 wavefronts
    probe.e2ttt_probe_lds.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                      ctypes.c_void_p]
    lout = torch.empty(ncu * 768, dtype=torch.int32, device="cuda")
    lds = {}
    for mode, name, lane_bytes in [(0, "ds_read_b128", 16), (1, "ds_read_b64_tr_b16", 8), (2, "ds_write_b128", 16)]:
        def launch(mode=mode):
            assert probe.e2ttt_probe_lds(mode, 12, 1000, ctypes.c_void_p(lout.data_ptr()), ncu, sp) == 0
        t = timed(launch)
        lds[name + "_B_per_ns_per_CU"] = 12 * 1000 * 16 * 64 * lane_bytes / (t * 1e9)
    res["lds"] = lds
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    rgrid = ncu * 16
    rout = torch.empty(rgrid * 256, dtype=torch.float32, device="cuda")

    def read():
        assert probe.e2ttt_probe_read(ctypes.c_void_p(src.data_ptr()), n // 4, ctypes.c_void_p(rout.data_ptr()),
                                      rgrid, sp) == 0
    res["hbm_read_GBs"] = n * 4 / timed(read) / 1e9
    dst = torch.empty_like(src)
    res["hbm_copy_GBs"] = 2 * n * 4 / timed(lambda: dst.copy_(src)) / 1e9
    res["note"] = ("min over 5 timed launches after 2 warm-up launches; 1 GiB buffers; "
                   "the roofline in the benchmark line is priced against the vendor peaks")
    return res


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="swiglu_1p3b", choices=list(synth.CONFIGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true",
                    help="time back-to-back calls (no 512 MiB cache flush before each timed call)")
    ap.add_argument("--backward", action="store_true", help="time the backward pass instead of the forward")
    ap.add_argument("--train", action="store_true",
                    help="time a training step: forward saving states, then backward from them")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--precise", action="store_true",
                    help="forward: E2TTT_FLAG_PRECISE (hi/lo bf16 operands on the SwiGLU MFMA path)")
    ap.add_argument("--graph", action="store_true",
                    help="forward: capture the call in a HIP graph once and time its replays")
    ap.add_argument("--peaks", action="store_true",
                    help="measure the chip's bf16 MFMA and HBM ceilings instead (one JSON line)")
    ap.add_argument("--copy-calibrate", type=int, default=0, metavar="MiB",
                    help="first run a plain fp32 copy kernel over MiB of data (3 launches), so that a counter "
                         "profile of this command holds the HBM counters of a copy of known size")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the (batch, head) recurrences would shard across GPUs without communication).",
              file=sys.stderr)
        return 2

    import torch
    import chunk_weight_rnn_amd as e2
    lib = e2.library()

    if args.copy_calibrate > 0:
        n = args.copy_calibrate * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    if args.peaks:
        print(json.dumps(run_peaks(torch)), flush=True)
        return 0
    cfg = synth.CONFIGS[args.config]
    if args.backward:
        print(json.dumps(run_backward(args, cfg, lib, e2, torch)), flush=True)
        return 0
    if args.train:
        print(json.dumps(run_train(args, cfg, lib, e2, torch)), flush=True)
        return 0
    x = {n: t.cuda() for n, t in synth.make_inputs(cfg, seed=0).items()}
    out = torch.empty_like(x["q"])
    W = torch.empty_like(x["W0"])
    M = torch.empty_like(x["M0"])
    desc = e2._lib.make_desc(cfg.kind, cfg.loss, cfg.io_dtype, cfg.B, cfg.H, cfg.T, cfg.D, cfg.Hd, cfg.chunk,
                             cfg.flags | (e2._lib.FLAG_PRECISE if args.precise else 0))
    ws_bytes = int(lib.e2ttt_workspace_size(ctypes.byref(desc)))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    hs = ctypes.c_void_p(stream.cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    hev = HipEvents(4 * max(args.steps, 1))

    def step(i=None, stream_handle=None):
        evs = None
        if i is not None:
            evs = (ctypes.c_void_p * 4)(*hev.ev[4 * i:4 * i + 4])
        st = lib.e2ttt_chunk_forward_events(ctypes.byref(desc), p(x["q"]), p(x["k"]), p(x["v"]), p(x["eta"]),
                                            p(x["alpha"]), p(x["beta"]), p(x["W0"]), p(x["M0"]), p(out), p(W),
                                            p(M), p(ws), ctypes.c_size_t(ws_bytes), stream_handle or hs, evs)
        if st != 0:
            raise e2.E2TTTError("e2ttt_chunk_forward_events", st)

    graph = None
    if args.graph:  # the whole call captured once, then replayed
        def on_current():
            step(stream_handle=ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            on_current()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            on_current()
    flush = Flusher(torch, not args.no_flush)
    gev = HipEvents(2 * max(args.steps, 1)) if graph else None
    for _ in range(args.warmup):
        graph.replay() if graph else step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        flush()
        if graph:
            assert gev.rt.hipEventRecord(gev.ev[2 * i], hs) == 0
            graph.replay()
            assert gev.rt.hipEventRecord(gev.ev[2 * i + 1], hs) == 0
        else:
            step(i)
    torch.cuda.synchronize()
    wall_ms = 1e3 * (time.perf_counter() - t0) / args.steps

    st_ms = None
    if not graph:
        stages = {"logscan": [], "loop": [], "apply": []}
        calls = []
        for i in range(args.steps):
            e = hev.ev[4 * i:4 * i + 4]
            stages["logscan"].append(hev.elapsed_ms(e[0], e[1]))
            stages["loop"].append(hev.elapsed_ms(e[1], e[2]))
            stages["apply"].append(hev.elapsed_ms(e[2], e[3]))
            calls.append(hev.elapsed_ms(e[0], e[3]))
        st_ms = {k: sum(v) / len(v) for k, v in stages.items()}
    else:
        calls = [gev.elapsed_ms(gev.ev[2 * i], gev.ev[2 * i + 1]) for i in range(args.steps)]
    call = stats(calls)
    ms_step = call["median"]

    tokens = cfg.B * cfg.T
    fpt = flops_per_token_head(cfg)
    heads_tokens = cfg.B * cfg.H * cfg.T
    path = int(lib.e2ttt_path(ctypes.byref(desc)))
    peak = PEAK_BF16_TFLOPS if path in (1, 2) else PEAK_F32_TFLOPS
    loop_kernel = {0: "generic_kernel", 1: "swiglu_loop_kernel", 2: "swiglu_loop_kernel", 3: "f32_chunk_kernel",
                   4: "f32_split_kernel"}[path]
    if path == 1:  # the chunk loop's form follows the grid (16- or 32-unit slices when they fit at once)
        ncu = torch.cuda.get_device_properties(0).multi_processor_count
        if cfg.B * cfg.H * (cfg.Hd // 32) <= ncu:
            loop_kernel = "swiglu_loop_bs_kernel"
    # the fp32 kernels compute the chunk outputs inside the chunk loop
    loop_stages = ("grad", "aggregate") if path in (1, 2) else ("grad", "aggregate", "apply")
    loop_flops = sum(fpt[k] for k in loop_stages) * heads_tokens
    loop_tflops = loop_flops / (st_ms["loop"] * 1e-3) / 1e12 if st_ms else None
    call_flops = sum(fpt.values()) * heads_tokens
    call_tflops = call_flops / (ms_step * 1e-3) / 1e12
    traffic = measured_traffic(0.0) if args.config == "swiglu_1p3b" and not args.precise else None

    res = {
        "metric": METRIC,
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.io_dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.notes}", "kind": cfg.kind, "loss": cfg.loss, "B": cfg.B,
                   "H": cfg.H, "T": cfg.T, "D": cfg.D, "Hd": cfg.Hd, "chunk": cfg.chunk, "io": cfg.io_dtype,
                   "state": "f32", "momentum": cfg.momentum, "chunk_avg": cfg.chunk_avg,
                   "precise": bool(args.precise)},
        "roofline": None if graph else {
            "bound": "mfma", "kernel": loop_kernel,
            "achieved": loop_tflops, "peak": peak, "unit": "TFLOP/s", "frac": loop_tflops / peak,
            "traffic": traffic,
            "per_launch": f"{sum(fpt[k] for k in loop_stages)} flop/token/head x {heads_tokens} "
                          f"token-heads = {loop_flops:.4g} flop"},
        "path": path,
        "whole_call": {"tflops": call_tflops, "frac_of_peak": call_tflops / peak,
                       "hbm_alg_GBs": alg_bytes(cfg) / (ms_step * 1e-3) / 1e9},
        "stages_ms": st_ms,
        "timing": timing_record(call, wall_ms, args),
    }
    if graph:
        res["graph"] = "each step replays one HIP graph of the whole call (no per-stage events)"
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, args.cpu_budget)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
