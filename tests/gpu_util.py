"""Helpers for GPU parity tests: run the HIP path and the oracle on the same
seeded inputs and compare them tensor by tensor (and chunk by chunk).

Error measure: err(x, r) = max|x - r| / max(max|r|, FLOOR) with FLOOR = 1e-12.
Every input here is O(0.01..1); a value below 1e-12 can only arise as a
product of several decayed factors (the fast-weight gradients are quadratic
in W, and alpha ~ 0.98 per token shrinks W by ~1e-3 per 256-token chunk), and
its fp32 evaluation underflows.  The floor turns the comparison of such
values into an absolute one at 1e-12 x tol, far below any input's scale.
Where the exact state overflows (the MLP/MSE workload diverges), chunks whose
reference is non-finite or above 1e3 are reported as diverged and not compared.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synth

TOL = {"f32": 1e-4, "bf16": 2e-2}
FLOOR = 1e-12
DIVERGED = 1e3


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def err(x, r) -> float:
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if x.size == 0:
        return 0.0
    return float(np.max(np.abs(x - r)) / max(float(np.max(np.abs(r))), FLOOR))


def to_dev(x: dict) -> dict:
    return {n: t.cuda() for n, t in x.items()}


def run_gpu(cfg: synth.Config, x: dict, force_generic=False, in_place=False, momentum=None, chunk_avg=None,
            precise=False):
    import chunk_weight_rnn_amd as e2
    momentum = cfg.momentum if momentum is None else momentum
    chunk_avg = cfg.chunk_avg if chunk_avg is None else chunk_avg
    d = to_dev(x)
    kw = {}
    if in_place:
        kw = dict(W_end=d["W0"], M_end=d["M0"] if momentum else None)
    out, W, M = e2.chunk_forward(d["q"], d["k"], d["v"], d["eta"], d["alpha"], d["beta"], d["W0"], d["M0"],
                                 chunk=cfg.chunk, kind=cfg.kind, loss=cfg.loss, Hd=cfg.Hd,
                                 force_generic=force_generic, momentum=momentum, chunk_avg=chunk_avg,
                                 precise=precise, **kw)
    torch.cuda.synchronize()
    return out.float().cpu(), W.cpu(), (M.cpu() if M is not None else None)


def run_oracle(cfg: synth.Config, x: dict, keep=False, momentum=None, chunk_avg=None):
    momentum = cfg.momentum if momentum is None else momentum
    chunk_avg = cfg.chunk_avg if chunk_avg is None else chunk_avg
    f = lambda t: t.double().numpy()
    with np.errstate(over="ignore", invalid="ignore"):
        return oracle.chunk_forward(cfg.kind, cfg.loss, f(x["q"]), f(x["k"]), f(x["v"]), f(x["eta"]),
                                    f(x["alpha"]), f(x["beta"]), f(x["W0"]), f(x["M0"]), cfg.chunk, cfg.Hd,
                                    keep=keep, momentum=momentum, chunk_avg=chunk_avg)


def _diverged(r) -> bool:
    return (not np.all(np.isfinite(r))) or float(np.max(np.abs(r))) > DIVERGED


def errors(cfg: synth.Config, got, ref, W0) -> dict:
    """Per-tensor errors: every W / M matrix, the update W_end - W0, and the
    output chunk by chunk (key out[c]).  Diverged references map to None."""
    out_g, W_g, M_g = [None if t is None else np.asarray(t, dtype=np.float64) for t in got]
    out_r, W_r, M_r = ref
    assert (M_g is None) == (M_r is None), "momentum output present on one side only"
    W0 = np.asarray(W0, dtype=np.float64)
    e = {}
    for c in range(-(-cfg.T // cfg.chunk)):  # the last chunk may be shorter
        sl = slice(c * cfg.chunk, min((c + 1) * cfg.chunk, cfg.T))
        r = out_r[:, :, sl]
        e[f"out[{c}]"] = None if _diverged(r) else err(out_g[:, :, sl], r)
    with np.errstate(invalid="ignore", over="ignore"):
        pairs = [("W", W_g, W_r), ("dW", W_g - W0, W_r - W0)] + ([("M", M_g, M_r)] if M_r is not None else [])
    for tag, g, r in pairs:
        mg = oracle.unpack(cfg.kind, g, cfg.D, cfg.Hd)
        mr = oracle.unpack(cfg.kind, r, cfg.D, cfg.Hd)
        for n in mg:
            e[f"{tag}.{n}"] = None if _diverged(mr[n]) else err(mg[n], mr[n])
    return e


def assert_close(cfg: synth.Config, got, ref, W0, tol=None, out_tol=None, allow_diverged=False):
    tol = TOL[cfg.io_dtype] if tol is None else tol
    out_tol = tol if out_tol is None else out_tol
    e = errors(cfg, got, ref, W0)
    compared = {n: v for n, v in e.items() if v is not None}
    diverged = [n for n, v in e.items() if v is None]
    if not allow_diverged:
        assert not diverged, f"{cfg.name}: reference diverged in {diverged}"
    assert "out[0]" in compared
    for n, v in compared.items():
        if n.startswith("out"):
            continue
        g = np.asarray(got[1] if n.startswith(("W", "dW")) else got[2])
        assert np.all(np.isfinite(g)), f"{cfg.name}: non-finite GPU state"
    worst = {}
    for n, v in compared.items():
        key = "out" if n.startswith("out") else n
        worst[key] = max(worst.get(key, 0.0), v)
    note(f"  {cfg.name}: " + ", ".join(f"{n}={v:.2e}" for n, v in worst.items())
         + (f"; diverged (not compared): {len(diverged)} tensors/chunks" if diverged else ""))
    bad = {n: v for n, v in compared.items() if v > (out_tol if n.startswith("out") else tol)}
    assert not bad, f"{cfg.name}: tolerance exceeded: {bad}"
    return e


def persistent_gates(cfg: synth.Config, x: dict) -> dict:
    """Full-shape input variant whose state stays well inside fp32 range over
    the whole sequence: slower decay (and, for the MLP/MSE fast weight, a
    1/D loss scale expressed through eta).  Everything else as drawn."""
    x = dict(x)
    g = torch.Generator().manual_seed(1234)
    z = torch.randn(x["alpha"].shape, generator=g)
    if cfg.kind == "mlp":
        x["alpha"] = torch.sigmoid(8.0 + z)
        x["eta"] = x["eta"] / cfg.D
    elif cfg.T > 4096:
        x["alpha"] = torch.sigmoid(7.5 + z)
    else:
        x["alpha"] = torch.sigmoid(6.0 + z)
    return x
