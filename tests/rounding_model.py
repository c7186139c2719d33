"""A CPU model of where the SwiGLU MFMA path rounds to bf16 (analysis aid for
the tests; it is neither the oracle nor the GPU path, and imports neither the
GPU package nor anything the kernels use).

The chunk loop's arithmetic, written out in float64 with explicit bf16
roundings at the points where the kernels round (the kernels accumulate in
fp32; at these sizes that is far below the bf16 roundings):

* grad operands: the chunk-start weights W1, W3, W2 as bf16 (precise form:
  a hi/lo pair, hi = bf16(w), lo = bf16(w - hi));
* the three per-token factors handed to the aggregation, a = hv h3 silu'(h1),
  b = hv silu(h1), u = silu(h1) h3 (hv = V W2^T): in fp32, as the kernels
  hand them over (factors_rounded: as bf16, or with precise as the hi/lo
  pairs the precise kernel hands over);
* the coefficient-scaled aggregation operands -cM x, cW x as bf16
  (precise: hi/lo of c x);
* the state in fp32 between chunks; the scalar kernels' outputs in fp32;
* the output from bf16 chunk-start weights, the hidden activations
  silu(h1) h3 as bf16, and the result rounded to bf16.

The closed-form transition is the oracle's (M <- Bb M + G^M,
W <- A W - gamma M_old - G^W), its scalar kernels taken from
oracle.chunk_coefficients and rounded to fp32.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle


def _rb(x):
    return x.to(torch.bfloat16).to(torch.float64)


def _hilo_sum(x):
    hi = _rb(x)
    return hi + _rb(x - hi)


def swiglu_bf16_path(cfg, x, precise: bool = False, factors_rounded: bool = False, hilo_grad=()):
    """(out, W_end, M_end) of the bf16 MFMA path's rounding model for one
    SwiGLU / negative-dot workload (a shorter last chunk when T % chunk != 0).
    factors_rounded: the factors a, b, u are rounded to bf16 before the
    coefficient scaling as well as after it (a form of the chunk loop that
    handed them over in bf16); otherwise they are scaled in fp32 and rounded
    once.  hilo_grad: names among "W1", "W3", "W2" whose grad operand is a
    hi/lo pair while the rest of the path stays bf16 (precise: all of them,
    and the aggregation operands too)."""
    D, Hd, C, T, B, H = cfg.D, cfg.Hd, cfg.chunk, cfg.T, cfg.B, cfg.H
    op = _hilo_sum if precise else _rb
    gop = {name: (_hilo_sum if (precise or name in hilo_grad) else _rb) for name in ("W1", "W3", "W2")}
    q, k, v = (x[n].double() for n in ("q", "k", "v"))
    W = x["W0"].double().clone()
    M = x["M0"].double().clone()
    n = D * Hd
    f32 = lambda y: torch.from_numpy(np.asarray(y, dtype=np.float32)).double()
    out = torch.zeros(B, H, T, D, dtype=torch.float64)
    for c0 in range(0, T, C):
        L = min(C, T - c0)
        sl = slice(c0, c0 + L)
        # the chunk's scalar kernels (oracle), rounded to fp32 as the scan kernel writes them
        g = lambda name: x[name][:, :, sl].double().numpy().reshape(B, H, 1, L)
        m, w, A, Bb, gamma = oracle.chunk_coefficients(g("alpha"), g("beta"))
        e = g("eta")
        cM, cW = f32(m * e)[:, :, 0], f32(w * e)[:, :, 0]
        A, Bb, gamma = f32(A)[:, :, 0], f32(Bb)[:, :, 0], f32(gamma)[:, :, 0]
        W1 = W[..., :n].reshape(B, H, D, Hd)
        W3 = W[..., n:2 * n].reshape(B, H, D, Hd)
        W2 = W[..., 2 * n:].reshape(B, H, Hd, D)
        K, V, Q = k[:, :, sl], v[:, :, sl], q[:, :, sl]
        # grad products at the chunk-start weights and the factors
        h1, h3 = K @ gop["W1"](W1), K @ gop["W3"](W3)
        hv = V @ gop["W2"](W2).transpose(-1, -2)
        sg = torch.sigmoid(h1)
        s1 = h1 * sg
        ds = sg + s1 * (1 - sg)
        fa, fb, fu = hv * h3 * ds, hv * s1, s1 * h3
        if factors_rounded:
            fa, fb, fu = op(fa), op(fb), op(fu)
        # output from the bf16 snapshot of the chunk-start weights
        x1, x3 = Q @ _rb(W1), Q @ _rb(W3)
        out[:, :, sl] = _rb(_rb(x1 * torch.sigmoid(x1) * x3) @ _rb(W2))
        # transition with the old momentum, then the scaled aggregations
        cm, cw = cM[..., None], cW[..., None]
        Mold = M
        W = A[..., None] * W - gamma[..., None] * Mold
        M = Bb[..., None] * Mold
        Kt, Vt = K.transpose(-1, -2), V.transpose(-1, -2)
        gM = [Kt @ op(-cm * fa), Kt @ op(-cm * fb), (Vt @ op(-cm * fu)).transpose(-1, -2)]
        gW = [Kt @ op(cw * fa), Kt @ op(cw * fb), (Vt @ op(cw * fu)).transpose(-1, -2)]
        M = M + torch.cat([g.reshape(B, H, -1) for g in gM], -1)
        W = W + torch.cat([g.reshape(B, H, -1) for g in gW], -1)
        W, M = W.float().double(), M.float().double()
    return _rb(out).numpy(), W.numpy(), M.numpy()
