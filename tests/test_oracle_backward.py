"""Pins for the backward oracle (oracle/e2ttt_backward.py).

Each pin fixes it against something other than itself:
  BP1  its torch forward equals the numpy closed form of e2ttt_oracle;
  BP2  its gradients equal central finite differences of the numpy closed
       form along random directions (every input, every kind and variant);
  BP3  its gradients equal autograd through an independent per-token
       recurrence whose per-token gradients come from autograd (no written-out
       gradient formulas), with the fast-weight models of tests/autograd_ref;
  BP4  the map from cotangents to gradients is linear.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import e2ttt_backward as ob
from tests import autograd_ref as ar

CASES = [("linear", "mse"), ("mlp", "mse"), ("mlp", "negdot"), ("swiglu", "negdot"), ("swiglu", "mse")]


def _inputs(kind, B, H, T, D, Hd, seed, momentum=True):
    rng = np.random.default_rng(seed)
    P = oracle.param_count(kind, D, Hd)
    x = {}
    x["q"] = rng.standard_normal((B, H, T, D)) / math.sqrt(D)
    x["k"] = rng.standard_normal((B, H, T, D)) / math.sqrt(D)
    x["v"] = rng.standard_normal((B, H, T, D))
    x["eta"] = 0.1 * np.log1p(np.exp(rng.standard_normal((B, H, T))))
    x["alpha"] = 1 / (1 + np.exp(-(1.5 + rng.standard_normal((B, H, T)))))
    x["beta"] = 1 / (1 + np.exp(-(0.5 + rng.standard_normal((B, H, T)))))
    x["W0"] = rng.standard_normal((B, H, P)) / math.sqrt(D)
    x["M0"] = 0.3 * rng.standard_normal((B, H, P)) / math.sqrt(D)
    cot = {"dout": rng.standard_normal((B, H, T, D)), "dW_end": rng.standard_normal((B, H, P)),
           "dM_end": rng.standard_normal((B, H, P))}
    if not momentum:
        x["beta"] = x["M0"] = cot["dM_end"] = None
    return x, cot


def _objective(kind, loss, x, cot, chunk, Hd, momentum, chunk_avg):
    out, W, M = oracle.chunk_forward(kind, loss, x["q"], x["k"], x["v"], x["eta"], x["alpha"], x["beta"],
                                     x["W0"], x["M0"], chunk, Hd, momentum=momentum, chunk_avg=chunk_avg)
    f = np.sum(out * cot["dout"]) + np.sum(W * cot["dW_end"])
    if momentum:
        f += np.sum(M * cot["dM_end"])
    return f


def _grads(kind, loss, x, cot, chunk, Hd, momentum=True, chunk_avg=False):
    return ob.chunk_backward(kind, loss, x["q"], x["k"], x["v"], x["eta"], x["alpha"], x["beta"], x["W0"],
                             x["M0"], cot["dout"], cot["dW_end"], cot["dM_end"], chunk, Hd, momentum=momentum,
                             chunk_avg=chunk_avg)


# --------------------------------------------------------------------------
# BP1: the torch forward is the numpy closed form
# --------------------------------------------------------------------------
@pytest.mark.parametrize("kind,loss", CASES)
@pytest.mark.parametrize("momentum,chunk_avg,T", [(True, False, 12), (False, False, 12), (True, True, 12),
                                                  (True, False, 11)])
def test_bp1_torch_forward_equals_numpy(kind, loss, momentum, chunk_avg, T):
    D, Hd, chunk = (5, 7, 4) if kind != "linear" else (6, 0, 4)
    x, _ = _inputs(kind, 1, 2, T, D, Hd, seed=1, momentum=momentum)
    ref = oracle.chunk_forward(kind, loss, x["q"], x["k"], x["v"], x["eta"], x["alpha"], x["beta"], x["W0"],
                               x["M0"], chunk, Hd, momentum=momentum, chunk_avg=chunk_avg)
    P = x["W0"].shape[-1]
    t = lambda a, *tail: torch.tensor(np.asarray(a).reshape(2, *tail))
    beta = t(x["beta"], T) if momentum else torch.zeros(2, T, dtype=torch.float64)
    M0 = t(x["M0"], P) if momentum else torch.zeros(2, P, dtype=torch.float64)
    out, W, M = ob.chunk_forward_torch(kind, loss, t(x["q"], T, D), t(x["k"], T, D), t(x["v"], T, D),
                                       t(x["eta"], T), t(x["alpha"], T), beta, t(x["W0"], P), M0, chunk, Hd,
                                       momentum, chunk_avg)
    assert oracle.rel_err(out.numpy().reshape(ref[0].shape), ref[0]) < 1e-13
    assert oracle.rel_err(W.numpy().reshape(ref[1].shape), ref[1]) < 1e-13
    if momentum:
        assert oracle.rel_err(M.numpy().reshape(ref[2].shape), ref[2]) < 1e-13


# --------------------------------------------------------------------------
# BP2: central finite differences of the numpy closed form
# --------------------------------------------------------------------------
@pytest.mark.parametrize("kind,loss", CASES)
@pytest.mark.parametrize("momentum,chunk_avg,T", [(True, False, 9), (False, False, 9), (True, True, 8)])
def test_bp2_finite_differences(kind, loss, momentum, chunk_avg, T):
    D, Hd, chunk = (4, 5, 3) if kind != "linear" else (4, 0, 3)
    x, cot = _inputs(kind, 1, 2, T, D, Hd, seed=2, momentum=momentum)
    g = _grads(kind, loss, x, cot, chunk, Hd, momentum, chunk_avg)
    rng = np.random.default_rng(7)
    h = 1e-5
    for name in ob.INPUTS:
        if x[name] is None:
            assert g[name] is None
            continue
        d = rng.standard_normal(x[name].shape)
        xp = dict(x, **{name: x[name] + h * d})
        xm = dict(x, **{name: x[name] - h * d})
        fd = (_objective(kind, loss, xp, cot, chunk, Hd, momentum, chunk_avg)
              - _objective(kind, loss, xm, cot, chunk, Hd, momentum, chunk_avg)) / (2 * h)
        an = float(np.sum(g[name] * d))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)


def test_bp2_catches_a_dropped_gate_gradient():
    """The finite-difference check sees a gradient that misses one token's term."""
    kind, loss, chunk, D, Hd, T = "swiglu", "negdot", 3, 4, 5, 6
    x, cot = _inputs(kind, 1, 1, T, D, Hd, seed=5)
    g = _grads(kind, loss, x, cot, chunk, Hd)
    g["alpha"][0, 0, 2] = 0.0  # planted mistake
    d = np.zeros_like(x["alpha"])
    d[0, 0, 2] = 1.0
    h = 1e-5
    fd = (_objective(kind, loss, dict(x, alpha=x["alpha"] + h * d), cot, chunk, Hd, True, False)
          - _objective(kind, loss, dict(x, alpha=x["alpha"] - h * d), cot, chunk, Hd, True, False)) / (2 * h)
    assert abs(fd) > 1e-6 and abs(fd - np.sum(g["alpha"] * d)) > 1e-6


# --------------------------------------------------------------------------
# BP3: autograd through an independent per-token recurrence
# --------------------------------------------------------------------------
def _brute_objective(kind, loss, leaves, cot, chunk, D, Hd, momentum):
    """<dout, out> + <dW, W_end> + <dM, M_end> of one (b, h) by the per-token
    recurrence, per-token gradients at the chunk-start weights by autograd."""
    q, k, v, eta, alpha = leaves["q"], leaves["k"], leaves["v"], leaves["eta"], leaves["alpha"]
    T = q.shape[0]
    W = leaves["W0"]
    M = leaves["M0"] if momentum else torch.zeros_like(W)
    obj = 0.0
    for c0 in range(0, T, chunk):
        Wc = W
        mats = ar.split(kind, Wc, D, Hd)
        for t in range(c0, min(c0 + chunk, T)):
            obj = obj + (ar.model(kind, mats, q[t]) * cot["dout"][t]).sum()
        for t in range(c0, min(c0 + chunk, T)):
            ell = ar.loss_fn(loss, ar.model(kind, mats, k[t]), v[t])
            (g,) = torch.autograd.grad(ell, Wc, create_graph=True)
            if momentum:
                M = leaves["beta"][t] * M + eta[t] * g
                W = alpha[t] * W - M
            else:
                W = alpha[t] * W - eta[t] * g
    obj = obj + (W * cot["dW_end"]).sum()
    if momentum:
        obj = obj + (M * cot["dM_end"]).sum()
    return obj


@pytest.mark.parametrize("kind,loss", CASES)
@pytest.mark.parametrize("momentum,T", [(True, 8), (False, 8), (True, 7)])
def test_bp3_autograd_of_the_recurrence(kind, loss, momentum, T):
    D, Hd, chunk = (4, 5, 4) if kind != "linear" else (5, 0, 4)
    x, cot = _inputs(kind, 1, 2, T, D, Hd, seed=3, momentum=momentum)
    g = _grads(kind, loss, x, cot, chunk, Hd, momentum)
    for h in range(2):
        leaves = {n: torch.tensor(x[n][0, h], requires_grad=True) for n in ob.INPUTS if x[n] is not None}
        c = {n: torch.tensor(a[0, h]) for n, a in cot.items() if a is not None}
        obj = _brute_objective(kind, loss, leaves, c, chunk, D, Hd, momentum)
        names = list(leaves)
        ref = torch.autograd.grad(obj, [leaves[n] for n in names])
        for n, r in zip(names, ref):
            assert oracle.rel_err(g[n][0, h], r.numpy()) < 1e-10, n


# --------------------------------------------------------------------------
# BP4: linear in the cotangents
# --------------------------------------------------------------------------
def test_bp4_linear_in_cotangents():
    kind, loss, chunk, D, Hd, T = "swiglu", "negdot", 4, 4, 6, 8
    x, c1 = _inputs(kind, 1, 2, T, D, Hd, seed=4)
    _, c2 = _inputs(kind, 1, 2, T, D, Hd, seed=5)
    g1 = _grads(kind, loss, x, c1, chunk, Hd)
    g2 = _grads(kind, loss, x, c2, chunk, Hd)
    c3 = {n: 2.0 * c1[n] - 0.5 * c2[n] for n in c1}
    g3 = _grads(kind, loss, x, c3, chunk, Hd)
    for n in ob.INPUTS:
        assert oracle.rel_err(g3[n], 2.0 * g1[n] - 0.5 * g2[n]) < 1e-12, n
    zero = {n: np.zeros_like(a) for n, a in c1.items()}
    gz = _grads(kind, loss, x, zero, chunk, Hd)
    assert all(np.all(gz[n] == 0) for n in ob.INPUTS)
