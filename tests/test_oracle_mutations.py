"""The pins must catch plausible mistakes: each test plants one mistake in the
oracle (monkeypatched, CPU only) and checks that a pin comparison then fails."""
import numpy as np
import pytest
import torch

import oracle
import oracle.e2ttt_oracle as eo
from tests import autograd_ref as ar
from tests.test_oracle_pins import _rand_inputs, _run


def _p1_err(kind, loss, chunk=4):
    D, Hd = 5, 7
    x = _rand_inputs(kind, 1, 2, 3 * chunk, D, Hd, seed=77)
    ref = _run(oracle.brute_force, kind, loss, x, chunk, Hd)
    got = _run(oracle.chunk_forward, kind, loss, x, chunk, Hd)
    return max(oracle.rel_err(a, b) for a, b in zip(got, ref))


def _p8_err(kind, loss):
    rng = np.random.default_rng(2)
    D, Hd, N = 5, 7, 3
    P = oracle.param_count(kind, D, Hd)
    p = rng.standard_normal(P) / np.sqrt(D)
    K = rng.standard_normal((N, D))
    V = rng.standard_normal((N, D))
    fac = eo.grad_factors(kind, loss, eo.unpack(kind, p, D, Hd), K, V)
    err = 0.0
    for i in range(N):
        c = np.eye(N)[i]
        g = eo.pack(kind, eo.weighted_grad_sum(kind, fac, K, c))
        ga = ar.token_grad(kind, loss, torch.tensor(p), torch.tensor(K[i]), torch.tensor(V[i]), D, Hd).numpy()
        err = max(err, oracle.rel_err(g, ga))
    return err


def test_unmutated_baseline():
    assert _p1_err("swiglu", "negdot") < 1e-12
    assert _p8_err("swiglu", "negdot") < 1e-12


def test_dropped_gamma_term_is_caught(monkeypatch):
    orig = eo.chunk_coefficients

    def bad(alpha, beta):
        m, w, A, Bb, gamma = orig(alpha, beta)
        return m, w, A, Bb, 0.0 * gamma
    monkeypatch.setattr(eo, "chunk_coefficients", bad)
    assert _p1_err("swiglu", "negdot") > 1e-6


def test_off_by_one_momentum_kernel_is_caught(monkeypatch):
    orig = eo.chunk_coefficients

    def bad(alpha, beta):
        m, w, A, Bb, gamma = orig(alpha, beta)
        return m * beta, w, A, Bb, gamma  # includes beta_i itself
    monkeypatch.setattr(eo, "chunk_coefficients", bad)
    assert _p1_err("mlp", "mse") > 1e-6


def test_wrong_silu_derivative_is_caught(monkeypatch):
    monkeypatch.setattr(eo, "dsilu", lambda x: eo.sigmoid(x))
    assert _p8_err("swiglu", "negdot") > 1e-6
    assert _p8_err("mlp", "mse") > 1e-6


def test_transposed_operand_is_caught(monkeypatch):
    orig = eo.weighted_grad_sum

    def bad(kind, fac, K, c):
        out = orig(kind, fac, K, c)
        if kind == "linear":
            out["W"] = np.swapaxes(out["W"], -1, -2)
        return out
    monkeypatch.setattr(eo, "weighted_grad_sum", bad)
    assert _p8_err("linear", "mse") > 1e-6


def test_sign_flip_in_loss_gradient_is_caught(monkeypatch):
    orig = eo._dloss_dy
    monkeypatch.setattr(eo, "_dloss_dy", lambda loss, Y, V: -orig(loss, Y, V))
    assert _p8_err("swiglu", "negdot") > 1e-6
