"""Pins for the oracle's variants: the no-momentum recurrence and the
chunk-averaged kernels.  Each test fixes the variant against something other
than its own closed form: the no-momentum per-token definition (brute force),
torch autograd SGD, the already-pinned momentum form, and the cases where the
chunk average reduces to the per-token kernels exactly.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests import autograd_ref as ar
from tests.test_oracle_pins import CASES, _rand_inputs


def _run(fn, kind, loss, x, chunk, Hd, **kw):
    return fn(kind, loss, x["q"], x["k"], x["v"], x["eta"], x["alpha"], x["beta"],
              x["W0"], x["M0"], chunk, Hd, **kw)


# --------------------------------------------------------------------------
# NM1: no-momentum closed form == its per-token definition
#      W_t = alpha_t W_{t-1} - eta_t g_t (gradients frozen at chunk start)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("kind,loss", CASES)
@pytest.mark.parametrize("chunk", [1, 3, 16])
def test_nm1_closed_form_equals_brute_force(kind, loss, chunk):
    D, Hd = 5, 7
    x = _rand_inputs(kind, 2, 2, 4 * chunk, D, Hd, seed=chunk + 300)
    ref = _run(oracle.brute_force, kind, loss, x, chunk, Hd, momentum=False)
    got = _run(oracle.chunk_forward, kind, loss, x, chunk, Hd, momentum=False)
    assert ref[2] is None and got[2] is None
    for a, b in zip(got[:2], ref[:2]):
        assert oracle.rel_err(a, b) < 1e-12


# --------------------------------------------------------------------------
# NM2: chunk size 1 -> token-wise decayed SGD with autograd gradients at the
#      current weights, written independently of the oracle
# --------------------------------------------------------------------------
@pytest.mark.parametrize("kind,loss", CASES)
def test_nm2_chunk1_is_decayed_sgd(kind, loss):
    D, Hd, T = 6, 9, 10
    x = _rand_inputs(kind, 1, 2, T, D, Hd, seed=311)
    out, W, M = _run(oracle.chunk_forward, kind, loss, x, 1, Hd, momentum=False)
    assert M is None
    for h in range(2):
        Wt = torch.tensor(x["W0"][0, h])
        for t in range(T):
            o = ar.output(kind, Wt, torch.tensor(x["q"][0, h, t]), D, Hd)
            assert oracle.rel_err(out[0, h, t], o.numpy()) < 1e-12
            g = ar.token_grad(kind, loss, Wt, torch.tensor(x["k"][0, h, t]), torch.tensor(x["v"][0, h, t]), D, Hd)
            Wt = x["alpha"][0, h, t] * Wt - x["eta"][0, h, t] * g
        assert oracle.rel_err(W[0, h], Wt.numpy()) < 1e-12


# --------------------------------------------------------------------------
# NM3: alpha = 1 -> plain gradient descent over the chunk: the chunk-end
#      weight is W0 - sum_t eta_t g_t(W0), gradients from autograd
# --------------------------------------------------------------------------
@pytest.mark.parametrize("kind,loss", CASES)
def test_nm3_no_decay_is_summed_gradient_step(kind, loss):
    D, Hd, C = 5, 6, 8
    x = _rand_inputs(kind, 1, 1, C, D, Hd, seed=312, gates=(1.0, 0.5))
    _, W, _ = _run(oracle.chunk_forward, kind, loss, x, C, Hd, momentum=False)
    W0 = torch.tensor(x["W0"][0, 0])
    step = sum(x["eta"][0, 0, t] * ar.token_grad(kind, loss, W0, torch.tensor(x["k"][0, 0, t]),
                                                 torch.tensor(x["v"][0, 0, t]), D, Hd) for t in range(C))
    assert oracle.rel_err(W[0, 0], (W0 - step).numpy()) < 1e-12


# --------------------------------------------------------------------------
# NM4: constant decay -> w_i = a^(C-1-i), A = a^C (geometric closed form)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("a", [0.97, 0.5, 1.0, 0.0])
@pytest.mark.parametrize("C", [1, 7, 64])
def test_nm4_constant_decay_powers(a, C):
    w, A = oracle.chunk_coefficients_nomomentum(np.full(C, a))
    i = np.arange(C)
    assert np.allclose(w, np.power(a, C - 1 - i), rtol=1e-13, atol=0)
    assert math.isclose(float(A), a ** C, rel_tol=1e-13, abs_tol=0)


# --------------------------------------------------------------------------
# NM5: the no-momentum weight path equals the (pinned) momentum form run with
#      beta = 0 and M0 = 0 (where M_t = eta_t g_t and W_t = alpha_t W_{t-1} - M_t)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("kind,loss", CASES)
def test_nm5_equals_momentum_form_with_beta_zero(kind, loss):
    D, Hd, C = 5, 7, 6
    x = _rand_inputs(kind, 1, 3, 3 * C, D, Hd, seed=313)
    y = dict(x, beta=np.zeros_like(x["beta"]), M0=np.zeros_like(x["M0"]))
    out_m, W_m, _ = _run(oracle.chunk_forward, kind, loss, y, C, Hd)
    out_n, W_n, _ = _run(oracle.chunk_forward, kind, loss, x, C, Hd, momentum=False)
    assert oracle.rel_err(out_n, out_m) < 1e-13
    assert oracle.rel_err(W_n, W_m) < 1e-13


# --------------------------------------------------------------------------
# AV1: chunk size 1 -> the chunk average is the per-token kernel itself
# --------------------------------------------------------------------------
@pytest.mark.parametrize("kind,loss", CASES)
@pytest.mark.parametrize("momentum", [True, False])
def test_av1_chunk1_equals_per_token(kind, loss, momentum):
    D, Hd, T = 5, 6, 9
    x = _rand_inputs(kind, 1, 2, T, D, Hd, seed=321)
    ref = _run(oracle.chunk_forward, kind, loss, x, 1, Hd, momentum=momentum)
    got = _run(oracle.chunk_forward, kind, loss, x, 1, Hd, momentum=momentum, chunk_avg=True)
    for a, b in zip(got, ref):
        if b is not None:
            assert oracle.rel_err(a, b) == 0.0


# --------------------------------------------------------------------------
# AV2: equal tokens within each chunk (same k, v) and a constant learning rate
#      per chunk -> sum_i mean(w) eta g = sum_i w_i eta g, so the averaged and
#      per-token transitions coincide (a sum in place of the mean, or averaging
#      the wrong quantity, breaks this); with distinct tokens they differ
# --------------------------------------------------------------------------
@pytest.mark.parametrize("kind,loss", CASES)
@pytest.mark.parametrize("momentum", [True, False])
def test_av2_equal_tokens_reduce_to_per_token(kind, loss, momentum):
    D, Hd, C, nc = 5, 6, 8, 3
    x = _rand_inputs(kind, 1, 2, C * nc, D, Hd, seed=322)
    y = dict(x)
    for n in ("k", "v"):
        y[n] = np.repeat(x[n][:, :, ::C], C, axis=2)
    y["eta"] = np.repeat(x["eta"][:, :, ::C], C, axis=2)
    ref = _run(oracle.chunk_forward, kind, loss, y, C, Hd, momentum=momentum)
    got = _run(oracle.chunk_forward, kind, loss, y, C, Hd, momentum=momentum, chunk_avg=True)
    for a, b in zip(got, ref):
        if b is not None:
            assert oracle.rel_err(a, b) < 1e-12
    ref = _run(oracle.chunk_forward, kind, loss, x, C, Hd, momentum=momentum)
    got = _run(oracle.chunk_forward, kind, loss, x, C, Hd, momentum=momentum, chunk_avg=True)
    assert oracle.rel_err(got[1], ref[1]) > 1e-6


# --------------------------------------------------------------------------
# AV3: alpha = beta = 1 -> m_i = 1 and w_i = C - i (i = 0..C-1), so the
#      averaged coefficients are cM_t = eta_t and cW_t = (C + 1)/2 eta_t, with
#      each token keeping its own learning rate
# --------------------------------------------------------------------------
@pytest.mark.parametrize("C", [1, 5, 32])
def test_av3_unit_gates_closed_form(C):
    x = _rand_inputs("linear", 1, 2, 2 * C, 4, 0, seed=323, gates=(1.0, 1.0))
    *_, inter = oracle.chunk_forward("linear", "mse", x["q"], x["k"], x["v"], x["eta"], x["alpha"], x["beta"],
                                     x["W0"], x["M0"], C, 0, keep=True, chunk_avg=True)
    eta = x["eta"].reshape(2, 2 * C)
    for c, it in enumerate(inter):
        e = eta[:, c * C:(c + 1) * C]
        assert np.allclose(it["cM"], e, rtol=1e-14, atol=0)
        assert np.allclose(it["cW"], (C + 1) / 2 * e, rtol=1e-14, atol=0)
