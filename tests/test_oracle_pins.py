"""Pins for the fp64 oracle: each test fixes part of it against something other
than itself (the brute-force definition, torch autograd, finite differences,
closed forms of special gates, algebraic invariants).

The pages print no worked example or intermediate value, so there are no
page-printed fixtures; every pin below is mathematical.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests import autograd_ref as ar

CASES = [("linear", "mse"), ("linear", "negdot"), ("mlp", "mse"), ("mlp", "negdot"),
         ("swiglu", "negdot"), ("swiglu", "mse")]


def _rand_inputs(kind, B, H, T, D, Hd, seed, m0=0.3, gates="random"):
    rng = np.random.default_rng(seed)
    P = oracle.param_count(kind, D, Hd)
    q = rng.standard_normal((B, H, T, D))
    k = rng.standard_normal((B, H, T, D))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, T, D))
    eta = 0.1 * np.log1p(np.exp(rng.standard_normal((B, H, T))))
    if gates == "random":
        alpha = 1 / (1 + np.exp(-(1.0 + rng.standard_normal((B, H, T)))))
        beta = 1 / (1 + np.exp(-(0.5 + rng.standard_normal((B, H, T)))))
    else:
        alpha, beta = gates
        alpha = np.broadcast_to(alpha, (B, H, T)).copy()
        beta = np.broadcast_to(beta, (B, H, T)).copy()
    W0 = rng.standard_normal((B, H, P)) / math.sqrt(D)
    M0 = m0 * rng.standard_normal((B, H, P)) / math.sqrt(D)
    return dict(q=q, k=k, v=v, eta=eta, alpha=alpha, beta=beta, W0=W0, M0=M0)


def _run(fn, kind, loss, x, chunk, Hd, **kw):
    return fn(kind, loss, x["q"], x["k"], x["v"], x["eta"], x["alpha"], x["beta"],
              x["W0"], x["M0"], chunk, Hd, **kw)


# --------------------------------------------------------------------------
# P1: closed form == brute-force per-token recurrence with frozen gradients
# --------------------------------------------------------------------------
@pytest.mark.parametrize("kind,loss", CASES)
@pytest.mark.parametrize("chunk", [1, 2, 3, 16])
def test_p1_closed_form_equals_brute_force(kind, loss, chunk):
    D, Hd = (6, 10) if kind != "linear" else (7, 0)
    x = _rand_inputs(kind, 2, 2, 4 * chunk, D, Hd, seed=chunk)
    ref = _run(oracle.brute_force, kind, loss, x, chunk, Hd)
    got = _run(oracle.chunk_forward, kind, loss, x, chunk, Hd)
    for a, b in zip(got, ref):
        assert oracle.rel_err(a, b) < 1e-12


def test_p1_edge_gates_zero_alpha_beta():
    """alpha = 0 and beta = 0 inside a chunk: still exact, no NaN."""
    kind, loss, chunk, D, Hd = "swiglu", "negdot", 8, 5, 7
    x = _rand_inputs(kind, 1, 2, 32, D, Hd, seed=3)
    x["alpha"][0, 0, [3, 11, 20]] = 0.0
    x["beta"][0, 1, [0, 7, 8, 31]] = 0.0
    x["eta"][0, 0, 5] = 0.0
    ref = _run(oracle.brute_force, kind, loss, x, chunk, Hd)
    got = _run(oracle.chunk_forward, kind, loss, x, chunk, Hd)
    for a, b in zip(got, ref):
        assert np.all(np.isfinite(a))
        assert oracle.rel_err(a, b) < 1e-12


# --------------------------------------------------------------------------
# P2: alpha = beta = 1 -> plain momentum SGD
# --------------------------------------------------------------------------
@pytest.mark.parametrize("C", [1, 5, 64])
def test_p2_unit_gates_coefficients(C):
    m, w, A, Bb, gamma = oracle.chunk_coefficients(np.ones(C), np.ones(C))
    assert np.array_equal(m, np.ones(C))
    assert np.array_equal(w, np.arange(C, 0, -1, dtype=np.float64))  # C-i+1 for i=1..C
    assert A == 1.0 and Bb == 1.0 and gamma == float(C)


@pytest.mark.parametrize("kind,loss", CASES[:5])
def test_p2_unit_gates_momentum_sgd(kind, loss):
    D, Hd, C = 5, 6, 6
    x = _rand_inputs(kind, 1, 1, C, D, Hd, seed=7, gates=(1.0, 1.0))
    out, W, M = _run(oracle.chunk_forward, kind, loss, x, C, Hd)
    p0 = torch.tensor(x["W0"][0, 0])
    Mt = torch.tensor(x["M0"][0, 0])
    Wt = p0.clone()
    for i in range(C):  # M += eta g(W0); W -= M
        g = ar.token_grad(kind, loss, p0, torch.tensor(x["k"][0, 0, i]), torch.tensor(x["v"][0, 0, i]), D, Hd)
        Mt = Mt + x["eta"][0, 0, i] * g
        Wt = Wt - Mt
    assert oracle.rel_err(W[0, 0], Wt.numpy()) < 1e-13
    assert oracle.rel_err(M[0, 0], Mt.numpy()) < 1e-13


# --------------------------------------------------------------------------
# P3: beta = 0 -> decayed SGD, momentum keeps only the last token
# --------------------------------------------------------------------------
def test_p3_zero_beta_coefficients():
    rng = np.random.default_rng(1)
    C = 9
    alpha = rng.uniform(0.2, 1.0, C)
    m, w, A, Bb, gamma = oracle.chunk_coefficients(alpha, np.zeros(C))
    assert np.array_equal(m, np.eye(C)[-1])
    for i in range(C):
        assert abs(w[i] - math.prod(alpha[i + 1:])) <= 1e-15
    assert gamma == 0.0 and Bb == 0.0
    assert abs(A - math.prod(alpha)) < 1e-15


@pytest.mark.parametrize("kind,loss", CASES[:5])
def test_p3_zero_beta_decayed_sgd(kind, loss):
    D, Hd, C = 5, 6, 7
    rng = np.random.default_rng(11)
    x = _rand_inputs(kind, 1, 1, C, D, Hd, seed=9, gates=(rng.uniform(0.5, 1.0, C), 0.0))
    out, W, M = _run(oracle.chunk_forward, kind, loss, x, C, Hd)
    p0 = torch.tensor(x["W0"][0, 0])
    Wt = p0.clone()
    g = None
    for i in range(C):  # W_t = alpha_t W_{t-1} - eta_t g_t(W0)
        g = ar.token_grad(kind, loss, p0, torch.tensor(x["k"][0, 0, i]), torch.tensor(x["v"][0, 0, i]), D, Hd)
        Wt = x["alpha"][0, 0, i] * Wt - x["eta"][0, 0, i] * g
    assert oracle.rel_err(W[0, 0], Wt.numpy()) < 1e-13
    assert oracle.rel_err(M[0, 0], (x["eta"][0, 0, C - 1] * g).numpy()) < 1e-13


# --------------------------------------------------------------------------
# P4: chunk size 1 -> exact token-wise TTT (gradients at the current weights)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("kind,loss", CASES)
def test_p4_chunk1_is_tokenwise_ttt(kind, loss):
    D, Hd, T = 6, 9, 12
    x = _rand_inputs(kind, 1, 2, T, D, Hd, seed=21)
    out, W, M = _run(oracle.chunk_forward, kind, loss, x, 1, Hd)
    for h in range(2):
        Wt = torch.tensor(x["W0"][0, h])
        Mt = torch.tensor(x["M0"][0, h])
        for t in range(T):
            o = ar.output(kind, Wt, torch.tensor(x["q"][0, h, t]), D, Hd)
            assert oracle.rel_err(out[0, h, t], o.numpy()) < 1e-12
            g = ar.token_grad(kind, loss, Wt, torch.tensor(x["k"][0, h, t]), torch.tensor(x["v"][0, h, t]), D, Hd)
            Mt = x["beta"][0, h, t] * Mt + x["eta"][0, h, t] * g
            Wt = x["alpha"][0, h, t] * Wt - Mt
        assert oracle.rel_err(W[0, h], Wt.numpy()) < 1e-12
        assert oracle.rel_err(M[0, h], Mt.numpy()) < 1e-12


# --------------------------------------------------------------------------
# P5: constant gates -> geometric sums
# --------------------------------------------------------------------------
@pytest.mark.parametrize("a,b", [(0.97, 0.8), (0.5, 0.5), (0.8, 0.97), (1.0, 0.9), (0.3, 1.0)])
@pytest.mark.parametrize("C", [1, 7, 256])
def test_p5_constant_gates_geometric(a, b, C):
    m, w, A, Bb, gamma = oracle.chunk_coefficients(np.full(C, a), np.full(C, b))
    for i in range(1, C + 1):  # 1-indexed token i
        n = C - i + 1
        ref_w = n * a ** (n - 1) if a == b else (a ** n - b ** n) / (a - b)
        assert abs(w[i - 1] - ref_w) <= 1e-13 * max(1.0, ref_w)
        assert abs(m[i - 1] - b ** (C - i)) <= 1e-13
    assert abs(A - a ** C) < 1e-13 and abs(Bb - b ** C) < 1e-13
    ref_g = b * w[0]
    assert abs(gamma - ref_g) <= 1e-13 * max(1.0, ref_g)


def test_gamma_equals_beta1_w1_and_bound():
    rng = np.random.default_rng(5)
    for C in (1, 2, 17, 300):
        al = rng.uniform(0, 1, C)
        be = rng.uniform(0, 1, C)
        m, w, A, Bb, gamma = oracle.chunk_coefficients(al, be)
        assert abs(gamma - be[0] * w[0]) <= 1e-13 * max(1, gamma)
        assert np.all(w <= np.arange(C, 0, -1) + 1e-12) and np.all(w >= 0)


# --------------------------------------------------------------------------
# P6: semigroup -- splitting a chunk's frozen-gradient transition
# --------------------------------------------------------------------------
@pytest.mark.parametrize("j", [1, 5, 11])
def test_p6_semigroup(j):
    rng = np.random.default_rng(j)
    C, P = 12, 20
    g = rng.standard_normal((C, P))
    eta = rng.uniform(0, 0.2, C)
    al = rng.uniform(0.3, 1, C)
    be = rng.uniform(0.0, 1, C)
    W0 = rng.standard_normal(P)
    M0 = rng.standard_normal(P)
    W_full, M_full = oracle.closed_form_transition(g, eta, al, be, W0, M0)
    W1, M1 = oracle.closed_form_transition(g[:j], eta[:j], al[:j], be[:j], W0, M0)
    W2, M2 = oracle.closed_form_transition(g[j:], eta[j:], al[j:], be[j:], W1, M1)
    assert oracle.rel_err(W2, W_full) < 1e-13
    assert oracle.rel_err(M2, M_full) < 1e-13


# --------------------------------------------------------------------------
# P7: resume -- two calls with carried state equal one call
# --------------------------------------------------------------------------
@pytest.mark.parametrize("kind,loss", CASES[:5])
def test_p7_resume(kind, loss):
    D, Hd, C = 6, 8, 4
    x = _rand_inputs(kind, 2, 1, 5 * C, D, Hd, seed=31)
    full = _run(oracle.chunk_forward, kind, loss, x, C, Hd)
    T1 = 2 * C
    a = {n: (t[:, :, :T1] if t.ndim >= 3 and n not in ("W0", "M0") else t) for n, t in x.items()}
    out1, W1, M1 = _run(oracle.chunk_forward, kind, loss, a, C, Hd)
    b = {n: (t[:, :, T1:] if t.ndim >= 3 and n not in ("W0", "M0") else t) for n, t in x.items()}
    b["W0"], b["M0"] = W1, M1
    out2, W2, M2 = _run(oracle.chunk_forward, kind, loss, b, C, Hd)
    assert np.array_equal(np.concatenate([out1, out2], axis=2), full[0])
    assert np.array_equal(W2, full[1]) and np.array_equal(M2, full[2])


# --------------------------------------------------------------------------
# P8: per-token gradients vs autograd and central finite differences
# --------------------------------------------------------------------------
@pytest.mark.parametrize("kind,loss", CASES)
def test_p8_gradients_vs_autograd_and_fd(kind, loss):
    rng = np.random.default_rng(2)
    D, Hd, N = 5, 7, 4
    P = oracle.param_count(kind, D, Hd)
    p = rng.standard_normal(P) / math.sqrt(D)
    K = rng.standard_normal((N, D))
    V = rng.standard_normal((N, D))
    mats = oracle.unpack(kind, p, D, Hd)
    fac = oracle.grad_factors(kind, loss, mats, K, V)
    for i in range(N):
        c = np.zeros(N)
        c[i] = 1.0
        g = oracle.pack(kind, oracle.weighted_grad_sum(kind, fac, K, c))
        ga = ar.token_grad(kind, loss, torch.tensor(p), torch.tensor(K[i]), torch.tensor(V[i]), D, Hd).numpy()
        assert oracle.rel_err(g, ga) < 1e-13
        # central differences of the token loss
        h = 1e-5
        fd = np.empty(P)
        for j in range(P):
            e = np.zeros(P)
            e[j] = h
            lp = ar.token_loss(kind, loss, torch.tensor(p + e), torch.tensor(K[i]), torch.tensor(V[i]), D, Hd)
            lm = ar.token_loss(kind, loss, torch.tensor(p - e), torch.tensor(K[i]), torch.tensor(V[i]), D, Hd)
            fd[j] = (lp - lm) / (2 * h)
        assert oracle.rel_err(g, fd) < 1e-8
    # outputs vs the torch model
    Y = oracle.fast_weight_forward(kind, mats, K)
    for i in range(N):
        assert oracle.rel_err(Y[i], ar.output(kind, torch.tensor(p), torch.tensor(K[i]), D, Hd).numpy()) < 1e-13


def test_token_grads_match_weighted_sum():
    rng = np.random.default_rng(4)
    for kind, loss in CASES:
        D, Hd, N = 4, 6, 5
        P = oracle.param_count(kind, D, Hd)
        p = rng.standard_normal(P)
        K = rng.standard_normal((N, D))
        V = rng.standard_normal((N, D))
        mats = oracle.unpack(kind, p, D, Hd)
        c = rng.standard_normal(N)
        g = oracle.pack(kind, oracle.token_grads(kind, loss, mats, K, V))
        s = oracle.pack(kind, oracle.weighted_grad_sum(kind, oracle.grad_factors(kind, loss, mats, K, V), K, c))
        assert oracle.rel_err(np.einsum("i,ip->p", c, g), s) < 1e-13


# --------------------------------------------------------------------------
# P9: linearity in eta with M0 = 0
# --------------------------------------------------------------------------
@pytest.mark.parametrize("kind,loss", CASES[:5])
def test_p9_linear_in_eta(kind, loss):
    D, Hd, C = 5, 6, 8
    x = _rand_inputs(kind, 1, 2, C, D, Hd, seed=41, m0=0.0)
    out, W, M, inter = oracle.chunk_forward(kind, loss, x["q"], x["k"], x["v"], x["eta"], x["alpha"],
                                            x["beta"], x["W0"], x["M0"], C, Hd, keep=True)
    s = 2.5
    y = dict(x)
    y["eta"] = s * x["eta"]
    out2, W2, M2, inter2 = oracle.chunk_forward(kind, loss, y["q"], y["k"], y["v"], y["eta"], y["alpha"],
                                                y["beta"], y["W0"], y["M0"], C, Hd, keep=True)
    A = inter[0]["A"][:, None].reshape(1, 2, 1)
    assert oracle.rel_err(M2, s * M) < 1e-13
    assert oracle.rel_err(W2 - A * x["W0"], s * (W - A * x["W0"])) < 1e-12
    assert oracle.rel_err(inter2[0]["GM"], s * inter[0]["GM"]) < 1e-13
    assert oracle.rel_err(inter2[0]["GW"], s * inter[0]["GW"]) < 1e-13


def test_pack_unpack_roundtrip():
    rng = np.random.default_rng(0)
    for kind in oracle.KINDS:
        P = oracle.param_count(kind, 4, 6)
        p = rng.standard_normal((3, P))
        assert np.array_equal(oracle.pack(kind, oracle.unpack(kind, p, 4, 6)), p)


def test_rejects_bad_chunk():
    x = _rand_inputs("linear", 1, 1, 10, 3, 0, seed=0)
    with pytest.raises(ValueError):
        _run(oracle.chunk_forward, "linear", "mse", x, 0, 0)


# --------------------------------------------------------------------------
# Ragged tail (T % C != 0): the last chunk holds the remaining tokens
# --------------------------------------------------------------------------
@pytest.mark.parametrize("kind,loss", CASES)
@pytest.mark.parametrize("C,r", [(4, 1), (4, 3), (16, 5), (7, 6)])
@pytest.mark.parametrize("momentum", [True, False])
def test_tail_closed_form_equals_brute_force(kind, loss, C, r, momentum):
    D, Hd = 5, 7
    x = _rand_inputs(kind, 1, 2, 2 * C + r, D, Hd, seed=C * 10 + r)
    ref = oracle.brute_force(kind, loss, x["q"], x["k"], x["v"], x["eta"], x["alpha"], x["beta"], x["W0"],
                             x["M0"], C, Hd, momentum=momentum)
    got = _run(oracle.chunk_forward, kind, loss, x, C, Hd, momentum=momentum)
    for a, b in zip(got, ref):
        if b is not None:
            assert oracle.rel_err(a, b) < 1e-12


@pytest.mark.parametrize("kind,loss", CASES)
@pytest.mark.parametrize("C,r", [(4, 3), (16, 9)])
def test_tail_equals_separate_call_on_the_remainder(kind, loss, C, r):
    """n whole chunks then a call with chunk = r on the remaining r tokens,
    state carried between the calls, is the ragged call."""
    D, Hd, n = 5, 6, 3
    x = _rand_inputs(kind, 1, 2, n * C + r, D, Hd, seed=C + r + 50)
    out, W, M = _run(oracle.chunk_forward, kind, loss, x, C, Hd)
    cut = lambda d, lo, hi: {k: (v[:, :, lo:hi] if v.ndim >= 3 and k not in ("W0", "M0") else v) for k, v in d.items()}
    a = cut(x, 0, n * C)
    o1, W1, M1 = _run(oracle.chunk_forward, kind, loss, a, C, Hd)
    b = cut(x, n * C, n * C + r)
    b["W0"], b["M0"] = W1, M1
    o2, W2, M2 = _run(oracle.chunk_forward, kind, loss, b, r, Hd)
    assert oracle.rel_err(out, np.concatenate([o1, o2], axis=2)) < 1e-13
    assert oracle.rel_err(W, W2) < 1e-13
    assert oracle.rel_err(M, M2) < 1e-13


def test_chunk_longer_than_sequence_is_one_chunk():
    x = _rand_inputs("swiglu", 1, 2, 13, 4, 5, seed=61)
    a = _run(oracle.chunk_forward, "swiglu", "negdot", x, 64, 5)
    b = _run(oracle.chunk_forward, "swiglu", "negdot", x, 13, 5)
    for u, v in zip(a, b):
        assert oracle.rel_err(u, v) == 0.0
