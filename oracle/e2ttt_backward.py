"""fp64 CPU oracle for the backward pass of the E2-TTT chunk update.

TEST INFRASTRUCTURE, under the same rules as ``e2ttt_oracle``: only the test
suite, the smoke check and the benchmark's CPU-baseline leg may import or call
it; it shares no code with the GPU library and never imports it.

Definition.  The pages ("Rethinking Expressivity and Efficiency in Test-Time
Training": abstract and atlas summary "Approach") describe the forward chunk
update and claim training throughput for it; the backward pass is the plain
derivative of that update.  Given cotangents (dout, dW_end, dM_end) of the
forward outputs (out, W_end, M_end), it returns the vector-Jacobian product

    dX = d/dX [ <dout, out> + <dW_end, W_end> + <dM_end, M_end> ]

for X in q, k, v, eta, alpha, beta, W0, M0 (the gradients a training step
needs).  The forward is written here in torch, fp64, with the same steps, in
the same order, as ``e2ttt_oracle.chunk_forward`` (chunk output at the
chunk-start weights, per-token backward factors, scalar kernels as plain
products, the two weighted aggregations, the transition with the chunk-start
momentum), and torch.autograd evaluates the derivative.  Nothing is fused or
reordered beyond those steps.

Pins (tests/test_oracle_backward.py): the torch forward equals
``e2ttt_oracle.chunk_forward``; the gradients equal central finite
differences of ``e2ttt_oracle.chunk_forward`` along random directions, and
equal autograd through an independent per-token recurrence whose per-token
gradients come from autograd itself rather than from written-out formulas;
the cotangent map is linear.  No function here is "parity unpinned".
"""
from __future__ import annotations

import numpy as np
import torch

INPUTS = ("q", "k", "v", "eta", "alpha", "beta", "W0", "M0")


def _unpack(kind, p, D, Hd):
    lead = p.shape[:-1]
    if kind == "linear":
        return {"W": p.reshape(*lead, D, D)}
    n = D * Hd
    if kind == "mlp":
        return {"W1": p[..., :n].reshape(*lead, Hd, D), "W2": p[..., n:2 * n].reshape(*lead, D, Hd)}
    if kind == "swiglu":
        return {"W1": p[..., :n].reshape(*lead, D, Hd), "W3": p[..., n:2 * n].reshape(*lead, D, Hd),
                "W2": p[..., 2 * n:3 * n].reshape(*lead, Hd, D)}
    raise ValueError(f"unknown kind {kind!r}")


def _pack(kind, mats):
    names = {"linear": ("W",), "mlp": ("W1", "W2"), "swiglu": ("W1", "W3", "W2")}[kind]
    return torch.cat([mats[n].reshape(*mats[n].shape[:-2], -1) for n in names], dim=-1)


def _silu(x):
    return x * torch.sigmoid(x)


def _dsilu(x):
    s = torch.sigmoid(x)
    return s * (1.0 + x * (1.0 - s))


def _T(x):
    return x.transpose(-1, -2)


def _forward_rows(kind, mats, X):
    """y = f_W(x) for every row of X (fast weights of the atlas summary's "Key results")."""
    if kind == "linear":
        return X @ _T(mats["W"])
    if kind == "mlp":
        return _silu(X @ _T(mats["W1"])) @ _T(mats["W2"])
    return (_silu(X @ mats["W1"]) * (X @ mats["W3"])) @ mats["W2"]


def _factors(kind, loss, mats, K, V):
    """Per-token backward factors of the fast-weight loss at ``mats``."""
    def dy_of(Y):
        return Y - V if loss == "mse" else -V
    if kind == "linear":
        return {"dy": dy_of(K @ _T(mats["W"]))}
    if kind == "mlp":
        z = K @ _T(mats["W1"])
        a = _silu(z)
        dy = dy_of(a @ _T(mats["W2"]))
        return {"dy": dy, "a": a, "dz": (dy @ mats["W2"]) * _dsilu(z)}
    h1, h3 = K @ mats["W1"], K @ mats["W3"]
    u = _silu(h1) * h3
    dy = dy_of(u @ mats["W2"])
    du = dy @ _T(mats["W2"])
    return {"dy": dy, "u": u, "dh1": du * h3 * _dsilu(h1), "dh3": du * _silu(h1)}


def _weighted_sum(kind, fac, K, c):
    """sum_i c_i g_i (one weighted gradient aggregation of the atlas summary's "Approach")."""
    cc = c[..., :, None]
    if kind == "linear":
        return {"W": _T(cc * fac["dy"]) @ K}
    if kind == "mlp":
        return {"W1": _T(cc * fac["dz"]) @ K, "W2": _T(cc * fac["dy"]) @ fac["a"]}
    return {"W1": _T(K) @ (cc * fac["dh1"]), "W3": _T(K) @ (cc * fac["dh3"]), "W2": _T(cc * fac["u"]) @ fac["dy"]}


def _excl_mask(C, dtype):
    """mask[i, s] = 1 where s > i (the tokens after token i)."""
    idx = torch.arange(C)
    return (idx[None, :] > idx[:, None]).to(dtype)


def _suffix_prod(x):
    """prod_{s>i} x_s for every i (last axis), as plain products."""
    C = x.shape[-1]
    mk = _excl_mask(C, x.dtype)
    return torch.prod(mk * x[..., None, :] + (1.0 - mk), dim=-1)


def _coefficients(alpha, beta):
    """Momentum kernel m, weight kernel w and A, Bb, gamma of one chunk, each a
    plain product or sum of products of the gates (atlas summary, "Approach"):
    m_i = prod_{s>i} beta_s, w_i = sum_{tau>=i} prod_{s>tau} alpha_s prod_{i<s<=tau} beta_s,
    A = prod alpha, Bb = prod beta, gamma = sum_tau prod_{s>tau} alpha_s prod_{s<=tau} beta_s."""
    C = alpha.shape[-1]
    a = _suffix_prod(alpha)
    m = _suffix_prod(beta)
    mk = _excl_mask(C, beta.dtype)
    # bprod[i, tau] = prod_{i<s<=tau} beta_s (1 for tau <= i)
    bprod = torch.cumprod(mk * beta[..., None, :] + (1.0 - mk), dim=-1)
    upper = 1.0 - _excl_mask(C, beta.dtype).transpose(0, 1)  # [i, tau] = 1 where tau >= i
    w = torch.sum(upper * bprod * a[..., None, :], dim=-1)
    A = torch.prod(alpha, dim=-1)
    Bb = torch.prod(beta, dim=-1)
    gamma = torch.sum(a * torch.cumprod(beta, dim=-1), dim=-1)
    return m, w, A, Bb, gamma


def chunk_forward_torch(kind, loss, q, k, v, eta, alpha, beta, W0, M0, chunk, Hd=0, momentum=True,
                        chunk_avg=False):
    """The forward closed form on torch fp64 tensors [BH, ...]: (out, W_end, M_end)."""
    BH, T, D = q.shape
    W, M = W0, M0
    outs = []
    for c0 in range(0, T, chunk):
        sl = slice(c0, min(c0 + chunk, T))  # the last chunk may be shorter
        mats = _unpack(kind, W, D, Hd)
        outs.append(_forward_rows(kind, mats, q[:, sl]))
        fac = _factors(kind, loss, mats, k[:, sl], v[:, sl])
        if momentum:
            m, w, A, Bb, gamma = _coefficients(alpha[:, sl], beta[:, sl])
        else:
            w, A = _suffix_prod(alpha[:, sl]), torch.prod(alpha[:, sl], dim=-1)
            m, Bb, gamma = torch.zeros_like(w), torch.zeros_like(A), torch.zeros_like(A)
        if chunk_avg:
            m = m.mean(dim=-1, keepdim=True).expand_as(m)
            w = w.mean(dim=-1, keepdim=True).expand_as(w)
        cM, cW = m * eta[:, sl], w * eta[:, sl]
        GM = _pack(kind, _weighted_sum(kind, fac, k[:, sl], cM))
        GW = _pack(kind, _weighted_sum(kind, fac, k[:, sl], cW))
        W, M = A[:, None] * W - gamma[:, None] * M - GW, Bb[:, None] * M + GM
    out = torch.cat(outs, dim=1) if outs else torch.zeros_like(q)
    return out, W, M


def chunk_backward(kind, loss, q, k, v, eta, alpha, beta, W0, M0, dout, dW_end, dM_end, chunk, Hd=0,
                   momentum=True, chunk_avg=False):
    """Gradients of <dout, out> + <dW_end, W_end> + <dM_end, M_end> (numpy in,
    numpy out, fp64).

    Shapes as ``e2ttt_oracle.chunk_forward``: q, k, v, dout [B, H, T, D];
    eta, alpha, beta [B, H, T]; W0, M0, dW_end, dM_end [B, H, P].  Returns a
    dict with keys q, k, v, eta, alpha, beta, W0, M0 (gradients of the same
    shapes).  Without momentum beta, M0 and dM_end may be None and the
    gradients of beta and M0 are None.
    """
    if chunk <= 0:
        raise ValueError("the chunk size must be positive")
    B, H, T, D = np.shape(q)
    BH = B * H
    P = np.shape(W0)[-1]

    def leaf(x, tail):
        return torch.tensor(np.asarray(x, dtype=np.float64).reshape(BH, *tail), requires_grad=True)

    xs = {"q": leaf(q, (T, D)), "k": leaf(k, (T, D)), "v": leaf(v, (T, D)), "eta": leaf(eta, (T,)),
          "alpha": leaf(alpha, (T,)), "W0": leaf(W0, (P,))}
    if momentum:
        xs["beta"] = leaf(beta, (T,))
        xs["M0"] = leaf(M0, (P,))
        b_, m_ = xs["beta"], xs["M0"]
    else:
        b_, m_ = torch.zeros(BH, T, dtype=torch.float64), torch.zeros(BH, P, dtype=torch.float64)
    out, W, M = chunk_forward_torch(kind, loss, xs["q"], xs["k"], xs["v"], xs["eta"], xs["alpha"], b_,
                                    xs["W0"], m_, chunk, Hd, momentum, chunk_avg)
    f = lambda x, tail: torch.tensor(np.asarray(x, dtype=np.float64).reshape(BH, *tail))
    obj = (out * f(dout, (T, D))).sum() + (W * f(dW_end, (P,))).sum()
    if momentum:
        obj = obj + (M * f(dM_end, (P,))).sum()
    leaves = [xs[n] for n in INPUTS if n in xs]
    grads = torch.autograd.grad(obj, leaves, allow_unused=True)
    res = {n: None for n in INPUTS}
    shapes = {"q": (B, H, T, D), "k": (B, H, T, D), "v": (B, H, T, D), "eta": (B, H, T), "alpha": (B, H, T),
              "beta": (B, H, T), "W0": (B, H, P), "M0": (B, H, P)}
    for n, g in zip([n for n in INPUTS if n in xs], grads):
        res[n] = (np.zeros(shapes[n]) if g is None else g.detach().numpy().reshape(shapes[n]))
    return res
