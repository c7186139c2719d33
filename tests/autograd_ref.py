"""Independent torch (fp64, CPU) fast-weight models used to pin the oracle.

Written directly from the model definitions, without the oracle's
hand-derived backward formulas: gradients come from torch.autograd.
"""
from __future__ import annotations

import torch


def shapes(kind: str, D: int, Hd: int):
    if kind == "linear":
        return [("W", (D, D))]
    if kind == "mlp":
        return [("W1", (Hd, D)), ("W2", (D, Hd))]
    return [("W1", (D, Hd)), ("W3", (D, Hd)), ("W2", (Hd, D))]


def split(kind, p: torch.Tensor, D: int, Hd: int) -> dict:
    out, off = {}, 0
    for name, shp in shapes(kind, D, Hd):
        n = shp[0] * shp[1]
        out[name] = p[off:off + n].reshape(shp)
        off += n
    return out


def model(kind, mats: dict, x: torch.Tensor) -> torch.Tensor:
    """f_W(x) for a single token vector x [D]."""
    if kind == "linear":
        return mats["W"] @ x
    if kind == "mlp":
        return mats["W2"] @ torch.nn.functional.silu(mats["W1"] @ x)
    h1 = x @ mats["W1"]
    h3 = x @ mats["W3"]
    return (torch.nn.functional.silu(h1) * h3) @ mats["W2"]


def loss_fn(loss: str, y: torch.Tensor, v: torch.Tensor) -> torch.Tensor:
    if loss == "mse":
        return 0.5 * ((y - v) ** 2).sum()
    return -(y * v).sum()


def token_grad(kind, loss, p, k, v, D, Hd) -> torch.Tensor:
    """Gradient of token loss wrt the packed parameter vector p (fp64)."""
    p = p.detach().clone().requires_grad_(True)
    ell = loss_fn(loss, model(kind, split(kind, p, D, Hd), k), v)
    (g,) = torch.autograd.grad(ell, p)
    return g.detach()


def token_loss(kind, loss, p, k, v, D, Hd) -> float:
    with torch.no_grad():
        return float(loss_fn(loss, model(kind, split(kind, p, D, Hd), k), v))


def output(kind, p, x, D, Hd) -> torch.Tensor:
    with torch.no_grad():
        return model(kind, split(kind, p, D, Hd), x)
