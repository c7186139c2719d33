"""Seeded synthetic inputs for the E2-TTT chunk update.

This module is shared by the oracle-based tests, the GPU parity tests, the
benchmark and the smoke check.  It only draws random numbers and shapes them
into the input distributions below; it contains none of the chunk update's
arithmetic (no gradients, no coefficients, no state transition), and it
imports neither the oracle nor the GPU package.

Input recipe (the pages train 340M/1.3B hybrid models at 2K context and test
16K extrapolation -- "Rethinking Expressivity and Efficiency in Test-Time
Training", atlas summary, Key results / Experimental setup; no dataset item is
used, these tensors stand in for the per-head inputs of the TTT branch):

* draw order from one ``torch.Generator`` seeded with ``seed``:
  q, k, v, z_eta, z_alpha, z_beta, then the initial fast weight, then M0;
* q, k ~ N(0, 1) per element, L2-normalised along the head dim in fp32
  (``x / max(||x||, 1e-12)``), then cast to the I/O dtype (bf16 rounds to
  nearest even);
* v ~ N(0, 1), cast to the I/O dtype;
* eta = 0.1 * softplus(z), alpha = sigmoid(4 + z), beta = sigmoid(2 + z),
  z ~ N(0, 1), all fp32, shape [B, H, T];
* initial fast weight: every entry ~ N(0, 1/D), drawn once per head (shape
  [H, P]) and shared by every batch row, fp32;
* M0 = m0_scale * N(0, 1/D) per entry (zero by default).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

KIND_IDS = {"linear": 0, "mlp": 1, "swiglu": 2}
LOSS_IDS = {"mse": 0, "negdot": 1}


def param_count(kind: str, D: int, Hd: int) -> int:
    """Floats per (batch, head) in the packed fast-weight vector."""
    if kind == "linear":
        return D * D
    if kind == "mlp":
        return 2 * D * Hd
    if kind == "swiglu":
        return 3 * D * Hd
    raise ValueError(kind)


@dataclass(frozen=True)
class Config:
    name: str
    kind: str
    loss: str
    B: int
    H: int
    T: int
    D: int
    Hd: int
    chunk: int
    io_dtype: str  # "f32" or "bf16"
    notes: str = ""
    flags: int = 0  # variant flags of the C ABI: 2 = no momentum, 4 = chunk-averaged kernels

    @property
    def momentum(self) -> bool:
        return not (self.flags & 2)

    @property
    def chunk_avg(self) -> bool:
        return bool(self.flags & 4)

    @property
    def P(self) -> int:
        return param_count(self.kind, self.D, self.Hd)

    @property
    def tokens(self) -> int:
        return self.B * self.T

    def with_(self, **kw) -> "Config":
        d = dict(self.__dict__)
        d.update(kw)
        return Config(**d)


# The five workloads.  Shapes follow the paper's 340M/1.3B hybrid layers
# (16 heads x 128 head dim at 1.3B) at 2K training context and the 8x (16K)
# length-extrapolation setting.
CONFIGS = {
    "tiny_linear": Config("tiny_linear", "linear", "mse", 1, 1, 256, 32, 0, 16, "f32",
                          "linear fast weight 32x32, loss 0.5||Wk-v||^2"),
    "mlp_fp32": Config("mlp_fp32", "mlp", "mse", 2, 4, 2048, 64, 128, 64, "f32",
                       "2-layer SiLU MLP 64->128->64, MSE loss"),
    "swiglu_340m": Config("swiglu_340m", "swiglu", "negdot", 4, 8, 2048, 128, 256, 256, "bf16",
                          "SwiGLU 128/256, negative-dot loss"),
    "swiglu_1p3b_c64": Config("swiglu_1p3b_c64", "swiglu", "negdot", 8, 16, 2048, 128, 256, 64, "bf16",
                              "1.3B-shaped TTT branch, chunk 64"),
    "swiglu_1p3b": Config("swiglu_1p3b", "swiglu", "negdot", 8, 16, 2048, 128, 256, 256, "bf16",
                          "1.3B-shaped TTT branch, chunk 256"),
    "swiglu_1p3b_c1024": Config("swiglu_1p3b_c1024", "swiglu", "negdot", 8, 16, 2048, 128, 256, 1024, "bf16",
                                "1.3B-shaped TTT branch, chunk 1024"),
    "swiglu_16k": Config("swiglu_16k", "swiglu", "negdot", 1, 16, 16384, 128, 256, 256, "bf16",
                         "16K length extrapolation, state carried over 64 chunks"),
    # the variants on the 1.3B-shaped workload
    "swiglu_1p3b_nomom": Config("swiglu_1p3b_nomom", "swiglu", "negdot", 8, 16, 2048, 128, 256, 256, "bf16",
                                "1.3B-shaped TTT branch, chunk 256, no momentum", flags=2),
    "swiglu_1p3b_avg": Config("swiglu_1p3b_avg", "swiglu", "negdot", 8, 16, 2048, 128, 256, 256, "bf16",
                              "1.3B-shaped TTT branch, chunk 256, chunk-averaged kernels", flags=4),
    # streaming: one 256-token chunk per call, state carried in from the previous call
    "swiglu_1p3b_stream": Config("swiglu_1p3b_stream", "swiglu", "negdot", 8, 16, 256, 128, 256, 256, "bf16",
                                 "1.3B-shaped TTT branch, streaming: one chunk per call"),
    # the 16K extrapolation sequence streamed one chunk per call (one row)
    "swiglu_16k_stream": Config("swiglu_16k_stream", "swiglu", "negdot", 1, 16, 256, 128, 256, 256, "bf16",
                                "1.3B-shaped TTT branch, 16K sequence streamed: one chunk of one row per call"),
    # a ragged sequence: 7 whole chunks and a 208-token tail
    "swiglu_1p3b_tail": Config("swiglu_1p3b_tail", "swiglu", "negdot", 8, 16, 2000, 128, 256, 256, "bf16",
                               "1.3B-shaped TTT branch, T = 7 x 256 + 208"),
}


def _normalise(x: torch.Tensor) -> torch.Tensor:
    n = x.norm(dim=-1, keepdim=True).clamp_min(1e-12)
    return x / n


def make_inputs(cfg: Config, seed: int = 0, m0_scale: float = 0.0) -> dict:
    """Draw one seeded input set for ``cfg`` as CPU tensors.

    Returns q, k, v ([B,H,T,D], I/O dtype), eta, alpha, beta ([B,H,T] fp32),
    W0, M0 ([B,H,P] fp32, contiguous).
    """
    g = torch.Generator().manual_seed(seed)
    B, H, T, D = cfg.B, cfg.H, cfg.T, cfg.D
    io = torch.bfloat16 if cfg.io_dtype == "bf16" else torch.float32
    q = _normalise(torch.randn(B, H, T, D, generator=g)).to(io).contiguous()
    k = _normalise(torch.randn(B, H, T, D, generator=g)).to(io).contiguous()
    v = torch.randn(B, H, T, D, generator=g).to(io).contiguous()
    z_eta = torch.randn(B, H, T, generator=g)
    z_alpha = torch.randn(B, H, T, generator=g)
    z_beta = torch.randn(B, H, T, generator=g)
    eta = (0.1 * torch.nn.functional.softplus(z_eta)).contiguous()
    alpha = torch.sigmoid(4.0 + z_alpha).contiguous()
    beta = torch.sigmoid(2.0 + z_beta).contiguous()
    P = cfg.P
    w_head = torch.randn(H, P, generator=g) / (D ** 0.5)
    W0 = w_head.unsqueeze(0).expand(B, H, P).contiguous()
    m_head = torch.randn(B, H, P, generator=g) / (D ** 0.5)
    M0 = (m0_scale * m_head).contiguous()
    return dict(q=q, k=k, v=v, eta=eta, alpha=alpha, beta=beta, W0=W0, M0=M0)


def make_cotangents(cfg: Config, seed: int = 1, state_scale: float = 1.0) -> dict:
    """Seeded cotangents for the backward pass, as CPU tensors: dout
    [B,H,T,D] ~ N(0, 1) in the I/O dtype (the gradient arriving at the chunk
    outputs), dW_end and dM_end [B,H,P] ~ state_scale * N(0, 1/D) fp32 (the
    gradient arriving at the final state; 0 when the final state is unused)."""
    g = torch.Generator().manual_seed(seed)
    io = torch.bfloat16 if cfg.io_dtype == "bf16" else torch.float32
    dout = torch.randn(cfg.B, cfg.H, cfg.T, cfg.D, generator=g).to(io).contiguous()
    dW = (state_scale * torch.randn(cfg.B, cfg.H, cfg.P, generator=g) / (cfg.D ** 0.5)).contiguous()
    dM = (state_scale * torch.randn(cfg.B, cfg.H, cfg.P, generator=g) / (cfg.D ** 0.5)).contiguous()
    return dict(dout=dout, dW_end=dW, dM_end=dM)


def head_slice(inputs: dict, heads: list[tuple[int, int]]) -> dict:
    """Select a list of (b, h) pairs as a new B=1, H=len(heads) input set."""
    out = {}
    for name, t in inputs.items():
        out[name] = torch.stack([t[b, h] for b, h in heads], dim=0).unsqueeze(0).contiguous()
    return out
