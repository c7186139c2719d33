"""GPU parity of the portable fp32 backward (every fast-weight kind and loss)
against the fp64 backward oracle, through the C ABI.  Bounds: 1e-4 for fp32
I/O (the forward's), 2e-2 for bf16 I/O; error measure max|x - r| / max|r| per
tensor as in the other parity tests."""
import numpy as np
import pytest

import synth
from tests.gpu_util import persistent_gates
from tests.test_gpu_backward import _compare, _gpu, _oracle

pytestmark = pytest.mark.gpu


def _cfg(kind, loss, io, B, H, T, D, Hd, chunk, flags=0):
    return synth.Config(f"gbwd_{kind}_{loss}_{io}_T{T}_C{chunk}_f{flags}", kind, loss, B, H, T, D, Hd, chunk, io,
                        "portable backward", flags)


CASES = [
    ("linear", "mse", "f32", 1, 2, 48, 16, 0, 16, 0),
    ("linear", "negdot", "f32", 1, 2, 40, 16, 0, 16, 2),     # no momentum, ragged tail
    ("mlp", "mse", "f32", 1, 2, 64, 16, 24, 16, 0),
    ("mlp", "negdot", "f32", 1, 2, 50, 16, 24, 16, 4),       # chunk-averaged, ragged tail
    ("swiglu", "mse", "f32", 1, 2, 48, 16, 24, 16, 0),
    ("swiglu", "negdot", "f32", 1, 2, 40, 16, 24, 16, 2),
    ("swiglu", "negdot", "bf16", 1, 2, 96, 32, 40, 32, 0),   # a shape the MFMA path does not take
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}-{c[2]}-f{c[9]}")
def test_generic_backward_small(case):
    cfg = _cfg(*case)
    x = synth.make_inputs(cfg, seed=0, m0_scale=0.5 if cfg.momentum else 0.0)
    c = synth.make_cotangents(cfg, seed=1)
    tol = 1e-4 if cfg.io_dtype == "f32" else 2e-2
    _compare(cfg, _gpu(cfg, x, c), _oracle(cfg, x, c), tol=tol)


def test_generic_backward_tiny_linear_full():
    """The tiny linear workload (B=1, H=1, T=256, chunk 16, D=32) at full size."""
    cfg = synth.CONFIGS["tiny_linear"]
    x = synth.make_inputs(cfg, seed=0, m0_scale=0.5)
    c = synth.make_cotangents(cfg, seed=1)
    _compare(cfg, _gpu(cfg, x, c), _oracle(cfg, x, c), tol=1e-4)


def test_generic_backward_mlp_full_size():
    """The MLP workload (B=2, H=4, T=2048, chunk 64, 64 -> 128 -> 64) at full
    size, with the slower-decay gates that keep its state in fp32 range."""
    cfg = synth.CONFIGS["mlp_fp32"]
    x = persistent_gates(cfg, synth.make_inputs(cfg, seed=0))
    c = synth.make_cotangents(cfg, seed=1)
    _compare(cfg, _gpu(cfg, x, c), _oracle(cfg, x, c), tol=1e-4)


def test_forced_generic_matches_mfma_backward():
    """The same SwiGLU bf16 call through both backward paths."""
    cfg = synth.Config("gbwd_vs_mfma", "swiglu", "negdot", 1, 2, 192, 128, 128, 64, "bf16", "")
    x = synth.make_inputs(cfg, seed=3, m0_scale=0.5)
    c = synth.make_cotangents(cfg, seed=4)
    ref = _oracle(cfg, x, c)
    _compare(cfg, _gpu(cfg, x, c, force_generic=True), ref)
    _compare(cfg, _gpu(cfg, x, c), ref)
