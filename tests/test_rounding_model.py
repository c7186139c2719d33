"""How the bf16 MFMA path's roundings drive its error over several chunks,
shown on the CPU with a model of its bf16 roundings (tests/rounding_model.py).

Inputs: a 64-unit SwiGLU head, T = 768 in three 256-token chunks, the stated
gates, momentum driven at half the W0 scale (M0 = 0.5 N(0, 1/D)), seed 15.
The model rounds where the kernels round and reproduces what the GPU gave:

- the kernels' form: the per-token factors scaled by the tokens'
  coefficients in fp32 and rounded to bf16 once.  GPU output errors 4.55e-3,
  3.83e-3, 6.34e-3 over the three chunks, state W 3.46e-3, M 7.15e-3;
- a form that rounded the factors to bf16 before the scaling as well: GPU
  output errors 4.6e-3, 1.1e-2, 2.75e-2, growing chunk after chunk past the
  2e-2 bound;
- hi/lo operands (the precise form): the state stays within ~1e-5 of the
  oracle and the output error is the bf16 output path's own (< 1e-2).
"""
import numpy as np
import pytest

import oracle
import synth
from tests import rounding_model as rm


def _case(Hd=64, T=768, seed=15):
    cfg = synth.CONFIGS["swiglu_1p3b"].with_(name="rounding", B=1, H=2, T=T, Hd=Hd, chunk=256)
    x = synth.make_inputs(cfg, seed=seed, m0_scale=0.5)
    f = lambda t: t.double().numpy()
    ref = oracle.chunk_forward(cfg.kind, cfg.loss, *(f(x[n]) for n in ("q", "k", "v", "eta", "alpha", "beta",
                                                                        "W0", "M0")), cfg.chunk, cfg.Hd)
    return cfg, x, ref


def _errs(cfg, got, ref):
    C = cfg.chunk
    out = [oracle.rel_err(got[0][:, :, c * C:(c + 1) * C], ref[0][:, :, c * C:(c + 1) * C])
           for c in range(cfg.T // C)]
    return out, oracle.rel_err(got[1], ref[1]), oracle.rel_err(got[2], ref[2])


def test_single_rounding_matches_the_gpu():
    cfg, x, ref = _case()
    out, eW, eM = _errs(cfg, rm.swiglu_bf16_path(cfg, x), ref)
    # the GPU gave 4.55e-3, 3.83e-3, 6.34e-3; W 3.46e-3, M 7.15e-3
    assert out == pytest.approx([4.55e-3, 3.83e-3, 6.34e-3], rel=0.05)
    assert eW == pytest.approx(3.46e-3, rel=0.05) and eM == pytest.approx(7.15e-3, rel=0.05)
    assert max(out) < 1e-2


def test_factors_rounded_twice_drift_over_chunks():
    cfg, x, ref = _case()
    out, eW, eM = _errs(cfg, rm.swiglu_bf16_path(cfg, x, factors_rounded=True), ref)
    # the GPU gave 4.6e-3, 1.1e-2, 2.75e-2 with this form
    assert out[0] == pytest.approx(4.6e-3, rel=0.1)
    assert out[1] == pytest.approx(1.1e-2, rel=0.1)
    assert out[2] == pytest.approx(2.75e-2, rel=0.1)
    assert out[0] < out[1] < out[2] and out[2] > 2e-2
    assert eW > 5e-3 and eM > 1e-2


def test_hilo_operands_follow_the_recurrence():
    """The precise form hands the factors over as hi/lo pairs and splits the
    scaled operands again."""
    cfg, x, ref = _case()
    out, eW, eM = _errs(cfg, rm.swiglu_bf16_path(cfg, x, precise=True, factors_rounded=True), ref)
    assert max(out) < 1e-2
    assert eW < 1e-4 and eM < 1e-4


def test_wider_head_same_picture():
    """A 128-unit head over four chunks (seed 14): rounding the factors twice
    drifts past 2e-2, once stays within the bound (the GPU gave 3.90e-3,
    3.55e-3, 1.10e-2, 3.93e-3), hi/lo operands follow the recurrence."""
    cfg, x, ref = _case(Hd=128, T=1024, seed=14)
    out_2, _, _ = _errs(cfg, rm.swiglu_bf16_path(cfg, x, factors_rounded=True), ref)
    out_1, _, _ = _errs(cfg, rm.swiglu_bf16_path(cfg, x), ref)
    out_p, eW, eM = _errs(cfg, rm.swiglu_bf16_path(cfg, x, precise=True, factors_rounded=True), ref)
    assert max(out_2) > 2e-2
    assert out_1 == pytest.approx([3.90e-3, 3.55e-3, 1.10e-2, 3.93e-3], rel=0.05)
    assert max(out_p) < 1e-2 and eW < 1e-4 and eM < 1e-4


def test_model_without_roundings_is_the_oracle():
    """Sanity of the model itself: the same code with every rounding removed
    (float64 throughout) reproduces the oracle's state to 1e-6 (the scalar
    kernels stay fp32)."""
    cfg, x, ref = _case()
    saved = rm._rb, rm._hilo_sum
    try:
        rm._rb = rm._hilo_sum = lambda t: t
        got = rm.swiglu_bf16_path(cfg, x, factors_rounded=True)
    finally:
        rm._rb, rm._hilo_sum = saved
    _, eW, eM = _errs(cfg, got, ref)
    assert eW < 1e-6 and eM < 1e-6
    assert np.all(np.isfinite(got[0]))
