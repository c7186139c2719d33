"""The seeded input generator: determinism, shapes, dtypes and distributions."""
import torch

import synth


def test_deterministic_and_shapes():
    cfg = synth.CONFIGS["tiny_linear"]
    a = synth.make_inputs(cfg, seed=0)
    b = synth.make_inputs(cfg, seed=0)
    for n in a:
        assert torch.equal(a[n], b[n])
    assert a["q"].shape == (1, 1, 256, 32) and a["q"].dtype == torch.float32
    assert a["W0"].shape == (1, 1, 32 * 32)
    c = synth.make_inputs(cfg, seed=1)
    assert not torch.equal(a["q"], c["q"])


def test_bf16_and_distributions():
    cfg = synth.CONFIGS["swiglu_340m"].with_(B=2, H=2, T=512)
    x = synth.make_inputs(cfg)
    assert x["q"].dtype == torch.bfloat16 and x["k"].dtype == torch.bfloat16
    n = x["k"].float().norm(dim=-1)
    assert torch.allclose(n, torch.ones_like(n), atol=1e-2)
    assert x["W0"].shape == (2, 2, 3 * 128 * 256)
    assert torch.equal(x["W0"][0], x["W0"][1])  # shared over the batch
    assert float(x["alpha"].min()) > 0 and float(x["alpha"].max()) < 1
    assert 0.02 < float(x["eta"].mean()) < 0.2
    assert float(x["M0"].abs().max()) == 0.0
    assert float(synth.make_inputs(cfg, m0_scale=0.5)["M0"].abs().max()) > 0


def test_config_table():
    for cfg in synth.CONFIGS.values():
        assert cfg.T >= 1 and cfg.chunk >= 1
        assert cfg.P == synth.param_count(cfg.kind, cfg.D, cfg.Hd)
