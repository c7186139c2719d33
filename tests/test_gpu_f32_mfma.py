"""GPU parity of the fp32 MFMA path (e2ttt_path 3: linear and MLP fast weights
with fp32 I/O) through the C ABI, against the fp64 oracle (bar 1e-4, the fp32
I/O tolerance) and against the portable fp32 kernel on the same inputs.

Shapes span one and several 16x16 tiles per wavefront, chunks of one token,
chunks shorter than, equal to and longer than the 64-token block (several
blocks per chunk), and ragged last chunks."""
import pytest
import torch

import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CASES = [
    # kind, loss, B, H, T, D, Hd, chunk
    ("linear", "mse", 1, 2, 37, 16, 0, 1),       # one-token chunks
    ("linear", "mse", 1, 1, 256, 32, 0, 16),     # the tiny linear workload's shape
    ("linear", "negdot", 2, 2, 250, 64, 0, 100),  # two blocks per chunk, a 50-token last chunk
    ("linear", "mse", 1, 3, 96, 48, 0, 32),
    ("mlp", "mse", 1, 2, 512, 64, 128, 64),      # the MLP workload's head shape
    ("mlp", "mse", 2, 1, 200, 32, 64, 48),       # 48-token blocks, an 8-token last chunk
    ("mlp", "negdot", 1, 2, 400, 16, 48, 130),   # three blocks per chunk (64 + 64 + 2)
    ("mlp", "mse", 1, 2, 256, 48, 80, 64),       # 5 column tiles: every tile reads its own B operand
    ("mlp", "negdot", 1, 1, 64, 64, 128, 16),
    ("mlp", "mse", 1, 2, 192, 64, 48, 64),       # 3 hidden slices: each writes 22 of the 64 output rows
    ("mlp", "negdot", 2, 1, 130, 64, 32, 64),    # 2 hidden slices (32 output rows each), a 2-token last chunk
]


def _cfg(case, flags=0):
    kind, loss, B, H, T, D, Hd, C = case
    return synth.Config(f"f32mfma_{kind}_{loss}_D{D}_H{Hd}_C{C}_T{T}_f{flags}", kind, loss, B, H, T, D, Hd, C, "f32",
                        flags=flags)


def _inputs(cfg, seed):
    x = synth.make_inputs(cfg, seed=seed, m0_scale=0.5 if cfg.momentum else 0.0)
    if cfg.kind == "mlp" and cfg.loss == "mse":
        x["eta"] = x["eta"] / cfg.D  # the stated eta makes MLP/MSE diverge within a few chunks
    return x


@pytest.mark.parametrize("flags", [0, 2, 4], ids=["momentum", "no_momentum", "chunk_avg"])
@pytest.mark.parametrize("i", range(len(CASES)))
def test_f32_mfma_parity(i, flags):
    import chunk_weight_rnn_amd as e2
    e2.library()
    cfg = _cfg(CASES[i], flags)
    gu.note(f"fp32 MFMA case {cfg.name}")
    assert e2.path(cfg.kind, cfg.loss, "f32", cfg.B, cfg.H, cfg.T, cfg.D, cfg.Hd, cfg.chunk, flags=flags) in (3, 4)
    x = _inputs(cfg, seed=30 + i)
    got = gu.run_gpu(cfg, x)
    ref = gu.run_oracle(cfg, x)
    gu.assert_close(cfg, got, ref, x["W0"].numpy())
    # the portable fp32 kernel on the same inputs: same arithmetic up to the
    # order of the fp32 sums
    por = gu.run_gpu(cfg, x, force_generic=True)
    for name, a, b in zip(("out", "W_end", "M_end"), got, por):
        if a is not None:
            e = gu.err(a.numpy(), b.numpy())
            assert e < 2e-5, f"{cfg.name}: {name} differs from the portable kernel by {e:.2e}"


def test_f32_mfma_in_place_and_deterministic():
    import chunk_weight_rnn_amd as e2
    e2.library()
    cfg = _cfg(CASES[4])
    x = _inputs(cfg, seed=41)
    a = gu.run_gpu(cfg, x)
    b = gu.run_gpu(cfg, x)
    c = gu.run_gpu(cfg, x, in_place=True)
    for s, t, u in zip(a, b, c):
        assert torch.equal(s, t) and torch.equal(s, u)


def test_f32_mfma_full_mlp_workload_persistent():
    """The MLP workload (B=2, H=4, T=2048, chunk 64) at full size, slow-decay
    gates (alpha = sigmoid(8 + z), eta / D) so that all 32 chunks stay in
    fp32 range; compared with the oracle on every chunk."""
    import chunk_weight_rnn_amd as e2
    e2.library()
    cfg = synth.CONFIGS["mlp_fp32"]
    assert e2.path(cfg.kind, cfg.loss, "f32", cfg.B, cfg.H, cfg.T, cfg.D, cfg.Hd, cfg.chunk) == 4  # hidden slices
    x = gu.persistent_gates(cfg, synth.make_inputs(cfg, seed=0, m0_scale=0.5))
    got = gu.run_gpu(cfg, x)
    gu.assert_close(cfg, got, gu.run_oracle(cfg, x), x["W0"].numpy())
