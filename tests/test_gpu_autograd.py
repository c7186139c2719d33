"""chunk_update (the differentiable op) on the GPU: torch.autograd through it
gives exactly what chunk_backward returns for the same cotangents, and its
gradients match the fp64 oracle."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import note
from tests.test_gpu_backward import SMALL, _compare, _oracle

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("momentum", [True, False])
def test_autograd_matches_chunk_backward(momentum):
    import chunk_weight_rnn_amd as e2
    cfg = SMALL.with_(flags=0 if momentum else 2, name=f"autograd_mom{int(momentum)}")
    note(f"case {cfg.name}")
    x = {n: t.cuda() for n, t in synth.make_inputs(cfg, seed=10, m0_scale=0.5 if momentum else 0.0).items()}
    c = {n: t.cuda() for n, t in synth.make_cotangents(cfg, seed=11).items()}
    leaves = {n: t.clone().requires_grad_(True) for n, t in x.items()}
    out, W, M = e2.chunk_update(leaves["q"], leaves["k"], leaves["v"], leaves["eta"], leaves["alpha"],
                                leaves["beta"], leaves["W0"], leaves["M0"], chunk=cfg.chunk, kind=cfg.kind,
                                loss=cfg.loss, Hd=cfg.Hd, momentum=momentum)
    obj = (out.float() * c["dout"].float()).sum() + (W * c["dW_end"]).sum()
    if momentum:
        assert M is not None
        obj = obj + (M * c["dM_end"]).sum()
    else:
        assert M is None
    obj.backward()
    torch.cuda.synchronize()
    g = e2.chunk_backward(x["q"], x["k"], x["v"], x["eta"], x["alpha"], x["beta"], x["W0"], x["M0"], c["dout"],
                          c["dW_end"], c["dM_end"], chunk=cfg.chunk, Hd=cfg.Hd, momentum=momentum)
    torch.cuda.synchronize()
    for n in ("q", "k", "v", "eta", "alpha", "W0") + (("beta", "M0") if momentum else ()):
        assert torch.equal(leaves[n].grad, g[n]), n
    got = {n: (None if g[n] is None else g[n].float().cpu().numpy()) for n in g}
    _compare(cfg, got, _oracle(cfg, {n: t.cpu() for n, t in x.items()}, {n: t.cpu() for n, t in c.items()}))


def test_autograd_unused_outputs():
    """Only out feeds the loss (the usual training case): the state cotangents are zero."""
    import chunk_weight_rnn_amd as e2
    cfg = SMALL.with_(name="autograd_out_only")
    x = {n: t.cuda() for n, t in synth.make_inputs(cfg, seed=12, m0_scale=0.5).items()}
    c = {n: t.cuda() for n, t in synth.make_cotangents(cfg, seed=13, state_scale=0.0).items()}
    leaves = {n: t.clone().requires_grad_(True) for n, t in x.items()}
    out, _, _ = e2.chunk_update(*[leaves[n] for n in ("q", "k", "v", "eta", "alpha", "beta", "W0", "M0")],
                                chunk=cfg.chunk, Hd=cfg.Hd)
    (out.float() * c["dout"].float()).sum().backward()
    g = e2.chunk_backward(x["q"], x["k"], x["v"], x["eta"], x["alpha"], x["beta"], x["W0"], x["M0"], c["dout"],
                          c["dW_end"], c["dM_end"], chunk=cfg.chunk, Hd=cfg.Hd)
    torch.cuda.synchronize()
    for n in ("q", "k", "v", "eta", "alpha", "beta", "W0", "M0"):
        assert torch.equal(leaves[n].grad, g[n]), n
    assert np.isfinite(leaves["alpha"].grad.cpu().numpy()).all()
