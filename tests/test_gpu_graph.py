"""The forward and backward entry points captured in a HIP graph (through
torch.cuda.CUDAGraph) and replayed: every replay, with eager calls between the
replays, must equal the eager result bit for bit.  The entry points record only
kernel launches on the caller's stream, so they can be captured."""
import pytest
import torch

import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _args(d):
    return (d["q"], d["k"], d["v"], d["eta"], d["alpha"], d["beta"], d["W0"], d["M0"])


@pytest.mark.parametrize("chunk", [256, 64])
def test_forward_graph_replay(chunk):
    import chunk_weight_rnn_amd as e2
    cfg = synth.CONFIGS["swiglu_1p3b"].with_(name="graph", B=2, H=4, T=512, chunk=chunk)
    gu.note(f"forward graph replay chunk={chunk}")
    d = gu.to_dev(synth.make_inputs(cfg, seed=3, m0_scale=0.5))
    kw = dict(chunk=cfg.chunk, kind=cfg.kind, loss=cfg.loss, Hd=cfg.Hd)
    ref = e2.chunk_forward(*_args(d), **kw)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        e2.chunk_forward(*_args(d), **kw)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        got = e2.chunk_forward(*_args(d), **kw)
    for rep in range(4):
        other = e2.chunk_forward(*_args(d), **kw)  # eager work between replays
        for t in got:
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b, c in zip(("out", "W_end", "M_end"), got, ref, other):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"
            assert torch.equal(c, b), f"eager call {rep}: {name} differs"


def test_forward_graph_replay_mlp_split():
    """The MLP split over hidden slices (one persistent launch whose slices meet
    through per-head counters in the workspace; a small kernel zeroes the
    counters first): replays and eager calls in between must agree."""
    import chunk_weight_rnn_amd as e2
    cfg = synth.CONFIGS["mlp_fp32"].with_(name="graph_mlp", T=512)
    assert e2.path(cfg.kind, cfg.loss, "f32", cfg.B, cfg.H, cfg.T, cfg.D, cfg.Hd, cfg.chunk) == 4
    gu.note("forward graph replay, MLP split")
    x = synth.make_inputs(cfg, seed=6, m0_scale=0.5)
    x["eta"] = x["eta"] / cfg.D
    d = gu.to_dev(x)
    kw = dict(chunk=cfg.chunk, kind=cfg.kind, loss=cfg.loss, Hd=cfg.Hd)
    ref = e2.chunk_forward(*_args(d), **kw)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        e2.chunk_forward(*_args(d), **kw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        got = e2.chunk_forward(*_args(d), **kw)
    for rep in range(4):
        other = e2.chunk_forward(*_args(d), **kw)
        for t in got:
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b, c in zip(("out", "W_end", "M_end"), got, ref, other):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"
            assert torch.equal(c, b), f"eager call {rep}: {name} differs"


def test_backward_graph_replay():
    import chunk_weight_rnn_amd as e2
    cfg = synth.CONFIGS["swiglu_1p3b"].with_(name="graph_bwd", B=1, H=4, T=512, chunk=256)
    gu.note("backward graph replay")
    d = gu.to_dev(synth.make_inputs(cfg, seed=4, m0_scale=0.5))
    c = gu.to_dev(synth.make_cotangents(cfg, seed=5))
    kw = dict(chunk=cfg.chunk, Hd=cfg.Hd)
    ref = e2.chunk_backward(*_args(d), c["dout"], c["dW_end"], c["dM_end"], **kw)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        e2.chunk_backward(*_args(d), c["dout"], c["dW_end"], c["dM_end"], **kw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        got = e2.chunk_backward(*_args(d), c["dout"], c["dW_end"], c["dM_end"], **kw)
    for rep in range(3):
        e2.chunk_backward(*_args(d), c["dout"], c["dW_end"], c["dM_end"], **kw)
        for t in got.values():
            if t is not None:
                t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for name in ref:
            if ref[name] is None:
                continue
            assert torch.equal(got[name], ref[name]), f"replay {rep}: d{name} differs from the eager call"
