"""GPU parity for a ragged tail (T % chunk != 0: a shorter last chunk) and for
streaming (the sequence fed in pieces with the state carried between calls),
against the fp64 oracle.  Tolerances as in test_gpu_parity.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _e2():
    import chunk_weight_rnn_amd as e2
    e2.library()
    return e2


@pytest.mark.parametrize("T,C", [(100, 64), (1, 64), (1000, 256), (1030, 1024), (2047, 1024), (29, 8), (5000, 2048),
                                 (700, 320), (900, 512)])
@pytest.mark.parametrize("momentum,chunk_avg", [(True, False), (False, True)])
def test_logscan_tail(T, C, momentum, chunk_avg):
    e2 = _e2()
    gu.note(f"logscan tail T={T} C={C} momentum={momentum} avg={chunk_avg}")
    B, H = 2, 2
    g = torch.Generator().manual_seed(T + 3 * C)
    eta = 0.1 * torch.nn.functional.softplus(torch.randn(B, H, T, generator=g))
    alpha = torch.sigmoid(4 + torch.randn(B, H, T, generator=g))
    beta = torch.sigmoid(2 + torch.randn(B, H, T, generator=g))
    cM, cW, scal = e2.logscan(eta.cuda(), alpha.cuda(), beta.cuda(), chunk=C, momentum=momentum,
                              chunk_avg=chunk_avg)
    torch.cuda.synchronize()
    nc = -(-T // C)
    assert tuple(scal.shape) == (B, H, nc, 4)
    got_cM, got_cW, s = (t.cpu().double().numpy() for t in (cM, cW, scal))
    a, b, e = (t.double().numpy() for t in (alpha, beta, eta))
    for c in range(nc):
        sl = slice(c * C, min((c + 1) * C, T))
        if momentum:
            m, w, A, Bb, gamma = oracle.chunk_coefficients(a[..., sl], b[..., sl])
        else:
            w, A = oracle.chunk_coefficients_nomomentum(a[..., sl])
            m = np.zeros_like(w)
            m[..., -1] = 1.0
            Bb = gamma = np.zeros_like(A)
        if chunk_avg:
            m, w = oracle.chunk_mean(m), oracle.chunk_mean(w)
        assert gu.err(got_cM[..., sl], m * e[..., sl]) < 1e-5, c
        assert gu.err(got_cW[..., sl], w * e[..., sl]) < 1e-5, c
        assert gu.err(s[..., c, 0], A) < 1e-5
        assert gu.err(s[..., c, 1], Bb) < 1e-5
        assert gu.err(s[..., c, 2], gamma) < 1e-5


# MFMA path: tails of 1 token, a partial half-block, exactly one half-block,
# a half-block plus one, a whole block, and several blocks
MFMA_TAILS = [
    dict(B=1, H=2, Hd=128, chunk=64, T=2 * 64 + 1),
    dict(B=1, H=2, Hd=192, chunk=128, T=2 * 128 + 31),
    dict(B=2, H=1, Hd=128, chunk=128, T=128 + 32),
    dict(B=1, H=2, Hd=64, chunk=256, T=256 + 33),
    dict(B=1, H=3, Hd=256, chunk=256, T=3 * 256 + 64),
    dict(B=2, H=2, Hd=128, chunk=256, T=256 + 200),
    dict(B=1, H=2, Hd=128, chunk=512, T=100),
    # the Hd = 256 output kernel with one partial item: a single token, and
    # one row short of a whole 256-token item
    dict(B=2, H=2, Hd=256, chunk=256, T=1),
    dict(B=1, H=3, Hd=256, chunk=512, T=255),
]


@pytest.mark.parametrize("i", range(len(MFMA_TAILS)))
@pytest.mark.parametrize("momentum", [True, False])
def test_swiglu_mfma_tail(i, momentum):
    e2 = _e2()
    c = MFMA_TAILS[i]
    cfg = synth.CONFIGS["swiglu_1p3b"].with_(name=f"tail{i}_m{int(momentum)}", **c)
    gu.note(f"mfma tail case {i} momentum={momentum}: {c}")
    assert e2.path("swiglu", "negdot", "bf16", cfg.B, cfg.H, cfg.T, cfg.D, cfg.Hd, cfg.chunk) == 1
    x = synth.make_inputs(cfg, seed=60 + i, m0_scale=0.5)
    got = gu.run_gpu(cfg, x, momentum=momentum)
    ref = gu.run_oracle(cfg, x, momentum=momentum)
    gu.assert_close(cfg, got, ref, x["W0"].numpy())


@pytest.mark.parametrize("kind,loss", [("linear", "mse"), ("mlp", "mse"), ("swiglu", "negdot")])
@pytest.mark.parametrize("chunk,T", [(16, 3 * 16 + 5), (7, 30), (64, 10)])
def test_generic_tail(kind, loss, chunk, T):
    _e2()
    base = synth.CONFIGS["mlp_fp32"] if kind == "mlp" else synth.CONFIGS["tiny_linear"]
    cfg = base.with_(name=f"gtail_{kind}", kind=kind, loss=loss, B=2, H=2, T=T, D=16,
                     Hd=24 if kind != "linear" else 0, chunk=chunk, io_dtype="f32")
    gu.note(f"generic tail {kind}/{loss} chunk={chunk} T={T}")
    x = synth.make_inputs(cfg, seed=T, m0_scale=0.5)
    if kind == "mlp":
        x["eta"] = x["eta"] / cfg.D
    got = gu.run_gpu(cfg, x, force_generic=True)
    ref = gu.run_oracle(cfg, x)
    gu.assert_close(cfg, got, ref, x["W0"].numpy())


def test_swiglu_1p3b_tail_full_size():
    """The 1.3B-shaped workload at full B, H, Hd, chunk with a ragged tail:
    two whole chunks and 100 tokens."""
    _e2()
    cfg = synth.CONFIGS["swiglu_1p3b"]
    cfg = cfg.with_(name="1p3b_tail", T=2 * cfg.chunk + 100)
    gu.note("1p3b tail")
    x = synth.make_inputs(cfg, seed=0)
    got = gu.run_gpu(cfg, x)
    ref = gu.run_oracle(cfg, x)
    gu.assert_close(cfg, got, ref, x["W0"].numpy())


@pytest.mark.parametrize("name,momentum", [("swiglu_1p3b", True), ("swiglu_1p3b", False), ("mlp_fp32", True)])
def test_streaming_chunk_by_chunk(name, momentum):
    """Streaming: the sequence arrives one chunk per call (the last call a
    ragged remainder) with the state carried between calls; outputs and the
    final state equal the single call bit for bit."""
    e2 = _e2()
    base = synth.CONFIGS[name]
    cfg = base.with_(B=1, H=2, T=4 * base.chunk + base.chunk // 2 + 3)
    gu.note(f"streaming {name} momentum={momentum} T={cfg.T}")
    x = gu.to_dev(synth.make_inputs(cfg, seed=9, m0_scale=0.5))
    kw = dict(chunk=cfg.chunk, kind=cfg.kind, loss=cfg.loss, Hd=cfg.Hd, momentum=momentum)
    full = e2.chunk_forward(x["q"], x["k"], x["v"], x["eta"], x["alpha"], x["beta"], x["W0"], x["M0"], **kw)
    sl = lambda t, a, b: t[:, :, a:b].contiguous()
    W, M, outs = x["W0"], x["M0"], []
    for t0 in range(0, cfg.T, cfg.chunk):
        t1 = min(t0 + cfg.chunk, cfg.T)
        o, W, M = e2.chunk_forward(*(sl(x[n], t0, t1) for n in ("q", "k", "v", "eta", "alpha", "beta")), W, M,
                                   **kw)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs, dim=2), full[0])
    assert torch.equal(W, full[1])
    if momentum:
        assert torch.equal(M, full[2])


@pytest.mark.parametrize("flags", [0, 2, 4])
def test_streaming_folded_scan(flags):
    """Streaming on a grid of 64-unit slices (B=8, H=16): a call of one
    256-token chunk takes the chunk loop that computes the scalar kernels in
    its own prologue, a call of five chunks takes the separate scan launch.
    One chunk per call (the last a ragged remainder), state carried, equals
    the single call bit for bit: with momentum, without (flags 2) and with
    chunk-averaged kernels (flags 4)."""
    e2 = _e2()
    cfg = synth.CONFIGS["swiglu_1p3b"].with_(T=4 * 256 + 128 + 5, flags=flags)
    momentum, avg = not (flags & 2), bool(flags & 4)
    gu.note(f"streaming, folded scan, B=8 H=16 T={cfg.T} flags={flags}")
    x = gu.to_dev(synth.make_inputs(cfg, seed=21, m0_scale=0.5 if momentum else 0.0))
    kw = dict(chunk=cfg.chunk, kind=cfg.kind, loss=cfg.loss, Hd=cfg.Hd, momentum=momentum, chunk_avg=avg)
    full = e2.chunk_forward(x["q"], x["k"], x["v"], x["eta"], x["alpha"], x["beta"], x["W0"], x["M0"], **kw)
    sl = lambda t, a, b: t[:, :, a:b].contiguous()
    W, M, outs = x["W0"], x["M0"], []
    for t0 in range(0, cfg.T, cfg.chunk):
        t1 = min(t0 + cfg.chunk, cfg.T)
        o, W, M = e2.chunk_forward(*(sl(x[n], t0, t1) for n in ("q", "k", "v", "eta", "alpha", "beta")), W, M,
                                   **kw)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs, dim=2), full[0])
    assert torch.equal(W, full[1])
    if momentum:
        assert torch.equal(M, full[2])


def test_folded_scan_single_chunk_oracle():
    """One 256-token chunk of the 1.3B-shaped layer (B=8, H=16, the streaming
    workload's call, scalar kernels computed inside the chunk loop) against
    the oracle on every head."""
    e2 = _e2()
    cfg = synth.CONFIGS["swiglu_1p3b"].with_(name="folded1", T=256)
    gu.note("folded scan, one chunk, B=8 H=16 T=256")
    x = synth.make_inputs(cfg, seed=22, m0_scale=0.5)
    assert e2.path(cfg.kind, cfg.loss, cfg.io_dtype, cfg.B, cfg.H, cfg.T, cfg.D, cfg.Hd, cfg.chunk) == 1
    got = gu.run_gpu(cfg, x)
    gu.assert_close(cfg, got, gu.run_oracle(cfg, x), x["W0"].numpy())


@pytest.mark.parametrize("name,momentum", [("swiglu_1p3b", True), ("swiglu_1p3b", False), ("mlp_fp32", True)])
def test_streaming_matches_oracle(name, momentum):
    """Streaming against the oracle directly: the sequence arrives one chunk
    per call (eight whole chunks and a ragged remainder) with the state
    carried between calls; every chunk's output and the final state are
    compared with one oracle pass over the whole sequence.  Slow-decay gates
    keep the carried state alive to the last chunk."""
    e2 = _e2()
    base = synth.CONFIGS[name]
    cfg = base.with_(name=f"stream_{name}", B=1, H=4, T=8 * base.chunk + 37, flags=0 if momentum else 2)
    gu.note(f"streaming vs oracle {name} momentum={momentum} T={cfg.T}")
    x = gu.persistent_gates(cfg, synth.make_inputs(cfg, seed=19, m0_scale=0.5 if momentum else 0.0))
    d = gu.to_dev(x)
    kw = dict(chunk=cfg.chunk, kind=cfg.kind, loss=cfg.loss, Hd=cfg.Hd, momentum=momentum)
    sl = lambda t, a, b: t[:, :, a:b].contiguous()
    W, M, outs = d["W0"], d["M0"], []
    for t0 in range(0, cfg.T, cfg.chunk):
        t1 = min(t0 + cfg.chunk, cfg.T)
        o, W, M = e2.chunk_forward(*(sl(d[n], t0, t1) for n in ("q", "k", "v", "eta", "alpha", "beta")), W, M,
                                   **kw)
        outs.append(o)
    torch.cuda.synchronize()
    got = (torch.cat(outs, dim=2).float().cpu(), W.cpu(), M.cpu() if momentum else None)
    gu.assert_close(cfg, got, gu.run_oracle(cfg, x), x["W0"].numpy())
