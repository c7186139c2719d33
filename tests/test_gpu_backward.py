"""GPU parity of the backward pass (e2ttt_chunk_backward through the C ABI)
against the fp64 backward oracle (autograd of the closed form), gradient by
gradient: dq, dk, dv, deta, dalpha, dbeta, dW0 (per matrix), dM0 (per matrix).

Error measure as in the forward tests: max|x - r| / max|r| per tensor,
bound 2e-2 for bf16 I/O (the forward's bound; the backward's operands are the
same bf16-rounded chunk-start weights and per-token terms).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import err, note

pytestmark = pytest.mark.gpu
TOL = 2e-2

SMALL = synth.Config("bwd_small", "swiglu", "negdot", 1, 2, 320, 128, 128, 128, "bf16",
                     "2.5 chunks of 128 (ragged tail of 64)")


def _gpu(cfg, x, c, force_generic=False, precise=False):
    import chunk_weight_rnn_amd as e2
    d = {n: t.cuda() for n, t in x.items()}
    dc = {n: t.cuda() for n, t in c.items()}
    note(f"  gpu backward {cfg.name}: B={cfg.B} H={cfg.H} T={cfg.T} C={cfg.chunk} flags={cfg.flags}")
    g = e2.chunk_backward(d["q"], d["k"], d["v"], d["eta"], d["alpha"], d["beta"], d["W0"], d["M0"],
                          dc["dout"], dc["dW_end"], dc["dM_end"], chunk=cfg.chunk, Hd=cfg.Hd, kind=cfg.kind,
                          loss=cfg.loss, momentum=cfg.momentum, chunk_avg=cfg.chunk_avg,
                          force_generic=force_generic, precise=precise)
    torch.cuda.synchronize()
    return {n: (None if t is None else t.float().cpu().numpy()) for n, t in g.items()}


def _oracle(cfg, x, c):
    f = lambda t: t.double().numpy()
    return oracle.chunk_backward(cfg.kind, cfg.loss, f(x["q"]), f(x["k"]), f(x["v"]), f(x["eta"]), f(x["alpha"]),
                                 f(x["beta"]), f(x["W0"]), f(x["M0"]), f(c["dout"]), f(c["dW_end"]),
                                 f(c["dM_end"]), cfg.chunk, cfg.Hd, momentum=cfg.momentum,
                                 chunk_avg=cfg.chunk_avg)


def _compare(cfg, got, ref, tol=TOL):
    errs = {}
    for n in ("q", "k", "v", "eta", "alpha", "beta"):
        if ref[n] is None or not cfg.momentum and n == "beta":
            assert got[n] is None
            continue
        errs["d" + n] = err(got[n], ref[n])
    for n in ("W0", "M0"):
        if not cfg.momentum and n == "M0":
            continue
        mg = oracle.unpack(cfg.kind, got[n], cfg.D, cfg.Hd)
        mr = oracle.unpack(cfg.kind, ref[n], cfg.D, cfg.Hd)
        for m in mg:
            errs[f"d{n}.{m}"] = err(mg[m], mr[m])
    note(f"  {cfg.name}: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for n, t in got.items():
        if t is not None:
            assert np.all(np.isfinite(t)), n
    bad = {k: v for k, v in errs.items() if v > tol}
    assert not bad, f"{cfg.name}: tolerance exceeded: {bad}"


@pytest.mark.parametrize("flags,state_scale", [(0, 1.0), (0, 0.0), (2, 1.0), (4, 1.0)],
                         ids=["momentum", "zero_state_cotangent", "no_momentum", "chunk_avg"])
def test_backward_small(flags, state_scale):
    cfg = SMALL.with_(flags=flags, name=f"bwd_small_f{flags}_s{state_scale:g}")
    note(f"case {cfg.name}")
    x = synth.make_inputs(cfg, seed=0, m0_scale=0.5 if cfg.momentum else 0.0)
    c = synth.make_cotangents(cfg, seed=1, state_scale=state_scale)
    _compare(cfg, _gpu(cfg, x, c), _oracle(cfg, x, c))


@pytest.mark.parametrize("T,chunk", [(64, 64), (256, 64), (200, 128), (512, 256)])
def test_backward_shapes(T, chunk):
    cfg = SMALL.with_(T=T, chunk=chunk, Hd=256, name=f"bwd_T{T}_C{chunk}")
    note(f"case {cfg.name}")
    x = synth.make_inputs(cfg, seed=2, m0_scale=0.5)
    c = synth.make_cotangents(cfg, seed=3)
    _compare(cfg, _gpu(cfg, x, c), _oracle(cfg, x, c))


@pytest.mark.parametrize("Hd,T,chunk", [(64, 128, 128), (64, 768, 64), (320, 256, 128)])
def test_backward_hidden_widths(Hd, T, chunk):
    """One 64-unit slice (one chunk; twelve 64-token chunks), and five slices
    (the weight kernel's slice grid and the token kernel's unit loop at other
    widths)."""
    cfg = SMALL.with_(T=T, chunk=chunk, Hd=Hd, name=f"bwd_Hd{Hd}_T{T}_C{chunk}")
    note(f"case {cfg.name}")
    x = synth.make_inputs(cfg, seed=7, m0_scale=0.5)
    c = synth.make_cotangents(cfg, seed=8)
    _compare(cfg, _gpu(cfg, x, c), _oracle(cfg, x, c))


def test_backward_two_group_grid():
    """A grid of 32-unit slices (24 heads of 256 units on 256 compute units):
    the forward recompute runs the block-slot loop with two unit groups per
    workgroup and writes the momentum snapshots from it."""
    cfg = SMALL.with_(H=24, T=512, chunk=256, Hd=256, name="bwd_two_group")
    note(f"case {cfg.name}")
    x = synth.make_inputs(cfg, seed=11, m0_scale=0.5)
    c = synth.make_cotangents(cfg, seed=12)
    _compare(cfg, _gpu(cfg, x, c), _oracle(cfg, x, c))


@pytest.mark.parametrize("Hd", [64, 128])
def test_backward_precise_multichunk(Hd):
    """The backward of a precise forward (E2TTT_FLAG_PRECISE) runs the portable
    fp32 backward: three 256-token chunks with a strongly driven momentum, the
    case where the bf16 operands drift (64- and 128-unit heads)."""
    cfg = SMALL.with_(T=768, chunk=256, Hd=Hd, name=f"bwd_precise_Hd{Hd}")
    note(f"case {cfg.name}")
    x = synth.make_inputs(cfg, seed=15, m0_scale=0.5)
    c = synth.make_cotangents(cfg, seed=16)
    _compare(cfg, _gpu(cfg, x, c, precise=True), _oracle(cfg, x, c))


def test_backward_full_size_every_head():
    """The 1.3B-shaped workload (B=8, H=16, T=2048, chunk 256) in one call,
    every (b, h) pair checked against the oracle, 16 heads at a time."""
    cfg = synth.CONFIGS["swiglu_1p3b"]
    note(f"case {cfg.name} backward")
    x = synth.make_inputs(cfg, seed=0, m0_scale=0.5)
    c = synth.make_cotangents(cfg, seed=1)
    got = _gpu(cfg, x, c)
    pairs = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    for i in range(0, len(pairs), 16):
        heads = pairs[i:i + 16]
        sub_cfg = cfg.with_(B=1, H=len(heads))
        ref = _oracle(sub_cfg, synth.head_slice(x, heads), synth.head_slice(c, heads))
        sub = {n: (None if t is None else np.stack([t[b, h] for b, h in heads])[None]) for n, t in got.items()}
        _compare(sub_cfg, sub, ref)


def test_backward_deterministic():
    cfg = SMALL
    x = synth.make_inputs(cfg, seed=4, m0_scale=0.5)
    c = synth.make_cotangents(cfg, seed=5)
    a = _gpu(cfg, x, c)
    b = _gpu(cfg, x, c)
    for n in a:
        if a[n] is not None:
            assert np.array_equal(a[n], b[n]), n


@pytest.mark.parametrize("T,chunk", [(1, 64), (63, 64), (64, 128), (130, 2048)], ids=lambda v: str(v))
def test_backward_short_sequences(T, chunk):
    """Sequences shorter than a block or than the chunk (one ragged chunk)."""
    cfg = SMALL.with_(T=T, chunk=chunk, name=f"bwd_short_T{T}_C{chunk}")
    note(f"case {cfg.name}")
    x = synth.make_inputs(cfg, seed=6, m0_scale=0.5)
    c = synth.make_cotangents(cfg, seed=7)
    _compare(cfg, _gpu(cfg, x, c), _oracle(cfg, x, c))


def test_backward_empty_sequence_passes_state_through():
    """T == 0: the state cotangents pass through unchanged; the others are empty."""
    import chunk_weight_rnn_amd as e2
    cfg = SMALL.with_(T=0, name="bwd_T0")
    x = {n: t.cuda() for n, t in synth.make_inputs(cfg, seed=8, m0_scale=0.5).items()}
    c = {n: t.cuda() for n, t in synth.make_cotangents(cfg, seed=9).items()}
    g = e2.chunk_backward(x["q"], x["k"], x["v"], x["eta"], x["alpha"], x["beta"], x["W0"], x["M0"], c["dout"],
                          c["dW_end"], c["dM_end"], chunk=cfg.chunk, Hd=cfg.Hd)
    torch.cuda.synchronize()
    assert torch.equal(g["W0"], c["dW_end"]) and torch.equal(g["M0"], c["dM_end"])
    assert g["q"].numel() == 0 and g["eta"].numel() == 0


def test_backward_empty_batch():
    import chunk_weight_rnn_amd as e2
    cfg = SMALL.with_(B=0, name="bwd_B0")
    x = {n: t.cuda() for n, t in synth.make_inputs(cfg, seed=8).items()}
    c = {n: t.cuda() for n, t in synth.make_cotangents(cfg, seed=9).items()}
    g = e2.chunk_backward(x["q"], x["k"], x["v"], x["eta"], x["alpha"], x["beta"], x["W0"], x["M0"], c["dout"],
                          c["dW_end"], c["dM_end"], chunk=cfg.chunk, Hd=cfg.Hd)
    torch.cuda.synchronize()
    assert all(t is None or t.numel() == 0 for t in g.values())


def test_backward_rejects_aliased_output():
    """An output that overlaps an input is refused before any launch."""
    import chunk_weight_rnn_amd as e2
    from chunk_weight_rnn_amd._lib import make_desc
    import ctypes
    cfg = SMALL
    x = {n: t.cuda() for n, t in synth.make_inputs(cfg, seed=8).items()}
    c = {n: t.cuda() for n, t in synth.make_cotangents(cfg, seed=9).items()}
    lib = e2.library()
    d = make_desc(cfg.kind, cfg.loss, cfg.io_dtype, cfg.B, cfg.H, cfg.T, cfg.D, cfg.Hd, cfg.chunk)
    ws = torch.empty(int(lib.e2ttt_backward_workspace_size(ctypes.byref(d))), dtype=torch.uint8, device="cuda")
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    out = {n: torch.empty_like(x[n]) for n in ("q", "k", "v", "eta", "alpha", "beta", "W0", "M0")}
    args = [p(x[n]) for n in ("q", "k", "v", "eta", "alpha", "beta", "W0", "M0")] + \
           [p(c["dout"]), p(c["dW_end"]), p(c["dM_end"])]
    outs = [p(out[n]) for n in ("q", "k", "v", "eta", "alpha", "beta", "W0", "M0")]
    outs[6] = p(x["W0"])  # dW0 written over W0
    st = lib.e2ttt_chunk_backward(ctypes.byref(d), *args, *outs, p(ws), ctypes.c_size_t(ws.numel()),
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 3


@pytest.mark.parametrize("case", ["swiglu_mfma", "swiglu_mfma_c64", "swiglu_nomom", "swiglu_folded", "mlp_portable",
                                  "linear_portable"])
def test_backward_from_saved_forward_states(case):
    """chunk_forward(save_states=True) then chunk_backward(saved=True) on one
    shared workspace gives the recomputing backward's result bit for bit."""
    import chunk_weight_rnn_amd as e2
    cfg = {"swiglu_mfma": SMALL, "swiglu_nomom": SMALL.with_(flags=2),
           "swiglu_mfma_c64": SMALL.with_(chunk=64),  # short chunks: the gradient waves store the snapshots
           # 64-unit slices, one chunk per gradient wave: the saving forward's chunk
           # loop computes the scalar kernels itself, the recompute launches the scan
           "swiglu_folded": SMALL.with_(B=8, H=16, T=448, Hd=256, chunk=256),
           "mlp_portable": synth.Config("saved_mlp", "mlp", "mse", 1, 2, 80, 16, 24, 32, "f32", ""),
           "linear_portable": synth.Config("saved_lin", "linear", "negdot", 1, 2, 80, 16, 0, 32, "f32", "")}[case]
    note(f"case saved {case}")
    x = {n: t.cuda() for n, t in synth.make_inputs(cfg, seed=14, m0_scale=0.5 if cfg.momentum else 0.0).items()}
    c = {n: t.cuda() for n, t in synth.make_cotangents(cfg, seed=15).items()}
    kw = dict(chunk=cfg.chunk, kind=cfg.kind, loss=cfg.loss, Hd=cfg.Hd, momentum=cfg.momentum)
    ws = e2.training_workspace(x["q"], **kw)
    fo = e2.chunk_forward(x["q"], x["k"], x["v"], x["eta"], x["alpha"], x["beta"], x["W0"], x["M0"], workspace=ws,
                          save_states=True, **kw)
    plain = e2.chunk_forward(x["q"], x["k"], x["v"], x["eta"], x["alpha"], x["beta"], x["W0"], x["M0"], **kw)
    gs = e2.chunk_backward(x["q"], x["k"], x["v"], x["eta"], x["alpha"], x["beta"], x["W0"], x["M0"], c["dout"],
                           c["dW_end"], c["dM_end"], workspace=ws, saved=True, **kw)
    gr = e2.chunk_backward(x["q"], x["k"], x["v"], x["eta"], x["alpha"], x["beta"], x["W0"], x["M0"], c["dout"],
                           c["dW_end"], c["dM_end"], **kw)
    torch.cuda.synchronize()
    for a, b in zip(fo, plain):
        assert (a is None and b is None) or torch.equal(a, b)
    for n in gs:
        assert (gs[n] is None and gr[n] is None) or torch.equal(gs[n], gr[n]), n
