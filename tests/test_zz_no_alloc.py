"""e2ttt_chunk_forward_noalloc: the forward without a workspace argument (its
scratch is the library's own per-GPU device array).  Through the C ABI it must
give e2ttt_chunk_forward's results bit for bit; two calls in a row, the second
on a smaller input, check that nothing the first call left in the scratch
leaks into the second.  Calls too large for the scratch are refused before
any device call."""
import ctypes

import pytest
import torch

import synth
from tests import gpu_util as gu


def _lib():
    import chunk_weight_rnn_amd as e2
    e2.library()
    return e2


def _call_both(e2, cfg, seed, m0_scale=0.5):
    x = gu.to_dev(synth.make_inputs(cfg, seed=seed, m0_scale=m0_scale))
    kw = dict(chunk=cfg.chunk, kind=cfg.kind, loss=cfg.loss, Hd=cfg.Hd, momentum=cfg.momentum,
              chunk_avg=cfg.chunk_avg)
    args = [x[n] for n in ("q", "k", "v", "eta", "alpha", "beta", "W0", "M0")]
    ref = e2.chunk_forward(*args, **kw)
    got = e2.chunk_forward_noalloc(*args, **kw)
    torch.cuda.synchronize()
    return x, ref, got


def _check(cfg, x, ref, got):
    for name, a, b in zip(("out", "W_end", "M_end"), got, ref):
        assert (a is None) == (b is None), name
        if a is not None:
            assert torch.equal(a, b), f"{cfg.name}: {name} differs from e2ttt_chunk_forward"
    # and the oracle's bar, as for the existing entry point
    gu.assert_close(cfg, tuple(None if t is None else t.float().cpu() for t in got),
                    gu.run_oracle(cfg, {n: t.cpu() for n, t in x.items()}), x["W0"].cpu().numpy())


@pytest.mark.gpu
def test_noalloc_matches_forward_twice_shrinking():
    """Two calls in a row: a 340M-shaped MFMA-path call (4 chunks), then a
    smaller one (fewer heads, shorter chunks, a ragged tail)."""
    e2 = _lib()
    big = synth.CONFIGS["swiglu_340m"].with_(name="noalloc_big", T=1024)
    small = synth.CONFIGS["swiglu_340m"].with_(name="noalloc_small", B=1, H=3, T=200, chunk=64)
    for cfg, seed in ((big, 21), (small, 22)):
        gu.note(f"noalloc {cfg.name}: B={cfg.B} H={cfg.H} T={cfg.T} C={cfg.chunk}")
        assert e2.workspace_size(cfg.kind, cfg.loss, cfg.io_dtype, cfg.B, cfg.H, cfg.T, cfg.D, cfg.Hd,
                                 cfg.chunk) <= e2._lib.NOALLOC_SCRATCH_BYTES
        x, ref, got = _call_both(e2, cfg, seed)
        _check(cfg, x, ref, got)


@pytest.mark.gpu
def test_noalloc_portable_path_and_variants():
    """The portable fp32 path (MLP / MSE) and the no-momentum variant, again a
    larger call followed by a smaller one."""
    e2 = _lib()
    mlp = synth.CONFIGS["mlp_fp32"].with_(name="noalloc_mlp", B=1, H=2, T=256)
    nomom = synth.CONFIGS["swiglu_340m"].with_(name="noalloc_nomom", B=1, H=2, T=128, chunk=64, flags=2)
    for cfg, seed, m0 in ((mlp, 23, 0.0), (nomom, 24, 0.0)):
        gu.note(f"noalloc {cfg.name}")
        x0 = synth.make_inputs(cfg, seed=seed, m0_scale=m0)
        if cfg.kind == "mlp":
            x0["eta"] = x0["eta"] / cfg.D  # keeps the MLP/MSE state in fp32 range
        x = gu.to_dev(x0)
        kw = dict(chunk=cfg.chunk, kind=cfg.kind, loss=cfg.loss, Hd=cfg.Hd, momentum=cfg.momentum)
        args = [x[n] for n in ("q", "k", "v", "eta", "alpha", "beta", "W0", "M0")]
        ref = e2.chunk_forward(*args, **kw)
        got = e2.chunk_forward_noalloc(*args, **kw)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert (a is None and b is None) or torch.equal(a, b)


@pytest.mark.gpu
def test_noalloc_serving_loop():
    """A serving loop: one 256-token chunk of a B = 2, H = 16 SwiGLU layer per
    call on a carried state, through the no-allocation entry point with
    preallocated outputs; every call's results equal e2ttt_chunk_forward's."""
    e2 = _lib()
    cfg = synth.CONFIGS["swiglu_1p3b"].with_(name="noalloc_serving", B=2, T=4 * 256)
    x = gu.to_dev(synth.make_inputs(cfg, seed=25, m0_scale=0.5))
    kw = dict(chunk=cfg.chunk, kind=cfg.kind, loss=cfg.loss, Hd=cfg.Hd)
    sl = lambda t, a, b: t[:, :, a:b].contiguous()
    W, M = x["W0"].clone(), x["M0"].clone()
    Wr, Mr = x["W0"].clone(), x["M0"].clone()
    out = torch.empty(cfg.B, cfg.H, cfg.chunk, cfg.D, dtype=torch.bfloat16, device="cuda")
    Wn, Mn = torch.empty_like(W), torch.empty_like(M)
    for t0 in range(0, cfg.T, cfg.chunk):
        args = [sl(x[n], t0, t0 + cfg.chunk) for n in ("q", "k", "v", "eta", "alpha", "beta")]
        e2.chunk_forward_noalloc(*args, W, M, out=out, W_end=Wn, M_end=Mn, **kw)
        ro, Wr, Mr = e2.chunk_forward(*args, Wr, Mr, **kw)
        torch.cuda.synchronize()
        assert torch.equal(out, ro) and torch.equal(Wn, Wr) and torch.equal(Mn, Mr)
        W, Wn = Wn, W
        M, Mn = Mn, M


def test_noalloc_refuses_oversized_call_before_device_work():
    """A call whose workspace exceeds the scratch returns
    E2TTT_ERR_SCRATCH_LIMIT (no device call happens first, so this runs
    without a GPU); E2TTT_FLAG_SAVE_STATES is refused."""
    from chunk_weight_rnn_amd import _lib as L
    lib = L.load()
    v = ctypes.c_void_p
    args = [v((1 << 40) + i * (1 << 33)) for i in range(11)]
    big = L.make_desc("swiglu", "negdot", "bf16", 8, 16, 2048, 128, 256, 256)
    assert lib.e2ttt_workspace_size(ctypes.byref(big)) > L.NOALLOC_SCRATCH_BYTES
    assert lib.e2ttt_chunk_forward_noalloc(ctypes.byref(big), *args, v(0)) == 6
    assert b"scratch" in lib.e2ttt_status_string(6)
    saving = L.make_desc("swiglu", "negdot", "bf16", 1, 1, 256, 128, 256, 256, L.FLAG_SAVE_STATES)
    assert lib.e2ttt_chunk_forward_noalloc(ctypes.byref(saving), *args, v(0)) == 1
    bad = L.make_desc("swiglu", "negdot", "bf16", 1, 1, 256, 128, 256, 0)  # chunk 0
    assert lib.e2ttt_chunk_forward_noalloc(ctypes.byref(bad), *args, v(0)) == 1
