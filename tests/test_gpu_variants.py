"""GPU parity of the variants against the fp64 oracle: the recurrence without
momentum (E2TTT_FLAG_NO_MOMENTUM) and the chunk-averaged kernels
(E2TTT_FLAG_CHUNK_AVG), on the scalar-kernel step alone, the SwiGLU MFMA path
(several tiles, slices and chunk sizes, and the 1.3B-shaped workload at full
size) and the portable fp32 path.  Tolerances as in test_gpu_parity.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

VARIANTS = [(False, False), (True, True), (False, True)]  # (momentum, chunk_avg)


def _e2():
    import chunk_weight_rnn_amd as e2
    e2.library()
    return e2


@pytest.mark.parametrize("momentum,chunk_avg", VARIANTS)
@pytest.mark.parametrize("T,C", [(2048, 256), (512, 64), (2048, 1024), (1200, 1200), (9, 3)])
def test_logscan_variants(momentum, chunk_avg, T, C):
    e2 = _e2()
    gu.note(f"logscan variant momentum={momentum} avg={chunk_avg} T={T} C={C}")
    B, H = 2, 3
    g = torch.Generator().manual_seed(T + C + 7)
    eta = 0.1 * torch.nn.functional.softplus(torch.randn(B, H, T, generator=g))
    alpha = torch.sigmoid(4 + torch.randn(B, H, T, generator=g))
    beta = torch.sigmoid(2 + torch.randn(B, H, T, generator=g))
    alpha[..., ::37] = 0.0
    cM, cW, scal = e2.logscan(eta.cuda(), alpha.cuda(), beta.cuda() if momentum else None, chunk=C,
                              momentum=momentum, chunk_avg=chunk_avg)
    torch.cuda.synchronize()
    nc = T // C
    a = alpha.double().numpy().reshape(B, H, nc, C)
    e = eta.double().numpy().reshape(B, H, nc, C)
    if momentum:
        m, w, A, Bb, gamma = oracle.chunk_coefficients(a, beta.double().numpy().reshape(B, H, nc, C))
    else:
        w, A = oracle.chunk_coefficients_nomomentum(a)
        m = np.zeros_like(w)
        m[..., -1] = 1.0
        Bb = gamma = np.zeros_like(A)
    if chunk_avg:
        m, w = oracle.chunk_mean(m), oracle.chunk_mean(w)
    s = scal.cpu().double().numpy()
    got_cM = cM.cpu().double().numpy().reshape(B, H, nc, C)
    got_cW = cW.cpu().double().numpy().reshape(B, H, nc, C)
    assert np.all(np.isfinite(got_cM)) and np.all(np.isfinite(got_cW)) and np.all(np.isfinite(s))
    assert gu.err(got_cM, m * e) < 1e-5
    assert gu.err(got_cW, w * e) < 1e-5
    assert gu.err(s[..., 0], A) < 1e-5
    assert gu.err(s[..., 1], Bb) < 1e-5
    assert gu.err(s[..., 2], gamma) < 1e-5


MFMA_CASES = [
    dict(B=1, H=1, T=64, Hd=64, chunk=64),
    dict(B=1, H=3, T=256, Hd=192, chunk=128),
    dict(B=2, H=3, T=384, Hd=128, chunk=64),
    dict(B=1, H=2, T=1024, Hd=320, chunk=256),
]


@pytest.mark.parametrize("momentum,chunk_avg", VARIANTS)
@pytest.mark.parametrize("i", range(len(MFMA_CASES)))
def test_swiglu_mfma_variants(momentum, chunk_avg, i):
    e2 = _e2()
    c = MFMA_CASES[i]
    cfg = synth.CONFIGS["swiglu_1p3b"].with_(name=f"var{i}_m{int(momentum)}a{int(chunk_avg)}", **c)
    gu.note(f"mfma variant momentum={momentum} avg={chunk_avg} case {i}: {c}")
    x = synth.make_inputs(cfg, seed=40 + i, m0_scale=0.5)
    x["alpha"][..., 1::19] = 1.0
    x["eta"][..., 3::31] = 0.0
    flags = (0 if momentum else 2) | (4 if chunk_avg else 0)
    assert e2.path("swiglu", "negdot", "bf16", cfg.B, cfg.H, cfg.T, cfg.D, cfg.Hd, cfg.chunk, flags) == 1
    got = gu.run_gpu(cfg, x, momentum=momentum, chunk_avg=chunk_avg)
    ref = gu.run_oracle(cfg, x, momentum=momentum, chunk_avg=chunk_avg)
    gu.assert_close(cfg, got, ref, x["W0"].numpy())


@pytest.mark.parametrize("momentum,chunk_avg", VARIANTS)
def test_swiglu_1p3b_variants_full_size(momentum, chunk_avg):
    """The 1.3B-shaped workload at full size in the benchmark's launch
    configuration, first two chunks (the state scale of test_config_prefix_state)."""
    _e2()
    cfg = synth.CONFIGS["swiglu_1p3b"]
    cfg = cfg.with_(T=2 * cfg.chunk)
    gu.note(f"1p3b variant momentum={momentum} avg={chunk_avg}")
    x = synth.make_inputs(cfg, seed=0)
    got = gu.run_gpu(cfg, x, momentum=momentum, chunk_avg=chunk_avg)
    ref = gu.run_oracle(cfg, x, momentum=momentum, chunk_avg=chunk_avg)
    gu.assert_close(cfg, got, ref, x["W0"].numpy())


@pytest.mark.parametrize("momentum,chunk_avg", VARIANTS)
@pytest.mark.parametrize("kind,loss", [("linear", "mse"), ("mlp", "mse"), ("swiglu", "negdot")])
@pytest.mark.parametrize("chunk", [1, 16])
def test_generic_variants(momentum, chunk_avg, kind, loss, chunk):
    _e2()
    base = synth.CONFIGS["mlp_fp32"] if kind == "mlp" else synth.CONFIGS["tiny_linear"]
    cfg = base.with_(name=f"gen_{kind}_m{int(momentum)}a{int(chunk_avg)}", kind=kind, loss=loss, B=2, H=2, T=4 * chunk,
                     D=16, Hd=24 if kind != "linear" else 0, chunk=chunk, io_dtype="f32")
    gu.note(f"generic variant {kind}/{loss} momentum={momentum} avg={chunk_avg} chunk={chunk}")
    x = synth.make_inputs(cfg, seed=chunk + 5, m0_scale=0.5)
    if kind == "mlp":  # the MLP/MSE state grows without bound at the drawn learning rates
        x["eta"] = x["eta"] / cfg.D
    got = gu.run_gpu(cfg, x, force_generic=True, momentum=momentum, chunk_avg=chunk_avg)
    ref = gu.run_oracle(cfg, x, momentum=momentum, chunk_avg=chunk_avg)
    gu.assert_close(cfg, got, ref, x["W0"].numpy())


def test_no_momentum_in_place_and_null_momentum_buffers():
    """Without momentum beta, M0 and M_end are never touched: the call works
    with them absent and updates W in place."""
    _e2()
    cfg = synth.CONFIGS["swiglu_1p3b"].with_(name="nm_inplace", B=1, H=2, T=512, Hd=128, chunk=128)
    x = synth.make_inputs(cfg, seed=77)
    ref = gu.run_oracle(cfg, x, momentum=False)
    got = gu.run_gpu(cfg, x, in_place=True, momentum=False)
    gu.assert_close(cfg, got, ref, x["W0"].numpy())
