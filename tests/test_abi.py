"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and validates descriptors and pointers (no GPU needed: only
entry points that return before touching a device are called)."""
import ctypes
import os
import re

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "e2ttt.h")


@pytest.fixture(scope="module")
def lib():
    from chunk_weight_rnn_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from chunk_weight_rnn_amd import build
        build.build()
    return _lib.load()


def _desc(kind="swiglu", loss="negdot", io="bf16", B=2, H=3, T=256, D=128, Hd=256, chunk=64, flags=0):
    from chunk_weight_rnn_amd._lib import make_desc
    return make_desc(kind, loss, io, B, H, T, D, Hd, chunk, flags)


def test_exports_every_declared_symbol(lib):
    names = set(re.findall(r"E2TTT_API[^;(]*?\b(e2ttt_\w+)\s*\(", open(HEADER).read()))
    assert len(names) == 13
    from chunk_weight_rnn_amd import _lib
    assert names == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_param_count_and_paths(lib):
    for cfg in synth.CONFIGS.values():
        d = _desc(cfg.kind, cfg.loss, cfg.io_dtype, cfg.B, cfg.H, cfg.T, cfg.D, cfg.Hd, cfg.chunk)
        assert lib.e2ttt_param_count(ctypes.byref(d)) == cfg.P
        path = lib.e2ttt_path(ctypes.byref(d))
        # linear / MLP: the fp32 MFMA path; the 8-head MLP workload split over hidden slices
        assert path == {"swiglu": 1, "linear": 3, "mlp": 4}[cfg.kind]
        assert lib.e2ttt_workspace_size(ctypes.byref(d)) > 0
    d = _desc(flags=1)
    assert lib.e2ttt_path(ctypes.byref(d)) == 0


def test_workspace_size_rules(lib):
    d = _desc(B=0)
    assert lib.e2ttt_workspace_size(ctypes.byref(d)) == 0
    d = _desc(T=0)
    assert lib.e2ttt_workspace_size(ctypes.byref(d)) == 0
    # a ragged tail is a shorter last chunk: two chunks, coefficient rows padded to 128
    d = _desc(T=100, chunk=64)
    assert lib.e2ttt_workspace_size(ctypes.byref(d)) == lib.e2ttt_workspace_size(ctypes.byref(_desc(T=128, chunk=64)))
    # MFMA path needs the snapshots: grows with the number of chunks
    a = lib.e2ttt_workspace_size(ctypes.byref(_desc(chunk=64)))
    b = lib.e2ttt_workspace_size(ctypes.byref(_desc(chunk=256)))
    assert a > b


def _ptrs(desc, base=1 << 40, gap=1 << 32):
    # 11 disjoint, 256-aligned fake device addresses (never dereferenced)
    return [base + i * gap for i in range(11)]


def _validate(lib, d, ptrs):
    arr = (ctypes.c_void_p * 11)(*[ctypes.c_void_p(p) for p in ptrs])
    return lib.e2ttt_validate(ctypes.byref(d), arr)


def test_validate_ok_and_in_place(lib):
    d = _desc()
    p = _ptrs(d)
    assert _validate(lib, d, p) == 0
    p2 = list(p)
    p2[9] = p2[6]   # W_end == W0
    p2[10] = p2[7]  # M_end == M0
    assert _validate(lib, d, p2) == 0


@pytest.mark.parametrize("field,value", [("kind", 7), ("loss", -1), ("io_dtype", 2), ("B", -1), ("D", 0),
                                         ("chunk", 0), ("Hd", 0)])
def test_validate_bad_desc(lib, field, value):
    d = _desc()
    setattr(d, field, value)
    assert _validate(lib, d, _ptrs(d)) == 1


def test_validate_ragged_tail_accepted(lib):
    for T, C in ((100, 64), (1, 64), (65, 64), (7, 3)):
        d = _desc(T=T, chunk=C)
        assert _validate(lib, d, _ptrs(d)) == 0


def test_validate_null_and_misaligned(lib):
    d = _desc()
    for i in range(11):
        p = _ptrs(d)
        p[i] = 0
        assert _validate(lib, d, p) == 1, i
    p = _ptrs(d)
    p[0] += 2  # q not 16-byte aligned
    assert _validate(lib, d, p) == 1
    p = _ptrs(d)
    p[3] += 4  # eta only needs 4-byte alignment
    assert _validate(lib, d, p) == 0
    # empty tensors may be null
    d0 = _desc(B=0)
    assert _validate(lib, d0, [0] * 11) == 0


def test_validate_aliasing(lib):
    d = _desc()
    p = _ptrs(d)
    p[8] = p[0] + 64  # out overlaps q
    assert _validate(lib, d, p) == 3
    p = _ptrs(d)
    p[9] = p[7]  # W_end == M0
    assert _validate(lib, d, p) == 3
    p = _ptrs(d)
    p[10] = p[9]  # M_end == W_end
    assert _validate(lib, d, p) == 3
    p = _ptrs(d)
    p[9] = p[6] + 16  # W_end partially overlapping W0
    assert _validate(lib, d, p) == 3


def test_validate_unsupported_shape(lib):
    d = _desc(kind="linear", loss="mse", io="f32", D=512, Hd=0)
    assert _validate(lib, d, _ptrs(d)) == 2
    d = _desc(kind="mlp", loss="mse", io="f32", D=64, Hd=2048)
    assert _validate(lib, d, _ptrs(d)) == 2
    # the MFMA path covers wide SwiGLU hidden layers
    d = _desc(Hd=2048)
    assert _validate(lib, d, _ptrs(d)) == 0


def test_chunk_forward_rejects_before_launch(lib):
    d = _desc(flags=1 << 20)  # unknown flag
    v = ctypes.c_void_p
    args = [v(1 << 40)] * 11
    assert lib.e2ttt_chunk_forward(ctypes.byref(d), *args, v(0), ctypes.c_size_t(0), v(0)) == 1
    d = _desc()
    args = [v((1 << 40) + i * (1 << 32)) for i in range(11)]
    # workspace missing
    assert lib.e2ttt_chunk_forward(ctypes.byref(d), *args, v(0), ctypes.c_size_t(0), v(0)) == 4
    # workspace too small
    assert lib.e2ttt_chunk_forward(ctypes.byref(d), *args, v(1 << 50), ctypes.c_size_t(16), v(0)) == 4
    assert lib.e2ttt_chunk_forward(None, *args, v(0), ctypes.c_size_t(0), v(0)) == 1
    assert lib.e2ttt_logscan(None, v(0), v(0), v(0), v(0), v(0), v(0), v(0)) == 1


def test_paths_of_narrow_heads_and_precise_flag(lib):
    """A 64-unit SwiGLU head takes the bf16 MFMA path (1); with
    E2TTT_FLAG_PRECISE the hi/lo-operand form of it (2); forcing the portable
    path wins over both (0).  A precise forward cannot save states for the
    MFMA backward (its backward is the portable one)."""
    from chunk_weight_rnn_amd._lib import FLAG_FORCE_GENERIC, FLAG_PRECISE, FLAG_SAVE_STATES
    for Hd in (64, 128, 256):
        assert lib.e2ttt_path(ctypes.byref(_desc(Hd=Hd, T=768, chunk=256))) == 1
        assert lib.e2ttt_path(ctypes.byref(_desc(Hd=Hd, T=768, chunk=256, flags=FLAG_PRECISE))) == 2
        assert lib.e2ttt_path(ctypes.byref(_desc(Hd=Hd, flags=FLAG_PRECISE | FLAG_FORCE_GENERIC))) == 0
    d = _desc(Hd=64, flags=FLAG_PRECISE)
    assert _validate(lib, d, _ptrs(d)) == 0
    d = _desc(Hd=64, flags=FLAG_PRECISE | FLAG_SAVE_STATES)
    assert _validate(lib, d, _ptrs(d)) == 2
    # same workspace as the bf16 MFMA path (snapshot layout)
    a = lib.e2ttt_workspace_size(ctypes.byref(_desc(Hd=64)))
    assert lib.e2ttt_workspace_size(ctypes.byref(_desc(Hd=64, flags=FLAG_PRECISE))) == a
    # the fp32 paths are unaffected by the flag
    d = _desc(kind="mlp", loss="mse", io="f32", D=64, Hd=128, flags=FLAG_PRECISE)
    assert lib.e2ttt_path(ctypes.byref(d)) == 4
    d = _desc(kind="mlp", loss="mse", io="f32", D=48, Hd=40, flags=FLAG_PRECISE)
    assert lib.e2ttt_path(ctypes.byref(d)) == 0


def test_fp32_mfma_path_shapes(lib):
    """Linear / MLP with fp32 I/O take the fp32 MFMA path (3) when D and Hd are
    multiples of 16 and a head's state fits 32 tiles of 16x16 per matrix;
    other shapes, bf16 I/O and E2TTT_FLAG_FORCE_GENERIC take the portable
    path (0)."""
    p = lambda **kw: lib.e2ttt_path(ctypes.byref(_desc(**kw)))
    assert p(kind="linear", loss="mse", io="f32", D=32, Hd=0, chunk=16) == 3
    assert p(kind="linear", loss="negdot", io="f32", D=64, Hd=0, chunk=100) == 3
    assert p(kind="mlp", loss="mse", io="f32", D=64, Hd=128, chunk=64) == 4      # 2 x 3 heads x 8 slices
    assert p(kind="mlp", loss="mse", io="f32", B=8, H=16, D=64, Hd=128, chunk=64) == 3  # 1024 slices: per head
    assert p(kind="mlp", loss="mse", io="f32", D=64, Hd=128, chunk=128) == 3     # chunks over 64 tokens
    assert p(kind="mlp", loss="negdot", io="f32", D=16, Hd=48, chunk=1) == 4
    assert p(kind="mlp", loss="mse", io="f32", D=48, Hd=40) == 0          # Hd not a multiple of 16
    assert p(kind="linear", loss="mse", io="f32", D=40, Hd=0) == 0        # D not a multiple of 16
    assert p(kind="mlp", loss="mse", io="f32", D=128, Hd=256) == 0        # 128 tiles per matrix
    assert p(kind="mlp", loss="mse", io="f32", D=128, Hd=64) == 0         # D > 64
    assert p(kind="mlp", loss="mse", io="f32", D=48, Hd=80) == 4
    assert p(kind="mlp", loss="mse", io="bf16", D=64, Hd=128) == 0        # bf16 I/O
    assert p(kind="mlp", loss="mse", io="f32", D=64, Hd=128, flags=1) == 0
    # the scalar kernels' outputs, and for few heads the hidden-slice split's
    # partial sums: partial Y and partial outputs [2][BH][S][64][D] (S = Hd / 16),
    # then one arrival counter per head and a time-out flag
    d = _desc(kind="mlp", loss="mse", io="f32", B=2, H=4, T=2048, D=64, Hd=128, chunk=64)
    split = (4 * (2 * 8 * 8 * 64 * 64 * 2 + 8 + 1) + 255) // 256 * 256  # partial sums, 8 head counters, a flag
    assert lib.e2ttt_workspace_size(ctypes.byref(d)) == 2 * 8 * 2048 * 4 + 8 * 32 * 16 + split
    # many heads fill the chip with one workgroup each: no split
    d = _desc(kind="mlp", loss="mse", io="f32", B=8, H=16, T=2048, D=64, Hd=128, chunk=64)
    assert lib.e2ttt_workspace_size(ctypes.byref(d)) == 2 * 128 * 2048 * 4 + 128 * 32 * 16
    # saving states for the portable backward is allowed from this path
    d = _desc(kind="mlp", loss="mse", io="f32", D=64, Hd=128, chunk=64, flags=8)
    assert _validate(lib, d, _ptrs(d)) == 0


def test_chunk_beyond_int32_rejected(lib):
    """Kernels take the chunk length as a 32-bit int: a longer chunk is
    refused rather than truncated (2^32 + 16 would otherwise run as 16)."""
    for c in ((1 << 31), (1 << 32) + 16):
        d = _desc(T=256, chunk=c)
        assert _validate(lib, d, _ptrs(d)) == 1
        assert lib.e2ttt_workspace_size(ctypes.byref(d)) == ctypes.c_size_t(-1).value
    d = _desc(T=256, chunk=(1 << 31) - 1)  # the largest chunk: one chunk of T tokens
    assert _validate(lib, d, _ptrs(d)) == 0


def test_logscan_validates_its_desc(lib):
    """e2ttt_logscan returns E2TTT_ERR_INVALID_ARG before any launch for
    unknown flags, a chunk outside [1, 2^31 - 1], negative sizes and
    misaligned pointers."""
    v = ctypes.c_void_p
    good = [v((1 << 40) + i * (1 << 32)) for i in range(6)]
    for d in (_desc(flags=1 << 20), _desc(chunk=(1 << 32) + 16), _desc(chunk=0), _desc(T=-1)):
        assert lib.e2ttt_logscan(ctypes.byref(d), *good, v(0)) == 1
    bad = list(good)
    bad[3] = v(good[3].value + 2)  # cM not float-aligned
    assert lib.e2ttt_logscan(ctypes.byref(_desc()), *bad, v(0)) == 1
    # null beta is only allowed without momentum
    nob = list(good)
    nob[2] = v(0)
    assert lib.e2ttt_logscan(ctypes.byref(_desc()), *nob, v(0)) == 1
    # an empty call touches nothing and succeeds
    assert lib.e2ttt_logscan(ctypes.byref(_desc(B=0)), *[v(0)] * 6, v(0)) == 0


def test_status_strings(lib):
    for s in range(7):
        assert lib.e2ttt_status_string(s)
    assert lib.e2ttt_status_string(99) == b"unknown status"


def test_binding_refuses_cpu_tensors(lib):
    import torch
    import chunk_weight_rnn_amd as e2
    x = synth.make_inputs(synth.CONFIGS["tiny_linear"])
    with pytest.raises(ValueError):
        e2.chunk_forward(x["q"], x["k"], x["v"], x["eta"], x["alpha"], x["beta"], x["W0"], x["M0"],
                         chunk=16, kind="linear", loss="mse")
    with pytest.raises(ValueError):
        e2.logscan(x["eta"], x["alpha"], x["beta"], chunk=16)
    assert isinstance(torch.__version__, str)


def test_validate_variant_flags(lib):
    # no momentum: beta (5), M0 (7) and M_end (10) are not used and may be null
    d = _desc(flags=2)
    p = _ptrs(d)
    p[5] = p[7] = p[10] = 0
    assert _validate(lib, d, p) == 0
    # ... and may then overlap anything (they are not read or written)
    p = _ptrs(d)
    p[10] = p[9]
    assert _validate(lib, d, p) == 0
    # the other pointers are still required
    p = _ptrs(d)
    p[9] = 0
    assert _validate(lib, d, p) == 1
    # with momentum they are required
    d = _desc(flags=4)
    p = _ptrs(d)
    p[7] = 0
    assert _validate(lib, d, p) == 1
    # both variants together, and with the portable path
    for f in (2 | 4, 1 | 2 | 4):
        d = _desc(flags=f)
        assert _validate(lib, d, _ptrs(d)) == 0
    # unknown flag bits are rejected
    d = _desc(flags=32)
    assert _validate(lib, d, _ptrs(d)) == 1
    assert lib.e2ttt_workspace_size(ctypes.byref(d)) == ctypes.c_size_t(-1).value


def _bwd_ptrs(d, momentum=True):
    # 19 disjoint fake device addresses, 1 GiB apart
    p = [(1 << 40) + i * (1 << 30) for i in range(19)]
    if not momentum:
        for i in (5, 7, 10, 16, 18):  # beta, M0, dM_end, dbeta, dM0
            p[i] = 0
    return p


def _validate_bwd(lib, d, p):
    arr = (ctypes.c_void_p * 19)(*[ctypes.c_void_p(x) for x in p])
    return lib.e2ttt_validate_backward(ctypes.byref(d), arr)


def test_backward_validation(lib):
    d = _desc()
    assert _validate_bwd(lib, d, _bwd_ptrs(d)) == 0
    assert lib.e2ttt_backward_workspace_size(ctypes.byref(d)) > 0
    # ragged tail, no momentum (unused pointers may be null), chunk average
    d = _desc(T=200)
    assert _validate_bwd(lib, d, _bwd_ptrs(d)) == 0
    d = _desc(flags=2)
    assert _validate_bwd(lib, d, _bwd_ptrs(d, momentum=False)) == 0
    d = _desc(flags=4)
    assert _validate_bwd(lib, d, _bwd_ptrs(d)) == 0
    # the portable backward takes what the MFMA path does not
    for ok in (_desc(kind="linear", loss="mse", io="f32", D=32, Hd=0), _desc(io="f32"), _desc(D=64),
               _desc(Hd=96), _desc(chunk=96), _desc(flags=1), _desc(kind="mlp", loss="mse", io="f32", D=64, Hd=128)):
        assert _validate_bwd(lib, ok, _bwd_ptrs(ok)) == 0
    # long chunks, and shapes neither path handles
    for bad in (_desc(chunk=4096, T=8192), _desc(kind="mlp", loss="mse", io="f32", D=64, Hd=2048),
                _desc(kind="linear", loss="mse", io="f32", D=512, Hd=0), _desc(D=256, Hd=2048)):
        assert _validate_bwd(lib, bad, _bwd_ptrs(bad)) == 2
    # every output must be disjoint from everything else (no in-place form)
    d = _desc()
    for o, i in ((17, 6), (18, 7), (11, 0), (14, 3), (12, 11)):
        p = _bwd_ptrs(d)
        p[o] = p[i]
        assert _validate_bwd(lib, d, p) == 3, (o, i)
    # null and misaligned pointers
    p = _bwd_ptrs(d)
    p[9] = 0
    assert _validate_bwd(lib, d, p) == 1
    p = _bwd_ptrs(d)
    p[12] += 4
    assert _validate_bwd(lib, d, p) == 1
    p = _bwd_ptrs(d)
    p[15] += 4  # dalpha needs 4-byte alignment only
    assert _validate_bwd(lib, d, p) == 0
    # the entry point validates before launching, and checks the workspace
    v = ctypes.c_void_p
    args = [v(x) for x in _bwd_ptrs(d)]
    assert lib.e2ttt_chunk_backward(ctypes.byref(d), *args, v(0), ctypes.c_size_t(0), v(0)) == 4
    bad = _desc(chunk=4096, T=8192)
    assert lib.e2ttt_chunk_backward(ctypes.byref(bad), *args, v(0), ctypes.c_size_t(0), v(0)) == 2


def test_very_long_sequences_take_the_portable_path(lib):
    """One head's K/V rows beyond 2 GiB leave the MFMA path (32-bit buffer offsets)."""
    d = _desc(B=1, H=1, T=(1 << 23) - 64)
    assert lib.e2ttt_path(ctypes.byref(d)) == 1
    d = _desc(B=1, H=1, T=1 << 23)
    assert lib.e2ttt_path(ctypes.byref(d)) == 0


def test_chunk_update_refuses_cpu_tensors(lib):
    import chunk_weight_rnn_amd as e2
    x = synth.make_inputs(synth.CONFIGS["tiny_linear"])
    with pytest.raises(ValueError):
        e2.chunk_update(x["q"], x["k"], x["v"], x["eta"], x["alpha"], x["beta"], x["W0"], x["M0"], chunk=16,
                        kind="linear", loss="mse")


def test_save_states_flag(lib):
    """With the save-states flag forward and backward share one workspace."""
    for d in (_desc(flags=8), _desc(flags=8 | 2), _desc(kind="mlp", loss="mse", io="f32", D=64, Hd=128, flags=8)):
        assert lib.e2ttt_workspace_size(ctypes.byref(d)) == lib.e2ttt_backward_workspace_size(ctypes.byref(d))
        assert _validate(lib, d, _ptrs(d)) == 0
    plain, saved = _desc(), _desc(flags=8)
    assert lib.e2ttt_workspace_size(ctypes.byref(saved)) > lib.e2ttt_workspace_size(ctypes.byref(plain))
    # where the backward is unsupported, so is saving for it
    d = _desc(chunk=4096, T=8192, flags=8)
    assert _validate(lib, d, _ptrs(d)) == 2
    assert _validate(lib, _desc(chunk=4096, T=8192), _ptrs(_desc(chunk=4096, T=8192))) == 0
