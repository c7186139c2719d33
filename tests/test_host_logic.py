"""Host-side logic added around the kernels (CPU only):

- the benchmark's code fingerprint, which keeps committed HBM counters valid
  across comment edits but not across code edits;
- the probe library's exports;
- the output kernel's wait counts: with a ring of NS stage buffers, each
  stage waits until at most (NS - 2) NI + NQ q loads are outstanding, where q
  is the number of query-load batches among the last NS - 1 stages (a bit
  mask in the kernel).  Modelled here on the kernel's issue order, that count
  must equal the number of loads issued after the stage's own copies, and the
  stage's copies must be covered.
"""
import ctypes
import os

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_fingerprint_ignores_comments_not_code(tmp_path):
    src = tmp_path / "k.hip"
    src.write_text("// header\nint f(int x) {\n    return x + 1;  // one\n}\n/* block\n comment */\n")
    fp = bench.code_fingerprint(str(src))
    src.write_text("// another header\nint f(int x) {\n  return x + 1;   // edited comment\n}\n")
    assert bench.code_fingerprint(str(src)) == fp
    src.write_text("// header\nint f(int x) {\n    return x + 2;  // one\n}\n")
    assert bench.code_fingerprint(str(src)) != fp


def test_probe_library_exports():
    path = os.path.join(ROOT, "chunk_weight_rnn_amd", "libe2ttt_probe.so")
    if not os.path.exists(path):
        pytest.skip("probe library not built")
    try:
        lib = ctypes.CDLL(path)
    except OSError as e:  # the HIP runtime may be absent on a build host
        pytest.skip(f"cannot load: {e}")
    for name in ("e2ttt_probe_mfma", "e2ttt_probe_read"):
        assert hasattr(lib, name), name


def _check_ring(NS, NI, NQ, nhb, nitems):
    ops = [("q", 0)] * NQ                      # the first item's queries, before every copy
    for g in range(NS - 1):                    # prologue: stages 0 .. NS-2
        ops += [("s", g)] * NI
    qmask = 0
    for gs in range(nitems * nhb):
        count = (NS - 2) * NI + NQ * min(bin(qmask).count("1"), 3)
        last = max(i for i, t in enumerate(ops) if t == ("s", gs))
        assert len(ops) - 1 - last == count, (NS, NI, nhb, gs)
        ops += [("s", gs + NS - 1)] * NI       # refill of the previous stage's buffer
        qmask = (qmask << 1) & ((1 << (NS - 1)) - 1)
        if gs % nhb == 0:                      # item start: the next item's query loads
            ops += [("q", gs // nhb + 1)] * NQ
            qmask |= 1


@pytest.mark.parametrize("NS,NI", [(6, 3), (3, 6), (3, 12)])  # 8-, 4- and 2-wavefront forms
@pytest.mark.parametrize("nhb", [2, 4, 6, 8, 10, 128])       # hidden width / 32
def test_output_ring_wait_counts(NS, NI, nhb):
    for nitems in (1, 2, 5):
        _check_ring(NS, NI, 8, nhb, nitems)
    # the mask never holds more batches than the switch in the kernel handles
    assert (NS - 1 + nhb - 1) // nhb <= 3
