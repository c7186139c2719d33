"""ctypes view of libe2ttt.so (the C ABI in include/e2ttt.h)."""
from __future__ import annotations

import ctypes
import os

# E2TTT_LIB names another build of the same library (the host-sanitized copy
# the CPU tests load); by default the in-tree libe2ttt.so.
LIB_PATH = os.environ.get("E2TTT_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libe2ttt.so")

KIND = {"linear": 0, "mlp": 1, "swiglu": 2}
LOSS = {"mse": 0, "negdot": 1}
DTYPE = {"f32": 0, "bf16": 1}
FLAG_FORCE_GENERIC = 1
FLAG_NO_MOMENTUM = 2
FLAG_CHUNK_AVG = 4
FLAG_SAVE_STATES = 8
FLAG_PRECISE = 16

STATUS = {0: "E2TTT_OK", 1: "E2TTT_ERR_INVALID_ARG", 2: "E2TTT_ERR_UNSUPPORTED", 3: "E2TTT_ERR_ALIAS",
          4: "E2TTT_ERR_WORKSPACE", 5: "E2TTT_ERR_HIP", 6: "E2TTT_ERR_SCRATCH_LIMIT"}
NOALLOC_SCRATCH_BYTES = 64 << 20  # E2TTT_NOALLOC_SCRATCH_BYTES

EXPORTS = ("e2ttt_param_count", "e2ttt_workspace_size", "e2ttt_path", "e2ttt_validate",
           "e2ttt_chunk_forward", "e2ttt_chunk_forward_events", "e2ttt_logscan", "e2ttt_status_string",
           "e2ttt_backward_workspace_size", "e2ttt_validate_backward", "e2ttt_chunk_backward",
           "e2ttt_chunk_backward_events", "e2ttt_chunk_forward_noalloc")


class Desc(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("loss", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("B", ctypes.c_int64), ("H", ctypes.c_int64),
                ("T", ctypes.c_int64), ("D", ctypes.c_int64), ("Hd", ctypes.c_int64),
                ("chunk", ctypes.c_int64)]


class E2TTTError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m chunk_weight_rnn_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    pd = ctypes.POINTER(Desc)
    lib.e2ttt_param_count.argtypes = [pd]
    lib.e2ttt_param_count.restype = i64
    lib.e2ttt_workspace_size.argtypes = [pd]
    lib.e2ttt_workspace_size.restype = sz
    lib.e2ttt_path.argtypes = [pd]
    lib.e2ttt_path.restype = ctypes.c_int
    lib.e2ttt_validate.argtypes = [pd, ctypes.POINTER(vp)]
    lib.e2ttt_validate.restype = ctypes.c_int
    lib.e2ttt_chunk_forward.argtypes = [pd] + [vp] * 11 + [vp, sz, vp]
    lib.e2ttt_chunk_forward.restype = ctypes.c_int
    lib.e2ttt_chunk_forward_events.argtypes = [pd] + [vp] * 11 + [vp, sz, vp, ctypes.POINTER(vp)]
    lib.e2ttt_chunk_forward_events.restype = ctypes.c_int
    lib.e2ttt_chunk_forward_noalloc.argtypes = [pd] + [vp] * 11 + [vp]
    lib.e2ttt_chunk_forward_noalloc.restype = ctypes.c_int
    lib.e2ttt_logscan.argtypes = [pd] + [vp] * 6 + [vp]
    lib.e2ttt_logscan.restype = ctypes.c_int
    lib.e2ttt_backward_workspace_size.argtypes = [pd]
    lib.e2ttt_backward_workspace_size.restype = sz
    lib.e2ttt_validate_backward.argtypes = [pd, ctypes.POINTER(vp)]
    lib.e2ttt_validate_backward.restype = ctypes.c_int
    lib.e2ttt_chunk_backward.argtypes = [pd] + [vp] * 19 + [vp, sz, vp]
    lib.e2ttt_chunk_backward.restype = ctypes.c_int
    lib.e2ttt_chunk_backward_events.argtypes = [pd] + [vp] * 19 + [vp, sz, vp, ctypes.POINTER(vp)]
    lib.e2ttt_chunk_backward_events.restype = ctypes.c_int
    lib.e2ttt_status_string.argtypes = [ctypes.c_int]
    lib.e2ttt_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def make_desc(kind: str, loss: str, io_dtype: str, B: int, H: int, T: int, D: int, Hd: int, chunk: int,
              flags: int = 0) -> Desc:
    return Desc(KIND[kind], LOSS[loss], DTYPE[io_dtype], flags, B, H, T, D, Hd, chunk)
