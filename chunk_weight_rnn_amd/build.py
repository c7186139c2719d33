"""Build libe2ttt.so in-tree with hipcc for gfx950.

    python -m chunk_weight_rnn_amd.build [--verbose] [--sanitize]

--sanitize builds a second copy, _build/san/libe2ttt.so, whose host code
(argument validation, workspace layout, dispatch) is instrumented with
AddressSanitizer and UndefinedBehaviorSanitizer (device code as usual); the
host-side ABI tests load it on the CPU with the sanitizer runtime preloaded.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libe2ttt.so")
PROBE_LIB = os.path.join(PKG, "libe2ttt_probe.so")  # microbenchmarks of the chip's ceilings (bench.py --peaks)
PROBE_SOURCES = ["probe.hip"]
SOURCES = ["abi.hip", "logscan.hip", "generic.hip", "generic_bwd.hip", "f32_mfma.hip", "swiglu_loop.hip",
           "swiglu_mfma.hip", "swiglu_bwd.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def _flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-fvisibility=hidden",
            # packed fp32 VALU ops are kept out of the device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument"]


# host-only sanitizers: every -fsanitize= sits right after -Xarch_host, so the
# device code is built without them
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_LIB = os.path.join(PKG, "_build", "san", "libe2ttt.so")


def sanitizer_runtime() -> str:
    """The clang AddressSanitizer runtime (with the UBSan handlers) that a
    process loading the sanitized library must preload."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang ASan runtime not found under /opt/rocm/llvm")
    return hits[-1]


def build_sanitized(verbose: bool = False) -> str:
    """The library with sanitized host code, in _build/san (not the product)."""
    cc = hipcc()
    objdir = os.path.dirname(SAN_LIB)
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src: str) -> str:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [cc, *_flags(), *SAN_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = SAN_LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *SAN_FLAGS, "-Xarch_host", "-shared-libsan", *objs,
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


def build(verbose: bool = False) -> str:
    cc = hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src: str) -> str:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [cc, *_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES + PROBE_SOURCES))

    def link(objects: list[str], lib: str) -> None:
        tmp = lib + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objects, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, lib)

    link(objs[:len(SOURCES)], LIB)
    link(objs[len(SOURCES):], PROBE_LIB)
    return LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized(verbose="--verbose" in sys.argv))
    else:
        print(build(verbose="--verbose" in sys.argv))
