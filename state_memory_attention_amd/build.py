"""Build libdart.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m state_memory_attention_amd.build [-v]

Each source is compiled to an object under ``_build/`` in parallel, then
linked into ``state_memory_attention_amd/libdart.so``.  The library is always
rebuilt: objects are not reused between calls.  The measurement probes go
into a library of their own, and a plain C program that calls libdart.so
through ``include/dart.h`` (``tests/c_abi/``) is built with gcc last.
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
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdart.so")

SOURCES = [
    "api.cpp",
    "general.hip",
    "chunk_states_mfma.hip",
    "sma_fwd_mfma.hip",
    "sma_decode_mfma.hip",
    "backward_general.hip",
    "decode_update.hip",
    "sma_bwd_mfma.hip",
    "rms_general.hip",
    "sma_fwd_rms_mfma.hip",
    "rms_backward.hip",
    "sma_bwd_rms_mfma.hip",
    "ssd.hip",
]
# Measurement support, not part of the library: a plain 16-byte-vector copy
# (calibrates the hardware memory-traffic counters), a streaming read and a
# matrix-core loop (two yardsticks), in a library of their own under probes/.
PROBE_DIR = os.path.join(PKG, "probes")
PROBE_SOURCE = os.path.join(PROBE_DIR, "probe_copy.hip")
PROBE_LIB = os.path.join(PROBE_DIR, "libdart_probe.so")

ARCH = "gfx950"
# Packed fp32 VALU forms are disabled for every HIP source.
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libdart.so")
    return path


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(os.path.basename(src))[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc(), f"--offload-arch={ARCH}", *COMMON_FLAGS, "-I", INCLUDE, "-I", CSRC,
           *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in line)  # host pass does not know the feature
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if verbose and out.strip():
        print(out, flush=True)
    return obj


def _link(objs, out, verbose):
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, out)


# A plain C program that uses libdart.so through include/dart.h and the HIP
# runtime only (tests/test_gpu_c_abi.py runs it on the GPU).
C_SMOKE_SOURCE = os.path.join(ROOT, "tests", "c_abi", "dart_c_smoke.c")
C_SMOKE_BIN = os.path.join(ROOT, "tests", "c_abi", "dart_c_smoke.bin")


def _build_c_smoke(verbose: bool) -> None:
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler found for tests/c_abi/dart_c_smoke.c")
    rel = os.path.relpath(PKG, os.path.dirname(C_SMOKE_BIN))
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE, "-I",
           os.path.join(rocm, "include"), C_SMOKE_SOURCE, "-L", PKG, "-ldart", "-L", os.path.join(rocm, "lib"),
           "-lamdhip64", "-lm", f"-Wl,-rpath,$ORIGIN/{rel}", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}",
           "-o", C_SMOKE_BIN]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C program failed to build:\n{r.stdout}{r.stderr}")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + [PROBE_SOURCE]
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    _link(objs[:-1], LIB, verbose)
    _link(objs[-1:], PROBE_LIB, verbose)
    _build_c_smoke(verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
