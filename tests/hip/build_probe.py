"""Build tests/hip/libqfa_probe.so, the test-only HIP library of GPU-side pins,
in-tree for gfx950 (hipcc cross-compiles without a GPU).

    python tests/hip/build_probe.py
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qfa_probe.hip")
LIB = os.path.join(HERE, "libqfa_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
]
SYMBOLS = ("probe_cvt", "probe_s_tile", "probe_s_tile_seeded", "probe_tile_rowsum", "probe_delta", "probe_exp2",
           "probe_lds_fill")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + [SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    ctypes.CDLL(tmp, mode=os.RTLD_NOW)
    os.replace(tmp, LIB)
    return LIB


def load():
    """The built probe library; raises if it has not been built."""
    if not os.path.exists(LIB):
        raise RuntimeError("%s is not built: run __graft_entry__.build() or %s" % (LIB, __file__))
    L = ctypes.CDLL(LIB)
    P, I, LG, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_long, ctypes.c_float
    L.probe_cvt.restype = I
    L.probe_cvt.argtypes = [I, P, LG, F, P]
    L.probe_s_tile.restype = I
    L.probe_s_tile.argtypes = [P, P, P, P, I, I, I, P]
    L.probe_s_tile_seeded.restype = I
    L.probe_s_tile_seeded.argtypes = [P, P, P, P, P, I, I, I, P]
    L.probe_tile_rowsum.restype = I
    L.probe_tile_rowsum.argtypes = [P, P, P, P]
    L.probe_delta.restype = I
    L.probe_delta.argtypes = [P, I, I, P, I, I, I, P]
    L.probe_exp2.restype = I
    L.probe_exp2.argtypes = [P, ctypes.c_long, P]
    L.probe_lds_fill.restype = I
    L.probe_lds_fill.argtypes = [ctypes.c_uint32, I, I]
    return L


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
