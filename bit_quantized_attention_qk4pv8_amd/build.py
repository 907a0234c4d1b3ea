"""Build libqfa.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m bit_quantized_attention_qk4pv8_amd.build

hipcc cross-compiles without a GPU.  Flags:
  -Xclang -target-feature -Xclang -packed-fp32-ops   no packed FP32 VALU ops
  -mllvm -amdgpu-mfma-vgpr-form                      MFMA accumulators in VGPRs
                                                     (no AGPR copies around the
                                                     softmax and rescale)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqfa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["api.hip", "quant.hip", "attn.hip", "prefill.hip"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the GPU-only target feature; that warning is expected
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    # Loading resolves every symbol (no GPU needed): a kernel whose host launch
    # stub went missing shows up here rather than at the first call.
    try:
        ctypes.CDLL(tmp, mode=os.RTLD_NOW)
    except OSError as e:
        os.remove(tmp)
        raise RuntimeError("built library does not load: %s" % e)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
