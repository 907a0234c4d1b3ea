"""Static check of the prefill kernels that keep O^T in fixed accumulation
registers (csrc/attn_common.h, ofix_*): only inline assembly may touch those
AGPRs.  The compiler does not know they hold a value between the statements,
so the kernels are correct only while the compiler allocates no AGPR of its
own in them.  This compiles prefill.hip to gfx950 assembly with the library's
flags and checks, for every such kernel, that
  - no AGPR appears outside the inline-assembly blocks,
  - the kernel descriptor reserves the D/2 AGPRs O^T occupies,
  - nothing spills.
CPU only (hipcc cross-compiles); skipped where hipcc is missing."""
import os
import re
import shutil
import subprocess

import pytest

from bit_quantized_attention_qk4pv8_amd import build as qbuild

# k_prefill<D, COMP, PV>: the method's format (PV 0) without compensation
FIXED_O = {64: "_ZN3qfa9k_prefillILi64ELb0ELi0EEEvNS_8AttnArgsEi",
           128: "_ZN3qfa9k_prefillILi128ELb0ELi0EEEvNS_8AttnArgsEi"}


@pytest.fixture(scope="module")
def prefill_asm(tmp_path_factory):
    if not (os.path.exists(qbuild.HIPCC) or shutil.which("hipcc")):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asm") / "prefill.s")
    flags = [f for f in qbuild.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [qbuild.HIPCC] + flags + ["--cuda-device-only", "-S", os.path.join(qbuild.CSRC, "prefill.hip"), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return open(out).read()


def _body(asm: str, name: str) -> list:
    m = re.search(r"^" + re.escape(name) + r":", asm, re.M)  # the label (a comment may follow)
    assert m, name
    end = asm.index("\n.Lfunc_end", m.start())
    return asm[m.start():end].split("\n")


def _descriptor(asm: str, name: str) -> dict:
    blk = asm[asm.index(".amdhsa_kernel " + name):]
    blk = blk[:blk.index(".end_amdhsa_kernel")]
    return {k: int(v) for k, v in re.findall(r"\.amdhsa_(\w+) (\d+)", blk)}


@pytest.mark.parametrize("D", sorted(FIXED_O))
def test_no_compiler_agpr_outside_fixed_o_asm(prefill_asm, D):
    name = FIXED_O[D]
    in_asm = False
    inside, outside = 0, []
    for line in _body(prefill_asm, name):
        if ";;#ASMSTART" in line:
            in_asm = True
            continue
        if ";;#ASMEND" in line:
            in_asm = False
            continue
        code = line.split(";")[0].strip()
        if not code or code.startswith("."):
            continue
        if re.search(r"\ba\[?\d", code):
            if in_asm:
                inside += 1
            else:
                outside.append(code)
    assert inside >= 2 * (D // 32) + D // 2, "fixed-O assembly not found in %s" % name
    assert not outside, "compiler-allocated AGPRs in %s: %s" % (name, outside[:5])


@pytest.mark.parametrize("D", sorted(FIXED_O))
def test_descriptor_reserves_fixed_o(prefill_asm, D):
    d = _descriptor(prefill_asm, FIXED_O[D])
    agprs = d["next_free_vgpr"] - d["accum_offset"]
    assert agprs >= D // 2, d
    assert d["next_free_vgpr"] <= 256, d      # two waves per SIMD
    assert d.get("private_segment_fixed_size", 0) == 0, d  # no spills to scratch
    meta = prefill_asm[prefill_asm.index(".name:           " + FIXED_O[D]):][:600]
    spill = re.findall(r"\.vgpr_spill_count:\s+(\d+)", meta)
    assert spill and int(spill[0]) == 0, meta
