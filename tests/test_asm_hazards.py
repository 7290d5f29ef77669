"""The direct-to-LDS loads of the MFMA kernel are inline asm, which the
compiler's hazard recognizer does not look into.  The CDNA3/CDNA4 ISA asks
for one wait state between an SALU write of M0 and a load that writes LDS, and
five between a VALU write of an SGPR (a v_readlane restoring a spilled address
base, say) and a vector memory instruction that reads it.  A load issued
without them can read a stale base and fault.  This compiles the kernel for
gfx950 (host only, no GPU) and checks that every such load in every
instantiation comes right after an s_nop of at least 5 wait states.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "diffusion_lm_speculative_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("src", ["verify_mfma.hip", "linear.hip", "stream_probe.hip"])
def test_every_lds_dma_load_follows_five_wait_states(tmp_path, src):
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
           "-o", str(out), os.path.join(CSRC, src)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    lines = [l.strip() for l in out.read_text().splitlines()]
    code = [l for l in lines if l and not l.startswith((";", ".", "//")) and not l.endswith(":")]
    loads = 0
    for i, ins in enumerate(code):
        if not ins.startswith(("global_load_lds", "buffer_load_lds")):
            continue
        loads += 1
        prev = code[i - 1] if i else ""
        m = re.match(r"s_nop\s+(\d+)", prev)
        assert m and int(m.group(1)) >= 4, f"LDS DMA load without 5 wait states before it: {prev!r} -> {ins!r}"
    assert loads > 0, "no direct-to-LDS loads found: the check would prove nothing"
