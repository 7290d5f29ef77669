"""The host side of libsimsd.so under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only, no GPU).

The library's sources are built again with the sanitizers on the host code
only (device code is unchanged and never runs here), and the C-ABI host tests
(argument validation, workspace sizing, extreme shapes) run in a child
process against that build with the sanitizer runtime preloaded.  Any
out-of-bounds access, use after free or undefined arithmetic in the host code
those tests reach stops the child with a report.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "diffusion_lm_speculative_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
RUNTIME = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
# host-only sanitizer flags (each one right after -Xarch_host)
SAN_FLAGS = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-omit-frame-pointer".split()


@pytest.mark.skipif(torch.cuda.is_available(), reason="host-only check; runs where no GPU is visible")
@pytest.mark.skipif(not (os.path.exists(HIPCC) and RUNTIME), reason="hipcc or the sanitizer runtime is missing")
def test_abi_host_paths_under_asan_and_ubsan(tmp_path):
    lib = tmp_path / "libsimsd_san.so"
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", *SAN_FLAGS, "-I", os.path.join(ROOT, "include"), *srcs, "-o", str(lib)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=900)
    env = dict(os.environ, SIMSD_LIBRARY=str(lib), LD_PRELOAD=RUNTIME[-1],
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-x",
                          "-s", "-p", "no:cacheprovider", "-k", "not every_declared_symbol"],
                         env=env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out
