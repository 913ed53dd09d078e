"""The C ABI layer (api.cpp, codebook.cpp, profile.cpp) built with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer against host-only stand-ins
of the HIP runtime and the kernel launchers (tests/sanitize/stubs.cpp), then
driven through every entry point with invalid and valid arguments
(tests/sanitize/reject.c). Needs no GPU; any sanitizer report fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_nf4_quantized_03_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
HIP = ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"]


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None, reason="no host compiler")
def test_abi_rejections_under_asan_ubsan(tmp_path):
    objs = []
    for name in ("api", "codebook", "profile"):
        o = str(tmp_path / f"{name}.o")
        _run(["g++", "-std=c++17", "-Wall", "-Werror"] + HIP + FLAGS + ["-c", os.path.join(CSRC, f"{name}.cpp"), "-o", o],
             tmp_path)
        objs.append(o)
    o = str(tmp_path / "stubs.o")
    _run(["g++", "-std=c++17"] + HIP + FLAGS + ["-c", os.path.join(SAN, "stubs.cpp"), "-o", o], tmp_path)
    objs.append(o)
    o = str(tmp_path / "reject.o")
    _run(["gcc", "-std=c11", "-Wall", "-Werror"] + FLAGS + ["-c", os.path.join(SAN, "reject.c"), "-o", o], tmp_path)
    exe = str(tmp_path / "reject")
    _run(["g++"] + FLAGS + [o] + objs + ["-o", exe], tmp_path)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and "reject: ok" in r.stdout, r.stdout[-4000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
