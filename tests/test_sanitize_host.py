"""CPU sanitizer run of the oracle and of the library's host-side logic.

tests/sanitize/driver.cpp drives the oracle (oracle/lbf_oracle.c) and every
library entry point's host checks (descriptor and argument validation, group
records, the K15H host helpers in lbf_api.cpp and lbf_host.cpp) over valid,
corrupted, truncated and random inputs, built here with AddressSanitizer and
UndefinedBehaviorSanitizer; device steps go to stand-ins that report no
device (tests/sanitize/hip_stubs.cpp).  Any sanitizer report fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_byte_split_amd", "csrc")
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _have_toolchain():
    return os.path.exists(CLANG) and os.path.exists(CLANG + "++") and os.path.isdir("/opt/rocm/include/hip")


@pytest.mark.skipif(not _have_toolchain(), reason="needs the ROCm clang and HIP headers")
def test_oracle_and_host_logic_under_asan_ubsan(tmp_path):
    inc = ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
    objs = []

    def cc(src, lang, extra):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        comp = CLANG if lang == "c" else CLANG + "++"
        std = ["-std=c11"] if lang == "c" else ["-std=c++17"]
        r = subprocess.run([comp, "-x", lang, *std, *SAN, *extra, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)

    cc(os.path.join(ROOT, "oracle", "lbf_oracle.c"), "c", [])
    for f in ("lbf_api.cpp", "lbf_host.cpp"):
        cc(os.path.join(CSRC, f), "c++", inc)
    for f in ("hip_stubs.cpp", "driver.cpp"):
        cc(os.path.join(ROOT, "tests", "sanitize", f), "c++", inc)
    exe = str(tmp_path / "sanitize_driver")
    r = subprocess.run([CLANG + "++", *SAN, *objs, "-o", exe, "-lm"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-6000:])
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-6000:]
    assert "checks clean" in r.stdout
