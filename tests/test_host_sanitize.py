"""Host AddressSanitizer / UndefinedBehaviorSanitizer run of the C-ABI layer
(abi.cpp) and the pack-table builders (pack_tables.cpp).

The device launchers are replaced by host stubs that count their calls
(tests/host_sanitize/stubs.cpp); tests/host_sanitize/driver.cpp fuzzes every
entry point with boundary arguments and checks that a rejected call launches
nothing, that explicit valid calls reach their launcher, and that the table
builders fill buffers of exactly the reported size.  Any invalid memory
access or undefined arithmetic aborts the run (-fno-sanitize-recover)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "packed_attention_amd", "csrc")
HS = os.path.join(ROOT, "tests", "host_sanitize")
ROCM = "/opt/rocm"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(os.path.join(ROCM, "include", "hip")),
                    reason="needs g++ and the HIP headers")
def test_abi_and_pack_tables_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", os.path.join(ROCM, "include"),
           os.path.join(CSRC, "abi.cpp"), os.path.join(CSRC, "pack_tables.cpp"),
           os.path.join(HS, "stubs.cpp"), os.path.join(HS, "driver.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe]
    b = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    assert b.returncode == 0, b.stdout[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("MF_DEBUG", None)
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600, env=env)
    out = r.stdout
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert "0 failure(s)" in out, out[-2000:]
