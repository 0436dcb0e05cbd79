"""The C ABI's argument handling built for the host with AddressSanitizer and
UndefinedBehaviorSanitizer: gdn_api.cpp (every check the entry points make before a HIP
call) and plan.cpp (the workspace sizing) linked with recording stubs in place of the kernel
launchers (tests/abi_host/abi_check.cpp) and a C caller (tests/abi_host/abi_c_caller.c), which
may store any int in an enum.  The driver runs valid, invalid and extreme calls on every entry
point and checks the statuses and the arguments the launchers would receive.  CPU only."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_attention_token_chunked_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "abi_host")
ROCM_INCLUDE = "/opt/rocm/include"
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
INC = ["-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE, "-I", os.path.join(ROOT, "include"), "-I", CSRC]


@pytest.mark.skipif(not (shutil.which("gcc") and shutil.which("g++") and os.path.isdir(ROCM_INCLUDE)),
                    reason="needs gcc, g++ and the HIP headers")
def test_abi_checks_clean_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    c_obj = str(tmp_path / "abi_c_caller.o")
    exe = str(tmp_path / "abi_check")
    subprocess.run(["gcc", "-std=c11", *SAN, *INC, "-c", os.path.join(HOST, "abi_c_caller.c"), "-o", c_obj],
                   check=True, capture_output=True, text=True)
    subprocess.run(["g++", "-std=c++17", *SAN, *INC, os.path.join(CSRC, "gdn_api.cpp"), os.path.join(CSRC, "plan.cpp"),
                    os.path.join(HOST, "abi_check.cpp"), c_obj, "-o", exe], check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=99",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=98")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report
    assert "abi_check ok" in r.stdout and "runtime error" not in report and "AddressSanitizer" not in report, report
