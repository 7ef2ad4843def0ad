"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the CPU parts
(no GPU): the oracle (plain C, gcc) with a driver that calls every oracle
entry point, and the C ABI's host code (abi.cpp, g++, host-only, with the
HIP runtime and the kernel launchers replaced by stand-ins) with a driver
that calls every host helper and every compute entry point's validation.
Any sanitizer report aborts the program (-fno-sanitize-recover=all)."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, "%s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr)
    return r.stdout


@pytest.fixture(scope="module")
def tmp():
    d = tempfile.mkdtemp(prefix="minikv_san_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def test_oracle_under_sanitizers(tmp):
    exe = os.path.join(tmp, "oracle_driver")
    _run(["gcc", "-std=c11", "-ffp-contract=off", "-Wall"] + SAN +
         [os.path.join(ROOT, "oracle", "minikv_oracle.c"),
          os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-lm", "-o", exe], tmp)
    out = _run([exe], tmp)
    assert "ok: 0 failures" in out


def test_abi_host_code_under_sanitizers(tmp):
    exe = os.path.join(tmp, "abi_driver")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           "-D__HIP_PLATFORM_AMD__"]
    _run(["g++", "-std=c++17", "-Wall"] + SAN + inc +
         [os.path.join(ROOT, "bit_quantized_attention_two_amd", "csrc", "abi.cpp"),
          os.path.join(ROOT, "tests", "sanitize", "host_stubs.cpp"),
          os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), "-o", exe], tmp)
    out = _run([exe], tmp)
    assert "ok: 0 failures" in out
