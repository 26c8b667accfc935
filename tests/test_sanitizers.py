"""Host code under AddressSanitizer, UndefinedBehaviorSanitizer and (for the
lock-free exchange protocol) ThreadSanitizer, CPU only:

  * the fp64 oracle (tests/oracle_san_check.c includes oracle/iabn_oracle.c);
  * the C ABI's host code, api.cpp, with stub launchers (tests/abi_host_check.cpp);
  * the host replay of every kernel's index arithmetic (tests/index_check.cpp);
  * the group exchange protocol with one host thread per workgroup
    (tests/group_check.cpp), also under ThreadSanitizer.

A sanitizer report aborts the program (-fno-sanitize-recover), so a clean exit
with "OK" means no report.  The HIP compiler's host pass gets the sanitizer
flags through -Xarch_host (its device pass is not sanitized)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "place_batchnorm_activation_amd", "csrc")
INC = os.path.join(ROOT, "include")
TESTS = os.path.join(ROOT, "tests")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd_build, cmd_run, timeout=300):
    b = subprocess.run(cmd_build, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-4000:]
    r = subprocess.run(cmd_run, capture_output=True, text=True, timeout=timeout, env=ENV)
    assert r.returncode == 0, (r.stdout + r.stderr)[-6000:]
    assert r.stdout.strip().splitlines()[-1].startswith("OK"), r.stdout[-2000:]
    assert "runtime error" not in r.stderr, r.stderr[-4000:]


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san_check")
    _run(["gcc", "-std=c99", "-ffp-contract=off"] + SAN +
         [os.path.join(TESTS, "oracle_san_check.c"), "-o", exe, "-lm"], [exe])


def test_c_abi_host_code_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_host_check")
    _run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + INC,
          "-I" + CSRC] + SAN +
         [os.path.join(TESTS, "abi_host_check.cpp"), os.path.join(CSRC, "api.cpp"), "-o", exe],
         [exe])


def test_index_math_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "index_check")
    host_san = []
    for f in SAN:
        host_san += ["-Xarch_host", f] if f.startswith("-fsanitize") or f.startswith(
            "-fno-sanitize") else [f]
    _run(["/opt/rocm/bin/hipcc", "-std=c++17", "-I" + INC, "-I" + CSRC] + host_san +
         [os.path.join(TESTS, "index_check.cpp"), "-o", exe], [exe, "20"], timeout=600)


@pytest.mark.parametrize("san", ["address,undefined", "thread"])
def test_group_exchange_under_sanitizers(tmp_path, san):
    exe = str(tmp_path / ("group_check_" + san.replace(",", "_")))
    flags = ["-fsanitize=" + san, "-fno-sanitize-recover=all", "-g", "-O1"]
    _run(["g++", "-std=c++17", "-pthread", "-Wno-unknown-pragmas",
          "-I" + os.path.join(TESTS, "hostshim"), "-I" + CSRC] + flags +
         [os.path.join(TESTS, "group_check.cpp"), "-o", exe], [exe], timeout=600)
