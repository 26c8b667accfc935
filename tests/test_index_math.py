"""Host replay of every kernel's index arithmetic (CPU only): builds
tests/index_check.cpp against the library's plan and walk helpers and runs it."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_kernel_index_math(tmp_path):
    exe = str(tmp_path / "index_check")
    subprocess.run(["/opt/rocm/bin/hipcc", "-O2", "-std=c++17",
                    "-I" + os.path.join(ROOT, "include"),
                    "-I" + os.path.join(ROOT, "place_batchnorm_activation_amd", "csrc"),
                    os.path.join(ROOT, "tests", "index_check.cpp"), "-o", exe],
                   check=True, capture_output=True)
    out = subprocess.run([exe, "300"], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("OK")
