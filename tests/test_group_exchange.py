"""Host run of the group exchange protocol (CPU only): builds tests/group_check.cpp
against the library's own group.hpp, with one host thread per workgroup, and runs
it -- member-order sums in one- and two-level groups over many calls on one
workspace, torn and stale partials rejected, and NaN instead of a hang when a
member never publishes, with the timeout recorded in the workspace's status word."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_group_exchange_protocol(tmp_path):
    exe = str(tmp_path / "group_check")
    subprocess.run(["g++", "-O2", "-std=c++17", "-pthread", "-Wall", "-Wno-unknown-pragmas",
                    "-I" + os.path.join(ROOT, "tests", "hostshim"),
                    "-I" + os.path.join(ROOT, "place_batchnorm_activation_amd", "csrc"),
                    os.path.join(ROOT, "tests", "group_check.cpp"), "-o", exe],
                   check=True, capture_output=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.strip().endswith("OK")
