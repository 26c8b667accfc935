"""bench.py's command-line contract that needs no GPU (CPU only)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert out.returncode == 2
    assert "one GPU" in out.stderr and out.stdout == ""


def test_kernel_source_digest_tracks_every_kernel_source():
    sys.path.insert(0, ROOT)
    import inspect

    import bench
    csrc = os.path.join(ROOT, "place_batchnorm_activation_amd", "csrc")
    # every file with device code or kernel tiling (launch.hpp only declares host
    # launchers)
    kernels = {f for f in os.listdir(csrc) if f.endswith((".hip", ".hpp"))} - {"launch.hpp"}
    src = inspect.getsource(bench.kernel_source_digest)
    for f in kernels:
        assert '"%s"' % f in src, f


def test_kernel_digest_ignores_comments_but_not_code():
    sys.path.insert(0, ROOT)
    import bench
    a = 'int f(int x) { return x + 1; }  // one\n/* two */ const char* s = "// kept";\n'
    b = '// another comment\nint f(int x) {\n    return x + 1;   /* changed */\n}\nconst char* s = "// kept";'
    c = 'int f(int x) { return x + 2; }\nconst char* s = "// kept";'
    d = 'int f(int x) { return x + 1; }\nconst char* s = "// changed";'
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)
    assert bench._code_only(a) != bench._code_only(d)
