"""No kernel of the library uses scratch memory (register spills), checked on the
compiler's per-kernel resource report (CPU only).  The build keeps the report
next to each object file and refuses spills itself; when the report of the last
build is missing or older than the sources, this test compiles the device code
again to get it."""
import concurrent.futures
import importlib.util
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    path = os.path.join(ROOT, "place_batchnorm_activation_amd", "build.py")
    spec = importlib.util.spec_from_file_location("_iabn_build_for_test", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _report(b, src: str, digest: str, tmp_path) -> str:
    path = b.remarks_path(src)
    if os.path.exists(path):
        with open(path) as fh:
            text = fh.read()
        if text.startswith("# source digest %s\n" % digest):
            return text
    cmd = ([b.HIPCC] + b.COMMON + b.DEVICE + b.REMARKS +
           ["-x", "hip", "--cuda-device-only", "-c", os.path.join(b.CSRC, src),
            "-o", str(tmp_path / (src + ".o"))])
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stderr[-4000:]
    return r.stderr


def test_no_kernel_uses_scratch(tmp_path):
    b = _build_module()
    digest = b.source_digest()
    hip = [s for s in b.SOURCES if s.endswith(".hip")]
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(hip)) as ex:
        reports = list(ex.map(lambda s: _report(b, s, digest, tmp_path), hip))
    kernels = {}
    for text in reports:
        kernels.update(b.scratch_use(text))
    assert len(kernels) > 300, "resource report covers only %d kernels" % len(kernels)
    spills = {k: v for k, v in kernels.items() if v}
    assert not spills, spills


def test_spill_detection_reads_the_report():
    """The report parser finds a kernel's scratch figure (a planted report)."""
    b = _build_module()
    text = ("x.hip:1:1: remark: Function Name: _Z1kv [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 12 [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:9:1: remark: Function Name: _Z1jv [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:9:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]\n")
    assert b.scratch_use(text) == {"_Z1kv": 12, "_Z1jv": 0}
