"""The C ABI's host code (kvq_host.cpp) built with AddressSanitizer and UndefinedBehaviorSanitizer and driven by
tests/host_sanitize/abi_driver.cpp, with the kernel launchers replaced by stubs (launch_stubs.cpp) so that every
host path (validation, size and region arithmetic, split planning, workspace checks, error returns) runs without
a GPU. The sanitizer flags apply to host code only (each -fsanitize= behind -Xarch_host). CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_decode_attention_append_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_sanitize")
HIPCC = "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]
FLAGS = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "--offload-arch=gfx950",
         "-Wno-unused-command-line-argument",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


def test_host_code_under_asan_and_ubsan(tmp_path):
    objs = []
    for src in (os.path.join(CSRC, "kvq_host.cpp"), os.path.join(HERE, "launch_stubs.cpp"),
                os.path.join(HERE, "abi_driver.cpp")):
        obj = str(tmp_path / (os.path.splitext(os.path.basename(src))[0] + ".o"))
        _run([HIPCC, *FLAGS, *SAN, "-c", src, "-o", obj])
        objs.append(obj)
    exe = str(tmp_path / "abi_driver")
    _run([HIPCC, *SAN, *objs, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-6000:]
    assert "runtime error" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert "0 failed checks" in r.stdout
