"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): every source of the library is compiled with the sanitizers on
its host side only (device code as usual), linked into a driver that calls
each entry point on the paths that refuse or answer before any device work
(tests/sanitize/abi_host_check.cpp), and run; any sanitizer report fails."""
import glob
import os
import shutil
import subprocess

import pytest

from tests.helpers import ROOT

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def test_abi_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    srcs = sorted(glob.glob(os.path.join(ROOT, "grouped_gemm_02_amd", "csrc", "*.hip")))
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    objs = []
    procs = []
    for src in srcs:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        procs.append(subprocess.Popen([HIPCC, *flags, *SAN, "-c", src, "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
        objs.append(obj)
    for p in procs:
        out, _ = p.communicate(timeout=900)
        assert p.returncode == 0, out[-3000:]
    driver = os.path.join(ROOT, "tests", "sanitize", "abi_host_check.cpp")
    dobj = str(tmp_path / "abi_host_check.o")
    r = subprocess.run([HIPCC, *flags, *SAN, "-c", driver, "-o", dobj], capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    exe = str(tmp_path / "abi_host_check")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN, dobj, *objs, "-o", exe], capture_output=True,
                       text=True, timeout=900)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "abi host checks passed" in out, out[-3000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-3000:]
