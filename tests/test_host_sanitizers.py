"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

The library's sources are compiled with the sanitizers on the host code only
(device code for gfx950 as usual), linked with tests/host/sanitize_driver.cpp,
and the driver runs every entry point's validation layer on invalid, extreme
and boundary arguments: calls that are rejected (or answered, for the
workspace-size queries) before any device work, so no GPU is needed.  A
sanitizer report or a wrong status fails the test."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from sparse_attention_08_amd import _build  # noqa: E402

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]


def test_validation_layer_under_sanitizers(tmp_path):
    try:
        cc = _build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    clang = os.path.join(os.path.dirname(os.path.realpath(cc)), "..", "lib", "llvm", "bin", "clang++")
    if not os.path.exists(clang):
        clang = "/opt/rocm/lib/llvm/bin/clang++"
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={_build.ARCH}",
             f"-I{_build.INCLUDE}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    objs, jobs = [], []
    for s in _build.SOURCES:
        o = str(tmp_path / s.replace(".hip", ".o"))
        objs.append(o)
        jobs.append([cc, *flags, *SAN, "-c", os.path.join(_build.CSRC, s), "-o", o])
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4)) as ex:
        for p in ex.map(lambda c: subprocess.run(c, capture_output=True, text=True), jobs):
            assert p.returncode == 0, p.stderr[-3000:]
    drv_o = str(tmp_path / "drv.o")
    p = subprocess.run([clang, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=all", f"-I{_build.INCLUDE}", "-c",
                        os.path.join(ROOT, "tests", "host", "sanitize_driver.cpp"), "-o", drv_o],
                       capture_output=True, text=True)
    assert p.returncode == 0, p.stderr[-3000:]
    exe = str(tmp_path / "drv")
    p = subprocess.run([cc, f"--offload-arch={_build.ARCH}", *SAN, drv_o, *objs, "-o", exe],
                       capture_output=True, text=True)
    assert p.returncode == 0, p.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    p = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert p.returncode == 0 and "OK (0 failures)" in p.stdout, p.stdout[-3000:] + p.stderr[-3000:]
