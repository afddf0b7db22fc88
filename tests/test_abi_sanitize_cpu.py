"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every translation unit of the library is compiled as shipped (for gfx950),
with the sanitizers on the host code only, linked with
``tests/abi_sanitize_driver.cpp``, and run here; the argument checks and plan
arithmetic are exactly the shipped ones.  The
driver makes only calls that validation must reject, and pure queries
(workspace sizes, plans) over the whole accepted domain; it refuses to run
where a GPU is visible.  A sanitizer report or a wrong status fails the test.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from backward_rmsnorm_fwd_amd import build as lib_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "abi_sanitize_driver.cpp")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]

pytestmark = pytest.mark.skipif(not os.path.exists(lib_build.hipcc()) and
                                shutil.which("hipcc") is None, reason="hipcc not found")


def _compile(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    return res.returncode, cmd, res.stdout + res.stderr


def test_host_validation_under_sanitizers(tmp_path):
    hipcc = lib_build.hipcc()
    inc = ["-I", os.path.join(ROOT, "include")]
    common = [f"--offload-arch={lib_build.ARCH}", "-O1", "-g", "-std=c++17", *SAN, *inc]
    objs, cmds = [], []
    for src, defs, name in lib_build.UNITS + [(DRIVER, [], "driver.o")]:
        obj = str(tmp_path / name)
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmds.append([hipcc, *common, *lang, *defs, "-c", src, "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        for rc, cmd, out in ex.map(_compile, cmds):
            assert rc == 0, f"{' '.join(cmd)}\n{out}"
    exe = str(tmp_path / "abi_sanitize")
    rc, cmd, out = _compile([hipcc, f"--offload-arch={lib_build.ARCH}", *SAN, *objs, "-o", exe])
    assert rc == 0, out
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = res.stdout + res.stderr
    if res.returncode == 77:
        pytest.skip(out.strip())
    assert res.returncode == 0, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
    assert ", 0 failures" in out, out
