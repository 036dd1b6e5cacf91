"""The library's host code (front end: validation, FIFO pool, plans, schedule;
serving-policy simulator) built with AddressSanitizer and
UndefinedBehaviorSanitizer on the host side only (device code is compiled
as usual; each -fsanitize= follows -Xarch_host), linked into
tests/sanitize/host_driver.cpp, and run on the CPU: every check of the
driver must hold and the sanitizers must report nothing."""

import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from decode_kv_cache_kara_amd import build  # noqa: E402

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


@pytest.mark.timeout(600)
@pytest.mark.skipif(not os.path.exists(build.HIPCC), reason="hipcc not installed")
def test_host_code_under_address_and_ub_sanitizers():
    tmp = tempfile.mkdtemp(prefix="kara_san_")
    try:
        objs = []
        cmds = []
        for src in build.SOURCES:
            o = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            cmds.append([build.HIPCC] + build.FLAGS + SAN + ["-c", os.path.join(build.CSRC, src), "-o", o])
            objs.append(o)
        drv = os.path.join(tmp, "host_driver.o")
        cmds.append([build.HIPCC] + build.FLAGS + SAN +
                    ["-c", os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"), "-o", drv])
        import concurrent.futures
        with concurrent.futures.ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as pool:
            list(pool.map(build._run, cmds))
        exe = os.path.join(tmp, "host_driver")
        build._run([build.HIPCC, "--offload-arch=gfx950"] + SAN + objs + [drv] + build.LINK_LIBS + ["-o", exe])
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
        report = r.stdout + r.stderr
        assert r.returncode == 0, report[-4000:]
        assert "all checks passed" in r.stdout
        assert "ERROR: AddressSanitizer" not in report and "runtime error" not in report, report[-4000:]
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
