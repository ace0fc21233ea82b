"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/sanitize/validation_driver.cpp is compiled together with every HIP
source of the library, with both sanitizers on the host side only (each
-fsanitize= follows -Xarch_host; the gfx950 device code is built as usual),
and run on the CPU: it sweeps the workspace planners over shapes at and past
every limit and calls every entry point with invalid arguments, all of which
return before any HIP call.  Any sanitizer report or failed check fails the
test.  The executable is cached in _build/ under a digest of its sources.
"""

import hashlib
import os
import subprocess

import pytest

from lm_head_chunked_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "sanitize", "validation_driver.cpp")


def _sources():
    return [os.path.join(build.CSRC, s) for s in build.SOURCES] + [DRIVER]


def _digest():
    h = hashlib.sha256()
    for f in _sources() + [os.path.join(build.INCLUDE, "lmce.h"), os.path.join(build.CSRC, "lmce_internal.h"),
                           os.path.join(build.CSRC, "lmce_device.h")]:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


@pytest.fixture(scope="module")
def driver_exe():
    if not os.path.exists(build.hipcc()):
        pytest.skip("hipcc not available")
    out_dir = os.path.join(ROOT, "_build")
    os.makedirs(out_dir, exist_ok=True)
    exe = os.path.join(out_dir, f"validation_asan_{_digest()}")
    if not os.path.exists(exe):
        for old in os.listdir(out_dir):  # builds of older sources
            if old.startswith("validation_asan_"):
                os.remove(os.path.join(out_dir, old))
        flags = [f for f in build.flags() if f != "-fPIC"]
        cmd = [build.hipcc(), *flags, "-O1", "-g", "-fno-omit-frame-pointer",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-sanitize-recover=undefined", *_sources(), "-o", exe + ".tmp"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        os.replace(exe + ".tmp", exe)
    return exe


def test_host_code_is_clean_under_asan_and_ubsan(driver_exe):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([driver_exe], capture_output=True, text=True, env=env, timeout=300)
    report = r.stdout + r.stderr
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-3000:]
    assert r.returncode == 0, report[-3000:]
    assert "all checks passed" in r.stdout
