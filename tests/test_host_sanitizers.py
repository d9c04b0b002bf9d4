"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

1. The C ABI's host side (csrc/api.cpp: validation, workspace layout, launch
   sequence), compiled with the sanitizers on the host pass only and linked
   against recording stand-ins for the kernel launchers, driven over a grid of
   valid and invalid parameter blocks (tests/sanitize/host_driver.cpp). The
   stand-ins also check that every workspace array handed to a kernel lies
   inside the caller's buffer.
2. The CPU oracle on tiny random inputs over many shapes
   (tests/sanitize/oracle_driver.c).
No GPU is used: nothing is launched.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
OUT = os.path.join(ROOT, "_build", "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r.returncode, r.stdout, "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)


@pytest.mark.slow
def test_abi_host_code_under_asan_and_ubsan():
    if shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    os.makedirs(OUT, exist_ok=True)
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "long_context_sparse_cell_amd", "csrc")]
    # the sanitizers apply to the host pass only (each -fsanitize= right after -Xarch_host)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    common = ["hipcc", "-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer"]
    objs = []
    for src in (os.path.join(ROOT, "long_context_sparse_cell_amd", "csrc", "api.cpp"),
                os.path.join(SAN, "launch_stubs.hip"), os.path.join(SAN, "host_driver.cpp")):
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        rc, _, err = _run(common + san + inc + ["-c", src, "-o", obj])
        assert rc == 0, err
        objs.append(obj)
    exe = os.path.join(OUT, "host_driver")
    rc, _, err = _run(["hipcc", "--offload-arch=gfx950"] + san + objs + ["-o", exe])
    assert rc == 0, err
    rc, out, err = _run([exe], env=ENV, timeout=600)
    print(out)
    assert rc == 0, out + err
    assert "0 failed checks" in out
    assert "runtime error" not in err and "AddressSanitizer" not in err, err


@pytest.mark.slow
def test_oracle_under_asan_and_ubsan():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_driver")
    rc, _, err = _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-ffp-contract=off",
                       "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                       os.path.join(SAN, "oracle_driver.c"), "-o", exe, "-lm"])
    assert rc == 0, err
    rc, out, err = _run([exe], env=ENV, timeout=600)
    print(out)
    assert rc == 0, out + err
    assert "0 failures" in out
    assert "runtime error" not in err and "AddressSanitizer" not in err, err
