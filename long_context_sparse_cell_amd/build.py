"""Compile the HIP library libfsl.so (gfx950) in place, next to this file.

Each source is compiled to an object on its own (in parallel), then linked;
every kernel is launched from the file that defines it, so no relocatable
device code is needed.
"""
import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libfsl.so")
OBJ_DIR = os.path.join(ROOT, "_build", "fsl")

# no packed fp32 instructions anywhere in device code
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def sources():
    csrc = os.path.join(HERE, "csrc")
    return sorted(glob.glob(os.path.join(csrc, "*.hip"))) + sorted(glob.glob(os.path.join(csrc, "*.cpp")))


def _filter(stderr: str) -> str:
    return "\n".join(l for l in stderr.splitlines() if "packed-fp32-ops" not in l)


def _compile(src: str, verbose: bool):
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = ["hipcc"] + DEVICE_FLAGS + ["-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(HERE, "csrc"),
                                      "-c", "-o", obj, src]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    return src, obj, r.returncode, _filter(r.stderr)


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Build libfsl.so for gfx950 with hipcc and return its path."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(os.cpu_count() or 1, 16)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, verbose), srcs))
    failed = [r for r in results if r[2] != 0]
    for src, _, rc, err in results:
        if err.strip() and (rc != 0 or verbose):
            sys.stderr.write(err + "\n")
    if failed:
        raise RuntimeError("hipcc failed on " + ", ".join(os.path.basename(r[0]) for r in failed))
    tmp = LIB + ".tmp"
    cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [r[1] for r in results]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(_filter(r.stderr) + "\n")
        raise RuntimeError("hipcc failed linking libfsl.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
