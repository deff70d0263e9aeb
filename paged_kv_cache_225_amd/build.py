"""Build libpaged_kv.so for gfx950 with hipcc, in-tree next to this file.

Every .hip file (and host-only .cpp file) under csrc/ is compiled to an object in
parallel, then linked into one shared library. Packed fp32 instructions are disabled for the device code.
Run as ``python -m paged_kv_cache_225_amd.build``.

``build_host_sanitized()`` (``python -m paged_kv_cache_225_amd.build --host-sanitized``)
builds the same sources with AddressSanitizer and UndefinedBehaviorSanitizer on their host
side only (the device code is compiled as usual and never run), linked into the executable
_build/san/pkv_host_checks with the driver tests/native/host_checks.cpp, which exercises the
library's host code on the CPU. The build is skipped when the sources and flags are unchanged.
"""
from __future__ import annotations

import concurrent.futures as cf
import ctypes
import glob
import hashlib
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libpaged_kv.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = os.environ.get("PKV_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str, obj_dir: str) -> str:
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    obj_dir = os.path.join(ROOT, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir), srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    # every symbol must resolve: a kernel whose host launch stub went missing shows up here
    try:
        ctypes.CDLL(tmp, mode=os.RTLD_NOW)
    except OSError as e:
        raise RuntimeError(f"built library does not load: {e}") from e
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(srcs)} sources", flush=True)
    return LIB_PATH


# host-side sanitizers: each -fsanitize= applies to the host compilation only
SANITIZE_FLAGS = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-g",
]
SAN_DIR = os.path.join(ROOT, "_build", "san")
SAN_EXE = os.path.join(SAN_DIR, "pkv_host_checks")
SAN_DRIVER = os.path.join(ROOT, "tests", "native", "host_checks.cpp")


def build_host_sanitized(verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    srcs.append(SAN_DRIVER)
    deps = srcs + sorted(glob.glob(os.path.join(CSRC, "*.hpp"))) + [os.path.join(INCLUDE, "paged_kv.h")]
    h = hashlib.sha256(" ".join(COMMON_FLAGS + SANITIZE_FLAGS).encode())
    for d in deps:
        h.update(d.encode())
        with open(d, "rb") as f:
            h.update(f.read())
    stamp = SAN_EXE + ".sha256"
    if os.path.exists(SAN_EXE) and os.path.exists(stamp) and open(stamp).read() == h.hexdigest():
        return SAN_EXE
    os.makedirs(SAN_DIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(SAN_DIR, os.path.basename(src) + ".o")
        cmd = [hipcc(), *COMMON_FLAGS, *SANITIZE_FLAGS, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    cmd = [hipcc(), f"--offload-arch={ARCH}", *SANITIZE_FLAGS, *objs, "-o", SAN_EXE]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    with open(stamp, "w") as f:
        f.write(h.hexdigest())
    if verbose:
        print(f"built {SAN_EXE}", flush=True)
    return SAN_EXE


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv[1:]:
        build_host_sanitized(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
