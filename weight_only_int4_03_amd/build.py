"""Build the HIP library libw4a16.so for gfx950 (run: python -m weight_only_int4_03_amd.build).

Every source under csrc/ is compiled by hipcc in parallel, then linked into
one shared library next to this file.  Packed-FP32 VALU instructions are
disabled for the device code (-packed-fp32-ops).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "libw4a16.so")
BUILD_DIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-munsafe-fp-atomics",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _headers_mtime() -> float:
    hs = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    hs.append(os.path.join(INCLUDE, "w4a16.h"))
    return max(os.path.getmtime(h) for h in hs)


def _compile(src: str, incremental: bool = False) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    if incremental and os.path.exists(obj) and os.path.getmtime(obj) > max(
            os.path.getmtime(src), _headers_mtime()):
        return obj
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
    return obj


def build(verbose: bool = False, incremental: bool = False) -> str:
    """Compile every source (incremental: only those newer than their object
    file, for development) and link the library."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, incremental), srcs))
    tmp = LIBRARY + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, LIBRARY)
    if verbose:
        print("built", LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    build(verbose=True, incremental="--incremental" in sys.argv)
    sys.exit(0)
