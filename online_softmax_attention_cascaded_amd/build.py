"""Build of the HIP library ``librf.so`` for gfx950 (MI355X), in-tree.

Compiles every ``csrc/*.hip`` file with hipcc into ``_build/`` and links them
into ``librf.so`` next to this file. ``python -m online_softmax_attention_cascaded_amd.build``
does the same from the command line.
"""

import concurrent.futures
import glob
import hashlib
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
SRC_DIR = os.path.join(PKG_DIR, "csrc")
HEADER = os.path.join(os.path.dirname(PKG_DIR), "include", "rf.h")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "librf.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # Keep the compiler from forming packed fp32 VALU ops.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def source_digest():
    """Hash of what librf.so is built from: every csrc source and header, the
    public header and the compiler flags. Compiled into the library as
    rf_build_id(); the binding refuses a library whose id differs."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(SRC_DIR, "*.hip")) + glob.glob(os.path.join(SRC_DIR, "*.hpp")))
    for f in files + [HEADER]:
        h.update(os.path.basename(f).encode() + b"\0")
        with open(f, "rb") as fh:
            h.update(fh.read())
        h.update(b"\0")
    h.update(" ".join(HIPCC_FLAGS).encode())
    return h.hexdigest()[:16]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build librf.so")
    return path


def _compile(src, digest):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, f'-DRF_BUILD_ID="{digest}"', "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose=False):
    """Compile all sources and link librf.so. Always recompiles."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(SRC_DIR, "*.hip")))
    workers = min(len(sources), max(1, min(8, os.cpu_count() or 1)))
    digest = source_digest()
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda src: _compile(src, digest), sources))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(sources)} sources")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
