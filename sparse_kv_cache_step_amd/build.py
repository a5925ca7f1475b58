"""Build the gfx950 HIP library libshadowkv.so in-tree with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_PATH = os.path.join(PKG, "libshadowkv.so")
SOURCES = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))
HEADERS = sorted(glob.glob(os.path.join(PKG, "csrc", "*.h"))) + [os.path.join(ROOT, "include", "shadowkv.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 instructions stay off (only the device pass knows the
    # feature; the host pass prints a harmless warning about it)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
]


OBJ_DIR = os.path.join(PKG, "_build")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile every HIP source (one hipcc process each, in parallel) and
    link them into one shared library.  With force=False the library is
    rebuilt only when a source or header is newer."""
    if not force and os.path.exists(LIB_PATH):
        t = os.path.getmtime(LIB_PATH)
        if all(os.path.getmtime(f) <= t for f in SOURCES + HEADERS):
            return LIB_PATH
    from concurrent.futures import ThreadPoolExecutor

    os.makedirs(OBJ_DIR, exist_ok=True)
    compile_flags = [f for f in FLAGS if f != "-shared"]
    objs = [os.path.join(OBJ_DIR, os.path.basename(src) + ".o") for src in SOURCES]
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        list(ex.map(lambda so: _run([HIPCC, *compile_flags, "-c", "-o", so[1], so[0]], verbose),
                    zip(SOURCES, objs)))
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-fPIC", "-shared", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(force=True, verbose=True))
