"""Build of the HIP library ``libmoe.so`` for gfx950 (hipcc, in-tree).

Each ``csrc/*.hip`` file is compiled to an object in parallel, then linked
into ``sparse_moe_layer_wg_amd/libmoe.so``.  Beside it, ``libmoe.so.srcsha``
records a digest of every source the library is built from (and of the
compiler flags), so that a library older than its sources is never loaded.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import hashlib
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
STAMP = LIB + ".srcsha"
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    # keep the compiler from emitting packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def sources(csrc: str = CSRC, include: str = INCLUDE) -> list:
    """Every file the library is built from: csrc/*.hip, csrc/*.h, include/*.h."""
    return sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.h")) +
                  glob.glob(os.path.join(include, "*.h")))


def source_digest(paths=None) -> str:
    """sha256 over the sources' names and contents and the compiler flags."""
    h = hashlib.sha256(" ".join(HIPCC_FLAGS[:-4]).encode())
    for path in (sources() if paths is None else paths):
        h.update(os.path.basename(path).encode() + b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
        h.update(b"\0")
    return h.hexdigest()


def is_current(lib: str = LIB, stamp: str = STAMP, paths=None) -> bool:
    """True when `lib` exists and was built from the sources as they are now."""
    if not (os.path.exists(lib) and os.path.exists(stamp)):
        return False
    with open(stamp) as f:
        return f.read().strip() == source_digest(paths)


def _hipcc() -> str:
    for cand in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.sep not in cand or os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    digest = source_digest()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    hipcc = _hipcc()

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        cmd = [hipcc, *HIPCC_FLAGS, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        if verbose:
            print(" ".join(cmd))
        return obj, r.stderr

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(compile_one, srcs))
    objs = [o for o, _ in results]
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    with open(STAMP + ".tmp", "w") as f:
        f.write(digest + "\n")
    os.replace(STAMP + ".tmp", STAMP)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
