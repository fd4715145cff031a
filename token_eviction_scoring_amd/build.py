"""Compile the gfx950 eviction-pass library in-tree: token_eviction_scoring_amd/libtri.so.

    python -m token_eviction_scoring_amd.build
"""
from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libtri.so")
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("kernels.hip", "probe.hip", "noalloc.hip", "api.cpp")]

HIPCC_FLAGS = [
    "-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared",
    "-mcode-object-version=5",
    # packed fp32 VALU forms stay out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found")
    return exe


STAMP = LIB + ".sources-sha256"   # hash of the sources the library was built from


def sources_hash() -> str:
    """SHA-256 over every source and header the library is built from (content, not modification times)."""
    h = hashlib.sha256()
    files = SOURCES + [os.path.join(HERE, "csrc", f) for f in sorted(os.listdir(os.path.join(HERE, "csrc")))
                       if f.endswith(".h")]
    files += [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))]
    files += [os.path.abspath(__file__)]
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stale() -> bool:
    """True when the library is missing or was built from other sources than the current ones."""
    if not os.path.exists(LIB) or not os.path.exists(STAMP):
        return True
    with open(STAMP) as fh:
        return fh.read().strip() != sources_hash()


def ensure_built() -> str:
    """Build the library unless it is current."""
    return build() if stale() else LIB


def build(verbose: bool = False) -> str:
    digest = sources_hash()
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
           *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    with open(STAMP, "w") as fh:
        fh.write(digest + "\n")
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
