"""Build the HIP library libsa.so (gfx950) in-tree with hipcc.

Each source is compiled to an object for gfx950 only, then linked into
``causal_streaming_attention_amd/libsa.so``.  Packed fp32 VALU instructions
are disabled for device code (``-packed-fp32-ops``).
"""
from __future__ import annotations

import concurrent.futures
import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libsa.so")
# The source hash libsa.so was built from; the binding refuses a library whose
# hash differs from the sources beside it (a stale build).
HASH_FILE = LIB + ".srchash"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["sa_api.cpp", "sa_forward.hip", "sa_backward.hip", "sa_query.hip", "sa_static.hip"]
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# The kernels never form a NaN from finite inputs (masked scores are selected to -inf, empty rows
# are tested explicitly), so maxima need no NaN canonicalization; infinities keep their meaning.
KERNEL_FLAGS = ["-fno-honor-nans"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def source_hash() -> str:
    """Hash of everything libsa.so is built from: the sources, the headers, the C ABI header and the flags."""
    h = hashlib.sha256()
    names = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp", ".h")))
    for name in names:
        h.update(name.encode())
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    with open(os.path.join(ROOT, "include", "sa.h"), "rb") as f:
        h.update(f.read())
    h.update(" ".join(SOURCES + DEVICE_FLAGS + KERNEL_FLAGS + COMMON[:4]).encode())
    return h.hexdigest()[:16]


def _compile(src: str, out_dir: str, verbose: bool) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, *KERNEL_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and "unknown target feature" not in l.lower())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    out_dir = os.path.join(PKG, "_build")
    os.makedirs(out_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, out_dir, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", *DEVICE_FLAGS, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    with open(HASH_FILE + ".tmp", "w") as f:
        f.write(source_hash() + "\n")
    os.replace(HASH_FILE + ".tmp", HASH_FILE)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
