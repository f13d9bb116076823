"""Build libattn.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m attention_flash_attn_03_amd._build

Each csrc/*.hip file is compiled to an object in _build/ (in parallel), then
linked into attention_flash_attn_03_amd/libattn.so.  Always rebuilds.  The
library carries the SHA-256 of the sources it was built from
(attn_source_sha256), which the loader compares with the sources beside it.
"""
from __future__ import annotations

import glob
import hashlib
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
HEADER = os.path.join(os.path.dirname(PKG), "include", "attn.h")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# per-file additions: the narrow prefill kernel keeps its MFMA accumulators in
# ordinary VGPRs, so its 256 registers per wave form one pool
EXTRA_FLAGS = {"narrow.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def source_files() -> list:
    """Every file libattn.so is compiled from: the HIP sources, their headers and the C ABI header."""
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h"))) + [HEADER]


def source_digest() -> str:
    """SHA-256 over the names and contents of source_files()."""
    h = hashlib.sha256()
    for path in source_files():
        h.update(os.path.basename(path).encode() + b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _compile(src: str, digest: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *EXTRA_FLAGS.get(os.path.basename(src), []), '-DATTN_SOURCE_SHA256="%s"' % digest,
           "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, msgs))
    if msgs.strip():
        sys.stderr.write(msgs + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    digest = source_digest()
    with ThreadPoolExecutor(max(1, min(len(sources), os.cpu_count() or 1))) as ex:
        objs = list(ex.map(lambda src: _compile(src, digest), sources))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()
