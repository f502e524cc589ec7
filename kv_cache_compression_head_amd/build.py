"""Build libkvbank.so (gfx950) in-tree with hipcc.

Each HIP translation unit is compiled to an object in ``_build/`` (in
parallel) and linked into ``kv_cache_compression_head_amd/libkvbank.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkvbank.so")
ARCH = "gfx950"

SOURCES = ["kvb_api.hip", "kvb_gram.hip", "kvb_select.hip", "kvb_forcing.hip", "kvb_attention.hip", "kvb_rope.hip",
           "kvb_sequential.hip"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    # keep the compiler from emitting packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    f"-I{os.path.join(ROOT, 'include')}",
]


def source_files():
    """Every file the library is built from: the HIP sources and headers, the
    C header, and this script (which holds the flags)."""
    files = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith((".hip", ".hpp"))]
    return files + [os.path.join(ROOT, "include", "kvbank.h"), os.path.abspath(__file__)]


def source_hash() -> str:
    """SHA-256 (hex) over the names and bytes of source_files().  The build
    embeds it in the library (kvb_source_hash), and the loader refuses a
    library whose hash differs from the sources beside it."""
    h = hashlib.sha256()
    for f in source_files():
        h.update(os.path.basename(f).encode() + b"\0")
        with open(f, "rb") as fh:
            h.update(fh.read())
        h.update(b"\0")
    return h.hexdigest()


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra=()) -> str:
    """Compile every HIP source for gfx950 and link libkvbank.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, (os.cpu_count() or 4)))
    tag = [f'-DKVB_SOURCE_HASH="{source_hash()}"']
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra) + tag), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
