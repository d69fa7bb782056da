"""Builds libdf11.so in-tree: host encoder with g++, the gfx950 decode and
encode kernels with hipcc, linked by hipcc.  Run as ``python -m huffman_decode_block_amd.build``.

Next to the library it writes ``libdf11.so.stamp``: a hash of the sources it
was built from (every file under ``csrc/`` and ``include/``, comments and
layout excluded) and of the compile flags.  The binding refuses a library
whose stamp does not match the sources in the tree, so a forgotten rebuild
cannot make tests or measurements describe old code."""
from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdf11.so")
STAMP = LIB + ".stamp"

HOST_SOURCES = ["df11_encode.cpp", "df11_tables.cpp", "df11_capi.cpp"]
HIP_SOURCES = ["df11_decode.hip", "df11_gpu_encode.hip", "df11_reference.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
# packed-fp32 instructions are disabled for every HIP translation unit
HIP_FLAGS = ["-O3", f"--offload-arch={ARCH}", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC]
HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-pthread", "-Wall", "-Wextra", "-I", INCLUDE, "-I", CSRC]


def code_tokens(src: str) -> str:
    """The source with comments removed and whitespace runs collapsed, so that
    a change of comments alone keeps the code's identity."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if src.startswith("//", i):
            i = src.find("\n", i)
            i = n if i < 0 else i
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def _flags_without_paths(flags):
    """Compile flags minus include directories (absolute paths differ between
    checkouts of the same tree)."""
    out, skip = [], False
    for f in flags:
        if skip:
            skip = False
        elif f == "-I":
            skip = True
        else:
            out.append(f)
    return out


def source_files() -> list:
    """Every source the library is built from, relative to the repository root."""
    files = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp", ".h"))]
    files += [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h")]
    return sorted(os.path.relpath(f, ROOT) for f in files)


def source_stamp() -> str:
    """Identity of what a build of the current tree would produce: the code of
    every source file (comments and layout excluded) and the compile flags."""
    h = hashlib.sha256()
    h.update(" ".join([ARCH, *_flags_without_paths(HIP_FLAGS), "|", *_flags_without_paths(HOST_FLAGS)]).encode())
    for rel in source_files():
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(f"\n== {rel}\n".encode())
            h.update(code_tokens(f.read()).encode())
    return h.hexdigest()[:16]


def built_stamp():
    """The stamp written by the build of the library in the tree, or None."""
    try:
        with open(STAMP, encoding="utf-8") as f:
            return f.read().strip() or None
    except OSError:
        return None


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        _run(["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        _run([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    stamp = source_stamp()  # taken before compiling: an edit during the build makes it stale
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp, "-pthread"], verbose)
    os.replace(tmp, LIB)
    with open(STAMP + ".tmp", "w", encoding="utf-8") as f:
        f.write(stamp + "\n")
    os.replace(STAMP + ".tmp", STAMP)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
