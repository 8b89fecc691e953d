"""Builds the HIP library `libtf_prefill.so` for gfx950 with hipcc (in-tree).

Every source under `csrc/` is compiled to an object in `_build/` (in parallel), then
linked into `dense_transformer_prefill_amd/libtf_prefill.so`. The library links the HIP
runtime and the C/C++ runtime only.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtf_prefill.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["abi.cpp", "k_gemm.hip", "k_rows.hip", "k_attn.hip", "k_quant.hip", "k_noalloc.hip"]

# Packed-fp32 VALU instructions are disabled in device code (they are generated only
# by the compiler; disabling them keeps every fp32 op a plain VOP).
FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def source_files():
    """Every file the library is compiled from (kernels, host code, headers)."""
    inc = os.path.join(ROOT, "include")
    files = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC))
             if f.endswith((".hip", ".cpp", ".h"))]
    return files + [os.path.join(inc, f) for f in sorted(os.listdir(inc)) if f.endswith(".h")]


def sources_sha256() -> str:
    """sha256 over the library's source files (names and contents, in a fixed order)."""
    import hashlib
    h = hashlib.sha256()
    for f in source_files():
        h.update(os.path.relpath(f, ROOT).encode() + b"\0")
        h.update(open(f, "rb").read())
    return h.hexdigest()


def _git_head() -> str:
    """The repository's HEAD commit, with "+dirty" when a library source differs from it."""
    try:
        head = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True,
                              text=True, timeout=10).stdout.strip()
        dirty = subprocess.run(["git", "-C", ROOT, "status", "--porcelain", "--",
                                *[os.path.relpath(f, ROOT) for f in source_files()]],
                               capture_output=True, text=True, timeout=10).stdout.strip()
        return (head or "unknown") + ("+dirty" if dirty else "")
    except Exception:
        return "unknown"


def build(verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    info = [f'-DTF_BUILD_SOURCES="{sources_sha256()}"', f'-DTF_BUILD_GIT="{_git_head()}"']
    for s in SOURCES:
        src = os.path.join(CSRC, s)
        obj = os.path.join(BUILD, os.path.splitext(s)[0] + ".o")
        lang = ["-x", "hip"] if s.endswith(".hip") else []
        defs = info if s == "abi.cpp" else []
        cmds.append([HIPCC, *FLAGS, *extra_flags, *defs, *lang, "-c", src, "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max(1, min(len(cmds), os.cpu_count() or 1))) as ex:
        outs = list(ex.map(_run, cmds))
    if verbose:
        for c, o in zip(cmds, outs):
            print(" ".join(c))
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
