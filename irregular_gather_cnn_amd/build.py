"""Builds libdeft.so (the gfx950 deformable convolution library) in-tree.

hipcc compiles every source under csrc/ for gfx950 (packed-fp32 instructions
disabled) and links them into irregular_gather_cnn_amd/libdeft.so.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdeft.so")
SOURCES = ["deft_sample.hip", "deft_gemm.hip", "deft_gemm_dl.hip", "deft_igemm.hip", "deft_dwconv.hip",
           "deft_dwpw.hip", "deft_backward.hip", "deft_noalloc.hip", "deft_host.cpp"]
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Wall", "-Wno-unused-result",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _hipcc() -> str:
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.isabs(c) and os.path.exists(c):
            return c
    return "hipcc"


def _compile(src: str, obj_dir: str = OBJ, extra=()) -> str:
    out = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [_hipcc()] + FLAGS + list(extra) + lang + ["-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, msgs))
    if msgs.strip():
        sys.stderr.write(msgs + "\n")
    return out


def build(lib: str = LIB, defines=()) -> str:
    """Compile all sources and link `lib` (default: the in-tree libdeft.so);
    `defines` are extra -D options.  Returns the library's path."""
    obj_dir = OBJ if not defines else OBJ + "_" + "_".join(d.replace("=", "") for d in defines)
    os.makedirs(obj_dir, exist_ok=True)
    extra = ["-D" + d for d in defines]
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda src: _compile(src, obj_dir, extra), SOURCES))
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % (r.stdout + r.stderr))
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    # python build.py [OUT.so [DEFINE ...]], e.g. a variant with the hardware
    # workgroup order: python build.py libdeft_noswizzle.so DEFT_XCD_SWIZZLE=0
    if len(sys.argv) > 1:
        print(build(os.path.abspath(sys.argv[1]), tuple(sys.argv[2:])))
    else:
        print(build())
