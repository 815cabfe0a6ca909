"""Build libyoco.so (the gfx950 HIP kernels and their C ABI) and
libyoco_ceiling.so (the achievable-bandwidth probes) in the package folder.

Run as ``python -m cross_layer_shared_amd.build`` or call ``build()``. Every
call recompiles; objects go to ``_build/`` at the repository root.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libyoco.so")
SOURCES = ["yoco_api.cpp", "compose.hip", "compose_backward.hip", "decode.hip", "decode_mfma.hip", "decode_noalloc.hip",
           "prefill.hip"]
CEILING_LIB = os.path.join(PKG, "libyoco_ceiling.so")
CEILING_SOURCES = ["ceiling.hip"]
ARCH = "gfx950"

# Packed-fp32 instructions are switched off for the device code (the target
# feature is unknown to the host pass, which only warns).
FLAGS = ["-O3", "-std=c++20", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [_hipcc(), *lang, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def _link(lib: str, objs: list[str]) -> None:
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES) + len(CEILING_SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES + CEILING_SOURCES))
    _link(LIB, objs[:len(SOURCES)])
    _link(CEILING_LIB, objs[len(SOURCES):])
    if verbose:
        print(f"built {LIB} and {CEILING_LIB}")
    return LIB


if __name__ == "__main__":
    build()
