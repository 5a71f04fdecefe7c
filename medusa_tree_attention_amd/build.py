"""Build libmedusa.so in-tree: host C++ tree compiler + HIP kernels for gfx950."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmedusa.so")
INCLUDE = os.path.join(ROOT, "include")

HIP_SOURCES = ["attn.hip", "attn_mfma.hip", "attn_noalloc.hip", "accept.hip", "compact.hip", "heads.hip",
               "probe.hip"]
CPP_SOURCES = ["tree_compile.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-I", INCLUDE, "-I", CSRC,
    # packed fp32 instructions stay off (hipcc's host pass warns about the feature name)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# weights of the greedy tree must be plain binary64 products
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-ffp-contract=off", "-I", INCLUDE,
             "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__"]


def _run(cmds):
    procs = [(c, subprocess.Popen(c, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)) for c in cmds]
    failed = []
    for cmd, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        if p.returncode != 0:
            failed.append((cmd, out))
        elif "error" in out.lower():
            sys.stderr.write(out)
    if failed:
        for cmd, out in failed:
            sys.stderr.write(" ".join(cmd) + "\n" + out + "\n")
        raise RuntimeError("libmedusa build failed")


def build(verbose: bool = True) -> str:
    """Compile every source and link ``libmedusa.so``; always recompiles."""
    os.makedirs(BUILD, exist_ok=True)
    objs, cmds = [], []
    for src in CPP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmds.append(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmds.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    if verbose:
        print(f"[build] compiling {len(cmds)} sources for gfx950", flush=True)
    _run(cmds)
    tmp = LIB + ".tmp"
    _run([[HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]])
    shutil.move(tmp, LIB)
    if verbose:
        print(f"[build] wrote {LIB}", flush=True)
    return LIB


HOST_SANITIZED = os.path.join(BUILD, "libmedusa_host_sanitized.so")


def build_host_sanitized(verbose: bool = True) -> str:
    """The host C++ (tree compile and node budget) alone, built with AddressSanitizer and
    UndefinedBehaviorSanitizer into a CPU-only library for the host tests.  It is loaded
    with the ASan runtime preloaded; it exports only the host entry points."""
    os.makedirs(BUILD, exist_ok=True)
    tmp = HOST_SANITIZED + ".tmp"
    _run([["g++", "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-Wall", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-I", INCLUDE, *[os.path.join(CSRC, src) for src in CPP_SOURCES], "-o", tmp]])
    shutil.move(tmp, HOST_SANITIZED)
    if verbose:
        print(f"[build] wrote {HOST_SANITIZED}", flush=True)
    return HOST_SANITIZED


if __name__ == "__main__":
    if sys.argv[1:] == ["host-sanitized"]:
        build_host_sanitized()
    else:
        build()
