"""Build libgdn.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Usage: python -m gated_deltanet_state_gdn_amd.build  (or call build()).
Each source compiles to its own object in _build/ (in parallel), then hipcc
links the shared library next to this file.  Packed-fp32 instruction
selection is disabled for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgdn.so")
SOURCES = ["gdn_api.cpp", "gdn_decode.hip", "gdn_spec.hip", "gdn_copy.hip", "gdn_mamba2.hip", "gdn_replay.hip", "gdn_prefill.hip"]
ARCH = os.environ.get("GDN_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-x", "hip",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    return r.stdout


def build(verbose: bool = False, defines=(), lib_path: str = LIB, build_dir: str = BUILD) -> str:
    """Compile every source and link ``lib_path``; ``defines`` are extra -D tuning macros."""
    os.makedirs(build_dir, exist_ok=True)
    objs = []
    cmds = []
    dflags = [f"-D{d}" for d in defines]
    for src in SOURCES:
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, *dflags, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 4)) as ex:
        outs = list(ex.map(_run, cmds))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = lib_path + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
