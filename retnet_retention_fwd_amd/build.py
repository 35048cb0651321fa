"""Build libretention_fwd.so in-tree with hipcc for gfx950.

    python -m retnet_retention_fwd_amd.build          # build (always recompiles)

The library is written next to this file so it travels with the source tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB_NAME = "libretention_fwd.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

SOURCES = ["api.cpp", "profile.cpp", "backward.cpp", "generic_chunk.hip", "decode.hip", "mfma_chunk.hip", "chunk64.hip", "calib.hip",
           "bwd_kernels.hip", "msr.hip"]

# Packed-fp32 instructions are disabled for all device code (the compiler would
# otherwise form v_pk_* fp32 ops from ordinary float code).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the retention library)")


def objects_cmds(tmp: str):
    cmds = []
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(tmp, src + ".o")
        cmd = [hipcc(), "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-I", INCLUDE, "-I", CSRC,
               "-Wall", "-Wno-unused-function", "-c", path, "-o", obj]
        if src.endswith(".hip"):
            cmd[1:1] = ["-x", "hip"]
            cmd += DEVICE_FLAGS
        cmds.append(cmd)
        objs.append(obj)
    return cmds, objs


def build(verbose: bool = True) -> str:
    """Compile every source and link the shared library; returns its path."""
    with tempfile.TemporaryDirectory(prefix="retn_build_") as tmp:
        cmds, objs = objects_cmds(tmp)
        procs = []
        for cmd in cmds:
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        failed = False
        for cmd, p in procs:
            out, _ = p.communicate()
            text = out.decode(errors="replace")
            # hipcc's host pass does not know the device-only feature flag; that note is harmless
            lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
            if lines and verbose:
                print("\n".join(lines), flush=True)
            if p.returncode != 0:
                failed = True
                print(f"FAILED: {' '.join(cmd)}", file=sys.stderr, flush=True)
        if failed:
            raise RuntimeError("building the retention library failed")
        tmp_lib = os.path.join(tmp, LIB_NAME)
        link = [hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp_lib] + objs
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.run(link, check=True)
        shutil.copyfile(tmp_lib, LIB_PATH + ".tmp")
        os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build())
