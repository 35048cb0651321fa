"""Build libretention_fwd.so in-tree with hipcc for gfx950.

    python -m retnet_retention_fwd_amd.build          # build (always recompiles)
    python -m retnet_retention_fwd_amd.build --host-sanitize   # ASan/UBSan host copy (temporary dir)

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

SOURCES = ["api.cpp", "profile.cpp", "backward.cpp", "generic_chunk.hip", "decode.hip", "mfma_chunk.hip", "chunk64.hip", "chunkw.hip", "calib.hip", "noalloc.hip",
           "bwd_kernels.hip", "msr.hip"]

# Packed-fp32 instructions are disabled for all device code (the compiler would
# otherwise form v_pk_* fp32 ops from ordinary float code).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the retention library)")


# Host-only AddressSanitizer and UndefinedBehaviorSanitizer (device code is built as
# usual): every -fsanitize= follows -Xarch_host, so no GPU code is instrumented.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
SANITIZED_LIB_NAME = "libretention_fwd_hostsan.so"


def objects_cmds(tmp: str, sanitize: bool = False):
    cmds = []
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(tmp, src + ".o")
        cmd = [hipcc(), "-O1" if sanitize else "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-I",
               INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function", "-c", path, "-o", obj]
        if src.endswith(".hip"):
            cmd[1:1] = ["-x", "hip"]
            cmd += DEVICE_FLAGS
        if sanitize:
            cmd += HOST_SANITIZE
        cmds.append(cmd)
        objs.append(obj)
    return cmds, objs


def build(verbose: bool = True, sanitize: bool = False, out_dir: str = HERE) -> str:
    """Compile every source and link the shared library into out_dir; returns its path.
    sanitize: build a host-sanitized copy (SANITIZED_LIB_NAME) for the validation tests
    instead; it needs the sanitizer runtime preloaded to load."""
    lib_name = SANITIZED_LIB_NAME if sanitize else LIB_NAME
    lib_path = os.path.join(out_dir, lib_name)
    with tempfile.TemporaryDirectory(prefix="retn_build_") as tmp:
        cmds, objs = objects_cmds(tmp, sanitize)
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
        tmp_lib = os.path.join(tmp, lib_name)
        link = [hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp_lib] + objs
        if sanitize:
            # the objects already carry their device code: the host compiler links them
            # with the HIP runtime and the host sanitizer runtimes
            rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
            link = [os.path.join(rocm, "llvm", "bin", "clang++"), "-shared", "-fPIC", "-o", tmp_lib] + objs + [
                "-L" + os.path.join(rocm, "lib"), "-Wl,-rpath," + os.path.join(rocm, "lib"), "-lamdhip64",
                "-fsanitize=address,undefined", "-shared-libsan"]
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.run(link, check=True)
        shutil.copyfile(tmp_lib, lib_path + ".tmp")
        os.replace(lib_path + ".tmp", lib_path)
    return lib_path


def sanitizer_runtime() -> str:
    """Path of the ROCm clang's shared AddressSanitizer runtime (to preload), or ''."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    clang = os.path.join(rocm, "llvm", "bin", "clang++")
    try:
        out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                             text=True, check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return ""
    return out if os.path.isabs(out) and os.path.exists(out) else ""


if __name__ == "__main__":
    if "--host-sanitize" in sys.argv[1:]:
        print(build(sanitize=True, out_dir=tempfile.mkdtemp(prefix="retn_hostsan_")))
    else:
        print(build())
